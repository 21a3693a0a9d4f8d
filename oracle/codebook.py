"""Oracle: the Lloyd-Max codebook variant of the INT2 demotion and its dequantisation.

Test infrastructure only: nothing outside tests/, the smoke check and the CPU baseline of
the benchmark may import this package.

Source: the QbitAI article on OSCAR, section comparing OSCAR with TurboQuant: the code
repository combines the attention-aware rotation with a stronger Lloyd-Max codebook in
place of the uniform INT2 levels. The article gives nothing beyond that name; the
readings below are this library's.

Readings:
  * one codebook per (layer, KV head, K or V): four levels l_0 <= l_1 <= l_2 <= l_3 in
    units of the group's scale above its zero point, so a code c dequantises to
    z16 + s16 l_c; the uniform INT2 levels are (0, 1, 2, 3). Scale and zero point are
    those of the uniform scheme (clip ratio, s = (hi - lo) / 3, fp16 each), so a row's
    range is the same with or without the codebook;
  * the levels are multiples of 1/16 in [0, 3], held as integers k = 16 l in [0, 48];
  * code = the nearest level to t = fl64(fl64(y - z16) / s16); at the midpoint of two
    levels the even index wins (for the uniform levels this is round half to even and
    the clamp to [0, 3]); every code is 0 when s16 == 0;
  * the codebook is fitted offline by the Lloyd-Max iteration (S. P. Lloyd, "Least squares
    quantization in PCM"; J. Max, "Quantizing for minimum distortion", 1960) on samples of
    t from calibration rows, starting from the uniform levels: cells are bounded by the
    midpoints of neighbouring levels, and each level moves to the mean of its cell (a
    level whose cell is empty stays). The fitted levels are then rounded to sixteenths,
    clamped to [0, 48] and made strictly increasing.
"""

from __future__ import annotations

import numpy as np

from . import quant

UNIFORM16 = np.array([0, 16, 32, 48])


def lloyd_max(samples, levels, iters: int = 200, tol: float = 0.0):
    """Lloyd-Max iteration in fp64. Returns (levels, mse_history): the levels after the
    last iteration and the mean squared error of the nearest-level quantiser before each
    iteration and after the last."""
    x = np.sort(np.asarray(samples, np.float64).ravel())
    lv = np.array(levels, np.float64)
    history = []
    for _ in range(iters):
        edges = (lv[:-1] + lv[1:]) / 2.0
        cell = np.searchsorted(edges, x, side="left")  # x == edge goes to the lower cell
        history.append(float(np.mean((x - lv[cell]) ** 2)))
        new = lv.copy()
        for j in range(len(lv)):
            members = x[cell == j]
            if members.size:
                new[j] = members.mean()
        moved = np.max(np.abs(new - lv))
        lv = new
        if moved <= tol:
            break
    edges = (lv[:-1] + lv[1:]) / 2.0
    cell = np.searchsorted(edges, x, side="left")
    history.append(float(np.mean((x - lv[cell]) ** 2)))
    return lv, history


def sixteenths(levels) -> np.ndarray:
    """Levels (units of the scale) as integers k = 16 l: nearest, clamped to [0, 48],
    then made strictly increasing (each at least one above the previous, counting up
    from the bottom, then each at most one below the next, counting down from the top)."""
    k = np.clip(np.rint(np.asarray(levels, np.float64) * 16.0), 0, 48).astype(np.int64)
    for j in range(1, len(k)):
        k[j] = max(k[j], k[j - 1] + 1)
    k[-1] = min(k[-1], 48)
    for j in range(len(k) - 2, -1, -1):
        k[j] = min(k[j], k[j + 1] - 1)
    return k


def thresholds(k16) -> np.ndarray:
    """Midpoints between neighbouring levels, in units of the scale (exact in fp64)."""
    k = np.asarray(k16, np.float64)
    return (k[:-1] + k[1:]) / 32.0


def codes_from_t(t, k16) -> np.ndarray:
    """Nearest level to t, the even index at a midpoint."""
    th = thresholds(k16)
    t = np.asarray(t, np.float64)
    return ((t > th[0]).astype(np.int64) + (t >= th[1]) + (t > th[2])).astype(np.uint8)


def boundary_distance(t, k16) -> np.ndarray:
    """Distance from t to the nearest midpoint between levels."""
    th = thresholds(k16)
    t = np.asarray(t, np.float64)
    return np.min(np.abs(t[..., None] - th), axis=-1)


def quantize_rows(x, r, clip: float, k16):
    """Demote rows x [N, 128] with rotation r and clip ratio `clip` (as quant.quantize_rows)
    against the codebook k16 (four sixteenths). The scale and zero point are those of
    quant.quantize_rows; only the code decisions differ. Returns (codes, s16, z16, margin),
    margin being the distance of t to the nearest midpoint (inf where s16 == 0)."""
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    _, s16, z16, _ = quant.quantize_rows(x, r, clip)
    rt = np.ascontiguousarray(r.T)
    y, bound = quant.rotate_with_bound(x, r)
    s64 = s16.astype(np.float64)[:, None]
    z64 = z16.astype(np.float64)[:, None]
    zero_scale = s64 == 0.0
    safe_s = np.where(zero_scale, 1.0, s64)
    t = (y - z64) / safe_s
    # a t within reach of a midpoint is recomputed from the correctly rounded dot product
    near = (boundary_distance(t, k16) <= bound / safe_s * 4.0 + 1e-12) & ~zero_scale
    ii, jj = np.nonzero(near)
    t[ii, jj] = (quant.exact_dots(x, rt, ii, jj) - z64[ii, 0]) / safe_s[ii, 0]
    codes = np.where(zero_scale, 0, codes_from_t(t, k16)).astype(np.uint8)
    margin = np.where(zero_scale, np.inf, boundary_distance(t, k16))
    return codes, s16, z16, margin


def dequantize(codes, s16, z16, k16) -> np.ndarray:
    """z16 + s16 k[c] / 16 per row, fp64 (rotated basis)."""
    lv = np.asarray(k16, np.float64) / 16.0
    s = np.asarray(s16, dtype=np.float64)[..., None]
    z = np.asarray(z16, dtype=np.float64)[..., None]
    return lv[np.asarray(codes, np.int64)] * s + z


def normalized_values(x, r, clip: float) -> np.ndarray:
    """Calibration samples t = (y - z16) / s16 of rows x (rows with s16 == 0 dropped)."""
    x = np.asarray(x, dtype=np.float64)
    _, s16, z16, _ = quant.quantize_rows(x, np.asarray(r, np.float64), clip)
    y = x @ np.asarray(r, np.float64)
    s = s16.astype(np.float64)
    keep = s > 0
    return ((y[keep] - z16.astype(np.float64)[keep, None]) / s[keep, None]).ravel()


def fit(x, r, clip: float, iters: int = 200) -> np.ndarray:
    """The codebook (sixteenths) of calibration rows x: Lloyd-Max from the uniform levels."""
    lv, _ = lloyd_max(normalized_values(x, r, clip), UNIFORM16 / 16.0, iters=iters)
    return sixteenths(lv)
