"""Host-side calibration of the clip ratios: per (layer, KV head, K or V), the ratio on the
grid 0.50, 0.51, ..., 1.00 whose uniform INT2 demotion reconstructs the calibration rows with
the least squared error in the rotated basis (the smallest ratio on a tie).

Source: the paper's abstract and the QbitAI article on OSCAR: the clipping thresholds are
estimated offline on calibration data and then fixed per layer. The criterion is not given
there; the least-squares reconstruction error is this library's reading. The demotion it
scores is the library's: y = x R, hi = c max y, lo = c min y, s = fp16((hi - lo) / 3),
z = fp16(lo), codes = clamp(round_half_even((y - z) / s), 0, 3), dequantised to z + code s.
"""

from __future__ import annotations

import numpy as np

from .extremes import rotate

GRID = np.round(np.arange(50, 101) / 100.0, 2)


def errors(rows, rot, grid=GRID) -> np.ndarray:
    """Squared reconstruction error of rows [N, 128] under rotation rot for each clip ratio
    (the scale and zero point from the rows' exact extremes, as the demotion kernels take
    them)."""
    y, ymax, ymin = rotate(rows, rot)
    out = np.empty(len(grid))
    for i, c in enumerate(grid):
        c32 = float(np.float32(c))
        hi, lo = c32 * ymax, c32 * ymin
        s = ((hi - lo) / 3.0).astype(np.float16).astype(np.float64)
        z = lo.astype(np.float16).astype(np.float64)
        safe = np.where(s > 0, s, 1.0)
        codes = np.where(s[:, None] > 0, np.clip(np.rint((y - z[:, None]) / safe[:, None]), 0, 3), 0)
        out[i] = float(np.sum((y - (z[:, None] + codes * s[:, None])) ** 2))
    return out


def best_clip(rows, rot, grid=GRID) -> float:
    """The clip ratio of least reconstruction error (the first on a tie)."""
    e = errors(rows, rot, grid)
    return float(grid[int(np.argmin(e))])


def layer_clips(calib_sets, rot_k_bits, rot_v_bits):
    """Per KV head, (clip_k, clip_v) float32 [Hkv] from each head's calibration keys and
    values (q, k, v) under its rotations (bf16 bits)."""
    def bf16(bits):
        return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)

    rk = bf16(rot_k_bits).reshape(-1, 128, 128)
    rv = bf16(rot_v_bits).reshape(-1, 128, 128)
    ck = [best_clip(k, rk[kv]) for kv, (_, k, _) in enumerate(calib_sets)]
    cv = [best_clip(v, rv[kv]) for kv, (_, _, v) in enumerate(calib_sets)]
    return np.array(ck, np.float32), np.array(cv, np.float32)
