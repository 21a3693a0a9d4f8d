"""Host-side calibration of the Lloyd-Max codebook variant: the four levels per (KV head,
K or V) that oscar_*_codebook read, fitted offline on calibration rows.

Source: the QbitAI article on OSCAR, section comparing OSCAR with TurboQuant: the code
release pairs the attention-aware rotation with a Lloyd-Max codebook in place of the
uniform INT2 levels, and rotations and clipping thresholds are calibrated offline. The
article gives only the name; the format is this library's: levels in sixteenths of the
group's scale above its zero point, k in [0, 48], strictly increasing (uniform INT2 is
0, 16, 32, 48).

The fit is the Lloyd-Max iteration (S. P. Lloyd, "Least squares quantization in PCM";
J. Max, "Quantizing for minimum distortion", 1960) on the normalised values
t = (y - z) / s of the calibration rows, y = x R, with the uniform scheme's scale and zero
point, started from the uniform levels: each level moves to the mean of the samples
nearer to it than to its neighbours (a sample on a midpoint counts for the lower cell; a
level with no samples stays), until no level moves. The result is rounded to sixteenths,
clamped to [0, 48] and made strictly increasing. Sample cell means come from prefix sums
over the sorted samples, so one iteration costs four binary searches.
"""

from __future__ import annotations

import numpy as np

from .extremes import rotate

UNIFORM = (0, 16, 32, 48)


def normalized_samples(rows, rot, clip: float) -> np.ndarray:
    """t = (y - z16) / s16 for every value of calibration rows [N, 128] (bf16 values) rotated by
    rot [128, 128]; rows whose fp16 scale is zero are dropped. The scale and zero point come
    from the rows' exact extremes, as the demotion kernels take them."""
    y, ymax, ymin = rotate(rows, rot)
    c = float(np.float32(clip))
    hi = c * ymax
    lo = c * ymin
    s = ((hi - lo) / 3.0).astype(np.float16).astype(np.float64)
    z = lo.astype(np.float16).astype(np.float64)
    keep = s > 0
    return ((y[keep] - z[keep, None]) / s[keep, None]).ravel()


def lloyd_max(samples, start=(0.0, 1.0, 2.0, 3.0), max_iters: int = 200) -> np.ndarray:
    """Four Lloyd-Max levels of the samples (fp64), from `start`."""
    t = np.sort(np.asarray(samples, np.float64).ravel())
    prefix = np.concatenate([[0.0], np.cumsum(t)])
    lv = np.array(start, np.float64)
    for _ in range(max_iters):
        cuts = np.searchsorted(t, (lv[:-1] + lv[1:]) / 2.0, side="right")
        bounds = np.concatenate([[0], cuts, [t.size]])
        new = lv.copy()
        for j in range(lv.size):
            a, b = bounds[j], bounds[j + 1]
            if b > a:
                new[j] = (prefix[b] - prefix[a]) / (b - a)
        if np.array_equal(new, lv):
            break
        lv = new
    return lv


def to_sixteenths(levels) -> np.ndarray:
    """Levels in units of the scale as integers 16 l: nearest, clamped to [0, 48], then each at
    least one above the one below it (from the bottom) and at most one below the one above
    it (from the top)."""
    k = [int(v) for v in np.clip(np.rint(np.asarray(levels, np.float64) * 16.0), 0, 48)]
    for j in range(1, 4):
        k[j] = max(k[j], k[j - 1] + 1)
    k[3] = min(k[3], 48)
    for j in (2, 1, 0):
        k[j] = min(k[j], k[j + 1] - 1)
    return np.array(k, np.int64)


def fit_levels(rows, rot, clip: float) -> np.ndarray:
    """The codebook (four sixteenths) of calibration rows under rotation rot and clip ratio."""
    t = normalized_samples(rows, rot, clip)
    if t.size == 0:
        return np.array(UNIFORM, np.int64)
    return to_sixteenths(lloyd_max(t))


def layer_codebooks(calib_sets, rot_k_bits, rot_v_bits, clip_k, clip_v):
    """Per KV head, the K and V codebooks ([Hkv, 4] each) fitted on each head's calibration
    (queries, keys, values): keys under R_K, values under R_V (rotation bits are bf16)."""
    def bf16(bits):
        return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)

    rk = bf16(rot_k_bits).reshape(-1, 128, 128)
    rv = bf16(rot_v_bits).reshape(-1, 128, 128)
    ks, vs = [], []
    for kv, (_, k, v) in enumerate(calib_sets):
        ks.append(fit_levels(k, rk[kv], float(np.asarray(clip_k).reshape(-1)[kv])))
        vs.append(fit_levels(v, rv[kv], float(np.asarray(clip_v).reshape(-1)[kv])))
    return np.stack(ks), np.stack(vs)
