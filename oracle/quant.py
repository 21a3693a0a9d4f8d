"""Oracle: demotion of one K or V vector to INT2 (rotate, clip, quantise).

Source: the QbitAI article on OSCAR, section on the serving path: the oldest recent
token is rotated, clipped, quantised and packed into INT2 history; INT2 has four levels;
dequantisation uses a scale and a zero point (asymmetric). The abstracts (arXiv v1/v2)
add that the clipping thresholds are fixed per layer and derived offline.

Normative steps for one bf16 vector x (128 values), rotation R (bf16 values) and clip
ratio c (a float32), with one group of 128 values per vector:
  1. y_j = sum_i x_i R_ij, taken as the correctly rounded fp64 value of the exact sum
     (every product of two bf16 values is exact in fp64);
  2. ymax = max_j y_j, ymin = min_j y_j;
  3. hi = fl64(c * ymax), lo = fl64(c * ymin);
  4. s = fl64(fl64(hi - lo) / 3); s16 = fp16(s), z16 = fp16(lo)  (nearest, ties to even,
     one rounding from fp64);
  5. t_j = fl64(fl64(y_j - z16) / s16); q_j = clamp(round-half-even(t_j), 0, 3);
     if s16 == 0 every q_j is 0.
Dequantised value: q_j * s16 + z16.

Readings: group = the whole 128-dim head vector; clip = scaling max and min by c; the
zero point is the fp16 lower clip value (not an integer offset); scale and zero point are
fp16 each (this is what makes a 32K-token request cost the 2.38 bits per element the
article reports); round half to even; codes clamp to [0, 3].

Exactness: step 1 is evaluated with a BLAS product plus an a-priori error bound
(|fl(x.r) - x.r| <= gamma_n sum|x_i r_i|); every entry whose value can change a decision
(a group extreme, or a code whose t lies within the bound of a rounding boundary) is
recomputed with math.fsum, which returns the correctly rounded exact sum.
"""

from __future__ import annotations

import math

import numpy as np

N_LEVELS = 4
BOUNDARIES = np.array([0.5, 1.5, 2.5])


def boundary_distance(t: np.ndarray) -> np.ndarray:
    """Distance from t to the nearest rounding boundary between levels (0.5, 1.5, 2.5)."""
    nearest = np.rint(np.clip(t, 0.5, 2.5) - 0.5) + 0.5
    return np.abs(t - nearest)


def fp32(x: float) -> float:
    """The float32 nearest to x, as a Python float (exact)."""
    return float(np.float32(x))


def fp16(x) -> np.ndarray:
    """Nearest fp16 (ties to even), from fp64 in one rounding step."""
    return np.asarray(x, dtype=np.float64).astype(np.float16)


def rotate_with_bound(x: np.ndarray, r: np.ndarray):
    """(y, bound): fp64 matrix product x @ r and a bound on |y - exact| per entry."""
    y = x @ r
    n = x.shape[1]
    gamma = n * 2.0 ** -53 / (1.0 - n * 2.0 ** -53)
    bound = 2.0 * gamma * (np.abs(x) @ np.abs(r))
    return y, bound


def exact_dot(x_row: np.ndarray, r_col: np.ndarray) -> float:
    return math.fsum((x_row * r_col).tolist())


def exact_dots(x: np.ndarray, rt: np.ndarray, ii: np.ndarray, jj: np.ndarray) -> np.ndarray:
    """Correctly rounded x[i] . rt[j] for every pair (ii[k], jj[k]) via math.fsum."""
    out = np.empty(len(ii))
    for a in range(0, len(ii), 1 << 15):
        prods = x[ii[a:a + (1 << 15)]] * rt[jj[a:a + (1 << 15)]]   # exact: bf16 x bf16
        out[a:a + len(prods)] = list(map(math.fsum, prods.tolist()))
    return out


def exact_rotation(x: np.ndarray, r: np.ndarray) -> np.ndarray:
    """Every y_ij by math.fsum (slow; for small inputs and cross-checks)."""
    out = np.empty((x.shape[0], r.shape[1]))
    for i in range(x.shape[0]):
        for j in range(r.shape[1]):
            out[i, j] = exact_dot(x[i], r[:, j])
    return out


def quantize_rows(x: np.ndarray, r: np.ndarray, clip: float):
    """Demote rows x [N, 128] (bf16 values as fp64) with rotation r [128, 128] (bf16
    values) and clip ratio `clip` (rounded to float32 first).

    Returns (codes uint8 [N,128], s16 float16 [N], z16 float16 [N], margin [N,128]).
    margin is the distance of t_j to the nearest rounding boundary (0.5, 1.5, 2.5), inf
    where s16 == 0; it is what the near-boundary tolerance on codes is judged by."""
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    c = fp32(clip)
    n = x.shape[0]
    rt = np.ascontiguousarray(r.T)
    y, bound = rotate_with_bound(x, r)

    # extremes: every entry whose bound interval reaches the largest (smallest) lower
    # (upper) bound may be the extreme; take the exact maximum (minimum) over those
    ymax = np.full(n, -np.inf)
    ymin = np.full(n, np.inf)
    top = y + bound >= (y - bound).max(axis=1, keepdims=True)
    bot = y - bound <= (y + bound).min(axis=1, keepdims=True)
    ii, jj = np.nonzero(top)
    np.maximum.at(ymax, ii, exact_dots(x, rt, ii, jj))
    ii, jj = np.nonzero(bot)
    np.minimum.at(ymin, ii, exact_dots(x, rt, ii, jj))

    hi = c * ymax
    lo = c * ymin
    s = (hi - lo) / 3.0
    s16 = fp16(s)
    z16 = fp16(lo)
    if not (np.all(np.isfinite(s16)) and np.all(np.isfinite(z16))):
        raise ValueError("clipped range exceeds fp16")
    s64 = s16.astype(np.float64)[:, None]
    z64 = z16.astype(np.float64)[:, None]
    zero_scale = (s64 == 0.0)
    safe_s = np.where(zero_scale, 1.0, s64)

    t = (y - z64) / safe_s
    near = boundary_distance(t) <= bound / safe_s * 4.0 + 1e-12
    near &= ~zero_scale
    ii, jj = np.nonzero(near)
    t[ii, jj] = (exact_dots(x, rt, ii, jj) - z64[ii, 0]) / safe_s[ii, 0]

    codes = np.clip(np.rint(t), 0, N_LEVELS - 1)
    codes = np.where(zero_scale, 0, codes).astype(np.uint8)
    margin = boundary_distance(t)
    margin = np.where(zero_scale, np.inf, margin)
    return codes, s16, z16, margin


def dequantize(codes: np.ndarray, s16: np.ndarray, z16: np.ndarray) -> np.ndarray:
    """q * s16 + z16 per row, fp64 (rotated basis)."""
    s = np.asarray(s16, dtype=np.float64)[..., None]
    z = np.asarray(z16, dtype=np.float64)[..., None]
    return codes.astype(np.float64) * s + z
