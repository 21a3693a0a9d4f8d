"""Oracle: the offline search for the clip ratio of one (layer, KV head, K or V).

Test infrastructure only: nothing outside tests/, the smoke check and the CPU baseline of
the benchmark may import this package.

Source: the paper's abstract (Hugging Face paper page, paper-check page) and the QbitAI
article on OSCAR: the rotations and the clipping thresholds are estimated offline on
calibration data and then fixed. The pages do not give the criterion; the reading here:

  * candidates c = 0.50, 0.51, ..., 1.00 (c as float32, as the demotion takes it);
  * the criterion is the mean squared reconstruction error of the calibration rows in
    the rotated basis, sum over rows and dims of (y - yhat)^2 with y = x R and yhat the
    dequantised value of the uniform INT2 demotion (quant.quantize_rows, exact y);
  * the smallest error wins, the smallest c on an exact tie.
"""

from __future__ import annotations

import numpy as np

from . import quant

GRID = np.round(np.arange(50, 101) / 100.0, 2)


def reconstruction_error(x, r, clip: float) -> float:
    """sum (y - yhat)^2 over the rows x [N, 128] under rotation r and clip ratio clip."""
    x = np.asarray(x, np.float64)
    codes, s16, z16, _ = quant.quantize_rows(x, np.asarray(r, np.float64), clip)
    y = quant.exact_rotation(x, np.asarray(r, np.float64)) if x.shape[0] <= 4 else _rotation(x, r)
    return float(np.sum((y - quant.dequantize(codes, s16, z16)) ** 2))


def _rotation(x, r):
    # y for the error itself: fp64 products summed by numpy (the codes above come from the
    # exact sums; the error only ranks the candidates)
    return np.asarray(x, np.float64) @ np.asarray(r, np.float64)


def search(x, r, grid=GRID):
    """(best clip ratio, errors per candidate) over the grid."""
    errs = np.array([reconstruction_error(x, r, float(c)) for c in grid])
    return float(grid[int(np.argmin(errs))]), errs
