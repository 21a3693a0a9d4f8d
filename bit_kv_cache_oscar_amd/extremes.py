"""Host-side rotation of calibration rows with exact extremes.

The demotion kernels take each group's extremes from the exact dot products: the products
of bf16 values are exact in fp64 and the sums are rounded once (QbitAI article on OSCAR,
serving-path section: rotate, clip, quantise to INT2 with a scale and zero point per
group). The scale and zero point (fp16) follow from the extremes, so offline calibration
that fits clip ratios or codebook levels from the same quantiser must take the same
extremes, not those of a BLAS product whose summation order may round differently.

rotate(rows, rot) returns the BLAS values y = x R together with the rows' exact maxima and
minima: every value within the BLAS error bound of a row's extreme (a few units of
2^-53 sum |x_i R_ij|, widened a hundredfold) is summed again with math.fsum, which rounds
the exact sum of the exact products once.
"""

from __future__ import annotations

import math

import numpy as np


def rotate(rows, rot):
    """(y [N, 128] fp64, ymax [N], ymin [N]) for bf16-valued rows [N, 128] and rotation
    [128, 128]; ymax and ymin are the correctly rounded exact extremes."""
    x = np.asarray(rows, np.float64)
    r = np.asarray(rot, np.float64)
    y = x @ r
    # the BLAS sums are within n 2^-53 sum |p| of the exact ones (any order, n = 128)
    tol = (np.abs(x) @ np.abs(r)) * (128 * 2.0 ** -53 * 100.0) + 1e-300
    hi_cut = (y + tol).max(axis=1)  # no exact value exceeds this
    lo_cut = (y - tol).min(axis=1)
    ymax = np.empty(len(x))
    ymin = np.empty(len(x))
    for i in range(len(x)):
        # values that may be the exact max / min: their upper (lower) end reaches the
        # largest lower end (smallest upper end)
        top = np.nonzero(y[i] + tol[i] >= (y[i] - tol[i]).max())[0]
        bot = np.nonzero(y[i] - tol[i] <= (y[i] + tol[i]).min())[0]
        ymax[i] = max(math.fsum(x[i] * r[:, j]) for j in top)
        ymin[i] = min(math.fsum(x[i] * r[:, j]) for j in bot)
        assert ymax[i] <= hi_cut[i] and ymin[i] >= lo_cut[i]
    return y, ymax, ymin
