"""The host calibration's exact extremes (bit_kv_cache_oscar_amd.extremes): the maxima and
minima of x R taken from exact products summed with a single rounding, as the demotion
kernels take them, including rows built so that the BLAS sum and the exact one round apart."""

import math

import numpy as np

import synth
from bit_kv_cache_oscar_amd.extremes import rotate


def _bf16(a):
    return synth.to_bf16_values(np.asarray(a, np.float32)).astype(np.float64)


def test_extremes_are_the_correctly_rounded_exact_ones():
    g = np.random.default_rng(3)
    x = _bf16(g.standard_normal((64, 128)) * np.exp(g.uniform(-8, 8, (64, 128))))
    r = _bf16(np.linalg.qr(g.standard_normal((128, 128)))[0])
    y, ymax, ymin = rotate(x, r)
    exact = np.array([[math.fsum(x[i] * r[:, j]) for j in range(128)] for i in range(64)])
    assert np.array_equal(ymax, exact.max(axis=1)) and np.array_equal(ymin, exact.min(axis=1))
    assert np.allclose(y, exact, rtol=0, atol=1e-9 * np.abs(exact).max())


def test_cancellation_rows():
    """Rows whose value is a small difference of huge products: a left-to-right fp64 sum
    rounds it wrong, the exact extremes do not."""
    x = np.zeros((3, 128))
    r = np.zeros((128, 128))
    # value j = 0: 2^60 - 2^60 + 1 ... as exact products; value j = 1: a plain 0.5
    x[:, 0], x[:, 1], x[:, 2] = 2.0 ** 30, 2.0 ** 30, 1.0
    r[0, 0], r[1, 0], r[2, 0] = 2.0 ** 30, -(2.0 ** 30), 0.75
    r[2, 1] = 0.5
    y, ymax, ymin = rotate(x, r)
    assert np.all(ymax == 0.75) and np.all(ymin == 0.0)
