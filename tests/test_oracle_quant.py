"""Pins for the oracle's INT2 demotion quantiser (CPU only)."""

import numpy as np
import pytest

from oracle import quant
from oracle.rotation import round_bf16, rotation_from_covariance

EYE = np.eye(128)


def _row(values):
    x = np.zeros(128)
    x[:len(values)] = values
    return x[None, :]


def test_identity_rotation_unit_clip_is_plain_minmax_int2():
    # R = I, c = 1: levels lo + k (hi - lo) / 3. Values 0..3 with hi = 3, lo = 0 give
    # scale 1, zero 0 and codes equal to the values themselves.
    vals = [3, 0, 1, 2, 2, 1, 0, 3]
    codes, s16, z16, _ = quant.quantize_rows(_row(vals), EYE, 1.0)
    assert s16[0] == 1.0 and z16[0] == 0.0
    assert list(codes[0, :8]) == vals
    assert np.all(codes[0, 8:] == 0)


def test_half_clip_ties_round_to_even_and_clamp():
    # c = 0.5 (exact in float32): hi = 1.5, lo = 0, s = 0.5, t = 2y.
    y = [3.0, 0.0, 0.25, 0.5, 0.75, 1.0, 1.25, 1.5]
    expect = [3, 0, 0, 1, 2, 2, 2, 3]   # t = 6->3 (clamp), 0, 0.5->0, 1, 1.5->2, 2, 2.5->2, 3
    codes, s16, z16, margin = quant.quantize_rows(_row(y), EYE, 0.5)
    assert s16[0] == 0.5 and z16[0] == 0.0
    assert list(codes[0, :8]) == expect
    assert margin[0, 2] == 0.0 and margin[0, 4] == 0.0 and margin[0, 6] == 0.0


def test_negative_zero_point_and_fp16_scale_rounding():
    # c = 1, y in [-1, 1]: s = 2/3 -> fp16(2/3) = 0.66650390625; z = -1
    codes, s16, z16, _ = quant.quantize_rows(_row([1.0, -1.0, 0.0, 0.3]), EYE, 1.0)
    assert z16[0] == -1.0
    assert float(s16[0]) == 0.66650390625
    # t = (y + 1) / s: 1 -> 3.0007 -> 3; -1 -> 0; 0 -> 1.50037 -> 2; 0.3 -> 1.9505 -> 2
    assert list(codes[0, :4]) == [3, 0, 2, 2]


def test_clip_ratio_is_taken_as_float32():
    c = quant.fp32(0.9)
    assert c == 0.89999997615814208984375
    codes, s16, z16, _ = quant.quantize_rows(_row([2.0, -2.0]), EYE, 0.9)
    assert z16[0] == np.float16(-2.0 * c)
    assert s16[0] == np.float16((2.0 * c - (-2.0 * c)) / 3.0)


def test_degenerate_constant_and_zero_vectors():
    x = np.stack([np.full(128, 2.5), np.zeros(128)])
    codes, s16, z16, margin = quant.quantize_rows(x, EYE, 0.9)
    assert s16[0] == 0.0 and z16[0] == np.float16(2.5 * quant.fp32(0.9))
    assert s16[1] == 0.0 and z16[1] == 0.0
    assert np.all(codes == 0) and np.all(np.isinf(margin))
    assert np.all(quant.dequantize(codes, s16, z16)[0] == float(z16[0]))


def _rotated_rows(n, seed=0, outliers=True):
    g = np.random.default_rng(seed)
    x = g.standard_normal((n, 128)).astype(np.float32)
    if outliers:
        x[:, [5, 17, 80, 99]] *= 20
    x = round_bf16(x.astype(np.float64))
    a = g.standard_normal((512, 128))
    r = round_bf16(rotation_from_covariance(a.T @ a))
    return x, r


def test_codes_are_the_nearest_level():
    # independent of the division-and-round formula: each code is the argmin over the four
    # levels z + k s of |y - level| (the clamp is the nearest end level)
    x, r = _rotated_rows(200)
    codes, s16, z16, margin = quant.quantize_rows(x, r, 0.9)
    y = quant.exact_rotation(x[:40], r)
    levels = z16[:40, None].astype(float) + np.arange(4)[None, :] * s16[:40, None].astype(float)
    nearest = np.abs(y[:, :, None] - levels[:, None, :]).argmin(-1)
    ok = margin[:40] > 1e-9
    assert ok.mean() > 0.99
    assert np.array_equal(codes[:40][ok], nearest[ok])


def test_reconstruction_error_bound_inside_clip_range():
    x, r = _rotated_rows(100, seed=1)
    codes, s16, z16, _ = quant.quantize_rows(x, r, 0.9)
    y = x @ r
    yhat = quant.dequantize(codes, s16, z16)
    s = s16.astype(float)[:, None]
    lo = z16.astype(float)[:, None]
    inside = (y >= lo) & (y <= lo + 3 * s)
    assert np.all(np.abs(y - yhat)[inside] <= s.repeat(128, 1)[inside] / 2 + 1e-9)
    # scale is a third of the clipped range, to fp16 precision
    c = quant.fp32(0.9)
    rng_ = c * (y.max(1) - y.min(1))
    assert np.allclose(s[:, 0] * 3, rng_, rtol=2e-3)


def test_fast_extremes_equal_exhaustive_fsum():
    # rows with a wide dynamic range stress the error-bound candidate logic
    g = np.random.default_rng(3)
    x = g.standard_normal((60, 128)) * np.exp(g.uniform(-12, 6, (60, 128)))
    x = round_bf16(x)
    _, r = _rotated_rows(1, seed=4)
    codes, s16, z16, _ = quant.quantize_rows(x, r, 0.9)
    y = quant.exact_rotation(x, r)
    c = quant.fp32(0.9)
    hi, lo = c * y.max(1), c * y.min(1)
    assert np.array_equal(s16, ((hi - lo) / 3.0).astype(np.float16))
    assert np.array_equal(z16, lo.astype(np.float16))
    t = (y - z16.astype(float)[:, None]) / s16.astype(float)[:, None]
    assert np.array_equal(codes, np.clip(np.rint(t), 0, 3).astype(np.uint8))


def test_fp16_conversion_is_single_rounding():
    # 1 + 2^-11 + 2^-40 would round to 1.0 through float32 (double rounding); direct is 1 + 2^-10
    assert quant.fp16(1.0 + 2 ** -11 + 2 ** -40) == np.float16(1.0 + 2 ** -10)
    assert quant.fp16(1.0 + 2 ** -11) == np.float16(1.0)


def test_overflowing_range_is_rejected():
    with pytest.raises(ValueError):
        quant.quantize_rows(_row([1e6, -1e6]), EYE, 1.0)


def test_boundary_distance_matches_brute_force():
    t = np.random.default_rng(9).uniform(-2, 6, 5000)
    brute = np.abs(t[:, None] - quant.BOUNDARIES[None, :]).min(1)
    assert np.array_equal(quant.boundary_distance(t), brute)
