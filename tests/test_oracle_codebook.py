"""Pins for the oracle's Lloyd-Max codebook variant (CPU only).

The fitter is pinned to the published 2-bit Lloyd-Max quantiser of the unit Gaussian
(J. Max, "Quantizing for minimum distortion", IRE Trans. Information Theory, 1960,
table for N = 4: outputs +-0.4528 and +-1.510, inner decision level +-0.9816, mean
squared error 0.1175) and to the uniform density, whose optimal quantiser is uniform.
The code decisions are pinned to round-half-even for the uniform levels and to exact
rational brute force for random codebooks."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import attention, codebook, quant
from oracle.rotation import round_bf16, rotation_from_covariance

EYE = np.eye(128)


def test_lloyd_max_on_the_unit_gaussian_gives_the_published_quantiser():
    g = np.random.default_rng(1960)
    x = g.standard_normal(2_000_000)
    lv, hist = codebook.lloyd_max(x, [-1.5, -0.5, 0.5, 1.5], iters=300, tol=1e-9)
    assert np.allclose(lv, [-1.510, -0.4528, 0.4528, 1.510], atol=6e-3)
    edges = (lv[:-1] + lv[1:]) / 2
    assert np.allclose(edges, [-0.9816, 0.0, 0.9816], atol=6e-3)
    assert abs(hist[-1] - 0.1175) < 1.5e-3


def test_lloyd_max_on_a_uniform_density_is_the_uniform_quantiser():
    # density uniform on [0, 3]: the optimal four levels are the cell centres 3/8 + 3k/4
    x = (np.arange(1_200_000) + 0.5) * (3.0 / 1_200_000)
    lv, _ = codebook.lloyd_max(x, [0.0, 1.0, 2.0, 3.0], iters=500, tol=1e-12)
    assert np.allclose(lv, [3 / 8, 9 / 8, 15 / 8, 21 / 8], atol=2e-3)


def test_lloyd_max_never_raises_the_error():
    g = np.random.default_rng(7)
    x = np.concatenate([g.standard_normal(50_000) * 0.3 + 0.4, g.exponential(0.8, 30_000)])
    _, hist = codebook.lloyd_max(x, [0.0, 1.0, 2.0, 3.0], iters=60)
    assert all(b <= a + 1e-15 for a, b in zip(hist, hist[1:]))
    assert hist[-1] < hist[0]


def test_sixteenths_round_clamp_and_separate():
    assert list(codebook.sixteenths([0.0, 1.0, 2.0, 3.0])) == [0, 16, 32, 48]
    assert list(codebook.sixteenths([-0.4, 0.51, 2.2, 3.9])) == [0, 8, 35, 48]
    assert list(codebook.sixteenths([1.0, 1.0, 1.0, 1.0])) == [16, 17, 18, 19]
    assert list(codebook.sixteenths([3.0, 3.0, 3.0, 3.0])) == [45, 46, 47, 48]
    assert list(codebook.sixteenths([0.0, 0.0, 0.0, 0.0])) == [0, 1, 2, 3]


def test_uniform_levels_decide_as_round_half_even_with_clamp():
    g = np.random.default_rng(3)
    t = np.concatenate([g.uniform(-2, 5, 20_000), np.arange(-8, 41) / 8.0])  # includes every tie
    got = codebook.codes_from_t(t, codebook.UNIFORM16)
    assert np.array_equal(got, np.clip(np.rint(t), 0, 3).astype(np.uint8))


def _exact_t(x_row, r_col, z16, s16):
    y = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x_row, r_col))
    return (y - Fraction(float(z16))) / Fraction(float(s16))


def _nearest_even(t: Fraction, k16):
    lv = [Fraction(int(k), 16) for k in k16]
    d = [abs(t - v) for v in lv]
    best = min(d)
    idx = [j for j in range(4) if d[j] == best]
    return idx[0] if len(idx) == 1 else next(j for j in idx if j % 2 == 0)


def test_codes_are_the_nearest_level_by_exact_arithmetic():
    g = np.random.default_rng(11)
    r = round_bf16(rotation_from_covariance(np.diag(g.uniform(0.5, 2.0, 128))))
    x = round_bf16(g.standard_normal((3, 128)))
    for k16 in ([0, 5, 30, 48], [2, 20, 27, 41], [0, 16, 32, 48]):
        codes, s16, z16, _ = codebook.quantize_rows(x, r, 0.93, k16)
        for i in range(3):
            for j in range(0, 128, 3):
                t = _exact_t(x[i], r[:, j], z16[i], s16[i])
                assert codes[i, j] == _nearest_even(t, k16), (k16, i, j)


def test_midpoint_ties_go_to_the_even_index():
    # R = I, c = 1, y in [0, 3]: s = 1, z = 0, t = y. Midpoints of (0, 8, 24, 48)/16 are
    # 0.25, 1.0 and 2.25; the values sit exactly on them.
    k16 = [0, 8, 24, 48]
    y = [3.0, 0.0, 0.25, 1.0, 2.25, 0.2, 1.1, 2.3]
    x = np.zeros((1, 128))
    x[0, :8] = y
    codes, s16, z16, margin = codebook.quantize_rows(x, EYE, 1.0, k16)
    assert s16[0] == 1.0 and z16[0] == 0.0
    assert list(codes[0, :8]) == [3, 0, 0, 2, 2, 0, 2, 3]
    assert margin[0, 2] == 0.0 and margin[0, 3] == 0.0 and margin[0, 4] == 0.0


def test_uniform_codebook_reduces_to_the_uniform_demotion():
    g = np.random.default_rng(5)
    r = round_bf16(rotation_from_covariance(np.diag(g.uniform(0.2, 3.0, 128))))
    x = round_bf16(g.standard_normal((64, 128)) * g.uniform(0.1, 4.0, (64, 1)))
    c1, s1, z1, _ = quant.quantize_rows(x, r, 0.9)
    c2, s2, z2, _ = codebook.quantize_rows(x, r, 0.9, codebook.UNIFORM16)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2) and np.array_equal(z1, z2)
    assert np.array_equal(quant.dequantize(c1, s1, z1), codebook.dequantize(c2, s2, z2, codebook.UNIFORM16))


def test_dequantize_maps_codes_to_levels():
    codes = np.array([[0, 1, 2, 3]], np.uint8)
    out = codebook.dequantize(codes, np.array([np.float16(0.5)]), np.array([np.float16(-1.0)]), [0, 4, 40, 48])
    assert list(out[0]) == [-1.0, -1.0 + 0.5 * 0.25, -1.0 + 0.5 * 2.5, -1.0 + 0.5 * 3.0]


def test_fitted_codebook_lowers_the_reconstruction_error_on_its_rows():
    g = np.random.default_rng(9)
    r = round_bf16(rotation_from_covariance(np.diag(np.linspace(0.1, 4.0, 128))))
    x = round_bf16(g.standard_normal((400, 128)) * np.linspace(0.2, 2.0, 128))
    k16 = codebook.fit(x, r, 0.95)
    assert np.all(np.diff(k16) > 0) and k16[0] >= 0 and k16[-1] <= 48
    y = x @ r

    def err(levels):
        c, s, z, _ = codebook.quantize_rows(x, r, 0.95, levels)
        return np.mean((codebook.dequantize(c, s, z, levels) - y) ** 2)

    assert err(k16) < 0.95 * err(codebook.UNIFORM16)


def test_decode_through_the_uniform_codebook_is_the_uniform_decode():
    g = np.random.default_rng(2)
    r = [round_bf16(rotation_from_covariance(np.diag(g.uniform(0.5, 2, 128)))) for _ in range(2)]
    rot = np.stack(r)
    hists = []
    for kv in range(2):
        xk = round_bf16(g.standard_normal((40, 128)))
        xv = round_bf16(g.standard_normal((40, 128)))
        kc, ks, kz, _ = quant.quantize_rows(xk, rot[kv], 0.9)
        vc, vs, vz, _ = quant.quantize_rows(xv, rot[kv], 0.9)
        hists.append((kc, ks, kz, vc, vs, vz))
    q = round_bf16(g.standard_normal((4, 128)))
    wk = round_bf16(g.standard_normal((2, 10, 128)))
    wv = round_bf16(g.standard_normal((2, 10, 128)))
    a = attention.decode(q, rot, rot, wk, wv, hists, 0.088)
    u = (codebook.UNIFORM16, codebook.UNIFORM16)
    b = attention.decode(q, rot, rot, wk, wv, hists, 0.088, codebooks=[u, u])
    assert np.array_equal(a, b)
    # a different codebook changes the dequantised history, hence the output
    c = attention.decode(q, rot, rot, wk, wv, hists, 0.088, codebooks=[([0, 8, 30, 48], [3, 18, 33, 45])] * 2)
    assert not np.allclose(a, c)


def test_multi_query_decode_through_codebooks():
    """decode_multi with codebooks: the uniform levels give the uniform multi-query decode
    exactly, and each token's output is decode() with the same codebook over its causal
    share of the window."""
    g = np.random.default_rng(12)
    rot = np.stack([round_bf16(rotation_from_covariance(np.diag(g.uniform(0.5, 2, 128))))])
    xk = round_bf16(g.standard_normal((30, 128)))
    xv = round_bf16(g.standard_normal((30, 128)))
    book = ([2, 20, 27, 41], [0, 5, 30, 48])
    kc, ks, kz, _ = codebook.quantize_rows(xk, rot[0], 0.9, book[0])
    vc, vs, vz, _ = codebook.quantize_rows(xv, rot[0], 0.9, book[1])
    hists = [(kc, ks, kz, vc, vs, vz)]
    q = round_bf16(g.standard_normal((3, 2, 128)))
    wk = round_bf16(g.standard_normal((1, 9, 128)))
    wv = round_bf16(g.standard_normal((1, 9, 128)))
    u = (codebook.UNIFORM16, codebook.UNIFORM16)
    assert np.array_equal(attention.decode_multi(q, rot, rot, wk, wv, hists, 0.088, codebooks=[u]),
                          attention.decode_multi(q, rot, rot, wk, wv, hists, 0.088))
    got = attention.decode_multi(q, rot, rot, wk, wv, hists, 0.088, codebooks=[book])
    for t in range(3):
        keep = 9 - (2 - t)
        ref = attention.decode(q[t], rot, rot, wk[:, :keep], wv[:, :keep], hists, 0.088, codebooks=[book])
        assert np.array_equal(got[t], ref)
    assert not np.allclose(got, attention.decode_multi(q, rot, rot, wk, wv, hists, 0.088))
