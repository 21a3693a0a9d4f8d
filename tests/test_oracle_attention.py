"""Pins for the oracle's decode attention and online-softmax merge (CPU only)."""

import math

import numpy as np

from oracle import attention as att
from oracle import quant
from oracle.rotation import bit_reversal_matrix, rotation_from_covariance


def brute_force(q, keys, values, sm_scale):
    """Softmax attention with plain Python loops."""
    s = [sm_scale * sum(a * b for a, b in zip(q, k)) for k in keys]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    tot = sum(w)
    return [sum(w[i] * values[i][d] for i in range(len(keys))) / tot for d in range(len(q))]


def test_split_merge_equals_single_softmax_at_every_split_point():
    g = np.random.default_rng(0)
    d, n = 8, 9
    q = g.standard_normal(d) * 3
    k = g.standard_normal((n, d)) * 3
    v = g.standard_normal((n, d))
    ref = np.array(brute_force(q.tolist(), k.tolist(), v.tolist(), 0.5))
    s = 0.5 * (k @ q)
    for a in range(n + 1):
        for b in range(a, n + 1):
            parts = [att.partial(s[:a], v[:a]), att.partial(s[a:b], v[a:b]), att.partial(s[b:], v[b:])]
            out = att.finalize(att.merge(parts))
            assert np.abs(out - ref).max() <= 1e-12


def test_empty_segments_contribute_nothing():
    v = np.ones((0, 4))
    m, l, acc = att.partial(np.zeros(0), v)
    assert m == -np.inf and l == 0.0 and not acc.any()
    only = att.partial(np.array([1.0, 2.0]), np.array([[1.0, 0, 0, 0], [0, 1.0, 0, 0]]))
    merged = att.merge([att.partial(np.zeros(0), v), only, att.partial(np.zeros(0), v)])
    assert merged[0] == only[0] and merged[1] == only[1]
    assert np.array_equal(att.finalize(att.merge([att.partial(np.zeros(0), v)])), np.zeros(4))


def _tiny_case(seed=1, n_hist=5, n_win=3, hq=2, hkv=1):
    g = np.random.default_rng(seed)
    a = g.standard_normal((512, 128))
    r = rotation_from_covariance(a.T @ a)          # fp64, orthogonal to 1e-15
    q = g.standard_normal((hq, 128))
    win_k = g.standard_normal((hkv, n_win, 128))
    win_v = g.standard_normal((hkv, n_win, 128))
    hk = g.standard_normal((n_hist, 128))
    hv = g.standard_normal((n_hist, 128))
    kc, ks, kz, _ = quant.quantize_rows(hk, r, 0.9)
    vc, vs, vz, _ = quant.quantize_rows(hv, r, 0.9)
    return q, r, win_k, win_v, (kc, ks, kz, vc, vs, vz)


def test_rotated_history_equals_attention_to_unrotated_dequantised_rows():
    # q_rot . khat = q . (khat R^T) and the V sum un-rotates by R^T: a transposed operand
    # anywhere would break this equality
    q, r, win_k, win_v, hist = _tiny_case()
    rk = np.stack([r])
    out = att.decode(q, rk, rk, win_k, win_v, [hist], 0.3)
    khat = quant.dequantize(hist[0], hist[1], hist[2]) @ r.T
    vhat = quant.dequantize(hist[3], hist[4], hist[5]) @ r.T
    keys = np.concatenate([win_k[0], khat]).tolist()
    vals = np.concatenate([win_v[0], vhat]).tolist()
    for h in range(2):
        ref = brute_force(q[h].tolist(), keys, vals, 0.3)
        assert np.abs(out[h] - ref).max() <= 1e-10


def test_decode_equals_split_and_merge_of_its_segments():
    q, r, win_k, win_v, hist = _tiny_case(seed=2, n_hist=11, n_win=4)
    out = att.decode_head(q[0], r, r, win_k[0], win_v[0], hist, 0.2)
    for cut in range(0, 12):
        hp = att.history_partials(q[0], r, hist, 0.2, [(0, cut), (cut, 11)])
        for wcut in range(0, 5):
            wp = att.window_partials(q[0], win_k[0], win_v[0], 0.2, [(0, wcut), (wcut, 4)])
            assert np.abs(att.merge_segments(hp, wp, r) - out).max() <= 1e-12


def test_lossless_quantisation_reduces_to_plain_attention():
    # R = bit-reversal permutation (exact in bf16), c = 1, and rows whose values lie on
    # {-1.5, -0.5, 0.5, 1.5} with both extremes present: scale 1, zero -1.5, codes exact, so
    # the three-segment decode equals plain attention over the raw rows
    g = np.random.default_rng(3)
    p = bit_reversal_matrix(128)
    grid = np.array([-1.5, -0.5, 0.5, 1.5])
    rows = grid[g.integers(0, 4, (2, 20, 128))]
    rows[:, :, 0], rows[:, :, 1] = -1.5, 1.5
    kc, ks, kz, _ = quant.quantize_rows(rows[0], p, 1.0)
    vc, vs, vz, _ = quant.quantize_rows(rows[1], p, 1.0)
    assert np.all(ks == 1.0) and np.all(kz == -1.5)
    assert np.array_equal(quant.dequantize(kc, ks, kz), rows[0] @ p)
    q = g.standard_normal((4, 128))
    win_k = g.standard_normal((1, 6, 128))
    win_v = g.standard_normal((1, 6, 128))
    pk = np.stack([p])
    out = att.decode(q, pk, pk, win_k, win_v, [(kc, ks, kz, vc, vs, vz)], 0.25)
    keys = np.concatenate([win_k[0], rows[0]]).tolist()
    vals = np.concatenate([win_v[0], rows[1]]).tolist()
    for h in range(4):
        assert np.abs(out[h] - brute_force(q[h].tolist(), keys, vals, 0.25)).max() <= 1e-12


def test_special_cases():
    q, r, win_k, win_v, hist = _tiny_case(seed=4)
    empty = tuple(np.asarray(x)[:0] for x in hist)
    # no history: plain BF16 attention over the window
    out = att.decode_head(q[0], r, r, win_k[0], win_v[0], empty, 0.4)
    assert np.abs(out - brute_force(q[0].tolist(), win_k[0].tolist(), win_v[0].tolist(), 0.4)).max() <= 1e-12
    # zero query: uniform weights, the mean of every value row (history un-rotated)
    vhat = quant.dequantize(hist[3], hist[4], hist[5]) @ r.T
    out = att.decode_head(np.zeros(128), r, r, win_k[0], win_v[0], hist, 0.4)
    assert np.abs(out - np.concatenate([win_v[0], vhat]).mean(0)).max() <= 1e-12
    # a single token: its value
    one = tuple(np.asarray(x)[:1] for x in hist)
    out = att.decode_head(q[0], r, r, win_k[0][:0], win_v[0][:0], one, 0.4)
    assert np.abs(out - vhat[0]).max() <= 1e-12


def test_gqa_heads_use_their_own_kv_head():
    g = np.random.default_rng(5)
    q = g.standard_normal((4, 128))
    win_k = g.standard_normal((2, 3, 128))
    win_v = g.standard_normal((2, 3, 128))
    eye = np.stack([np.eye(128)] * 2)
    empty = (np.zeros((0, 128), np.uint8), np.zeros(0, np.float16), np.zeros(0, np.float16),
             np.zeros((0, 128), np.uint8), np.zeros(0, np.float16), np.zeros(0, np.float16))
    out = att.decode(q, eye, eye, win_k, win_v, [empty, empty], 0.5)
    for h in range(4):
        kv = h // 2
        ref = brute_force(q[h].tolist(), win_k[kv].tolist(), win_v[kv].tolist(), 0.5)
        assert np.abs(out[h] - ref).max() <= 1e-12


def test_multi_query_tokens_see_the_window_up_to_their_own_position():
    # brute force with an explicit causal cut of the window: token t of T sees window slots
    # [0, n_w - (T - 1 - t)) and the whole (un-rotated, dequantised) history
    _, r, win_k, win_v, hist = _tiny_case(seed=5, n_hist=7, n_win=6)
    g = np.random.default_rng(6)
    n_tok = 4
    q = g.standard_normal((n_tok, 2, 128))
    rk = np.stack([r])
    out = att.decode_multi(q, rk, rk, win_k, win_v, [hist], 0.3)
    assert out.shape == (n_tok, 2, 128)
    khat = quant.dequantize(hist[0], hist[1], hist[2]) @ r.T
    vhat = quant.dequantize(hist[3], hist[4], hist[5]) @ r.T
    for t in range(n_tok):
        keep = 6 - (n_tok - 1 - t)
        keys = np.concatenate([win_k[0][:keep], khat]).tolist()
        vals = np.concatenate([win_v[0][:keep], vhat]).tolist()
        for h in range(2):
            ref = brute_force(q[t, h].tolist(), keys, vals, 0.3)
            assert np.abs(out[t, h] - ref).max() <= 1e-10


def test_multi_query_special_cases():
    q1, r, win_k, win_v, hist = _tiny_case(seed=7, n_hist=5, n_win=2)
    rk = np.stack([r])
    # one token is the single-query decode
    assert np.array_equal(att.decode_multi(q1[None], rk, rk, win_k, win_v, [hist], 0.3)[0],
                          att.decode(q1, rk, rk, win_k, win_v, [hist], 0.3))
    g = np.random.default_rng(8)
    q = g.standard_normal((4, 2, 128))
    out = att.decode_multi(q, rk, rk, win_k, win_v, [hist], 0.3)
    # the last token sees the whole window
    assert np.array_equal(out[3], att.decode(q[3], rk, rk, win_k, win_v, [hist], 0.3))
    # with more query tokens than window slots the first ones see the history alone
    empty = np.zeros((1, 0, 128))
    for t in (0, 1):
        assert np.array_equal(out[t], att.decode(q[t], rk, rk, empty, empty, [hist], 0.3))
