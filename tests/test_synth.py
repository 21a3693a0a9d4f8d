"""The seeded input generator: determinism, shapes and the workload structure."""

import numpy as np

import synth


def test_bf16_rounding_hand_cases():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -8 + 2 ** -20], np.float32)
    v = synth.to_bf16_values(x)
    assert list(v) == [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 1.0 + 2 ** -7]


def test_workload_shapes():
    w = synth.workload(2)
    assert (w.batch, w.n_q_heads, w.n_kv_heads, w.gq) == (1, 32, 8, 4)
    assert w.hist_len(0) == 32448 and w.win_len(0) == 320
    w3 = synth.workload(3)
    assert w3.hist_len(0) == 99680 and w3.permute_pages
    w4 = synth.workload(4)
    assert w4.batch == 64 and all(8192 <= c <= 16384 for c in w4.ctx_lens)
    assert w4.shared_pages == 63
    w5 = synth.workload(5)
    assert (w5.batch, w5.n_q_heads, w5.gq, w5.hist_len(0)) == (4, 64, 8, 130752)
    w1 = synth.workload(1)
    assert (w1.hist_len(0), w1.gq) == (1024, 1)


def test_rows_are_deterministic_and_sliceable():
    w = synth.workload(2).with_ctx([5000])
    k1, v1 = synth.kv_rows(w, 0, 3)
    k2, v2 = synth.kv_rows(w, 0, 3, 100, 900)
    assert np.array_equal(k1[100:900], k2) and np.array_equal(v1[100:900], v2)
    assert np.array_equal(synth.to_bf16_values(k1), k1)
    hk, hv = synth.history_rows(w, 0, 3)
    assert np.array_equal(hk, k1[64:5000 - 256])
    wk, wv = synth.window_rows(w, 0, 3)
    assert np.array_equal(wk, np.concatenate([k1[:64], k1[-256:]]))


def test_outliers_are_shared_by_keys_and_their_queries():
    w = synth.workload(2).with_ctx([2000])
    kq_ch, kf, qf, v_ch, vf = synth.outliers(w, 1)
    k, v = synth.kv_rows(w, 0, 1)
    rms = np.sqrt((k.astype(np.float64) ** 2).mean(0))
    assert set(np.argsort(-rms)[:4]) == set(kq_ch)
    q = synth.query(w, 0)
    assert np.all(np.abs(q[4:8][:, kq_ch]).mean() > 3 * np.abs(q[4:8]).mean())
    assert np.all((kf >= 10) & (kf <= 30))


def test_shared_prefix_rows_and_pages():
    w = synth.workload(4)
    w = w.with_ctx([4096 + 700, 4096 + 1500, 4096 + 64 * 3 + 320], capacity=16384)
    a, _ = synth.kv_rows(w, 0, 2, 0, 4096)
    b, _ = synth.kv_rows(w, 1, 2, 0, 4096)
    c, _ = synth.kv_rows(w, 1, 2, 4096, 4200)
    d, _ = synth.kv_rows(w, 0, 2, 4096, 4200)
    assert np.array_equal(a, b) and not np.array_equal(c, d)
    table, n_phys = synth.block_table(w)
    assert np.array_equal(table[0, :63], np.arange(63)) and np.array_equal(table[1, :63], np.arange(63))
    used = table[table >= 0]
    private = used[used >= 63]
    assert len(set(private.tolist())) == len(private)
    assert n_phys == 63 + sum(-(-w.hist_len(b) // 64) - 63 for b in range(3))


def test_permuted_pages_are_a_bijection():
    w = synth.workload(3).with_ctx([64 * 40 + 320 + 17])
    table, n_phys = synth.block_table(w)
    row = table[0, :41]
    assert sorted(row.tolist()) == list(range(41)) and n_phys == 41
    assert not np.array_equal(row, np.arange(41))
    assert np.all(table[0, 41:] == -1)


def test_window_rows_for_short_contexts():
    w = synth.workload(2).with_ctx([1, 40, 64, 100, 320, 321, 700])
    for b, L in enumerate(w.ctx_lens):
        k, v = synth.window_rows(w, b, 0)
        full_k, _ = synth.kv_rows(w, b, 0)
        assert len(k) == w.win_len(b) == min(L, 320)
        idx = list(range(min(L, 64))) + list(range(max(min(L, 64), L - 256), L))
        assert np.array_equal(k, full_k[idx])
        assert w.hist_len(b) == max(0, L - 320)
