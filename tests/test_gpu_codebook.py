"""GPU parity of the Lloyd-Max codebook variant (MI355X only), through the C ABI's
*_codebook entry points, against the oracle's codebook demotion and decode.

Codebooks are fitted by the oracle's Lloyd-Max fitter on the first rows of each KV head's
history (K and V separately), plus fixed ones: a skewed pair whose centre is not that of
the uniform levels, and the uniform levels themselves (which must reproduce the uniform
path)."""

from __future__ import annotations

import numpy as np
import pytest

import synth
from gpu_harness import assert_close, compare_history, rotations, windows
from oracle import attention as oatt
from oracle import codebook as ocb
from oracle import pages as opages
from oracle import quant as oquant
from test_gpu_parity import (DECODE_CASES, _demote_all, bf16, custom, make_cache, multi_split_counts, queries, say,
                             wide_splits)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SKEWED = ([0, 5, 30, 48], [2, 20, 27, 41])
UNIFORM = (list(ocb.UNIFORM16), list(ocb.UNIFORM16))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import bit_kv_cache_oscar_amd as ok
    ok.lib()


def fitted(w, rk, rv, n_rows=256):
    """Per KV head, the Lloyd-Max levels (sixteenths) of K and of V, fitted on the first
    n_rows history rows of request 0."""
    ks, vs = [], []
    for kv in range(w.n_kv_heads):
        hk, hv = synth.history_rows(w, 0, kv)
        ks.append(ocb.fit(hk[:n_rows].astype(np.float64), rk[kv], w.clip_ratio))
        vs.append(ocb.fit(hv[:n_rows].astype(np.float64), rv[kv], w.clip_ratio))
    return np.stack(ks), np.stack(vs)


def fixed(w, pair):
    return np.tile(np.array(pair[0]), (w.n_kv_heads, 1)), np.tile(np.array(pair[1]), (w.n_kv_heads, 1))


def oracle_history_cb(rows_k, rows_v, rk, rv, clip, klv, vlv):
    kc, ks, kz, km = ocb.quantize_rows(rows_k.astype(np.float64), rk, clip, klv)
    vc, vs, vz, vm = ocb.quantize_rows(rows_v.astype(np.float64), rv, clip, vlv)
    return (kc, ks, kz, vc, vs, vz), km, vm


def oracle_decode_cb(w, b, rk, rv, hists_b, klv, vlv):
    q = synth.query(w, b).astype(np.float64)
    wk, wv = windows(w, b)
    out = np.zeros((w.n_q_heads, 128))
    for h in range(w.n_q_heads):
        kv = h // w.gq
        out[h] = oatt.decode_head(q[h], rk[kv], rv[kv], wk[kv], wv[kv], hists_b[kv], w.sm_scale,
                                  codebook=(klv[kv], vlv[kv]))
    return out


CB_DECODE_CASES = [("c1", "fitted"), ("c2-4k", "fitted"), ("c5-gq8", "fitted"), ("gq16", "skewed"),
                   ("edges", "skewed"), ("gq1", "fitted"), ("c4-shared-ragged", "fitted")]


@pytest.mark.parametrize("case,book", CB_DECODE_CASES)
def test_codebook_decode_on_oracle_pages(case, book):
    """oscar_decode_codebook on a pool the oracle built with the codebook, at several split
    counts (one of them past 256 workgroups), twice per count."""
    from bit_kv_cache_oscar_amd import oscar_default_splits

    w = DECODE_CASES[case]()
    (rk_bits, rv_bits), (rk, rv) = rotations(w)
    klv, vlv = fitted(w, rk, rv) if book == "fitted" else fixed(w, SKEWED)
    table, n_phys = synth.block_table(w)
    pool = opages.new_pool(n_phys, w.n_kv_heads)
    refs = []
    for b in range(w.batch):
        hists = {}
        for kv in range(w.n_kv_heads):
            hk, hv = synth.history_rows(w, b, kv)
            hist, _, _ = oracle_history_cb(hk, hv, rk[kv], rv[kv], w.clip_ratio, klv[kv], vlv[kv])
            opages.pack_history(pool, table[b], kv, hist)
            hists[kv] = hist
        refs.append(oracle_decode_cb(w, b, rk, rv, hists, klv, vlv))
    c = make_cache(w, rk_bits, rv_bits, table, n_phys)
    c.set_codebook(klv, vlv)
    c.pool.copy_(torch.from_numpy(pool.reshape(-1)))
    q = queries(w)
    splits = {oscar_default_splits(c.desc, w.batch, int(w.hist_lens.max())), 1, 3, wide_splits(w)}
    for s in sorted(x for x in splits if x is not None):
        say(case, book, "codebook decode", "B", w.batch, "Hq", w.n_q_heads, "Hkv", w.n_kv_heads, "splits", s,
            "K levels", klv[0].tolist(), "V levels", vlv[0].tolist())
        c.set_splits(s)
        for rep in range(2):
            c.out.fill_(np.nan)
            got = c.decode_fused(q, w.sm_scale).cpu().numpy()
            for b in range(w.batch):
                assert_close(got[b], refs[b], f"{case} {book} b{b} splits {s} call {rep}")


@pytest.mark.parametrize("n", [1024, 40])
def test_codebook_demote_bitexact(n):
    """oscar_demote_codebook on the tiny workload's history (n >= 64: the matrix-core kernel;
    n < 64: the per-row kernel): scales bit-exact, codes equal outside the exemption band
    around the midpoints between levels."""
    w = synth.workload(1)
    (rk_bits, rv_bits), (rk, rv) = rotations(w)
    table, n_phys = synth.block_table(w)
    klv, vlv = fitted(w, rk, rv)
    c = make_cache(w, rk_bits, rv_bits, table, n_phys, with_windows=False)
    c.set_codebook(klv, vlv)
    hk, hv = synth.history_rows(w, 0, 0)
    hk, hv = hk[:n], hv[:n]
    j = np.arange(n)
    say("codebook demote c1", n, "K levels", klv[0].tolist(), "V levels", vlv[0].tolist())
    _demote_all(c, w, 0, table[0, j // 64], j % 64, hk[:, None, :], hv[:, None, :])
    torch.cuda.synchronize()
    ref, km, vm = oracle_history_cb(hk, hv, rk[0], rv[0], w.clip_ratio, klv[0], vlv[0])
    pool = c.pool.cpu().numpy().reshape(-1, w.n_kv_heads, opages.HEAD_BLOCK)
    got = opages.unpack_history(pool, table[0], 0, n)
    compare_history(got, ref, km, vm, f"codebook c1 n={n}")
    # the levels matter: the uniform codes differ from these
    uc, _, _, _ = oquant.quantize_rows(hk.astype(np.float64), rk[0], w.clip_ratio)
    assert not np.array_equal(uc, ref[0])


def test_codebook_uniform_levels_reproduce_the_uniform_pool():
    """The uniform levels (0, 16, 32, 48) through the codebook entry points demote as
    oscar_demote does (both kernels; codes equal to the oracle's uniform ones outside the
    exemption band, the per-row kernel's bytes identical) and decode to the oracle's
    uniform output."""
    w = custom("cbuni", 8, 2, [64 + 700 + 256], cfg=2)
    (rk_bits, rv_bits), (rk, rv) = rotations(w)
    table, n_phys = synth.block_table(w)
    n = w.hist_len(0)
    rows_k = np.stack([synth.history_rows(w, 0, kv)[0] for kv in range(w.n_kv_heads)], 1)
    rows_v = np.stack([synth.history_rows(w, 0, kv)[1] for kv in range(w.n_kv_heads)], 1)
    j = np.arange(n)
    pools = []
    for use_cb in (False, True):
        c = make_cache(w, rk_bits, rv_bits, table, n_phys)
        if use_cb:
            c.set_codebook(*fixed(w, UNIFORM))
        say("uniform levels, codebook path" if use_cb else "uniform levels, plain path", n)
        _demote_all(c, w, 0, table[0, j[:-30] // 64], j[:-30] % 64, rows_k[:-30], rows_v[:-30])  # bulk
        _demote_all(c, w, 0, table[0, j[-30:] // 64], j[-30:] % 64, rows_k[-30:], rows_v[-30:])  # rows
        torch.cuda.synchronize()
        pool = c.pool.cpu().numpy().reshape(n_phys, w.n_kv_heads, opages.HEAD_BLOCK)
        pools.append(pool.copy())
        c.set_splits(3)
        out = c.decode_fused(queries(w), w.sm_scale).cpu().numpy()
        hists = {}
        for kv in range(w.n_kv_heads):
            kc, ks, kz, km = oquant.quantize_rows(rows_k[:, kv].astype(np.float64), rk[kv], w.clip_ratio)
            vc, vs, vz, vm = oquant.quantize_rows(rows_v[:, kv].astype(np.float64), rv[kv], w.clip_ratio)
            hists[kv] = (kc, ks, kz, vc, vs, vz)
            gpu = opages.unpack_history(pool, table[0], kv, n)
            compare_history(gpu, hists[kv], km, vm, f"uniform levels, codebook path {use_cb}, kv{kv}")
        q = synth.query(w, 0).astype(np.float64)
        wk, wv = windows(w, 0)
        ref = np.stack([oatt.decode_head(q[h], rk[h // w.gq], rv[h // w.gq], wk[h // w.gq], wv[h // w.gq],
                                         hists[h // w.gq], w.sm_scale) for h in range(w.n_q_heads)])
        assert_close(out[0], ref, f"uniform levels, codebook path {use_cb}")
    # the per-row kernel decides every code exactly on both paths: its tokens' bytes agree
    for kv in range(w.n_kv_heads):
        a = opages.unpack_history(pools[0], table[0], kv, n)
        b = opages.unpack_history(pools[1], table[0], kv, n)
        for x, y in zip(a, b):
            assert np.array_equal(np.asarray(x)[-30:], np.asarray(y)[-30:])


def test_codebook_rows_kernel_exact_midpoint_ties():
    """Under R = I with clip 1, rows whose values sit exactly on the midpoints between the
    levels (0, 8, 24, 48) / 16 take the per-row kernel's compensated path: their codes must
    equal the oracle's exactly (the even index wins a midpoint)."""
    w = custom("cbties", 4, 2, [64 + 320], cfg=2)
    table = np.array([[0]], np.int32)
    eye_bits = np.zeros((2, 128, 128), np.uint16)
    eye_bits[:, np.arange(128), np.arange(128)] = 0x3F80
    c = make_cache(w, eye_bits, eye_bits, table, 1, with_windows=False)
    one = np.ones(2, np.float32)
    c.set_rotations(eye_bits, eye_bits, one, one)
    k16 = [0, 8, 24, 48]
    c.set_codebook(np.tile(k16, (2, 1)), np.tile([1, 9, 30, 47], (2, 1)))
    ties = np.resize(np.array([3.0, 0.0, 0.25, 1.0, 2.25, 0.2, 1.1, 2.3]), 128)            # s = 1, z = 0
    ties_v = np.resize(np.array([3.0, 0.0, 5 / 16, 39 / 32, 77 / 32, 2.0, 0.5]), 128)      # midpoints of V's levels
    plain = np.resize(np.array([-1.0, -0.375, 0.25, 0.625, 2.0]), 128)
    rows_k = np.stack([ties, plain, ties[::-1].copy()])[:, None, :].repeat(2, 1).astype(np.float32)
    rows_v = np.stack([ties_v, plain[::-1].copy(), ties_v[::-1].copy()])[:, None, :].repeat(2, 1).astype(np.float32)
    m = len(rows_k)
    j = np.arange(m)
    say("codebook rows kernel, exact midpoint ties", m)
    _demote_all(c, w, 0, table[0, j // 64], j % 64, rows_k, rows_v)
    torch.cuda.synchronize()
    pool = c.pool.cpu().numpy().reshape(1, 2, opages.HEAD_BLOCK)
    for kv in range(2):
        ref, km, vm = oracle_history_cb(rows_k[:, kv], rows_v[:, kv], np.eye(128), np.eye(128), 1.0, k16,
                                        [1, 9, 30, 47])
        got = opages.unpack_history(pool, table[0], kv, m)
        compare_history(got, ref, km, vm, f"codebook ties head {kv}")
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[3], ref[3]), "tie codes differ"
        assert np.any(km == 0.0) and np.any(vm == 0.0), "the rows must hold exact ties"


@pytest.mark.parametrize("case", ["c2-4k", "c5-gq8", "gq16"])
def test_codebook_step_demotes_then_decodes(case):
    """oscar_decode_step_codebook: all history tokens but the last through
    oscar_demote_codebook, the last through the step, which then decodes; pool bytes and
    output against the oracle's codebook demotion and decode."""
    from bit_kv_cache_oscar_amd import oscar_default_splits

    w = DECODE_CASES[case]()
    (rk_bits, rv_bits), (rk, rv) = rotations(w)
    klv, vlv = fitted(w, rk, rv)
    table, n_phys = synth.block_table(w)
    c = make_cache(w, rk_bits, rv_bits, table, n_phys)
    c.set_codebook(klv, vlv)
    last_k, last_v, last_p, last_s = [], [], [], []
    rows = {}
    for b in range(w.batch):
        n = w.hist_len(b)
        ks = np.stack([synth.history_rows(w, b, kv)[0] for kv in range(w.n_kv_heads)], 1)
        vs = np.stack([synth.history_rows(w, b, kv)[1] for kv in range(w.n_kv_heads)], 1)
        rows[b] = (ks, vs)
        j = np.arange(n)
        _demote_all(c, w, b, table[b, j[:-1] // 64], j[:-1] % 64, ks[:-1], vs[:-1])
        last_k.append(ks[-1])
        last_v.append(vs[-1])
        last_p.append(table[b, (n - 1) // 64])
        last_s.append((n - 1) % 64)
    s = oscar_default_splits(c.desc, w.batch, int(w.hist_lens.max()))
    c.set_splits(s)
    dev = torch.device("cuda")
    kr, vr = bf16(np.stack(last_k)), bf16(np.stack(last_v))
    pg = torch.tensor(last_p, dtype=torch.int32, device=dev)
    sl = torch.tensor(last_s, dtype=torch.int32, device=dev)
    say(case, "codebook step", "B", w.batch, "splits", s)
    got = c.step(kr, vr, pg, sl, queries(w), w.sm_scale).cpu().numpy()
    pool = c.pool.cpu().numpy().reshape(n_phys, w.n_kv_heads, opages.HEAD_BLOCK)
    for b in range(w.batch):
        hists = {}
        for kv in range(w.n_kv_heads):
            ks, vs = rows[b]
            ref, km, vm = oracle_history_cb(ks[:, kv], vs[:, kv], rk[kv], rv[kv], w.clip_ratio, klv[kv], vlv[kv])
            gpu = opages.unpack_history(pool, table[b], kv, w.hist_len(b))
            compare_history(gpu, ref, km, vm, f"{case} codebook b{b} kv{kv}")
            hists[kv] = ref
        assert_close(got[b], oracle_decode_cb(w, b, rk, rv, hists, klv, vlv), f"{case} codebook step b{b}")


# every KV head of the 32K workload; four pairs of the 100K and 128K workloads, the last
# request and the last KV head among them
FULL_SAMPLES_CB = {2: [(0, kv) for kv in range(8)], 3: [(0, 0), (0, 3), (0, 6), (0, 7)],
                   5: [(0, 0), (1, 4), (2, 1), (3, 7)]}


@pytest.mark.parametrize("cfg", [2, 3, 5])
def test_codebook_full_size_end_to_end_sampled(cfg):
    """The codebook variant at the workload's real size, as the benchmark runs it: per-head
    codebooks fitted on the calibration set, every history token demoted on the GPU against
    them, then oscar_decode_codebook with the default split count; sampled KV heads compared
    with the oracle (pool bytes and their query heads' outputs)."""
    from bit_kv_cache_oscar_amd import oscar_default_splits

    w = synth.workload(cfg)
    (rk_bits, rv_bits), (rk, rv) = rotations(w)
    cal = [synth.calibration_set(w, kv) for kv in range(w.n_kv_heads)]
    klv = np.stack([ocb.fit(cal[kv][1], rk[kv], w.clip_ratio) for kv in range(w.n_kv_heads)])
    vlv = np.stack([ocb.fit(cal[kv][2], rv[kv], w.clip_ratio) for kv in range(w.n_kv_heads)])
    table, n_phys = synth.block_table(w)
    c = make_cache(w, rk_bits, rv_bits, table, n_phys)
    c.set_codebook(klv, vlv)
    say("codebook full size", w.name, "pages", n_phys, "K levels", klv[0].tolist(), "V levels", vlv[0].tolist())
    for b in range(w.batch):
        n = w.hist_len(b)
        ks = np.stack([synth.kv_rows(w, b, kv, 64, 64 + n)[0] for kv in range(w.n_kv_heads)], 1)
        vs = np.stack([synth.kv_rows(w, b, kv, 64, 64 + n)[1] for kv in range(w.n_kv_heads)], 1)
        j = np.arange(n)
        _demote_all(c, w, b, table[b, j // 64], j % 64, ks, vs)
    s = oscar_default_splits(c.desc, w.batch, int(w.hist_lens.max()))
    c.set_splits(s)
    got = c.decode_fused(queries(w), w.sm_scale).cpu().numpy()
    pool = c.pool.cpu().numpy().reshape(n_phys, w.n_kv_heads, opages.HEAD_BLOCK)
    for b, kv in FULL_SAMPLES_CB[cfg]:
        say("codebook full size sample", w.name, "b", b, "kv", kv, "splits", s)
        hk, hv = synth.history_rows(w, b, kv)
        ref, km, vm = oracle_history_cb(hk, hv, rk[kv], rv[kv], w.clip_ratio, klv[kv], vlv[kv])
        gpu = opages.unpack_history(pool, table[b], kv, w.hist_len(b))
        compare_history(gpu, ref, km, vm, f"{w.name} codebook b{b} kv{kv}")
        q = synth.query(w, b).astype(np.float64)
        wk, wv = windows(w, b)
        for h in range(kv * w.gq, (kv + 1) * w.gq):
            r = oatt.decode_head(q[h], rk[kv], rv[kv], wk[kv], wv[kv], ref, w.sm_scale, codebook=(klv[kv], vlv[kv]))
            assert_close(got[b, h], r, f"{w.name} codebook b{b} h{h}")


@pytest.mark.parametrize("case,n_tok,book", [("c2-4k", 4, "fitted"), ("c5-gq8", 2, "skewed"), ("edges", 2, "fitted")])
def test_codebook_multi_query_on_oracle_pages(case, n_tok, book):
    """oscar_decode_multi_codebook: T query tokens per request over a codebook pool built by
    the oracle, causal over the window, twice per split count."""
    from bit_kv_cache_oscar_amd import oscar_decode_multi_codebook, oscar_decode_workspace_bytes

    w = DECODE_CASES[case]()
    (rk_bits, rv_bits), (rk, rv) = rotations(w)
    klv, vlv = fitted(w, rk, rv) if book == "fitted" and w.hist_len(0) > 0 else fixed(w, SKEWED)
    table, n_phys = synth.block_table(w)
    pool = opages.new_pool(n_phys, w.n_kv_heads)
    hists = []
    for b in range(w.batch):
        hb = []
        for kv in range(w.n_kv_heads):
            hk, hv = synth.history_rows(w, b, kv)
            hist, _, _ = oracle_history_cb(hk, hv, rk[kv], rv[kv], w.clip_ratio, klv[kv], vlv[kv])
            opages.pack_history(pool, table[b], kv, hist)
            hb.append(hist)
        hists.append(hb)
    c = make_cache(w, rk_bits, rv_bits, table, n_phys)
    c.set_codebook(klv, vlv)
    c.pool.copy_(torch.from_numpy(pool.reshape(-1)))
    qn = np.stack([synth.query_tokens(w, b, n_tok) for b in range(w.batch)])
    q = bf16(qn)
    books = [(klv[kv], vlv[kv]) for kv in range(w.n_kv_heads)]
    refs = []
    for b in range(w.batch):
        wk, wv = windows(w, b)
        refs.append(oatt.decode_multi(qn[b].astype(np.float64), rk, rv, wk, wv, hists[b], w.sm_scale, codebooks=books))
    for s in sorted(multi_split_counts(c.desc, w, n_tok)):
        ws = torch.zeros(oscar_decode_workspace_bytes(c.desc, w.batch * n_tok, s), dtype=torch.uint8, device="cuda")
        out = torch.empty((w.batch, n_tok, w.n_q_heads, 128), dtype=torch.float32, device="cuda")
        for rep in range(2):
            say(case, book, "codebook multi-query", "T", n_tok, "splits", s, "call", rep)
            out.fill_(np.nan)
            oscar_decode_multi_codebook(c.desc, q, c.rot_k, c.rot_v, c.codebook, c.pool, c.block_table, c.hist_len,
                                        c.k_win, c.v_win, c.win_len, w.sm_scale, s, ws, out)
            got = out.cpu().numpy()
            for b in range(w.batch):
                for t in range(n_tok):
                    assert_close(got[b, t], refs[b][t], f"{case} codebook multi b{b} t{t} splits {s} call {rep}")
