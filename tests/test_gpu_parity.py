"""GPU parity: every entry point against the oracle on seeded inputs (MI355X only).

Decode is checked on pools the oracle built (so demotion tolerances cannot leak into
decode parity), entry point by entry point and end to end; demotion is checked byte
by byte; the full-size workloads run the whole GPU path (demote every history token,
then decode) in the launch configuration the benchmark uses and are compared on
sampled KV heads."""

from __future__ import annotations

import numpy as np
import pytest

import synth
from gpu_harness import (assert_close, bits_to_f64, clips, compare_history, oracle_decode, oracle_history,
                         oracle_pool, rotations, windows)
from oracle import attention as oatt
from oracle import pages as opages

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import bit_kv_cache_oscar_amd as ok
    ok.lib()  # fails loudly if the library is not built


def say(*a):
    print("[case]", *a, flush=True)


def bf16(x) -> "torch.Tensor":
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda().to(torch.bfloat16)


def make_cache(w, rk_bits, rv_bits, table, n_phys, with_windows=True):
    from bit_kv_cache_oscar_amd.layer import LayerCache

    c = LayerCache(w.n_q_heads, w.n_kv_heads, w.batch, table.shape[1], n_phys)
    ck, cv = clips(w)
    c.set_rotations(rk_bits, rv_bits, ck, cv)
    c.set_block_table(table)
    c.set_hist_len(w.hist_lens)
    if with_windows:
        for b in range(w.batch):
            for kv in range(w.n_kv_heads):
                k, v = synth.window_rows(w, b, kv)
                c.set_window(b, kv, k, v)
        c.set_win_len(w.win_lens)
    return c


def queries(w):
    return bf16(np.stack([synth.query(w, b) for b in range(w.batch)]))


def custom(name, hq, hkv, ctx, cfg=2, **kw):
    base = synth.workload(cfg)
    return synth.Workload(cfg, name, len(ctx), hq, hkv, tuple(ctx), max(ctx),
                          outlier_fixed=base.outlier_fixed, **kw)


DECODE_CASES = {
    "c1": lambda: synth.workload(1),
    "c2-4k": lambda: synth.workload(2).with_ctx([4000]),
    "c3-6k-permuted": lambda: synth.workload(3).with_ctx([6000]),
    "c4-shared-ragged": lambda: synth.workload(4).with_ctx([4596, 5096, 3000, 4096 + 128 + 320 + 3], capacity=6000),
    "c5-gq8": lambda: synth.workload(5).with_ctx([3000, 2600]),
    "gq16": lambda: custom("gq16", 32, 2, [2500, 900]),
    "gq2": lambda: custom("gq2", 16, 8, [1500]),
    "edges": lambda: custom("edges", 8, 2, [100, 320, 321, 64 * 3 + 320, 1, 0 + 64 * 1 + 320 + 63]),
    "gq1": lambda: custom("gq1", 4, 4, [900, 1700]),
}


def wide_splits(w):
    """The smallest split count whose decode grid exceeds 256 workgroups (the fused decode
    then runs 4 waves per workgroup instead of 8), or None past the 256-split limit."""
    groups = w.batch * w.n_kv_heads * (w.gq // 8 if w.gq > 8 else 1)
    s = 256 // groups + 1
    return s if s <= 256 else None


@pytest.mark.parametrize("case", list(DECODE_CASES))
def test_decode_on_oracle_pages(case):
    w = DECODE_CASES[case]()
    (rk_bits, rv_bits), (rk, rv) = rotations(w)
    assert np.array_equal(bits_to_f64(rk_bits), rk) and np.array_equal(bits_to_f64(rv_bits), rv)
    pool, table, hists = oracle_pool(w, rk, rv)
    refs = [oracle_decode(w, b, rk, rv, hists[b]) for b in range(w.batch)]
    from bit_kv_cache_oscar_amd import oscar_default_splits

    c = make_cache(w, rk_bits, rv_bits, table, pool.shape[0])
    c.pool.copy_(torch.from_numpy(pool.reshape(-1)))
    q = queries(w)
    max_pages = int(np.max(-(-w.hist_lens // 64))) if w.batch else 0
    splits = {oscar_default_splits(c.desc, w.batch, int(w.hist_lens.max())), 1, 3, max_pages + 5, wide_splits(w)}
    for s in sorted(x for x in splits if x is not None):
        say(case, "decode", "B", w.batch, "Hq", w.n_q_heads, "Hkv", w.n_kv_heads, "ctx", w.ctx_lens, "splits", s)
        c.set_splits(s)
        out = c.decode(q, w.sm_scale)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        for b in range(w.batch):
            assert_close(got[b], refs[b], f"{case} b{b} splits {s}")
        # the two-launch path, twice in a row (its arrival counters must re-arm between calls)
        for rep in range(2):
            c.out.fill_(np.nan)
            got = c.decode_fused(q, w.sm_scale).cpu().numpy()
            for b in range(w.batch):
                assert_close(got[b], refs[b], f"{case} b{b} splits {s} fused call {rep}")


MULTI_CASES = {
    "c2-4k-T2": ("c2-4k", 2),
    "c2-4k-T4": ("c2-4k", 4),
    "gq2-T8": ("gq2", 8),
    "edges-T2": ("edges", 2),
    "c5-gq8-T2": ("c5-gq8", 2),
}


def multi_split_counts(desc, w, n_tok):
    """Split counts a multi-query test runs: the two-launch default, the one-launch count,
    3, and the smallest count whose grid no longer fits one launch (the two-launch path)."""
    from bit_kv_cache_oscar_amd import oscar_decode_multi_splits, oscar_default_splits, oscar_window_splits

    mh = int(w.hist_lens.max())
    gqt = w.n_q_heads // w.n_kv_heads * n_tok
    per_split = w.n_kv_heads * w.batch * (2 if gqt > 8 else 1)
    fixed = ((oscar_window_splits(desc) + 1) // 2 + 1) * w.n_kv_heads * w.batch
    two = max(1, (256 - fixed) // per_split + 1)
    return {oscar_default_splits(desc, w.batch, mh), oscar_decode_multi_splits(desc, w.batch, n_tok, mh), 3,
            min(two, 255)}


@pytest.mark.parametrize("name", list(MULTI_CASES))
def test_decode_multi_on_oracle_pages(name):
    """T query tokens per request over one pool: token t sees the whole history and the window
    up to its own position. The virtual (token, head) rows fill the fused kernels' head tiles
    (T x query heads per KV head up to 16, two head groups at 16)."""
    from bit_kv_cache_oscar_amd import oscar_decode_multi, oscar_decode_workspace_bytes, oscar_default_splits

    case, n_tok = MULTI_CASES[name]
    w = DECODE_CASES[case]()
    (rk_bits, rv_bits), (rk, rv) = rotations(w)
    pool, table, hists = oracle_pool(w, rk, rv)
    c = make_cache(w, rk_bits, rv_bits, table, pool.shape[0])
    c.pool.copy_(torch.from_numpy(pool.reshape(-1)))
    qn = np.stack([synth.query_tokens(w, b, n_tok) for b in range(w.batch)])
    q = bf16(qn)
    refs = []
    for b in range(w.batch):
        wk, wv = windows(w, b)
        refs.append(oatt.decode_multi(qn[b].astype(np.float64), rk, rv, wk, wv, hists[b], w.sm_scale))
    splits = multi_split_counts(c.desc, w, n_tok)
    for s in sorted(splits):
        ws = torch.zeros(oscar_decode_workspace_bytes(c.desc, w.batch * n_tok, s), dtype=torch.uint8, device="cuda")
        out = torch.empty((w.batch, n_tok, w.n_q_heads, 128), dtype=torch.float32, device="cuda")
        for rep in range(2):  # twice: the arrival counters must re-arm
            say(name, "multi-query decode", "B", w.batch, "T", n_tok, "Hq", w.n_q_heads, "splits", s, "call", rep)
            out.fill_(np.nan)
            oscar_decode_multi(c.desc, q, c.rot_k, c.rot_v, c.pool, c.block_table, c.hist_len, c.k_win, c.v_win,
                               c.win_len, w.sm_scale, s, ws, out)
            got = out.cpu().numpy()
            for b in range(w.batch):
                for t in range(n_tok):
                    assert_close(got[b, t], refs[b][t], f"{name} b{b} t{t} splits {s} call {rep}")
    # the last token of each request is a one-token decode of the same pool
    c.set_splits(max(splits))
    single = c.decode_fused(q[:, -1].contiguous(), w.sm_scale).cpu().numpy()
    for b in range(w.batch):
        assert_close(single[b], refs[b][-1], f"{name} b{b} one-token decode")


def _split_bounds(nh, s_total):
    n_pages = -(-nh // 64)
    pps = -(-n_pages // s_total) if s_total else 0
    out = []
    for s in range(s_total):
        a = min(nh, s * pps * 64)
        z = min(nh, (s + 1) * pps * 64)
        out.append((a, max(a, z)))
    return out


def _partials(buf, batch, hq, splits):
    raw = buf.cpu().numpy().view(np.float32)
    n = batch * hq * splits
    acc_off = -(-8 * n // 256) * 256 // 4
    m = raw[:n].reshape(batch, hq, splits)
    l = raw[n:2 * n].reshape(batch, hq, splits)
    acc = raw[acc_off:acc_off + n * 128].reshape(batch, hq, splits, 128)
    return m, l, acc


def _check_partial(gm, gl, gacc, ref, what):
    m, l, acc = ref
    if l == 0.0:
        assert gm == -np.inf and gl == 0.0 and not np.any(gacc), what
        return
    assert abs(gm / LOG2E - m) <= 1e-5 * max(1.0, abs(m)), what
    assert abs(gl - l) <= 1e-4 * l, what
    assert_close(gacc / gl, acc / l, what)


def test_int2_partials_match_oracle():
    from bit_kv_cache_oscar_amd import oscar_decode_int2, oscar_partials_bytes

    w = synth.workload(2).with_ctx([4000, 2000])
    (rk_bits, rv_bits), (rk, rv) = rotations(w)
    pool, table, hists = oracle_pool(w, rk, rv)
    c = make_cache(w, rk_bits, rv_bits, table, pool.shape[0], with_windows=False)
    c.pool.copy_(torch.from_numpy(pool.reshape(-1)))
    S = 7
    buf = torch.zeros(oscar_partials_bytes(c.desc, w.batch, S), dtype=torch.uint8, device="cuda")
    q = queries(w)
    say("int2 partials", w.ctx_lens, "splits", S)
    oscar_decode_int2(c.desc, q, c.rot_k, c.pool, c.block_table, c.hist_len, w.sm_scale, S, buf)
    torch.cuda.synchronize()
    gm, gl, gacc = _partials(buf, w.batch, w.n_q_heads, S)
    for b in range(w.batch):
        qb = synth.query(w, b).astype(np.float64)
        bounds = _split_bounds(w.hist_len(b), S)
        for h in range(0, w.n_q_heads, 5):
            kv = h // w.gq
            refs = oatt.history_partials(qb[h], rk[kv], hists[b][kv], w.sm_scale, bounds)
            for s, ref in enumerate(refs):
                _check_partial(gm[b, h, s], gl[b, h, s], gacc[b, h, s], ref, f"b{b} h{h} s{s}")


def test_bf16_partials_match_oracle():
    from bit_kv_cache_oscar_amd import oscar_decode_bf16, oscar_partials_bytes, oscar_window_splits

    w = custom("win", 32, 8, [5000, 70, 320, 1])
    (rk_bits, rv_bits), _ = rotations(w)
    table, n_phys = synth.block_table(w)
    c = make_cache(w, rk_bits, rv_bits, table, n_phys)
    ws = oscar_window_splits(c.desc)
    buf = torch.zeros(oscar_partials_bytes(c.desc, w.batch, ws), dtype=torch.uint8, device="cuda")
    q = queries(w)
    say("bf16 partials", w.ctx_lens)
    oscar_decode_bf16(c.desc, q, c.k_win, c.v_win, c.win_len, w.sm_scale, buf)
    torch.cuda.synchronize()
    gm, gl, gacc = _partials(buf, w.batch, w.n_q_heads, ws)
    for b in range(w.batch):
        qb = synth.query(w, b).astype(np.float64)
        wk, wv = windows(w, b)
        bounds = [(min(64 * i, w.win_len(b)), min(64 * i + 64, w.win_len(b))) for i in range(ws)]
        for h in range(0, w.n_q_heads, 3):
            kv = h // w.gq
            refs = oatt.window_partials(qb[h], wk[kv], wv[kv], w.sm_scale, bounds)
            for s, ref in enumerate(refs):
                _check_partial(gm[b, h, s], gl[b, h, s], gacc[b, h, s], ref, f"b{b} h{h} c{s}")


def test_merge_of_oracle_partials():
    from bit_kv_cache_oscar_amd import oscar_merge, oscar_partials_bytes, oscar_window_splits, layer_desc

    g = np.random.default_rng(11)
    B, HQ, HKV, S = 3, 8, 2, 5
    desc = layer_desc(HQ, HKV)
    ws = oscar_window_splits(desc)
    w = custom("merge", HQ, HKV, [2000] * B)
    (_, rv_bits), (_, rv) = rotations(w)

    def fill(splits, empty_rate):
        n = B * HQ * splits
        m = g.normal(0, 20, n)
        l = g.uniform(0.5, 50, n)
        acc = g.normal(0, 3, (n, 128)) * l[:, None]
        empty = g.random(n) < empty_rate
        m[empty], l[empty], acc[empty] = -np.inf, 0.0, 0.0
        return m, l, acc

    hm, hl, hacc = fill(S, 0.3)
    wm, wl, wacc = fill(ws, 0.3)
    # one (b, h) with everything empty: output 0
    for arr in (hm,):
        arr[:S] = -np.inf
    hl[:S], hacc[:S] = 0.0, 0.0
    wm[:ws], wl[:ws], wacc[:ws] = -np.inf, 0.0, 0.0

    def pack(m, l, acc, splits):
        n = B * HQ * splits
        buf = np.zeros(oscar_partials_bytes(desc, B, splits), np.uint8)
        f = buf.view(np.float32)
        f[:n] = (m * LOG2E).astype(np.float32)
        f[n:2 * n] = l
        off = -(-8 * n // 256) * 256 // 4
        f[off:off + n * 128] = acc.reshape(-1)
        return torch.from_numpy(buf).cuda()

    out = torch.zeros((B, HQ, 128), dtype=torch.float32, device="cuda")
    rvt = bf16(bits_to_f64(rv_bits).astype(np.float32))
    say("merge", B, HQ, HKV, S)
    oscar_merge(desc, pack(hm, hl, hacc, S), S, pack(wm, wl, wacc, ws), rvt, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b in range(B):
        for h in range(HQ):
            i = (b * HQ + h)
            hp = [(hm[i * S + s], hl[i * S + s], hacc[i * S + s]) for s in range(S)]
            wp = [(wm[i * ws + s], wl[i * ws + s], wacc[i * ws + s]) for s in range(ws)]
            # the GPU sees m rounded to float32 in log2 units; use the same m on the oracle side
            hp = [(float(np.float32(m * LOG2E)) / LOG2E, l, a) for m, l, a in hp]
            wp = [(float(np.float32(m * LOG2E)) / LOG2E, l, a) for m, l, a in wp]
            ref = oatt.merge_segments(hp, wp, rv[h // (HQ // HKV)])
            assert_close(got[b, h], ref, f"merge b{b} h{h}")
    assert not np.any(got[0, 0])


# ------------------------------------------------------------------------------ demotion


def _demote_all(c, w, b, pages_np, slots_np, rows_k, rows_v, chunk=1 << 16):
    pages_t = torch.from_numpy(pages_np.astype(np.int32)).cuda()
    slots_t = torch.from_numpy(slots_np.astype(np.int32)).cuda()
    for a in range(0, len(pages_np), chunk):
        z = min(len(pages_np), a + chunk)
        c.demote(bf16(rows_k[a:z]), bf16(rows_v[a:z]), pages_t[a:z], slots_t[a:z])


def _gpu_head_history(c, w, table_row, kv, n):
    pool = c.pool.cpu().numpy().reshape(-1, w.n_kv_heads, opages.HEAD_BLOCK)
    return opages.unpack_history(pool, table_row, kv, n)


def test_demote_config1_bitexact():
    w = synth.workload(1)
    (rk_bits, rv_bits), (rk, rv) = rotations(w)
    table, n_phys = synth.block_table(w)
    c = make_cache(w, rk_bits, rv_bits, table, n_phys, with_windows=False)
    n = w.hist_len(0)
    hk, hv = synth.history_rows(w, 0, 0)
    j = np.arange(n)
    say("demote c1", n)
    _demote_all(c, w, 0, table[0, j // 64], j % 64, hk[:, None, :], hv[:, None, :])
    torch.cuda.synchronize()
    ref, km, vm = oracle_history(w, 0, 0, rk, rv)
    flips = compare_history(_gpu_head_history(c, w, table[0], 0, n), ref, km, vm, "c1")
    assert flips == 0


def test_demote_random_order_on_stale_pages_and_overwrite():
    w = custom("stale", 8, 4, [64 * 3 + 320], cfg=2)
    (rk_bits, rv_bits), (rk, rv) = rotations(w)
    n_phys = 5
    table = np.array([[4, 1, 3]], np.int32)
    c = make_cache(w, rk_bits, rv_bits, table, n_phys, with_windows=False)
    g = np.random.default_rng(5)
    stale = g.integers(0, 256, n_phys * w.n_kv_heads * opages.HEAD_BLOCK, dtype=np.uint8)
    c.pool.copy_(torch.from_numpy(stale))
    n = 192
    rows_k = np.stack([synth.history_rows(w, 0, kv)[0] for kv in range(w.n_kv_heads)], 1)
    rows_v = np.stack([synth.history_rows(w, 0, kv)[1] for kv in range(w.n_kv_heads)], 1)
    order = g.permutation(n)
    say("demote stale pages, random order", n)
    for half in (order[:n // 2], order[n // 2:]):
        _demote_all(c, w, 0, table[0, half // 64], half % 64, rows_k[half], rows_v[half])
    # overwrite 40 slots with other rows
    redo = g.choice(n, 40, replace=False)
    other_k = rows_k[::-1].copy()
    other_v = rows_v[::-1].copy()
    _demote_all(c, w, 0, table[0, redo // 64], redo % 64, other_k[redo], other_v[redo])
    torch.cuda.synchronize()
    final_k, final_v = rows_k.copy(), rows_v.copy()
    final_k[redo], final_v[redo] = other_k[redo], other_v[redo]
    pool = c.pool.cpu().numpy().reshape(n_phys, w.n_kv_heads, opages.HEAD_BLOCK)
    from oracle import quant as oquant
    for kv in range(w.n_kv_heads):
        kc, ks, kz, km = oquant.quantize_rows(final_k[:, kv].astype(np.float64), rk[kv], w.clip_ratio)
        vc, vs, vz, vm = oquant.quantize_rows(final_v[:, kv].astype(np.float64), rv[kv], w.clip_ratio)
        got = opages.unpack_history(pool, table[0], kv, n)
        assert compare_history(got, (kc, ks, kz, vc, vs, vz), km, vm, f"head {kv}") == 0
    # untouched physical pages keep their bytes
    stale3 = stale.reshape(n_phys, w.n_kv_heads, opages.HEAD_BLOCK)
    assert np.array_equal(pool[0], stale3[0]) and np.array_equal(pool[2], stale3[2])


def test_demote_degenerate_rows():
    w = custom("degenerate", 4, 2, [64 + 320], cfg=2)
    (rk_bits, rv_bits), (rk, rv) = rotations(w)
    table = np.array([[0]], np.int32)
    c = make_cache(w, rk_bits, rv_bits, table, 1, with_windows=False)
    g = np.random.default_rng(6)
    rows = g.standard_normal((64, 2, 128)).astype(np.float32)
    rows[0] = 0.0
    rows[1] = 1.5
    rows[2, :, 7] = 3000.0
    rows[3] *= 1e-6
    rows = synth.to_bf16_values(rows)
    j = np.arange(64)
    say("demote degenerate rows")
    _demote_all(c, w, 0, table[0, j // 64], j % 64, rows, rows[::-1].copy())
    torch.cuda.synchronize()
    pool = c.pool.cpu().numpy().reshape(1, 2, opages.HEAD_BLOCK)
    from oracle import quant as oquant
    for kv in range(2):
        kc, ks, kz, km = oquant.quantize_rows(rows[:, kv].astype(np.float64), rk[kv], w.clip_ratio)
        vc, vs, vz, vm = oquant.quantize_rows(rows[::-1][:, kv].astype(np.float64), rv[kv], w.clip_ratio)
        got = opages.unpack_history(pool, table[0], kv, 64)
        assert compare_history(got, (kc, ks, kz, vc, vs, vz), km, vm, f"head {kv}") == 0
        assert ks[0] == 0 and got[1][0] == 0


def test_demote_rows_kernel_random_and_exact_ties():
    """Fewer than 64 tokens go through the per-row kernel. Random rows under the workload's
    rotations; then rows under R = I with clip 1 whose rotated values sit exactly on code
    boundaries (they round half to even) or whose minimum is exactly 0, where the kernel's
    error intervals cannot settle the decision and its compensated path decides: those
    codes must equal the oracle's exactly."""
    w = custom("rows", 4, 2, [64 + 320], cfg=2)
    (rk_bits, rv_bits), (rk, rv) = rotations(w)
    table = np.array([[0]], np.int32)
    c = make_cache(w, rk_bits, rv_bits, table, 1, with_windows=False)
    g = np.random.default_rng(8)
    n = 40
    rows_k = g.standard_normal((n, 2, 128)).astype(np.float32) * 3
    rows_v = g.standard_normal((n, 2, 128)).astype(np.float32)
    rows_k[5, :, 3] = 40.0  # an outlier channel
    rows_k[7] *= 1e-6       # fp16 subnormal scale and zero point
    rows_v[9] *= 2e-8       # scale near half the smallest fp16 subnormal
    rows_k, rows_v = synth.to_bf16_values(rows_k), synth.to_bf16_values(rows_v)
    j = np.arange(n)
    say("demote rows kernel, random", n)
    _demote_all(c, w, 0, table[0, j // 64], j % 64, rows_k, rows_v)
    torch.cuda.synchronize()
    pool = c.pool.cpu().numpy().reshape(1, 2, opages.HEAD_BLOCK)
    from oracle import quant as oquant
    for kv in range(2):
        kc, ks, kz, km = oquant.quantize_rows(rows_k[:, kv].astype(np.float64), rk[kv], w.clip_ratio)
        vc, vs, vz, vm = oquant.quantize_rows(rows_v[:, kv].astype(np.float64), rv[kv], w.clip_ratio)
        got = opages.unpack_history(pool, table[0], kv, n)
        assert compare_history(got, (kc, ks, kz, vc, vs, vz), km, vm, f"rows head {kv}") == 0

    eye_bits = np.zeros((2, 128, 128), np.uint16)
    eye_bits[:, np.arange(128), np.arange(128)] = 0x3F80
    one = np.ones(2, np.float32)
    c.set_rotations(eye_bits, eye_bits, one, one)
    ties_a = np.resize(np.array([0.0, 0.5, 1.0, 1.5, 2.0, 2.5, 3.0]), 128)       # min exactly 0, s = 1
    ties_b = np.resize(np.array([-1.0, -0.5, 0.0, 0.5, 1.0, 1.5, 2.0]), 128)     # z = -1, s = 1
    plain = np.resize(np.array([-1.0, -0.375, 0.25, 0.625, 2.0]), 128)           # no value near a boundary
    rows = np.stack([ties_a, ties_b, plain, ties_b[::-1].copy()])[:, None, :].repeat(2, 1).astype(np.float32)
    m = len(rows)
    j = np.arange(n, n + m)
    say("demote rows kernel, exact ties", m)
    _demote_all(c, w, 0, table[0, j // 64], j % 64, rows, rows[::-1].copy())
    torch.cuda.synchronize()
    pool = c.pool.cpu().numpy().reshape(1, 2, opages.HEAD_BLOCK)
    for kv in range(2):
        kc, ks, kz, km = oquant.quantize_rows(rows[:, kv].astype(np.float64), np.eye(128), 1.0)
        vc, vs, vz, vm = oquant.quantize_rows(rows[::-1][:, kv].astype(np.float64), np.eye(128), 1.0)
        got = opages.unpack_history(pool, table[0], kv, n + m)
        got = tuple(a[n:] for a in got)
        compare_history(got, (kc, ks, kz, vc, vs, vz), km, vm, f"ties head {kv}")
        assert np.array_equal(got[0], kc) and np.array_equal(got[3], vc), "tie codes differ"
        assert np.any(km == 0.0), "the rows must hold exact ties"


# ------------------------------------------------------------------- full-size workloads

# (request, KV head) pairs compared at full size: every KV head of the batch-1 workloads;
# at batch 64 and at 128K, ten and eight pairs spread over requests and heads, the last
# request and the last KV head among them
FULL_PAIRS = {
    2: [(0, kv) for kv in range(8)],
    3: [(0, kv) for kv in range(8)],
    4: [(0, 0), (7, 3), (15, 6), (22, 1), (31, 4), (40, 2), (48, 7), (56, 5), (63, 0), (63, 7)],
    5: [(0, 0), (0, 7), (1, 2), (1, 5), (2, 1), (2, 6), (3, 3), (3, 7)],
}


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_full_size_benchmarked_path(cfg):
    """The whole GPU path at the workload's real size, in the launch configuration the
    benchmark times: every history token but the last demoted through oscar_demote (the
    bulk kernel), then oscar_decode_step at the library's default split count, which
    demotes the last token of each request and decodes in two launches (prepare; attend =
    INT2 pass with the in-launch ticket merge). Then the attend launch alone, twice, on the
    workspace the step prepared (what the benchmark's roofline row times), oscar_decode
    (the two launches without demotion), the three separate passes, the one-launch step
    and the multi-query decode at the benchmark's T and split count. Pool bytes and the
    outputs of every query head (and query token) of the listed (request, KV head) pairs
    are compared with the oracle; every path must meet the decode tolerance."""
    from bit_kv_cache_oscar_amd import oscar_attend, oscar_default_splits

    w = synth.workload(cfg)
    (rk_bits, rv_bits), (rk, rv) = rotations(w)
    table, n_phys = synth.block_table(w)
    c = make_cache(w, rk_bits, rv_bits, table, n_phys)
    say("full size", w.name, "pages", n_phys)
    last_k, last_v, last_p, last_s = [], [], [], []
    for b in range(w.batch):
        n = w.hist_len(b)
        start = min(n, w.shared_pages * 64) if (w.shared_pages and b > 0) else 0
        assert n - 1 > start
        ks, vs = [], []
        for kv in range(w.n_kv_heads):
            k, v = synth.kv_rows(w, b, kv, 64 + start, 64 + n)
            ks.append(k)
            vs.append(v)
        ks, vs = np.stack(ks, 1), np.stack(vs, 1)
        j = np.arange(start, n)
        _demote_all(c, w, b, table[b, j[:-1] // 64], j[:-1] % 64, ks[:-1], vs[:-1])
        last_k.append(ks[-1])
        last_v.append(vs[-1])
        last_p.append(table[b, (n - 1) // 64])
        last_s.append((n - 1) % 64)
        del ks, vs
    s = oscar_default_splits(c.desc, w.batch, int(w.hist_lens.max()))
    c.set_splits(s)
    q = queries(w)
    dev = torch.device("cuda")
    pg = torch.tensor(np.array(last_p, np.int32), device=dev)
    sl = torch.tensor(np.array(last_s, np.int32), device=dev)
    say("full size step", w.name, "splits", s, "grid", s * w.n_kv_heads * max(1, w.gq // 8) * w.batch)
    outs = {"step": c.step(bf16(np.stack(last_k)), bf16(np.stack(last_v)), pg, sl, q, w.sm_scale).cpu().numpy()}
    for rep in range(2):
        say("full size attend alone", w.name, "call", rep)
        c.out.fill_(np.nan)
        oscar_attend(c.desc, c.rot_v, c.pool, c.block_table, c.hist_len, s, c.workspace, c.out)
        outs[f"attend {rep}"] = c.out.cpu().numpy()
    c.out.fill_(np.nan)
    say("full size two-launch decode", w.name)
    outs["decode_fused"] = c.decode_fused(q, w.sm_scale).cpu().numpy()
    c.out.fill_(np.nan)
    say("full size four entry points", w.name)
    outs["decode"] = c.decode(q, w.sm_scale).cpu().numpy()
    # the one-launch step at its own split count (what the benchmark's step times): the
    # same last tokens appended again (the same bytes), twice, then once without appending
    from bit_kv_cache_oscar_amd import oscar_decode_step_append_splits

    sa = oscar_decode_step_append_splits(c.desc, w.batch, int(w.hist_lens.max()))
    c.set_splits(sa)
    for rep in range(2):
        say("full size one-launch step", w.name, "splits", sa, "call", rep)
        c.out.fill_(np.nan)
        outs[f"one-launch {rep}"] = c.step_append(bf16(np.stack(last_k)), bf16(np.stack(last_v)), q,
                                                 w.sm_scale).cpu().numpy()
    c.out.fill_(np.nan)
    outs["one-launch decode"] = c.step_append(None, None, q, w.sm_scale).cpu().numpy()
    # the multi-query decode as the benchmark times it: T query tokens per request (T query
    # heads' worth of rows per KV head, 16 at most) at its own split count (one launch at
    # batch 1, prepare + attend at batch 4 and 64)
    from bit_kv_cache_oscar_amd import oscar_decode_multi, oscar_decode_multi_splits, oscar_decode_workspace_bytes

    n_tok = min(4, 16 // w.gq)
    qn = np.stack([synth.query_tokens(w, b, n_tok) for b in range(w.batch)])
    ms = oscar_decode_multi_splits(c.desc, w.batch, n_tok, int(w.hist_lens.max()))
    wsm = torch.zeros(oscar_decode_workspace_bytes(c.desc, w.batch * n_tok, ms), dtype=torch.uint8, device=dev)
    outm = torch.full((w.batch, n_tok, w.n_q_heads, 128), np.nan, dtype=torch.float32, device=dev)
    say("full size multi-query decode", w.name, "T", n_tok, "splits", ms)
    oscar_decode_multi(c.desc, bf16(qn), c.rot_k, c.rot_v, c.pool, c.block_table, c.hist_len, c.k_win, c.v_win,
                       c.win_len, w.sm_scale, ms, wsm, outm)
    got_m = outm.cpu().numpy()
    torch.cuda.synchronize()
    pool = c.pool.cpu().numpy().reshape(n_phys, w.n_kv_heads, opages.HEAD_BLOCK)
    for b, kv in FULL_PAIRS[cfg]:
        say("full size compare", w.name, "b", b, "kv", kv)
        ref_hist, km, vm = oracle_history(w, b, kv, rk, rv)
        gpu_hist = opages.unpack_history(pool, table[b], kv, w.hist_len(b))
        compare_history(gpu_hist, ref_hist, km, vm, f"{w.name} b{b} kv{kv}")
        heads = range(kv * w.gq, (kv + 1) * w.gq)
        ref = oracle_decode(w, b, rk, rv, {kv: ref_hist}, heads=heads)
        for name, got in outs.items():
            for h in heads:
                assert_close(got[b, h], ref[h], f"{w.name} {name} b{b} h{h}")
        wk, wv = windows(w, b)
        sl_h = slice(kv * w.gq, (kv + 1) * w.gq)
        ref_m = oatt.decode_multi(qn[b][:, sl_h].astype(np.float64), rk[kv:kv + 1], rv[kv:kv + 1], wk[kv:kv + 1],
                                  wv[kv:kv + 1], [ref_hist], w.sm_scale)
        for t in range(n_tok):
            for i, h in enumerate(heads):
                assert_close(got_m[b, t, h], ref_m[t, i], f"{w.name} multi-query b{b} t{t} h{h}")


STEP_CASES = ["c1", "c2-4k", "c4-shared-ragged", "c5-gq8", "gq16", "edges"]


@pytest.mark.parametrize("case", STEP_CASES)
def test_decode_step_demotes_then_decodes(case):
    """oscar_decode_step: every history token but the last of each request goes in through
    oscar_demote, the last ones through the step itself, which then decodes; the pool is
    compared byte by byte (with the exemption band) and the output with the oracle."""
    from bit_kv_cache_oscar_amd import oscar_default_splits

    w = DECODE_CASES[case]()
    (rk_bits, rv_bits), (rk, rv) = rotations(w)
    table, n_phys = synth.block_table(w)
    c = make_cache(w, rk_bits, rv_bits, table, n_phys)
    last_k, last_v, last_p, last_s = [], [], [], []
    for b in range(w.batch):
        n = w.hist_len(b)
        start = min(n, w.shared_pages * 64) if (w.shared_pages and b > 0) else 0
        if n == 0 or n - 1 < start:
            continue  # no history, or its last token belongs to the shared prefix demoted for request 0
        ks, vs = [], []
        for kv in range(w.n_kv_heads):
            k, v = synth.kv_rows(w, b, kv, 64 + start, 64 + n)
            ks.append(k)
            vs.append(v)
        ks, vs = np.stack(ks, 1), np.stack(vs, 1)
        j = np.arange(start, n)
        if n - 1 > start:
            _demote_all(c, w, b, table[b, j[:-1] // 64], j[:-1] % 64, ks[:-1], vs[:-1])
        last_k.append(ks[-1])
        last_v.append(vs[-1])
        last_p.append(table[b, (n - 1) // 64])
        last_s.append((n - 1) % 64)
    s = oscar_default_splits(c.desc, w.batch, int(w.hist_lens.max()))
    c.set_splits(s)
    dev = torch.device("cuda")
    if last_k:
        kr, vr = bf16(np.stack(last_k)), bf16(np.stack(last_v))
        pg = torch.tensor(last_p, dtype=torch.int32, device=dev)
        sl = torch.tensor(last_s, dtype=torch.int32, device=dev)
    else:
        kr = vr = pg = sl = None
    say(case, "step", "B", w.batch, "Hq", w.n_q_heads, "Hkv", w.n_kv_heads, "demoted in step", len(last_k), "splits", s)
    got = c.step(kr, vr, pg, sl, queries(w), w.sm_scale).cpu().numpy()
    pool = c.pool.cpu().numpy().reshape(n_phys, w.n_kv_heads, opages.HEAD_BLOCK)
    for b in range(w.batch):
        hists = {}
        for kv in range(w.n_kv_heads):
            ref_hist, km, vm = oracle_history(w, b, kv, rk, rv)
            gpu_hist = opages.unpack_history(pool, table[b], kv, w.hist_len(b))
            compare_history(gpu_hist, ref_hist, km, vm, f"{case} b{b} kv{kv}")
            hists[kv] = ref_hist
        ref = oracle_decode(w, b, rk, rv, hists)
        assert_close(got[b], ref, f"{case} step b{b}")


def plain_rotations(kind, n_kv):
    """(bits [n_kv, 128, 128] from the library's host builder, fp64 values from the oracle)
    for R = H P (Hadamard and bit reversal, no eigenbasis: the eigenbasis of a diagonal
    covariance with descending entries is the identity) or R = I (no rotation)."""
    from bit_kv_cache_oscar_amd import rotation as prot
    from oracle import rotation as orot

    if kind == "identity":
        bits = np.zeros((128, 128), np.uint16)
        bits[np.arange(128), np.arange(128)] = 0x3F80
        vals = np.eye(128)
    else:
        sigma = np.diag(np.arange(128, 0, -1).astype(np.float64))
        bits = prot.bf16_bits_from_f64(prot.rotation_fp64(sigma))
        vals = orot.round_bf16(orot.rotation_from_covariance(sigma))
        hp = orot.sylvester_hadamard(128) @ orot.bit_reversal_matrix(128)
        assert np.array_equal(vals, orot.round_bf16(hp))
    assert np.array_equal(bits_to_f64(bits), vals)
    return np.repeat(bits[None], n_kv, 0), np.repeat(vals[None], n_kv, 0)


@pytest.mark.parametrize("case", ["c2-4k", "c5-gq8", "c4-shared-ragged"])
@pytest.mark.parametrize("kind", ["hadamard", "identity"])
def test_plain_rotations_demote_and_decode(kind, case):
    """R = H P (Hadamard and bit reversal without the eigenbasis, the QuaRot-style baseline
    the pages compare with) and R = I (naive INT2): the whole history demoted on the GPU (the
    last token of each request through oscar_decode_step), then decoded through the step,
    the attend launch alone, oscar_decode and the four separate entry points; the pool and
    every output against the oracle."""
    from bit_kv_cache_oscar_amd import oscar_attend, oscar_default_splits

    w = DECODE_CASES[case]()
    rk_bits, rk = plain_rotations(kind, w.n_kv_heads)
    table, n_phys = synth.block_table(w)
    c = make_cache(w, rk_bits, rk_bits, table, n_phys)
    last_k, last_v, last_p, last_s = [], [], [], []
    hists = [[None] * w.n_kv_heads for _ in range(w.batch)]
    for b in range(w.batch):
        n = w.hist_len(b)
        start = min(n, w.shared_pages * 64) if (w.shared_pages and b > 0) else 0
        ks, vs = [], []
        for kv in range(w.n_kv_heads):
            k, v = synth.kv_rows(w, b, kv, 64 + start, 64 + n)
            ks.append(k)
            vs.append(v)
            hists[b][kv], _, _ = oracle_history(w, b, kv, rk, rk)
        ks, vs = np.stack(ks, 1), np.stack(vs, 1)
        j = np.arange(start, n)
        if n - 1 > start:
            _demote_all(c, w, b, table[b, j[:-1] // 64], j[:-1] % 64, ks[:-1], vs[:-1])
        if n - 1 >= start:
            last_k.append(ks[-1])
            last_v.append(vs[-1])
            last_p.append(table[b, (n - 1) // 64])
            last_s.append((n - 1) % 64)
    s = oscar_default_splits(c.desc, w.batch, int(w.hist_lens.max()))
    c.set_splits(s)
    q = queries(w)
    dev = torch.device("cuda")
    pg = torch.tensor(np.array(last_p, np.int32), device=dev)
    sl = torch.tensor(np.array(last_s, np.int32), device=dev)
    say(case, kind, "step", "B", w.batch, "splits", s)
    outs = {"step": c.step(bf16(np.stack(last_k)), bf16(np.stack(last_v)), pg, sl, q, w.sm_scale).cpu().numpy()}
    c.out.fill_(np.nan)
    oscar_attend(c.desc, c.rot_v, c.pool, c.block_table, c.hist_len, s, c.workspace, c.out)
    outs["attend"] = c.out.cpu().numpy()
    c.out.fill_(np.nan)
    outs["decode_fused"] = c.decode_fused(q, w.sm_scale).cpu().numpy()
    c.out.fill_(np.nan)
    outs["decode"] = c.decode(q, w.sm_scale).cpu().numpy()
    pool = c.pool.cpu().numpy().reshape(n_phys, w.n_kv_heads, opages.HEAD_BLOCK)
    for b in range(w.batch):
        for kv in range(w.n_kv_heads):
            ref_hist, km, vm = oracle_history(w, b, kv, rk, rk)
            gpu_hist = opages.unpack_history(pool, table[b], kv, w.hist_len(b))
            compare_history(gpu_hist, ref_hist, km, vm, f"{case} {kind} b{b} kv{kv}")
        ref = oracle_decode(w, b, rk, rk, hists[b])
        for name, got in outs.items():
            assert_close(got[b], ref, f"{case} {kind} {name} b{b}")


def _adversarial_rows(rk, g, n_each):
    """bf16 rows [4 n_each, 128] for one KV head's rotation rk (fp64 bf16 values):
    cancellation (x = y_t R^T rounded to bf16, with y_t two entries of +-1000 and the rest
    near 0.01, so most rotated values are sums of terms near 100 that cancel to a few units);
    mixed magnitudes (entries of 3000 and 0.001 in random dims); single spikes (x = c R_:,j,
    one large rotated value and the rest cancellation residue); and plain outlier rows."""
    rows = []
    for _ in range(n_each):
        yt = g.standard_normal(128) * 0.01
        yt[g.choice(128, 2, replace=False)] = g.choice([-1000.0, 1000.0], 2)
        rows.append(yt @ rk.T)
    for _ in range(n_each):
        x = g.standard_normal(128) * 1e-3
        big = g.choice(128, 64, replace=False)
        x[big] = g.standard_normal(64) * 3000.0
        rows.append(x)
    for _ in range(n_each):
        rows.append(g.uniform(5.0, 500.0) * g.choice([-1.0, 1.0]) * rk[:, g.integers(128)])
    for _ in range(n_each):
        x = g.standard_normal(128)
        x[g.choice(128, 4, replace=False)] *= 20.0
        rows.append(x)
    return synth.to_bf16_values(np.array(rows, np.float32))


def test_bulk_demotion_adversarial_rows_exact():
    """The matrix-core demotion kernel on rows built to stress its error bound: large
    cancellation (sum |x_i R_ij| hundreds of times |y_j|), mixed magnitudes (3000 next to
    0.001) and single spikes, with plain outlier rows beside them; every scale, zero point
    and code equal to the oracle's, with no code in the tolerated band allowed to differ."""
    w = custom("adversarial", 4, 2, [64 * 8 + 320], cfg=2)
    (rk_bits, rv_bits), (rk, rv) = rotations(w)
    table = np.array([list(range(8))], np.int32)
    c = make_cache(w, rk_bits, rv_bits, table, 8, with_windows=False)
    g = np.random.default_rng(31)
    n = 4 * 128
    rows_k = np.stack([_adversarial_rows(rk[kv], g, 128) for kv in range(2)], 1)
    rows_v = np.stack([_adversarial_rows(rv[kv], g, 128) for kv in range(2)], 1)
    perm = g.permutation(n)  # mixed within tiles
    rows_k, rows_v = rows_k[perm], rows_v[perm]
    j = np.arange(n)
    say("bulk demotion, adversarial rows", n)
    _demote_all(c, w, 0, table[0, j // 64], j % 64, rows_k, rows_v)
    torch.cuda.synchronize()
    pool = c.pool.cpu().numpy().reshape(8, 2, opages.HEAD_BLOCK)
    from oracle import quant as oquant
    for kv in range(2):
        kc, ks, kz, km = oquant.quantize_rows(rows_k[:, kv].astype(np.float64), rk[kv], w.clip_ratio)
        vc, vs, vz, vm = oquant.quantize_rows(rows_v[:, kv].astype(np.float64), rv[kv], w.clip_ratio)
        got = opages.unpack_history(pool, table[0], kv, n)
        assert compare_history(got, (kc, ks, kz, vc, vs, vz), km, vm, f"adversarial head {kv}") == 0


def _tie_rows(g, n):
    """Rows under R = I whose scale (max - min) / 3 is exactly halfway between two fp16
    values, with two values at the maximum and two at the minimum in each lane group's
    dims (d % 16) // 4 of the bulk kernel's layout, the rest strictly between."""
    def bf16_range(lo_e, hi_e):
        return np.concatenate([(1.0 + np.arange(128) / 128.0) * 2.0 ** e for e in range(lo_e, hi_e)])
    hi_vals, lo_vals = bf16_range(-1, 2), -bf16_range(-8, 2)
    s = (hi_vals[:, None] - lo_vals[None, :]) / 3.0
    ulp = 2.0 ** (np.floor(np.log2(s)) - 10)
    ties = np.argwhere(s == (np.floor(s / ulp) + 0.5) * ulp)
    pick = ties[g.choice(len(ties), n, replace=False)]
    d = np.arange(128)
    grp = (d % 16) // 4
    rows = np.empty((n, 128))
    for r, (i, j) in enumerate(pick):
        hi, lo = hi_vals[i], lo_vals[j]
        rows[r] = synth.to_bf16_values(g.uniform(lo + 0.25 * (hi - lo), hi - 0.25 * (hi - lo), 128).astype(np.float32))
        for gg in range(4):
            dims = d[grp == gg]
            rows[r, dims[:2]] = hi
            rows[r, dims[2:4]] = lo
    return rows


def test_bulk_demotion_many_open_tokens_exact():
    """Tiles whose every token leaves its fp16 scale open (exact ties under R = I, clip 1)
    and puts four extreme candidates in each of its lanes: eight candidates per side and
    token, so each of the kernel's 16-lane groups sums many in turn, over eight rounds of two
    tokens per wave and iteration, then the compensated sums
    that settle ties (to even); with random rows after them. Scales, zero points and codes
    equal to the oracle's."""
    w = custom("open tokens", 4, 2, [64 * 2 + 320], cfg=2)
    (rk_bits, rv_bits), _ = rotations(w)
    table = np.array([[0, 1]], np.int32)
    c = make_cache(w, rk_bits, rv_bits, table, 2, with_windows=False)
    eye_bits = np.zeros((2, 128, 128), np.uint16)
    eye_bits[:, np.arange(128), np.arange(128)] = 0x3F80
    one = np.ones(2, np.float32)
    c.set_rotations(eye_bits, eye_bits, one, one)
    g = np.random.default_rng(77)
    n_tie, n = 64, 96
    rows = np.empty((n, 2, 128), np.float32)
    for kv in range(2):
        rows[:n_tie, kv] = _tie_rows(g, n_tie)
        rows[n_tie:, kv] = synth.to_bf16_values(g.standard_normal((n - n_tie, 128)).astype(np.float32))
    j = np.arange(n)
    say("bulk demotion, open tokens", n)
    _demote_all(c, w, 0, table[0, j // 64], j % 64, rows, rows[::-1].copy())
    torch.cuda.synchronize()
    pool = c.pool.cpu().numpy().reshape(2, 2, opages.HEAD_BLOCK)
    from oracle import quant as oquant
    for kv in range(2):
        kc, ks, kz, km = oquant.quantize_rows(rows[:, kv].astype(np.float64), np.eye(128), 1.0)
        vc, vs, vz, vm = oquant.quantize_rows(rows[::-1][:, kv].astype(np.float64), np.eye(128), 1.0)
        got = opages.unpack_history(pool, table[0], kv, n)
        compare_history(got, (kc, ks, kz, vc, vs, vz), km, vm, f"open tokens head {kv}")
        for a, b in zip(got, (kc, ks, kz, vc, vs, vz)):
            assert np.array_equal(np.asarray(a), np.asarray(b)), "open-token demotion differs from the oracle"


def test_bulk_demotion_codes_on_every_bf16_t():
    """Rows under R = I with clip 1 holding 0 and 3 (so s16 = 1 and z16 = 0 exactly, and
    t = y) and, between them, every bf16 value from 1/4 to 3: the matrix-core kernel takes
    each code from the hardware's float-to-byte packing conversion unless the value lies
    within its error bound of a half-integer, so this pins that conversion's rounding to
    nearest at every representable t next to each code boundary (0.498 and 0.502 beside
    1/2, and so on), and the exact ties 1/2, 3/2 and 5/2 to even."""
    w = custom("every t", 4, 2, [64 * 2 + 320], cfg=2)
    (rk_bits, rv_bits), _ = rotations(w)
    table = np.array([[0, 1]], np.int32)
    c = make_cache(w, rk_bits, rv_bits, table, 2, with_windows=False)
    eye_bits = np.zeros((2, 128, 128), np.uint16)
    eye_bits[:, np.arange(128), np.arange(128)] = 0x3F80
    one = np.ones(2, np.float32)
    c.set_rotations(eye_bits, eye_bits, one, one)
    ts = np.concatenate([(1.0 + np.arange(128) / 128.0) * 2.0 ** e for e in (-2, -1, 0, 1)])
    ts = ts[ts <= 3.0]
    assert 0.5 in ts and 1.5 in ts and 2.5 in ts and len(ts) == 449
    g = np.random.default_rng(5)
    n = 128
    rows = np.empty((n, 2, 128), np.float32)
    for r in range(n):
        for kv in range(2):
            vals = np.resize(np.roll(ts, -126 * r - 61 * kv), 126)
            row = np.concatenate([[0.0, 3.0], vals])
            rows[r, kv] = row[g.permutation(128)]
    assert np.array_equal(synth.to_bf16_values(rows), rows)
    j = np.arange(n)
    say("bulk demotion, every bf16 t", n)
    _demote_all(c, w, 0, table[0, j // 64], j % 64, rows, rows[::-1].copy())
    torch.cuda.synchronize()
    pool = c.pool.cpu().numpy().reshape(2, 2, opages.HEAD_BLOCK)
    from oracle import quant as oquant
    for kv in range(2):
        kc, ks, kz, km = oquant.quantize_rows(rows[:, kv].astype(np.float64), np.eye(128), 1.0)
        vc, vs, vz, vm = oquant.quantize_rows(rows[::-1][:, kv].astype(np.float64), np.eye(128), 1.0)
        assert np.all(ks == 1.0) and np.all(kz == 0.0)
        got = opages.unpack_history(pool, table[0], kv, n)
        compare_history(got, (kc, ks, kz, vc, vs, vz), km, vm, f"every t head {kv}")
        for a, b in zip(got, (kc, ks, kz, vc, vs, vz)):
            assert np.array_equal(np.asarray(a), np.asarray(b)), "codes differ from the oracle"


@pytest.mark.parametrize("n", [40, 128])
def test_demotion_fp16_overflow_contract(n):
    """A row whose clipped range exceeds fp16 is outside the quantiser's domain (the oracle
    rejects it); both demotion kernels (per row below 64 tokens, matrix cores from 64) store
    the fp16 rounding of its scale and zero point (infinite) and codes 0, and leave the
    other rows of the call exact."""
    w = custom("overflow", 4, 2, [64 * 2 + 320], cfg=2)
    (rk_bits, rv_bits), (rk, rv) = rotations(w)
    table = np.array([[0, 1]], np.int32)
    c = make_cache(w, rk_bits, rv_bits, table, 2, with_windows=False)
    g = np.random.default_rng(5)
    rows = synth.to_bf16_values(g.standard_normal((n, 2, 128)).astype(np.float32))
    rows[3] = synth.to_bf16_values(np.full((2, 128), 1.0e5, np.float32) * g.choice([-1.0, 1.0], (2, 128)))
    j = np.arange(n)
    say("demotion overflow contract", n)
    _demote_all(c, w, 0, table[0, j // 64], j % 64, rows, rows[::-1].copy())
    torch.cuda.synchronize()
    pool = c.pool.cpu().numpy().reshape(2, 2, opages.HEAD_BLOCK)
    from oracle import quant as oquant
    keep = np.arange(n) != 3
    keep_v = np.arange(n) != n - 1 - 3
    for kv in range(2):
        got = opages.unpack_history(pool, table[0], kv, n)
        kcg, ksg, kzg, vcg, vsg, vzg = got
        with pytest.raises(ValueError):
            oquant.quantize_rows(rows[3:4, kv].astype(np.float64), rk[kv], w.clip_ratio)
        assert np.isinf(np.float64(ksg[3])) and np.isinf(np.float64(kzg[3])) and not np.any(kcg[3])
        assert np.isinf(np.float64(vsg[n - 4])) and not np.any(vcg[n - 4])
        kc, ks, kz, km = oquant.quantize_rows(rows[keep, kv].astype(np.float64), rk[kv], w.clip_ratio)
        vc, vs, vz, vm = oquant.quantize_rows(rows[::-1][keep_v, kv].astype(np.float64), rv[kv], w.clip_ratio)
        mine = (kcg[keep], ksg[keep], kzg[keep], vcg[keep_v], vsg[keep_v], vzg[keep_v])
        assert compare_history(mine, (kc, ks, kz, vc, vs, vz), km, vm, f"overflow call head {kv}") == 0


APPEND_CASES = {
    "c1": lambda: synth.workload(1),
    "c2-4k": lambda: synth.workload(2).with_ctx([4000]),
    "c3-6k-permuted": lambda: synth.workload(3).with_ctx([6000]),
    # every request's last history token past the shared prefix: appended tokens land in
    # pages of their own request
    "c4-shared-ragged": lambda: synth.workload(4).with_ctx([4596, 5096, 4500, 4096 + 128 + 320 + 3], capacity=6000),
    "c5-gq8": lambda: synth.workload(5).with_ctx([3000, 2600]),
    "gq16": lambda: custom("gq16", 32, 2, [2500, 900]),
    "gq2": lambda: custom("gq2", 16, 8, [1500]),
    "gq1": lambda: custom("gq1", 4, 4, [900, 1700]),
    "edges": lambda: custom("edges", 8, 2, [321, 64 * 3 + 320 + 1, 64 + 320, 64 * 5 + 320 + 63]),
}


def _fill_but_last(c, w, table):
    """Every history token but each request's last through oscar_demote; returns the last
    tokens' rows [B, Hkv, 128] (float32 bf16 values)."""
    last_k, last_v = [], []
    for b in range(w.batch):
        n = w.hist_len(b)
        start = min(n, w.shared_pages * 64) if (w.shared_pages and b > 0) else 0
        assert n - 1 >= start, "the appended token must lie in a page of its own request"
        ks, vs = [], []
        for kv in range(w.n_kv_heads):
            k, v = synth.kv_rows(w, b, kv, 64 + start, 64 + n)
            ks.append(k)
            vs.append(v)
        ks, vs = np.stack(ks, 1), np.stack(vs, 1)
        j = np.arange(start, n)
        if n - 1 > start:
            _demote_all(c, w, b, table[b, j[:-1] // 64], j[:-1] % 64, ks[:-1], vs[:-1])
        last_k.append(ks[-1])
        last_v.append(vs[-1])
    return np.stack(last_k), np.stack(last_v)


@pytest.mark.parametrize("case", list(APPEND_CASES))
def test_decode_step_append_one_launch(case):
    """oscar_decode_step_append: every history token but each request's last through
    oscar_demote, the last one appended by the one-launch step, which then decodes; the pool
    (every token) and the output against the oracle, at the one-launch default split count
    and at 3 splits; then the same launch without appending (the pool as it is), twice in a
    row (the arrival counters must re-arm). The split counts run largest first and then
    again: the workspace allocated for the largest serves the smaller ones, and its arrival
    counters move with the split count."""
    from bit_kv_cache_oscar_amd import oscar_decode_step_append_splits

    w = APPEND_CASES[case]()
    (rk_bits, rv_bits), (rk, rv) = rotations(w)
    table, n_phys = synth.block_table(w)
    c = make_cache(w, rk_bits, rv_bits, table, n_phys)
    lk, lv = _fill_but_last(c, w, table)
    refs = []
    for b in range(w.batch):
        hists = {}
        for kv in range(w.n_kv_heads):
            hists[kv], _, _ = oracle_history(w, b, kv, rk, rv)
        refs.append(oracle_decode(w, b, rk, rv, hists))
    q = queries(w)
    s = oscar_decode_step_append_splits(c.desc, w.batch, int(w.hist_lens.max()))
    for splits in ([s, 3, s] if s > 3 else [3]):
        c.set_splits(splits)
        say(case, "one-launch step", "B", w.batch, "Hq", w.n_q_heads, "Hkv", w.n_kv_heads, "splits", splits)
        c.out.fill_(np.nan)
        got = c.step_append(bf16(lk), bf16(lv), q, w.sm_scale).cpu().numpy()
        for b in range(w.batch):
            assert_close(got[b], refs[b], f"{case} one-launch step b{b} splits {splits}")
        pool = c.pool.cpu().numpy().reshape(n_phys, w.n_kv_heads, opages.HEAD_BLOCK)
        for b in range(w.batch):
            for kv in range(w.n_kv_heads):
                ref_hist, km, vm = oracle_history(w, b, kv, rk, rv)
                gpu_hist = opages.unpack_history(pool, table[b], kv, w.hist_len(b))
                compare_history(gpu_hist, ref_hist, km, vm, f"{case} one-launch pool b{b} kv{kv}")
        for rep in range(2):
            c.out.fill_(np.nan)
            got = c.step_append(None, None, q, w.sm_scale).cpu().numpy()
            for b in range(w.batch):
                assert_close(got[b], refs[b], f"{case} one-launch decode b{b} splits {splits} call {rep}")
        # the same calls prepared once (prepare=True) and issued twice: the same bits
        kk, vv = bf16(lk), bf16(lv)  # a prepared call keeps pointers only: the tensors stay alive here
        want = c.step_append(kk, vv, q, w.sm_scale).clone()
        call = c.step_append(kk, vv, q, w.sm_scale, prepare=True)
        for rep in range(2):
            c.out.fill_(np.nan)
            call()
            assert torch.equal(c.out, want), f"{case} prepared one-launch step splits {splits} call {rep}"
        want = c.decode_fused(q, w.sm_scale).clone()
        call = c.decode(q, w.sm_scale, prepare=True)
        c.out.fill_(np.nan)
        call()
        assert_close(c.out.cpu().numpy()[0], want.cpu().numpy()[0], f"{case} prepared three-launch decode")
