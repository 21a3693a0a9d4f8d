"""GPU parity of grouped pages (quantisation groups of 64 or 32 rotated dims) against the
group oracle (oracle/groups.py): oscar_demote_grouped bit-exact up to the rounding band,
oscar_decode_int2_grouped + oscar_decode_bf16 + oscar_merge within the decode tolerance,
and the one-group case of the grouped entry points against the one-group entry points."""

from __future__ import annotations

import ctypes

import numpy as np
import pytest

import synth
from gpu_harness import assert_close, clips, compare_history, rotations, windows
from oracle import attention as oatt
from oracle import groups as ogroups
from test_gpu_parity import DECODE_CASES, bf16, queries, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import bit_kv_cache_oscar_amd as ok
    ok.lib()


def grouped_cache(w, rk_bits, rv_bits, table, n_phys, group):
    from bit_kv_cache_oscar_amd.layer import LayerCache

    c = LayerCache(w.n_q_heads, w.n_kv_heads, w.batch, table.shape[1], n_phys, group_size=group)
    ck, cv = clips(w)
    c.set_rotations(rk_bits, rv_bits, ck, cv)
    c.set_block_table(table)
    c.set_hist_len(w.hist_lens)
    for b in range(w.batch):
        for kv in range(w.n_kv_heads):
            k, v = synth.window_rows(w, b, kv)
            c.set_window(b, kv, k, v)
    c.set_win_len(w.win_lens)
    return c


def oracle_history_grouped(w, b, kv, rk, rv, group, n=None):
    hk, hv = synth.history_rows(w, b, kv)
    if n is not None:
        hk, hv = hk[:n], hv[:n]
    kc, ks, kz, km = ogroups.quantize_rows_grouped(hk.astype(np.float64), rk[kv], w.clip_ratio, group)
    vc, vs, vz, vm = ogroups.quantize_rows_grouped(hv.astype(np.float64), rv[kv], w.clip_ratio, group)
    return (kc, ks, kz, vc, vs, vz), km, vm


def pack_grouped(pool, table_row, kv, hist, group):
    n = len(hist[1])
    for p in range(-(-n // 64)):
        r = slice(64 * p, min(n, 64 * p + 64))
        pool[table_row[p], kv] = ogroups.pack_page_grouped(*(a[r] for a in hist), group)


def unpack_grouped(pool, table_row, kv, n, group):
    parts = [[] for _ in range(6)]
    for p in range(-(-n // 64)):
        cnt = min(64, n - 64 * p)
        for lst, a in zip(parts, ogroups.unpack_page_grouped(pool[table_row[p], kv], group)):
            lst.append(a[:cnt])
    return tuple(np.concatenate(x) for x in parts)


def decode_refs(w, rk, rv, hists):
    refs = []
    for b in range(w.batch):
        q = synth.query(w, b).astype(np.float64)
        wk, wv = windows(w, b)
        out = np.zeros((w.n_q_heads, 128))
        for h in range(w.n_q_heads):
            kv = h // w.gq
            out[h] = oatt.decode_head(q[h], rk[kv], rv[kv], wk[kv], wv[kv], hists[b][kv], w.sm_scale)
        refs.append(out)
    return refs


@pytest.mark.parametrize("group", [64, 32])
@pytest.mark.parametrize("n", [1024, 40])
def test_grouped_demote_bitexact(group, n):
    """Every KV head of request 0's first n history rows of the tiny workload: per-group
    scales and zero points bit-exact, codes equal outside the band around rounding
    boundaries."""
    w = synth.workload(1)
    (rk_bits, rv_bits), (rk, rv) = rotations(w)
    table, n_phys = synth.block_table(w)
    c = grouped_cache(w, rk_bits, rv_bits, table, n_phys, group)
    j = np.arange(n)
    rows = [synth.history_rows(w, 0, kv) for kv in range(w.n_kv_heads)]
    hk = np.stack([r[0][:n] for r in rows], axis=1)
    hv = np.stack([r[1][:n] for r in rows], axis=1)
    say("grouped demote c1", "group", group, "n", n, "Hkv", w.n_kv_heads)
    pages = torch.from_numpy(table[0, j // 64].astype(np.int32)).cuda()
    slots = torch.from_numpy((j % 64).astype(np.int32)).cuda()
    c.demote(bf16(hk), bf16(hv), pages, slots)
    torch.cuda.synchronize()
    pool = c.pool.cpu().numpy().reshape(-1, w.n_kv_heads, ogroups.head_block_bytes(group))
    for kv in range(w.n_kv_heads):
        ref, km, vm = oracle_history_grouped(w, 0, kv, rk, rv, group, n)
        got = unpack_grouped(pool, table[0], kv, n, group)
        assert got[1].shape == (n, 128 // group)
        compare_history(got, ref, km, vm, f"grouped demote g{group} n={n} kv{kv}")


GROUPED_CASES = [("c1", 64), ("c1", 32), ("c2-4k", 32), ("c2-4k", 64), ("c5-gq8", 32), ("gq16", 64),
                 ("edges", 32), ("gq1", 64), ("gq2", 32)]


@pytest.mark.parametrize("case,group", GROUPED_CASES)
def test_grouped_decode_on_oracle_pages(case, group):
    """oscar_decode_int2_grouped, oscar_decode_bf16 and oscar_merge on a grouped pool the
    oracle built, at several split counts, twice per count."""
    from bit_kv_cache_oscar_amd import oscar_default_splits

    w = DECODE_CASES[case]()
    (rk_bits, rv_bits), (rk, rv) = rotations(w)
    table, n_phys = synth.block_table(w)
    pool = np.zeros((n_phys, w.n_kv_heads, ogroups.head_block_bytes(group)), np.uint8)
    hists = [[None] * w.n_kv_heads for _ in range(w.batch)]
    for b in range(w.batch):
        for kv in range(w.n_kv_heads):
            hists[b][kv], _, _ = oracle_history_grouped(w, b, kv, rk, rv, group)
            if len(hists[b][kv][1]):
                pack_grouped(pool, table[b], kv, hists[b][kv], group)
    refs = decode_refs(w, rk, rv, hists)
    c = grouped_cache(w, rk_bits, rv_bits, table, n_phys, group)
    c.pool.copy_(torch.from_numpy(pool.reshape(-1)))
    q = queries(w)
    max_pages = int(np.max(-(-w.hist_lens // 64)))
    splits = {oscar_default_splits(c.desc, w.batch, int(w.hist_lens.max())), 1, 3, max_pages + 5}
    for s in sorted(splits):
        say(case, "grouped decode", "group", group, "B", w.batch, "Hq", w.n_q_heads, "Hkv", w.n_kv_heads,
            "ctx", w.ctx_lens, "splits", s)
        c.set_splits(s)
        for rep in range(2):
            c.out.fill_(np.nan)
            got = c.decode(q, w.sm_scale).cpu().numpy()
            for b in range(w.batch):
                assert_close(got[b], refs[b], f"{case} g{group} b{b} splits {s} call {rep}")


@pytest.mark.parametrize("group", [32, 64])
def test_grouped_demote_then_decode(group):
    """The whole grouped path on the GPU: demote request 0's history of the 4K workload,
    then decode, against the oracle's demotion and decode."""
    w = DECODE_CASES["c2-4k"]()
    (rk_bits, rv_bits), (rk, rv) = rotations(w)
    table, n_phys = synth.block_table(w)
    c = grouped_cache(w, rk_bits, rv_bits, table, n_phys, group)
    hists = [[None] * w.n_kv_heads for _ in range(w.batch)]
    for b in range(w.batch):
        rows = [synth.history_rows(w, b, kv) for kv in range(w.n_kv_heads)]
        n = len(rows[0][0])
        j = np.arange(n)
        pages = torch.from_numpy(table[b, j // 64].astype(np.int32)).cuda()
        slots = torch.from_numpy((j % 64).astype(np.int32)).cuda()
        say("grouped step c2-4k", "group", group, "b", b, "n", n)
        c.demote(bf16(np.stack([r[0] for r in rows], 1)), bf16(np.stack([r[1] for r in rows], 1)), pages, slots)
        for kv in range(w.n_kv_heads):
            hists[b][kv], _, _ = oracle_history_grouped(w, b, kv, rk, rv, group)
    refs = decode_refs(w, rk, rv, hists)
    c.set_splits(7)
    got = c.decode(queries(w), w.sm_scale).cpu().numpy()
    for b in range(w.batch):
        assert_close(got[b], refs[b], f"grouped step g{group} b{b}")


def test_one_group_grouped_entries_match_the_one_group_path():
    """group_size 128 through the grouped entry points: the same page bytes as oscar_demote
    (the grouped layout with one group is the one-group layout) and partials that merge to
    the one-group decode's output within the decode tolerance."""
    import bit_kv_cache_oscar_amd._lib as L
    from test_gpu_parity import make_cache

    w = DECODE_CASES["c2-4k"]()
    (rk_bits, rv_bits), (rk, rv) = rotations(w)
    table, n_phys = synth.block_table(w)
    c = make_cache(w, rk_bits, rv_bits, table, n_phys)
    rows = [synth.history_rows(w, 0, kv) for kv in range(w.n_kv_heads)]
    n = 40  # the per-row kernel of oscar_demote
    j = np.arange(n)
    pages = torch.from_numpy(table[0, j // 64].astype(np.int32)).cuda()
    slots = torch.from_numpy((j % 64).astype(np.int32)).cuda()
    k = bf16(np.stack([r[0][:n] for r in rows], 1))
    v = bf16(np.stack([r[1][:n] for r in rows], 1))
    say("one-group grouped demote", "n", n)
    c.demote(k, v, pages, slots)
    want = c.pool.clone()
    c.pool.zero_()
    L.oscar_demote_grouped(c.desc, k, v, pages, slots, c.rot_k, c.rot_v, c.clip_k, c.clip_v, c.pool)
    torch.cuda.synchronize()
    assert torch.equal(c.pool, want)
    # decode: a full pool from the one-group demotion, then both INT2 passes
    c.pool.zero_()
    for b in range(w.batch):
        rows = [synth.history_rows(w, b, kv) for kv in range(w.n_kv_heads)]
        m = len(rows[0][0])
        jj = np.arange(m)
        c.demote(bf16(np.stack([r[0] for r in rows], 1)), bf16(np.stack([r[1] for r in rows], 1)),
                 torch.from_numpy(table[b, jj // 64].astype(np.int32)).cuda(),
                 torch.from_numpy((jj % 64).astype(np.int32)).cuda())
    q = queries(w)
    c.set_splits(5)
    ref = c.decode(q, w.sm_scale).clone()
    L.oscar_decode_int2_grouped(c.desc, q, c.rot_k, c.pool, c.block_table, c.hist_len, w.sm_scale, 5, c.partials)
    L.oscar_merge(c.desc, c.partials, 5, c.win_partials, c.rot_v, c.out)
    # the grouped pass sums in fp32, the one-group pass in exact integers: the decode bar
    got = c.out.cpu().numpy()
    ref = ref.cpu().numpy()
    for b in range(w.batch):
        assert_close(got[b], ref[b], f"one-group grouped decode vs one-group decode b{b}")
    assert ctypes.sizeof(L.LayerDesc) == 28


@pytest.mark.parametrize("group", [32, 64])
def test_grouped_full_size_sampled(group):
    """The grouped path at the 32K workload's real size (32768-token context, 32 query heads,
    8 KV heads): every history token demoted on the GPU, then decoded in three launches at
    about four pages per split and by the two-launch grouped step at the default split count
    (the benchmark's); every KV head compared with the oracle (pool contents and the outputs
    of its query heads)."""
    from test_gpu_parity import _demote_all

    w = synth.workload(2)
    (rk_bits, rv_bits), (rk, rv) = rotations(w)
    table, n_phys = synth.block_table(w)
    c = grouped_cache(w, rk_bits, rv_bits, table, n_phys, group)
    for b in range(w.batch):
        n = w.hist_len(b)
        ks, vs = [], []
        for kv in range(w.n_kv_heads):
            k, v = synth.kv_rows(w, b, kv, 64, 64 + n)
            ks.append(k)
            vs.append(v)
        j = np.arange(n)
        say("grouped full size", w.name, "group", group, "b", b, "tokens", n)
        _demote_all(c, w, b, table[b, j // 64], j % 64, np.stack(ks, 1), np.stack(vs, 1))
    from bit_kv_cache_oscar_amd import oscar_default_splits

    s = -(-(-(-int(w.hist_lens.max()) // 64)) // 4)
    c.set_splits(s)
    got = c.decode(queries(w), w.sm_scale).cpu().numpy()
    # the two-launch grouped step (nothing demoted) at the default split count
    c.set_splits(oscar_default_splits(c.desc, w.batch, int(w.hist_lens.max())))
    say("grouped full size step", w.name, "group", group, "splits", c.n_splits)
    got_step = c.step(None, None, None, None, queries(w), w.sm_scale).cpu().numpy()
    pool = c.pool.cpu().numpy().reshape(n_phys, w.n_kv_heads, ogroups.head_block_bytes(group))
    for b, kv in [(0, kv) for kv in range(w.n_kv_heads)]:
        say("grouped full size sample", w.name, "group", group, "b", b, "kv", kv, "splits", s)
        ref_hist, km, vm = oracle_history_grouped(w, b, kv, rk, rv, group)
        gpu_hist = unpack_grouped(pool, table[b], kv, w.hist_len(b), group)
        compare_history(gpu_hist, ref_hist, km, vm, f"{w.name} g{group} b{b} kv{kv}")
        q = synth.query(w, b).astype(np.float64)
        wk, wv = windows(w, b)
        for h in range(kv * w.gq, (kv + 1) * w.gq):
            ref = oatt.decode_head(q[h], rk[kv], rv[kv], wk[kv], wv[kv], ref_hist, w.sm_scale)
            assert_close(got[b, h], ref, f"{w.name} g{group} b{b} h{h}")
            assert_close(got_step[b, h], ref, f"{w.name} g{group} step b{b} h{h}")


@pytest.mark.parametrize("case,group", [("c2-4k", 32), ("c5-gq8", 64), ("gq16", 32)])
def test_grouped_step_demotes_then_decodes(case, group):
    """oscar_decode_step_grouped: every history token but the last of each request goes in
    through oscar_demote_grouped, the last ones through the step; the pool (every token of
    every KV head) and the output against the oracle, twice in a row."""
    w = DECODE_CASES[case]()
    (rk_bits, rv_bits), (rk, rv) = rotations(w)
    table, n_phys = synth.block_table(w)
    c = grouped_cache(w, rk_bits, rv_bits, table, n_phys, group)
    last_k, last_v, last_p, last_s = [], [], [], []
    hists = [[None] * w.n_kv_heads for _ in range(w.batch)]
    for b in range(w.batch):
        rows = [synth.history_rows(w, b, kv) for kv in range(w.n_kv_heads)]
        n = len(rows[0][0])
        assert n >= 2
        hk = np.stack([r[0] for r in rows], 1)
        hv = np.stack([r[1] for r in rows], 1)
        j = np.arange(n - 1)
        c.demote(bf16(hk[:-1]), bf16(hv[:-1]), torch.from_numpy(table[b, j // 64].astype(np.int32)).cuda(),
                 torch.from_numpy((j % 64).astype(np.int32)).cuda())
        last_k.append(hk[-1])
        last_v.append(hv[-1])
        last_p.append(table[b, (n - 1) // 64])
        last_s.append((n - 1) % 64)
        for kv in range(w.n_kv_heads):
            hists[b][kv], _, _ = oracle_history_grouped(w, b, kv, rk, rv, group)
    refs = decode_refs(w, rk, rv, hists)
    pages = torch.tensor(np.array(last_p, np.int32)).cuda()
    slots = torch.tensor(np.array(last_s, np.int32)).cuda()
    c.set_splits(5)
    q = queries(w)
    for rep in range(2):
        say(case, "grouped step", "group", group, "B", w.batch, "call", rep)
        c.out.fill_(np.nan)
        got = c.step(bf16(np.stack(last_k)), bf16(np.stack(last_v)), pages, slots, q, w.sm_scale).cpu().numpy()
        for b in range(w.batch):
            assert_close(got[b], refs[b], f"{case} g{group} step b{b} call {rep}")
    pool = c.pool.cpu().numpy().reshape(n_phys, w.n_kv_heads, ogroups.head_block_bytes(group))
    for b in range(w.batch):
        for kv in range(w.n_kv_heads):
            ref, km, vm = oracle_history_grouped(w, b, kv, rk, rv, group)
            got_h = unpack_grouped(pool, table[b], kv, w.hist_len(b), group)
            compare_history(got_h, ref, km, vm, f"{case} g{group} step pool b{b} kv{kv}")


@pytest.mark.parametrize("kind", ["hadamard", "identity"])
@pytest.mark.parametrize("group", [64, 32])
def test_grouped_plain_rotations(kind, group):
    """Grouped pages with R = H P (Hadamard and bit reversal, no eigenbasis: the QuaRot-style
    baseline) and R = I (naive INT2), the comparisons the pages draw for the bit-reversal's
    group balancing: the history of the 4K workload demoted on the GPU (the last token of
    each request through the grouped step), then decoded by the step and by the three
    separate passes; every token of the pool and every output against the oracle."""
    from test_gpu_parity import plain_rotations

    w = DECODE_CASES["c2-4k"]()
    rk_bits, rk = plain_rotations(kind, w.n_kv_heads)
    table, n_phys = synth.block_table(w)
    c = grouped_cache(w, rk_bits, rk_bits, table, n_phys, group)
    last_k, last_v, last_p, last_s = [], [], [], []
    hists = [[None] * w.n_kv_heads for _ in range(w.batch)]
    for b in range(w.batch):
        rows = [synth.history_rows(w, b, kv) for kv in range(w.n_kv_heads)]
        n = len(rows[0][0])
        hk = np.stack([r[0] for r in rows], 1)
        hv = np.stack([r[1] for r in rows], 1)
        j = np.arange(n - 1)
        c.demote(bf16(hk[:-1]), bf16(hv[:-1]), torch.from_numpy(table[b, j // 64].astype(np.int32)).cuda(),
                 torch.from_numpy((j % 64).astype(np.int32)).cuda())
        last_k.append(hk[-1])
        last_v.append(hv[-1])
        last_p.append(table[b, (n - 1) // 64])
        last_s.append((n - 1) % 64)
        for kv in range(w.n_kv_heads):
            hists[b][kv], _, _ = oracle_history_grouped(w, b, kv, rk, rk, group)
    refs = decode_refs(w, rk, rk, hists)
    pages = torch.tensor(np.array(last_p, np.int32)).cuda()
    slots = torch.tensor(np.array(last_s, np.int32)).cuda()
    c.set_splits(5)
    q = queries(w)
    say("grouped", kind, "group", group, "step")
    outs = {"step": c.step(bf16(np.stack(last_k)), bf16(np.stack(last_v)), pages, slots, q, w.sm_scale)
            .cpu().numpy()}
    c.out.fill_(np.nan)
    outs["decode"] = c.decode(q, w.sm_scale).cpu().numpy()
    pool = c.pool.cpu().numpy().reshape(n_phys, w.n_kv_heads, ogroups.head_block_bytes(group))
    for b in range(w.batch):
        for kv in range(w.n_kv_heads):
            ref, km, vm = oracle_history_grouped(w, b, kv, rk, rk, group)
            got_h = unpack_grouped(pool, table[b], kv, w.hist_len(b), group)
            compare_history(got_h, ref, km, vm, f"{kind} g{group} pool b{b} kv{kv}")
        for name, got in outs.items():
            assert_close(got[b], refs[b], f"{kind} g{group} {name} b{b}")
