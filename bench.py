"""Benchmark: the OSCAR decode step (each request's oldest recent token demoted into its INT2
history, the BF16 sink/recent pass, the INT2 history pass, the merge and the un-rotation) on
one MI355X, through oscar_decode_step_append: one launch when its workgroups fit the chip at
once (batch 1 at 32K and 100K tokens), else prepare + attend.

Workloads (rows, in this order by default): a Qwen3-8B-shaped layer at 32,768 tokens, batch
1 (the headline: `value`); the same layer at 100,000 tokens over randomly permuted pages; a
Qwen3-32B-shaped layer (64 query heads) at 131,072 tokens, batch 4; and batch 64 at 8K-16K
tokens sharing a 4,096-token prefix. All: 64 BF16 sink tokens, 256 BF16 recent tokens,
head_dim 128, 64-token pages, seeded synthetic N(0,1) data with per-head outlier channels,
rotations built by the library from synthetic calibration data. Steps cycle over layer
instances (separate pools, windows and rotations, sharing one block table) so every step
reads its KV pool from HBM, not from the 256 MB last-level cache.

Prints one JSON line. `value` is the headline step's algorithmic HBM bytes divided by its
time (GB/s). Each row (`rows`) has its step time and rate; `roofline` (the dominant kernel:
the one-launch step's kernel, or the attend launch of a two-launch step) against the 8 TB/s
HBM peak, timed with events on the launch stream, with `traffic` the HBM bytes per launch
from the committed counter summary under profiles/ while the kernel sources are unchanged;
and `cpu_baseline`, the CPU oracle timed on a bounded sample of the same workload. The
headline row also carries `multi_query` (oscar_decode_multi), `codebook` (the Lloyd-Max
codebook variant), `grouped` (groups of 64 and 32 dims), `calibration` and `bf16_baseline`
(plain BF16 decode of the same context); the 128K row carries `bulk_demote`.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "INT2 decode attention µs/step + achieved HBM GB/s (% of peak) at 32K–128K ctx"
HBM_PEAK_GBS = 8000.0
# MI355X's published fp32 peak (dense matrix cores, and the vector units with packed fp32:
# 256 CUs x 4 SIMDs x 32 FMA lanes per clock x 2 flops x 2.4 GHz)
FP32_PEAK_TFLOPS = 157.3
HIST_BYTES = 72          # per history token per KV head: 2 x 32 B codes + 2 x (fp16 s, fp16 z)
WIN_BYTES = 512          # per BF16 window token per KV head (K + V)
ROT_BYTES = 128 * 128 * 2
COPY_BYTES = 256 * 2 ** 20  # the plain copy whose counter readings calibrate FETCH_SIZE / WRITE_SIZE
CSRC = os.path.join(ROOT, "bit_kv_cache_oscar_amd", "csrc")
# the sources of the timed step kernels: a change to any of them retires the counter summaries
STEP_SOURCES = ("step.hip", "int2_pass.h", "merge_pass.h", "window_pass.h", "demote_pass.h", "grouped_pass.h",
                "device_common.h", "launch.h", "decode_int2.hip")
CONFIGS = (2, 3, 5, 4)  # headline first


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--configs", default=",".join(str(c) for c in CONFIGS),
                   help="workload configs, headline first (2: 32K, 3: 100K, 5: 128K B=4, 4: B=64)")
    p.add_argument("--config", type=int, default=0, help="one workload config only (overrides --configs)")
    p.add_argument("--layers", type=int, default=0, help="layer instances to cycle (0: enough for 512 MB)")
    p.add_argument("--splits", type=int, default=0, help="INT2 splits (0: library default)")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU oracle sample budget per row (0 disables)")
    p.add_argument("--extras", choices=("headline", "all", "none"), default="headline",
                   help="rows beyond the step (multi-query, codebook, grouped, calibration, BF16 baseline)")
    return p.parse_args()


def hist_tokens(w, unique):
    """History tokens the step reads: every request's own (logical), or with the shared
    prefix pages counted once (unique: what HBM must deliver at the least)."""
    n = int(sum(w.hist_lens))
    if unique and w.shared_pages:
        n -= (w.batch - 1) * w.shared_pages * 64
    return n


def step_bytes(w, unique=True):
    """Algorithmic bytes of one step: what the method must move, nothing of our workspace.
    Returns (step, attend launch) bytes."""
    hist = hist_tokens(w, unique) * w.n_kv_heads * HIST_BYTES
    win = int(sum(w.win_lens)) * w.n_kv_heads * WIN_BYTES
    rot = 2 * w.n_kv_heads * ROT_BYTES
    qo = w.batch * w.n_q_heads * 128 * (2 + 4)
    demote = w.batch * w.n_kv_heads * (2 * 256 + HIST_BYTES)
    # the attend launch: history pages, R_V for the un-rotation, the output
    attend = hist + w.n_kv_heads * ROT_BYTES + w.batch * w.n_q_heads * 128 * 4
    return hist + win + rot + qo + demote, attend


def step_source_hash():
    import hashlib

    h = hashlib.sha256()
    for f in STEP_SOURCES:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` ("append_kernel": the one-launch step's kernel,
    "main_kernel": the attend launch, "attend_codebook": the attend launch of the codebook
    variant, "multi_query": the one-launch multi-query decode, "grouped_pass_g64" / "_g32":
    the grouped INT2 pass alone, "grouped_attend_g64" / "_g32": the grouped step's attend
    launch) from the committed counter summary
    of this workload, or None when there is none or the kernel sources changed since it was
    taken. FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are each scaled by what the same
    counter reads for a plain copy of COPY_BYTES bytes in the same run."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    try:
        if kv.get("kernel_source_sha256") != step_source_hash():
            return None
        f = float(kv["fetch_kib_per_dispatch"]) * COPY_BYTES / float(kv["copy_fetch_kib"])
        wr = float(kv["write_kib_per_dispatch"]) * COPY_BYTES / float(kv["copy_write_kib"])
    except (KeyError, ValueError, ZeroDivisionError):
        return None
    return int(round(f + wr))


def timed_once(fn, stream, torch):
    """Milliseconds of one call of fn, with HIP events on `stream`."""
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    fn()
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop)


def blas_threads():
    try:
        from threadpoolctl import threadpool_info

        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def oracle_rotations(w, kv):
    """R_K, R_V of one KV head built by the oracle itself (bf16 values in fp64)."""
    import synth
    from oracle import rotation as orot

    if w.calib == "gram":
        r = orot.round_bf16(orot.rotation_from_covariance(orot.gram_covariance(synth.gram_matrix_source(w, kv))))
        return r, r
    q, k, v = synth.calibration_set(w, kv)
    return (orot.round_bf16(orot.rotation_from_covariance(orot.key_covariance(q))),
            orot.round_bf16(orot.rotation_from_covariance(orot.value_covariance(q, k, v, w.sm_scale))))


def cpu_baseline(w, budget_s):
    """The oracle, as it stands, on a bounded sample: demote one token of KV head 0 and
    decode that head's query heads over the full context, repeated until the budget is
    spent. Reported in the benchmark's unit (algorithmic GB/s)."""
    import synth
    from oracle import attention as oatt
    from oracle import quant as oquant

    kv = 0
    b = 0
    r_k, r_v = oracle_rotations(w, kv)
    rk, rv = {kv: r_k}, {kv: r_v}
    hk, hv = synth.history_rows(w, b, kv)
    kc, ks, kz, _ = oquant.quantize_rows(hk.astype(np.float64), rk[kv], w.clip_ratio)
    vc, vs, vz, _ = oquant.quantize_rows(hv.astype(np.float64), rv[kv], w.clip_ratio)
    hist = (kc, ks, kz, vc, vs, vz)
    wk, wv = synth.window_rows(w, b, kv)
    wk, wv = wk.astype(np.float64), wv.astype(np.float64)
    q = synth.query(w, b).astype(np.float64)
    step_k, step_v = hk[-1:].astype(np.float64), hv[-1:].astype(np.float64)
    reps, t0 = 0, time.perf_counter()
    while True:
        oquant.quantize_rows(step_k, rk[kv], w.clip_ratio)
        oquant.quantize_rows(step_v, rv[kv], w.clip_ratio)
        for h in range(kv * w.gq, (kv + 1) * w.gq):
            oatt.decode_head(q[h], rk[kv], rv[kv], wk, wv, hist, w.sm_scale)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    per_rep_bytes = (w.hist_len(b) * HIST_BYTES + w.win_len(b) * WIN_BYTES + 2 * ROT_BYTES
                     + w.gq * 128 * 6 + 2 * 256 + HIST_BYTES)
    rate = per_rep_bytes * reps / el
    total, _ = step_bytes(w)
    return {
        "value": round(rate / 1e9, 6),
        "unit": "GB/s",
        "cores": blas_threads(),
        "kind": "oracle",
        "sample": f"request 0, KV head 0 of {w.n_kv_heads} ({w.gq} query heads) over the full "
                  f"{w.ctx_lens[0]}-token context: demote one token + decode, {reps} repetitions in {el:.1f} s "
                  f"(oracle pool built beforehand, untimed); one repetition is "
                  f"{per_rep_bytes / total:.4f} of the step's bytes, and the whole step at this rate is the "
                  f"scaled figure",
        "sample_fraction_of_step": round(per_rep_bytes / total, 6),
        "us_per_step_scaled": round(total / rate * 1e6, 1),
    }


BULK_TOKENS = 32768  # the bulk-demotion workload: 262,144 K rows and 262,144 V rows at 8 KV heads


def bulk_demote(w, rk_bits, rv_bits, dev, stream, reps, codebook=None):
    """oscar_demote of BULK_TOKENS history tokens (every KV head, K and V) into fresh pages,
    timed with HIP events on the launch stream; rows drawn like the workload's history.
    With codebook = (K levels, V levels) [Hkv, 4], oscar_demote_codebook."""
    import torch

    import synth
    from bit_kv_cache_oscar_amd.layer import LayerCache

    n_pages = BULK_TOKENS // 64
    c = LayerCache(w.n_q_heads, w.n_kv_heads, 1, n_pages, n_pages, device=dev)
    clip = np.full(w.n_kv_heads, w.clip_ratio, np.float32)
    c.set_rotations(rk_bits, rv_bits, clip, clip)
    if codebook is not None:
        c.set_codebook(*codebook)
    ks, vs = [], []
    for kv in range(w.n_kv_heads):
        k, v = synth.kv_rows(w, 0, kv, 64, 64 + BULK_TOKENS)
        ks.append(k)
        vs.append(v)
    kk = torch.from_numpy(np.stack(ks, 1)).to(dev).to(torch.bfloat16)
    vv = torch.from_numpy(np.stack(vs, 1)).to(dev).to(torch.bfloat16)
    j = torch.arange(BULK_TOKENS, dtype=torch.int32, device=dev)
    pg, sl = (j // 64).contiguous(), (j % 64).contiguous()
    c.demote(kk, vv, pg, sl, stream)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(reps):
        c.demote(kk, vv, pg, sl, stream)
    stop.record(stream)
    torch.cuda.synchronize()
    us = start.elapsed_time(stop) * 1e3 / reps
    rows = 2 * BULK_TOKENS * w.n_kv_heads
    # 256 B in and 36 B out per row, and both rotations of every KV head
    nbytes = rows * (256 + 36) + w.n_kv_heads * 2 * ROT_BYTES
    return {
        "kernel": "demote_bulk_kernel (oscar_demote)" if codebook is None
                  else "demote_bulk_kernel<codebook> (oscar_demote_codebook)",
        "tokens": BULK_TOKENS,
        "rows": rows,
        "us": round(us, 3),
        "bound": "hbm",
        "achieved": round(nbytes / (us * 1e-6) / 1e9, 2),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "bytes": nbytes,
        "mfma_tflops": round(rows * 2 * 128 * 128 / (us * 1e-6) / 1e12, 2),
    }


BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak


class Setup:
    """One workload on the device: layer instances with filled pools, the step's inputs."""


def setup(cfg, args, dev, fill_rows_needed):
    import torch

    import synth
    from bit_kv_cache_oscar_amd import oscar_decode_step_append_splits, oscar_default_splits
    from bit_kv_cache_oscar_amd.layer import LayerCache
    from bit_kv_cache_oscar_amd.rotation import layer_rotations_from_calibration, layer_rotations_from_gram

    S = Setup()
    S.w = w = synth.workload(cfg)
    table, n_phys = synth.block_table(w)
    S.total_bytes, S.attend_bytes = step_bytes(w)
    S.logical_bytes, _ = step_bytes(w, unique=False)
    S.layers = args.layers or max(2, -(-512 * 2 ** 20 // max(S.logical_bytes, 1)))
    # rotations: the library's host builder from the synthetic calibration data
    if w.calib == "gram":
        S.rk_bits, S.rv_bits = layer_rotations_from_gram([synth.gram_matrix_source(w, kv) for kv in range(w.n_kv_heads)])
    else:
        S.rk_bits, S.rv_bits = layer_rotations_from_calibration(
            [synth.calibration_set(w, kv) for kv in range(w.n_kv_heads)], w.sm_scale)
    base = LayerCache(w.n_q_heads, w.n_kv_heads, w.batch, table.shape[1], n_phys, device=dev)
    S.clip = np.full(w.n_kv_heads, w.clip_ratio, np.float32)
    base.set_rotations(S.rk_bits, S.rv_bits, S.clip, S.clip)
    base.set_block_table(table)
    base.set_hist_len(w.hist_lens)
    base.set_win_len(w.win_lens)
    # fill: every history token but the last goes in by bulk demotion; the last one is the
    # token each timed step demotes from the recent window
    S.step_k = torch.zeros((w.batch, w.n_kv_heads, 128), dtype=torch.bfloat16, device=dev)
    S.step_v = torch.zeros_like(S.step_k)
    S.step_page = torch.zeros(w.batch, dtype=torch.int32, device=dev)
    S.step_slot = torch.zeros(w.batch, dtype=torch.int32, device=dev)
    S.fill_rows = []  # per request: the rows demoted by the fill (kept for the extra rows)
    for b in range(w.batch):
        n = w.hist_len(b)
        start = min(n, w.shared_pages * 64) if (w.shared_pages and b > 0) else 0
        ks, vs = [], []
        for kv in range(w.n_kv_heads):
            k, v = synth.kv_rows(w, b, kv, 64 + start, 64 + n)
            ks.append(k)
            vs.append(v)
            wk, wv = synth.window_rows(w, b, kv)
            base.set_window(b, kv, wk, wv)
        kk = torch.from_numpy(np.stack(ks, 1)).to(dev).to(torch.bfloat16)
        vv = torch.from_numpy(np.stack(vs, 1)).to(dev).to(torch.bfloat16)
        j = np.arange(start, n)
        pg = torch.from_numpy(table[b, j // 64].astype(np.int32)).to(dev)
        sl = torch.from_numpy((j % 64).astype(np.int32)).to(dev)
        if n - start > 1:
            base.demote(kk[:-1], vv[:-1], pg[:-1], sl[:-1])
            if fill_rows_needed:
                S.fill_rows.append((kk[:-1], vv[:-1], pg[:-1], sl[:-1]))
        S.step_k[b], S.step_v[b] = kk[-1], vv[-1]
        S.step_page[b], S.step_slot[b] = pg[-1], sl[-1]
    S.q = torch.from_numpy(np.stack([synth.query(w, b) for b in range(w.batch)])).to(dev).to(torch.bfloat16)
    # split counts: the two-launch default (attend launch), and the one-launch step's
    S.splits = args.splits or oscar_default_splits(base.desc, w.batch, int(w.hist_lens.max()))
    S.splits1 = args.splits or oscar_decode_step_append_splits(base.desc, w.batch, int(w.hist_lens.max()))
    base.set_splits(S.splits)
    S.insts = [base]
    for _ in range(S.layers - 1):
        c = LayerCache(w.n_q_heads, w.n_kv_heads, w.batch, table.shape[1], n_phys, device=dev)
        for name in ("pool", "k_win", "v_win", "rot_k", "rot_v", "clip_k", "clip_v"):
            getattr(c, name).copy_(getattr(base, name))
        # one request's page table and lengths serve every layer of a model
        c.block_table, c.hist_len, c.win_len = base.block_table, base.hist_len, base.win_len
        c.set_splits(S.splits)
        S.insts.append(c)
    S.base = base
    torch.cuda.synchronize()
    return S


def prepared(make):
    """A call per layer instance that make(c) builds once with the library's prepare=True (its
    arguments validated and marshalled then); later calls for that instance issue the C-ABI
    call alone, so that a timed loop measures the launches and not Python's checks (which
    take longer than a 32K step)."""
    cache = {}

    def call(c):
        f = cache.get(id(c))
        if f is None:
            f = cache[id(c)] = make(c)
        f()

    return call


def make_timer(S, stream, torch):
    def timed(fn, k):
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(k):
            fn(S.insts[i % S.layers])
        stop.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / k

    return timed


def pct(v):
    return [round(float(np.percentile(v, p)) * 1e3, 3) for p in (10, 50, 90)]


def step_row(S, args, stream, torch):
    """The step (oscar_decode_step_append) and its dominant kernel: times, rates, roofline."""
    from bit_kv_cache_oscar_amd import oscar_attend, oscar_decode_step_append_launches

    w = S.w
    launches = oscar_decode_step_append_launches(S.base.desc, w.batch, S.splits1)
    timed = make_timer(S, stream, torch)

    def make_step(c):
        c.n_splits = S.splits1
        return c.step_append(S.step_k, S.step_v, S.q, w.sm_scale, stream, prepare=True)

    def make_step2(c):  # the two-launch step, whose workspace the attend launch reads
        c.n_splits = S.splits
        return c.step(S.step_k, S.step_v, S.step_page, S.step_slot, S.q, w.sm_scale, stream, prepare=True)

    def make_attend(c):
        return oscar_attend(c.desc, c.rot_v, c.pool, c.block_table, c.hist_len, S.splits, c.workspace, c.out, stream,
                            prepare=True)

    step, step2, attend = prepared(make_step), prepared(make_step2), prepared(make_attend)

    for c in S.insts:  # every instance's workspaces allocated and prepared before any timing
        step2(c)
        step(c)
    for i in range(args.warmup):
        step(S.insts[i % S.layers])
    torch.cuda.synchronize()
    # timed region 1: whole steps back to back over the layer instances, then five more
    # regions for the spread (the reported figure stays the first region's)
    ms = timed(step, args.steps)
    rep_step = sorted([ms] + [timed(step, args.steps) for _ in range(5)])
    S.step_ms = ms
    row = {
        "workload": w.name,
        "entry": "oscar_decode_step_append (" + ("one launch" if launches == 1 else "prepare + attend") + ")",
        "batch": w.batch,
        "context_tokens": list(sorted(set(w.ctx_lens)))[:4] if len(set(w.ctx_lens)) <= 4 else
        [int(min(w.ctx_lens)), int(max(w.ctx_lens))],
        "q_heads": w.n_q_heads,
        "kv_heads": w.n_kv_heads,
        "int2_splits": S.splits1,
        "launches": launches,
        "layer_instances": S.layers,
        "us_per_step": round(ms * 1e3, 3),
        "us_per_step_p10_p50_p90": pct(rep_step),
        "step_bytes": S.total_bytes,
        "achieved_gbs": round(S.total_bytes / (ms * 1e-3) / 1e9, 2),
        "pct_of_hbm_peak": round(100 * S.total_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(w.batch / (ms * 1e-3), 1),
        "context_tokens_per_s": round(sum(w.ctx_lens) / (ms * 1e-3), 1),
    }
    if S.logical_bytes != S.total_bytes:
        row["bytes_note"] = ("step_bytes counts the shared prefix pages once (what HBM must deliver); "
                             "logical_step_bytes counts every request's own history")
        row["logical_step_bytes"] = S.logical_bytes
        row["logical_gbs"] = round(S.logical_bytes / (ms * 1e-3) / 1e9, 2)
    if launches == 1:
        # the one launch is the whole step: its kernel time is the step time measured above
        S.dominant_ms = ms
        roof = {
            "kernel": "append_kernel (oscar_decode_step_append: window, appended token, INT2 history, merge)",
            "bound": "hbm",
            "achieved": round(S.total_bytes / (ms * 1e-3) / 1e9, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(S.total_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(w.name, "append_kernel"),
            "us_per_launch": round(ms * 1e3, 3),
            "bytes_per_launch": S.total_bytes,
            "bytes_note": "the step's algorithmic bytes: history pages, window, R_K and R_V, query, output, "
                          "the appended token's rows and codes",
        }
    else:
        for i in range(max(2, args.warmup)):
            step2(S.insts[i % S.layers])
        attend_ms = timed(attend, args.steps)
        rep_attend = sorted([attend_ms] + [timed(attend, args.steps) for _ in range(5)])
        S.dominant_ms = attend_ms
        roof = {
            "kernel": "main_kernel (attend launch: INT2 history pass + merge)",
            "bound": "hbm",
            "achieved": round(S.attend_bytes / (attend_ms * 1e-3) / 1e9, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(S.attend_bytes / (attend_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(w.name, "main_kernel"),
            "us_per_launch": round(attend_ms * 1e3, 3),
            "us_per_launch_p10_p50_p90": pct(rep_attend),
            "bytes_per_launch": S.attend_bytes,
            "bytes_note": "history pages (shared prefix once) + R_V + output",
        }
        if S.logical_bytes != S.total_bytes:
            logical_attend = S.attend_bytes + (S.logical_bytes - S.total_bytes)
            roof["logical_bytes_per_launch"] = logical_attend
            roof["logical_gbs"] = round(logical_attend / (attend_ms * 1e-3) / 1e9, 2)
    if roof["traffic"] is not None:
        roof["traffic_gbs"] = round(roof["traffic"] / (roof["us_per_launch"] * 1e-6) / 1e9, 2)
        roof["traffic_frac"] = round(roof["traffic_gbs"] / HBM_PEAK_GBS, 4)
    row["roofline"] = roof
    return row


def extra_rows(S, args, stream, torch, dev, ceiling_gbs):
    """multi-query, grouped pages, codebook, calibration and BF16-baseline rows."""
    import synth
    from bit_kv_cache_oscar_amd import (oscar_decode_multi, oscar_decode_multi_splits, oscar_decode_workspace_bytes,
                                        oscar_window_splits)

    w, base, splits, layers, q = S.w, S.base, S.splits, S.layers, S.q
    step_k, step_v, step_page, step_slot = S.step_k, S.step_v, S.step_page, S.step_slot
    total_bytes, attend_bytes, ms = S.total_bytes, S.attend_bytes, S.step_ms
    rk_bits, rv_bits, clip, fill_rows = S.rk_bits, S.rv_bits, S.clip, S.fill_rows
    insts = S.insts
    out = {}

    def timed(fn, k):
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(k):
            fn(insts[i % layers])
        stop.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / k

    for c in insts:
        c.set_splits(splits)
    # timed region 3, the multi-query row: T query tokens per request over the same pools
    # (speculative verification reading the compressed prefix), oscar_decode_multi back to
    # back over the layer instances; T query heads' worth of rows per KV head, up to 16
    n_tok = min(4, 16 // w.gq)
    multi = None
    if n_tok >= 2:
        qm = torch.from_numpy(np.stack([synth.query_tokens(w, b, n_tok) for b in range(w.batch)])).to(dev)
        qm = qm.to(torch.bfloat16)
        msplits = oscar_decode_multi_splits(base.desc, w.batch, n_tok, int(w.hist_lens.max()))
        gqt = w.gq * n_tok
        m_items = (((oscar_window_splits(base.desc) + 1) // 2 + 1) * w.n_kv_heads * w.batch +
                   msplits * w.n_kv_heads * w.batch * (2 if gqt > 8 else 1))
        wsm = torch.zeros(oscar_decode_workspace_bytes(base.desc, w.batch * n_tok, msplits), dtype=torch.uint8,
                          device=dev)
        outm = torch.empty((w.batch, n_tok, w.n_q_heads, 128), dtype=torch.float32, device=dev)

        decode_multi = prepared(lambda c: oscar_decode_multi(
            c.desc, qm, c.rot_k, c.rot_v, c.pool, c.block_table, c.hist_len, c.k_win, c.v_win, c.win_len, w.sm_scale,
            msplits, wsm, outm, stream, prepare=True))

        for i in range(max(2, args.warmup)):
            decode_multi(insts[i % layers])
        multi_ms = timed(decode_multi, args.steps)
        launches_m = 1 if m_items <= 256 else 2
        hist = int(sum(w.hist_lens)) * w.n_kv_heads * HIST_BYTES
        win = int(sum(w.win_lens)) * w.n_kv_heads * WIN_BYTES
        mbytes = hist + win + 2 * w.n_kv_heads * ROT_BYTES + w.batch * n_tok * w.n_q_heads * 128 * (2 + 4)
        multi = {
            "entry": "oscar_decode_multi (no demotion)",
            "launches": launches_m,
            "n_splits": msplits,
            "query_tokens": n_tok,
            "us_per_call": round(multi_ms * 1e3, 3),
            "vs_one_token_step": round(multi_ms / ms, 3),
            "bound": "hbm",
            "achieved": round(mbytes / (multi_ms * 1e-3) / 1e9, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(mbytes / (multi_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "bytes_per_call": mbytes,
            "traffic": measured_traffic(w.name, "multi_query") if launches_m == 1 else None,
            "query_tokens_per_s": round(w.batch * n_tok / (multi_ms * 1e-3), 1),
        }

    # timed region 5, grouped pages (one scale and zero point per 64 or 32 rotated dims): the
    # same history demoted into grouped pools of every instance, then the three-launch decode
    # (oscar_decode_int2_grouped, oscar_decode_bf16, oscar_merge) and the grouped INT2 pass
    # alone, back to back over the instances
    from bit_kv_cache_oscar_amd import oscar_attend, oscar_decode_int2_grouped, oscar_default_splits
    from bit_kv_cache_oscar_amd.layer import LayerCache

    # the one-group baselines: the two-launch step and its attend launch alone, at the
    # two-launch default split count
    def make_one_step2(c):
        c.n_splits = splits
        return c.step(step_k, step_v, step_page, step_slot, q, w.sm_scale, stream, prepare=True)

    one_step2 = prepared(make_one_step2)
    one_attend = prepared(lambda c: oscar_attend(c.desc, c.rot_v, c.pool, c.block_table, c.hist_len, splits,
                                                 c.workspace, c.out, stream, prepare=True))

    for i in range(max(2, args.warmup)):
        one_step2(insts[i % layers])
    one_step2_ms = timed(one_step2, args.steps)
    one_attend_ms = timed(one_attend, args.steps)
    grouped_rows = {"one_group_step_us": round(one_step2_ms * 1e3, 3),
                    "one_group_attend_us": round(one_attend_ms * 1e3, 3)}
    for group in (64, 32):
        ng = 128 // group
        gins = []
        for i in range(layers):
            g = LayerCache(w.n_q_heads, w.n_kv_heads, w.batch, base.block_table.shape[1],
                           base.pool.numel() // (w.n_kv_heads * 4608), device=dev, group_size=group)
            for name in ("rot_k", "rot_v", "clip_k", "clip_v", "block_table", "hist_len", "k_win", "v_win",
                         "win_len"):
                getattr(g, name).copy_(getattr(base, name))
            if i == 0:
                for kk, vv, pg, sl in fill_rows:
                    g.demote(kk, vv, pg, sl, stream)
            else:
                g.pool.copy_(gins[0].pool)
            g.set_splits(oscar_default_splits(g.desc, w.batch, int(max(w.hist_lens))))
            gins.append(g)
        torch.cuda.synchronize()

        def g_decode(c):  # an unprepared call: it sets up each instance's partials
            c.decode(q, w.sm_scale, stream)

        def make_g_decode(c):
            return c.decode(q, w.sm_scale, stream, prepare=True)

        def make_g_int2(c):
            return oscar_decode_int2_grouped(c.desc, q, c.rot_k, c.pool, c.block_table, c.hist_len, w.sm_scale,
                                             c.n_splits, c.partials, stream, prepare=True)

        saved = insts
        insts = gins
        # split counts: the library default and about 16, 8, 4 and 2 pages per split (this
        # pass gains from more, smaller workgroups); the fastest is reported
        n_pg = -(-int(max(w.hist_lens)) // 64)
        sweep = {}
        for sp in sorted({gins[0].n_splits} | {max(1, min(65535, -(-n_pg // k))) for k in (16, 8, 4, 2)}):
            for c in gins:
                c.set_splits(sp)
            for i in range(max(2, args.warmup)):
                g_decode(insts[i % layers])
            sweep[sp] = timed(prepared(make_g_int2), args.steps)
        best = min(sweep, key=sweep.get)
        for c in gins:
            c.set_splits(best)
        g_decode(insts[0])
        g_ms = timed(prepared(make_g_decode), args.steps)
        g_int2_ms = timed(prepared(make_g_int2), args.steps)
        g_step = prepared(lambda c: c.step(step_k, step_v, step_page, step_slot, q, w.sm_scale, stream, prepare=True))

        # the two-launch grouped step at the library's default split count
        g_splits = oscar_default_splits(gins[0].desc, w.batch, int(max(w.hist_lens)))
        for c in gins:
            c.set_splits(g_splits)
        for i in range(max(2, args.warmup)):
            g_step(insts[i % layers])
        g_step_ms = timed(g_step, args.steps)
        insts = saved
        g_bytes = int(sum(w.hist_lens)) * w.n_kv_heads * (64 + 8 * ng) + w.n_kv_heads * ROT_BYTES + \
            w.batch * w.n_q_heads * 128 * 2
        grouped_rows[f"group_{group}"] = {
            "entry": "oscar_decode_int2_grouped + oscar_decode_bf16 + oscar_merge; pass alone: "
                     "oscar_decode_int2_grouped",
            "history_bytes_per_token_head": 64 + 8 * ng,
            "splits": gins[0].n_splits,
            "int2_pass_us_by_splits": {str(k): round(v * 1e3, 3) for k, v in sorted(sweep.items())},
            "us_per_decode": round(g_ms * 1e3, 3),
            "us_per_step": round(g_step_ms * 1e3, 3),
            "step_splits": g_splits,
            "step_entry": "oscar_decode_step_grouped (prepare: demotion, window pass, query; attend: grouped "
                          "matrix-core pass + merge)",
            "step_vs_one_group_step": round(g_step_ms / one_step2_ms, 3),
            "int2_pass_us_per_launch": round(g_int2_ms * 1e3, 3),
            "int2_pass_vs_one_group_attend": round(g_int2_ms / one_attend_ms, 3),
            "bound": "hbm",
            "achieved": round(g_bytes / (g_int2_ms * 1e-3) / 1e9, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(g_bytes / (g_int2_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(w.name, f"grouped_pass_g{group}"),
            "attend_traffic": measured_traffic(w.name, f"grouped_attend_g{group}"),
        }
        del gins
        torch.cuda.empty_cache()

    # timed region 4, the Lloyd-Max codebook variant: per-head K and V codebooks fitted on the
    # calibration set by the library's host calibration; the same history demoted against
    # them into every instance's pool; then whole steps and the attend launch alone, as above
    cb_row = None
    if w.calib != "gram":
        from bit_kv_cache_oscar_amd import oscar_attend_codebook
        from bit_kv_cache_oscar_amd.codebook import layer_codebooks

        klv, vlv = layer_codebooks([synth.calibration_set(w, kv) for kv in range(w.n_kv_heads)], rk_bits, rv_bits,
                                   clip, clip)
        base.set_codebook(klv, vlv)
        for kk, vv, pg, sl in fill_rows:
            base.demote(kk, vv, pg, sl)
        for c in insts[1:]:
            c.pool.copy_(base.pool)
            c.codebook = base.codebook

        step_cb = prepared(lambda c: c.step(step_k, step_v, step_page, step_slot, q, w.sm_scale, stream,
                                            prepare=True))
        attend_cb = prepared(lambda c: oscar_attend_codebook(c.desc, c.rot_v, c.codebook, c.pool, c.block_table,
                                                             c.hist_len, c.n_splits, c.workspace, c.out, stream,
                                                             prepare=True))

        for c in insts:  # every workspace prepared with the codebook before the attend timing
            step_cb(c)
        for i in range(args.warmup):
            step_cb(insts[i % layers])
        cb_ms = timed(step_cb, args.steps)
        cb_attend_ms = timed(attend_cb, args.steps)
        cb_row = {
            "entry": "oscar_decode_step_codebook (prepare + attend); attend alone: oscar_attend_codebook",
            "k_levels_head0": [int(x) for x in klv[0]],
            "v_levels_head0": [int(x) for x in vlv[0]],
            "us_per_step": round(cb_ms * 1e3, 3),
            "step_gbs": round(total_bytes / (cb_ms * 1e-3) / 1e9, 2),
            "attend_us_per_launch": round(cb_attend_ms * 1e3, 3),
            "bound": "hbm",
            "achieved": round(attend_bytes / (cb_attend_ms * 1e-3) / 1e9, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(attend_bytes / (cb_attend_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(w.name, "attend_codebook"),
        }
        del fill_rows

    # the calibration row: the covariances behind R_K and R_V (oscar_calib_covariances) from
    # the workload's 512-token calibration sequence of every KV head
    calib_row = None
    if w.calib != "gram":
        from bit_kv_cache_oscar_amd import oscar_calib_covariances, oscar_calib_workspace_bytes

        cal = [synth.calibration_set(w, kv) for kv in range(w.n_kv_heads)]
        n_cal = cal[0][1].shape[0]
        qc = torch.from_numpy(np.concatenate([c[0] for c in cal], axis=1)).to(dev).to(torch.bfloat16)
        kc = torch.from_numpy(np.stack([c[1] for c in cal], axis=1)).to(dev).to(torch.bfloat16)
        vc = torch.from_numpy(np.stack([c[2] for c in cal], axis=1)).to(dev).to(torch.bfloat16)
        wsc = torch.empty(oscar_calib_workspace_bytes(base.desc, n_cal), dtype=torch.uint8, device=dev)
        sig_k = torch.empty((w.n_kv_heads, 128, 128), dtype=torch.float32, device=dev)
        sig_v = torch.empty_like(sig_k)

        def calib():
            oscar_calib_covariances(base.desc, qc, kc, vc, w.sm_scale, wsc, sig_k, sig_v, stream)

        calib()
        reps = 20
        cal_ms = timed_once(lambda: [calib() for _ in range(reps)], stream, torch) / reps
        rows = n_cal * w.n_q_heads
        causal = w.n_q_heads * (n_cal * (n_cal + 1) // 2)
        # bf16 matrix-core work: the scores q k^T and the key Gram sum of q; fp32 matrix-core
        # work: the weighted value sums S V and the value Gram sum of S V. Each is priced at
        # its own peak: frac is the time a launch running both at peak would take, over the
        # measured time.
        bf16_flops = 2 * causal * 128 + 2 * rows * 128 * 128
        fp32_flops = 2 * causal * 128 + 2 * rows * 128 * 128
        ideal_s = bf16_flops / (BF16_PEAK_TFLOPS * 1e12) + fp32_flops / (FP32_PEAK_TFLOPS * 1e12)
        calib_row = {
            "entry": "oscar_calib_covariances (Sigma_K = sum Q^T Q, Sigma_V = sum (S V)^T (S V))",
            "tokens": n_cal,
            "us": round(cal_ms * 1e3, 3),
            "bound": "mfma",
            "bf16_flops": bf16_flops,
            "fp32_flops": fp32_flops,
            "achieved_bf16_tflops": round(bf16_flops / (cal_ms * 1e-3) / 1e12, 3),
            "achieved_fp32_tflops": round(fp32_flops / (cal_ms * 1e-3) / 1e12, 3),
            "peak_bf16_tflops": BF16_PEAK_TFLOPS,
            "peak_fp32_tflops": FP32_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(ideal_s / (cal_ms * 1e-3), 4),
            "frac_note": "(bf16 flops / bf16 peak + fp32 flops / fp32 peak) / measured time",
        }

    # the uncompressed baseline: plain BF16 decode attention over the same context held dense
    # (oscar_decode_dense_bf16), on instances cycled as above; the MI355X counterpart of the
    # pages' INT2-versus-BF16 decode comparison (context, not a target). Its cost does not
    # depend on the values: random bf16 rows.
    from bit_kv_cache_oscar_amd import oscar_decode_dense_bf16, oscar_dense_workspace_bytes

    cap = -(-int(max(w.ctx_lens)) // 64) * 64
    dense_bytes = 2 * w.batch * w.n_kv_heads * cap * 128 * 2
    n_dense = max(1, min(4, -(-512 * 2 ** 20 // dense_bytes)))
    lens_t = torch.tensor(list(w.ctx_lens), dtype=torch.int32, device=dev)
    dense = [(torch.randn((w.batch, w.n_kv_heads, cap, 128), device=dev).to(torch.bfloat16),
              torch.randn((w.batch, w.n_kv_heads, cap, 128), device=dev).to(torch.bfloat16)) for _ in range(n_dense)]
    ws_d = torch.empty(oscar_dense_workspace_bytes(base.desc, w.batch, cap), dtype=torch.uint8, device=dev)
    out_d = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.float32, device=dev)

    def dense_call(i):
        kd, vd = dense[i % n_dense]
        oscar_decode_dense_bf16(base.desc, q, kd, vd, lens_t, w.sm_scale, ws_d, out_d, stream)

    for i in range(max(2, args.warmup)):
        dense_call(i)
    dense_ms = timed_once(lambda: [dense_call(i) for i in range(args.steps)], stream, torch) / args.steps
    dense_alg = int(sum(w.ctx_lens)) * w.n_kv_heads * WIN_BYTES + w.batch * w.n_q_heads * 128 * (2 + 4)
    dense_row = {
        "entry": "oscar_decode_dense_bf16 (BF16 K/V of the whole context, no compression)",
        "us_per_call": round(dense_ms * 1e3, 3),
        "achieved": round(dense_alg / (dense_ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "frac": round(dense_alg / (dense_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "bytes_per_call": dense_alg,
        "int2_step_speedup": round(dense_ms / ms, 3),
        "int2_dominant_kernel_speedup": round(dense_ms / S.dominant_ms, 3),
        # against any BF16 decode of this context on this machine: its bytes at the measured read
        # ceiling (a bound no BF16 kernel can beat)
        "bf16_at_ceiling_us": round(dense_alg / (ceiling_gbs * 1e9) * 1e6, 3),
        "int2_step_speedup_vs_ceiling": round(dense_alg / (ceiling_gbs * 1e9) / (ms * 1e-3), 3),
        "kv_bytes_ratio": round(dense_alg / max(total_bytes, 1), 3),
    }
    del dense, ws_d, out_d

    if multi is not None:
        out["multi_query"] = multi
    if cb_row is not None:
        out["codebook"] = cb_row
    out["grouped"] = grouped_rows
    if calib_row is not None:
        out["calibration"] = calib_row
    out["bf16_baseline"] = dense_row
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this path has no multi-GPU mode (the pool shards by KV head "
              "or request with no exchange; see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    dev = torch.device("cuda:0")
    configs = [args.config] if args.config else [int(c) for c in args.configs.split(",") if c.strip()]
    stream = torch.cuda.current_stream()
    t_start = time.perf_counter()

    # one plain copy of known size (untimed): its FETCH_SIZE / WRITE_SIZE readings calibrate
    # the counters of the kernels in the same profiled run
    src = torch.empty(COPY_BYTES // 4, dtype=torch.int32, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst

    # measured stream ceiling of this machine: the library's read probe over 1 GiB, best of five
    from bit_kv_cache_oscar_amd import oscar_read_probe

    probe = torch.ones(2 ** 28, dtype=torch.int32, device=dev)
    probe_out = torch.zeros(4096, dtype=torch.int32, device=dev)
    oscar_read_probe(probe, probe_out, stream)
    ceil_ms = min(timed_once(lambda: oscar_read_probe(probe, probe_out, stream), stream, torch) for _ in range(5))
    del probe, probe_out
    ceiling_gbs = 2 ** 30 / (ceil_ms * 1e-3) / 1e9

    rows = []
    for i, cfg in enumerate(configs):
        headline = i == 0
        want_extras = args.extras == "all" or (args.extras == "headline" and headline)
        S = setup(cfg, args, dev, fill_rows_needed=want_extras)
        row = step_row(S, args, stream, torch)
        row["roofline"]["frac_of_measured_ceiling"] = round(
            row["roofline"]["achieved"] / ceiling_gbs, 4)
        if want_extras:
            row.update(extra_rows(S, args, stream, torch, dev, ceiling_gbs))
        if cfg == 5:
            # the bulk-demotion row of this workload (after the decode timing: it allocates)
            row["bulk_demote"] = bulk_demote(S.w, S.rk_bits, S.rv_bits, dev, stream, max(5, args.steps // 5))
        if args.cpu_seconds > 0:
            row["cpu_baseline"] = cpu_baseline(S.w, args.cpu_seconds)
        rows.append(row)
        print(f"[bench] {S.w.name}: {row['us_per_step']} us/step, roofline frac {row['roofline']['frac']}, "
              f"{time.perf_counter() - t_start:.0f} s elapsed", file=sys.stderr, flush=True)
        del S
        torch.cuda.empty_cache()

    h = rows[0]
    ms = h["us_per_step"] * 1e-3
    out = {
        "metric": METRIC,
        "value": h["achieved_gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "us_per_step": h["us_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {
            "workload": h["workload"],
            "batch": h["batch"],
            "context_tokens": h["context_tokens"],
            "q_heads": h["q_heads"],
            "kv_heads": h["kv_heads"],
            "head_dim": 128,
            "page_tokens": 64,
            "int2_splits": h["int2_splits"],
            "layer_instances": h["layer_instances"],
            "step": "oscar_decode_step_append: demote 1 token/request + BF16 pass + INT2 pass + merge",
        },
        "step_bytes": h["step_bytes"],
        "pct_of_hbm_peak": h["pct_of_hbm_peak"],
        "roofline": h["roofline"],
        "stream_ceiling": {"probe": "oscar_read_probe over 1 GiB (streaming 16-byte loads), best of 5",
                           "gbs": round(ceiling_gbs, 1), "frac_of_peak": round(ceiling_gbs / HBM_PEAK_GBS, 4)},
        "rows": {r["workload"]: r for r in rows},
        "wall_s": round(time.perf_counter() - t_start, 1),
    }
    if "cpu_baseline" in h:
        out["cpu_baseline"] = h["cpu_baseline"]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
