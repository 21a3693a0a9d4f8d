"""Test-side helpers: build one workload's inputs for both sides and the oracle's
expectations. Inputs come from synth; expectations come only from oracle/."""

from __future__ import annotations

import numpy as np

import synth
from oracle import attention as oatt
from oracle import pages as opages
from oracle import quant as oquant
from oracle import rotation as orot

MAX_ABS = 2e-3
REL_L2 = 1e-3
CODE_BAND = 1e-4        # near-boundary band of t in which a code may differ by one
CODE_FRACTION = 1e-4    # at most this fraction of codes may use the band


def bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return synth.bf16_value(bits).astype(np.float64)


def rotations(w: synth.Workload):
    """((rk_bits, rv_bits) from the library's host builder, (rk, rv) fp64 bf16 values from
    the oracle). The two must agree bit for bit; callers assert it."""
    from bit_kv_cache_oscar_amd import rotation as prot

    if w.calib == "gram":
        srcs = [synth.gram_matrix_source(w, kv) for kv in range(w.n_kv_heads)]
        rk_bits, rv_bits = prot.layer_rotations_from_gram(srcs)
        rk = np.stack([orot.round_bf16(orot.rotation_from_covariance(orot.gram_covariance(a))) for a in srcs])
        rv = rk.copy()
    else:
        cal = [synth.calibration_set(w, kv) for kv in range(w.n_kv_heads)]
        rk_bits, rv_bits = prot.layer_rotations_from_calibration(cal, w.sm_scale)
        rk = np.stack([orot.round_bf16(orot.rotation_from_covariance(orot.key_covariance(q))) for q, _, _ in cal])
        rv = np.stack([orot.round_bf16(orot.rotation_from_covariance(orot.value_covariance(q, k, v, w.sm_scale)))
                       for q, k, v in cal])
    return (rk_bits, rv_bits), (rk, rv)


def clips(w: synth.Workload):
    c = np.full(w.n_kv_heads, w.clip_ratio, np.float32)
    return c, c.copy()


def oracle_history(w, b, kv, rk, rv, n=None):
    """Oracle demotion of request b's history for one KV head:
    ((kc, ks, kz, vc, vs, vz), k_margin, v_margin)."""
    hk, hv = synth.history_rows(w, b, kv)
    if n is not None:
        hk, hv = hk[:n], hv[:n]
    kc, ks, kz, km = oquant.quantize_rows(hk.astype(np.float64), rk[kv], w.clip_ratio)
    vc, vs, vz, vm = oquant.quantize_rows(hv.astype(np.float64), rv[kv], w.clip_ratio)
    return (kc, ks, kz, vc, vs, vz), km, vm


def oracle_pool(w, rk, rv):
    """(pool uint8 [n_phys, Hkv, 4608], table, hists[b][kv]) built entirely by the oracle."""
    table, n_phys = synth.block_table(w)
    pool = opages.new_pool(n_phys, w.n_kv_heads)
    hists = [[None] * w.n_kv_heads for _ in range(w.batch)]
    for b in range(w.batch):
        for kv in range(w.n_kv_heads):
            hist, _, _ = oracle_history(w, b, kv, rk, rv)
            hists[b][kv] = hist
            opages.pack_history(pool, table[b], kv, hist)
    return pool, table, hists


def windows(w, b):
    """(win_k, win_v) [Hkv, n_w, 128] float64 of request b."""
    ks, vs = [], []
    for kv in range(w.n_kv_heads):
        k, v = synth.window_rows(w, b, kv)
        ks.append(k)
        vs.append(v)
    return np.stack(ks).astype(np.float64), np.stack(vs).astype(np.float64)


def oracle_decode(w, b, rk, rv, hists_b, heads=None):
    q = synth.query(w, b).astype(np.float64)
    wk, wv = windows(w, b)
    out = np.zeros((w.n_q_heads, 128))
    for h in (range(w.n_q_heads) if heads is None else heads):
        kv = h // w.gq
        out[h] = oatt.decode_head(q[h], rk[kv], rv[kv], wk[kv], wv[kv], hists_b[kv], w.sm_scale)
    return out


def assert_close(got, ref, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    max_abs = float(err.max()) if err.size else 0.0
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert max_abs <= MAX_ABS and rel <= REL_L2, f"{what}: max_abs {max_abs:.3e} rel_l2 {rel:.3e}"
    return max_abs, rel


def compare_history(gpu_hist, ref_hist, k_margin, v_margin, what=""):
    """Codes and scales of one head's history: scales bit-exact, codes equal except where
    the oracle's t lies within CODE_BAND of a rounding boundary (at most CODE_FRACTION)."""
    gkc, gks, gkz, gvc, gvs, gvz = gpu_hist
    rkc, rks, rkz, rvc, rvs, rvz = ref_hist
    for a, b, name in ((gks, rks, "k scale"), (gkz, rkz, "k zero"), (gvs, rvs, "v scale"), (gvz, rvz, "v zero")):
        ab = np.asarray(a, np.float16).view(np.uint16)
        bb = np.asarray(b, np.float16).view(np.uint16)
        bad = np.nonzero(ab != bb)[0]
        assert bad.size == 0, f"{what}: {name} differs at {bad[:5]}"
    total = 0
    for g, r, mg, name in ((gkc, rkc, k_margin, "k"), (gvc, rvc, v_margin, "v")):
        diff = g != r
        if diff.any():
            assert np.all(mg[diff] < CODE_BAND), f"{what}: {name} code differs away from a boundary"
            assert np.all(np.abs(g.astype(int) - r.astype(int))[diff] == 1)
        total += int(diff.sum())
    n = gkc.size + gvc.size
    assert total <= CODE_FRACTION * n, f"{what}: {total} of {n} codes differ"
    return total
