"""GPU parity of the calibration covariances (MI355X only): oscar_calib_covariances against
the oracle's key_covariance and value_covariance (fp64) on each workload's synthetic
calibration sequences, rounded to bf16 for both sides.

Tolerance, per entry (i, j), from the arithmetic. The GPU sums n = T * G products in fp32
(the bf16 products are exact), so |error| <= n 2^-24 sum_r |x_ri| |x_rj|. For the values each
attention output also carries the fp32 error of its scores: a score whose terms sum to at
most A in magnitude (log2 units) is off by at most 130 2^-24 A; that moves each softmax
weight by a relative 2 ln 2 of it (twice, numerator and sum), and the fp32 running sums over
T keys and the exp2 add (T + 10) 2^-24; with e the total, output entry O_ri is off by at most
e W_ri, W_ri = sum_u p_ru |v_ui|, so the Gram sums move by at most
e sum_r (W_ri |O_rj| + |O_ri| W_rj) more."""

import numpy as np
import pytest

import synth
from gpu_harness import rotations
from oracle import rotation as orot

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634


def calib_inputs(w):
    """bf16-rounded calibration sequences of every KV head: q [T, Hq, 128], k, v [T, Hkv, 128]."""
    cal = [synth.calibration_set(w, kv) for kv in range(w.n_kv_heads)]
    q = np.concatenate([orot.round_bf16(c[0]) for c in cal], axis=1)
    k = np.stack([orot.round_bf16(c[1]) for c in cal], axis=1)
    v = np.stack([orot.round_bf16(c[2]) for c in cal], axis=1)
    return q, k, v


@pytest.mark.parametrize("cfg,n_tok", [(2, 512), (5, 512), (4, 300), (2, 37)])
def test_calib_covariances_match_oracle(cfg, n_tok):
    from bit_kv_cache_oscar_amd import layer_desc, oscar_calib_covariances, oscar_calib_workspace_bytes

    w = synth.workload(cfg)
    q, k, v = calib_inputs(w)
    q, k, v = q[:n_tok], k[:n_tok], v[:n_tok]
    desc = layer_desc(w.n_q_heads, w.n_kv_heads)
    dev = torch.device("cuda")

    def t16(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev).to(torch.bfloat16)

    ws = torch.empty(oscar_calib_workspace_bytes(desc, n_tok), dtype=torch.uint8, device=dev)
    sk = torch.full((w.n_kv_heads, 128, 128), np.nan, dtype=torch.float32, device=dev)
    sv = torch.full_like(sk, np.nan)
    print("[case] calibration covariances", w.name, "T", n_tok, flush=True)
    for rep in range(2):
        oscar_calib_covariances(desc, t16(q), t16(k), t16(v), w.sm_scale, ws, sk, sv)
        gk, gv = sk.cpu().numpy().astype(np.float64), sv.cpu().numpy().astype(np.float64)
        if rep == 0:
            first = (gk.copy(), gv.copy())
    assert np.array_equal(first[0], gk) and np.array_equal(first[1], gv), "not deterministic"
    n = n_tok * w.gq
    for kv in range(w.n_kv_heads):
        qg = q[:, kv * w.gq:(kv + 1) * w.gq, :]
        rk = orot.key_covariance(qg)
        rv = orot.value_covariance(qg, k[:, kv], v[:, kv], w.sm_scale)
        aq = np.abs(qg).reshape(-1, 128)
        tol_k = n * 2.0 ** -24 * (aq.T @ aq)
        tol_v = np.zeros((128, 128))
        for g in range(w.gq):
            sc = orot.causal_softmax_scores(qg[:, g, :], k[:, kv], w.sm_scale)
            o = np.abs(sc @ v[:, kv])
            wabs = sc @ np.abs(v[:, kv])
            a = float(np.max(np.abs(w.sm_scale * qg[:, g, :]) @ np.abs(k[:, kv]).T)) * LOG2E
            e = 4 * np.log(2) * 130 * 2.0 ** -24 * a + (n_tok + 10) * 2.0 ** -24
            tol_v += e * (wabs.T @ o + o.T @ wabs) + n * 2.0 ** -24 * (o.T @ o)
        for got, ref, tol, name in ((gk[kv], rk, tol_k, "sigma_k"), (gv[kv], rv, tol_v, "sigma_v")):
            err = np.abs(got - ref)
            worst = float(np.max(err / (tol + 1e-300)))
            print(f"[case] {name} kv{kv}: max |err| / tol = {worst:.3e}, max rel {float(np.max(err) / np.max(np.abs(ref))):.2e}",
                  flush=True)
            assert worst <= 1.0, (name, kv, worst)
            assert np.array_equal(got, got.T)
        # a rotation built from the GPU's key covariance is orthogonal
        r = orot.rotation_from_covariance(gk[kv])
        assert np.abs(r.T @ r - np.eye(128)).max() < 1e-10
