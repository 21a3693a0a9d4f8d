"""GPU parity of the dense BF16 baseline (MI355X only): oscar_decode_dense_bf16 against the
oracle's plain softmax attention in fp64 over the same bf16 rows, at the decode tolerance."""

import numpy as np
import pytest

import synth
from gpu_harness import assert_close

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg,lens,cap", [(2, [4000, 1, 64], 4096), (5, [2500, 130], 2560), (1, [1344], 1344)])
def test_dense_bf16_decode_matches_plain_attention(cfg, lens, cap):
    from bit_kv_cache_oscar_amd import layer_desc, oscar_decode_dense_bf16, oscar_dense_workspace_bytes
    from oracle import attention as oatt

    base = synth.workload(cfg)
    w = base.with_ctx(lens)
    B = len(lens)
    k = np.zeros((B, w.n_kv_heads, cap, 128), np.float32)
    v = np.zeros_like(k)
    for b in range(B):
        for kv in range(w.n_kv_heads):
            kr, vr = synth.kv_rows(w, b, kv, 0, lens[b])
            k[b, kv, :lens[b]], v[b, kv, :lens[b]] = kr, vr
    q = np.stack([synth.query(w, b) for b in range(B)])
    dev = torch.device("cuda")

    def t16(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev).to(torch.bfloat16)

    desc = layer_desc(w.n_q_heads, w.n_kv_heads)
    ws = torch.empty(oscar_dense_workspace_bytes(desc, B, cap), dtype=torch.uint8, device=dev)
    out = torch.full((B, w.n_q_heads, 128), np.nan, dtype=torch.float32, device=dev)
    ln = torch.tensor(lens, dtype=torch.int32, device=dev)
    print("[case] dense bf16", w.name, "lens", lens, "capacity", cap, flush=True)
    oscar_decode_dense_bf16(desc, t16(q), t16(k), t16(v), ln, w.sm_scale, ws, out)
    got = out.cpu().numpy()
    for b in range(B):
        for h in range(w.n_q_heads):
            kv = h // w.gq
            ref = oatt.softmax_attention(q[b, h].astype(np.float64), k[b, kv, :lens[b]].astype(np.float64),
                                         v[b, kv, :lens[b]].astype(np.float64), w.sm_scale)
            assert_close(got[b, h], ref, f"dense b{b} h{h}")
