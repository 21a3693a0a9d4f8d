"""The decode step without a caller workspace (oscar_decode_step_noalloc) against
oscar_decode_step with one: the same kernels, so the same pool bytes and the same outputs
bit for bit, on two calls in a row, the second with a smaller input (fewer requests, fewer
query heads per KV head, a shorter history); and a request larger than the static array
rejected before anything is enqueued."""

from __future__ import annotations

import numpy as np
import pytest

import synth
from gpu_harness import assert_close, oracle_decode, oracle_pool, rotations
from test_gpu_parity import DECODE_CASES, bf16, make_cache, queries, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import bit_kv_cache_oscar_amd as ok
    ok.lib()


def _run(case):
    """(output and pool of oscar_decode_step, the same of oscar_decode_step_noalloc, oracle
    outputs) for one decode step that demotes each request's last history token."""
    import bit_kv_cache_oscar_amd as ok

    w = DECODE_CASES[case]()
    (rk_bits, rv_bits), (rk, rv) = rotations(w)
    pool, table, hists = oracle_pool(w, rk, rv)
    refs = [oracle_decode(w, b, rk, rv, hists[b]) for b in range(w.batch)]
    c = make_cache(w, rk_bits, rv_bits, table, pool.shape[0])
    c.set_splits(ok.oscar_default_splits(c.desc, w.batch, int(w.hist_lens.max())))
    q = queries(w)
    # the step demotes each request's last history token again, over the oracle's bytes
    lk, lv, lp, ls = [], [], [], []
    for b in range(w.batch):
        n = w.hist_len(b)
        ks = np.stack([synth.kv_rows(w, b, kv, 64 + n - 1, 64 + n)[0][0] for kv in range(w.n_kv_heads)])
        vs = np.stack([synth.kv_rows(w, b, kv, 64 + n - 1, 64 + n)[1][0] for kv in range(w.n_kv_heads)])
        lk.append(ks)
        lv.append(vs)
        lp.append(table[b, (n - 1) // 64])
        ls.append((n - 1) % 64)
    kr, vr = bf16(np.stack(lk)), bf16(np.stack(lv))
    pg = torch.tensor(np.array(lp, np.int32), device="cuda")
    sl = torch.tensor(np.array(ls, np.int32), device="cuda")
    base = torch.from_numpy(pool.reshape(-1)).cuda()
    c.pool.copy_(base)
    say(case, "oscar_decode_step with a workspace", "B", w.batch, "splits", c.n_splits)
    want = c.step(kr, vr, pg, sl, q, w.sm_scale).clone()
    want_pool = c.pool.clone()
    c.pool.copy_(base)
    got = torch.full_like(c.out, float("nan"))
    say(case, "oscar_decode_step_noalloc", "B", w.batch, "splits", c.n_splits)
    ok.oscar_decode_step_noalloc(c.desc, kr, vr, pg, sl, c.clip_k, c.clip_v, q, c.rot_k, c.rot_v, c.pool,
                                 c.block_table, c.hist_len, c.k_win, c.v_win, c.win_len, w.sm_scale, c.n_splits, got)
    torch.cuda.synchronize()
    return (want.cpu().numpy(), want_pool.cpu().numpy()), (got.cpu().numpy(), c.pool.cpu().numpy()), refs


def test_noalloc_step_matches_workspace_step_twice():
    # the second call is smaller: one request instead of two, 4 query heads per KV head
    # instead of 8, a 4K history instead of 2.5K-3K tokens over fewer pages
    for case in ("c5-gq8", "c2-4k"):
        (want, want_pool), (got, got_pool), refs = _run(case)
        assert np.array_equal(got_pool, want_pool), f"{case}: pool bytes differ"
        assert np.array_equal(got, want), f"{case}: outputs differ from oscar_decode_step"
        for b in range(len(refs)):
            assert_close(got[b], refs[b], f"{case} no-alloc step b{b}")


def test_noalloc_rejects_a_step_larger_than_the_static_array():
    import bit_kv_cache_oscar_amd as ok
    from bit_kv_cache_oscar_amd import _lib as L

    desc = L.layer_desc(32, 8)
    cap = ok.oscar_decode_step_noalloc_max_bytes()
    assert cap == 16 << 20
    assert L.oscar_decode_workspace_bytes(desc, 64, 256) > cap
    st = L.lib().oscar_decode_step_noalloc(
        desc, None, None, 0, None, None, None, None, None, None, None, None, None, 1, None, None, None, None, 64,
        0.088, 256, None, None)
    assert st == L.OSCAR_ERR_WORKSPACE
    assert b"static scratch" in L.lib().oscar_last_error()
