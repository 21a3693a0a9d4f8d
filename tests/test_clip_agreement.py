"""The library's host clip-ratio calibration (bit_kv_cache_oscar_amd/clip.py) against the
oracle's search on the workloads' synthetic calibration rows."""

import numpy as np
import pytest

import synth
from bit_kv_cache_oscar_amd import clip as hclip
from gpu_harness import rotations
from oracle import clip as oclip
from oracle.rotation import round_bf16


@pytest.mark.parametrize("cfg", [2, 5])
def test_library_clip_search_equals_oracle(cfg):
    w = synth.workload(cfg)
    (rk_bits, rv_bits), (rk, rv) = rotations(w)
    cal = [synth.calibration_set(w, kv) for kv in range(2)]
    cal = [(q, round_bf16(k[:128]), round_bf16(v[:128])) for q, k, v in cal]
    ck, cv = hclip.layer_clips(cal, rk_bits[:2], rv_bits[:2])
    for kv in range(2):
        bk, ek = oclip.search(cal[kv][1], rk[kv])
        bv, ev = oclip.search(cal[kv][2], rv[kv])
        assert float(ck[kv]) == pytest.approx(bk) and float(cv[kv]) == pytest.approx(bv), (kv, ck, cv, bk, bv)
        # the error curves agree too (they rank the candidates)
        assert np.allclose(hclip.errors(cal[kv][1], rk[kv]), ek, rtol=1e-9)
        assert 0.5 <= bk <= 1.0 and 0.5 <= bv <= 1.0


def test_library_clip_on_evenly_spaced_rows():
    g = np.random.default_rng(3)
    spaced = (2 * np.arange(128) + 1) / 128 - 1
    x = np.stack([g.permutation(spaced) for _ in range(16)])
    assert hclip.best_clip(x, np.eye(128)) in (0.75, 0.76)
