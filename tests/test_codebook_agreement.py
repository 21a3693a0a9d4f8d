"""The library's host codebook calibration (bit_kv_cache_oscar_amd/codebook.py) against
the oracle's Lloyd-Max fitter, and against the published 2-bit Lloyd-Max quantiser of the
unit Gaussian (J. Max, 1960: outputs +-0.4528, +-1.510)."""

import numpy as np
import pytest

import synth
from bit_kv_cache_oscar_amd import codebook as hcb
from gpu_harness import bits_to_f64, rotations
from oracle import codebook as ocb


@pytest.mark.parametrize("cfg", [2, 5])
def test_library_codebook_equals_oracle_codebook(cfg):
    w = synth.workload(cfg)
    (rk_bits, rv_bits), (rk, rv) = rotations(w)
    cal = [synth.calibration_set(w, kv) for kv in range(2)]
    clip = np.full(2, w.clip_ratio, np.float32)
    ks, vs = hcb.layer_codebooks(cal, rk_bits[:2], rv_bits[:2], clip, clip)
    for kv in range(2):
        _, k, v = cal[kv]
        assert list(ks[kv]) == list(ocb.fit(k, rk[kv], w.clip_ratio)), kv
        assert list(vs[kv]) == list(ocb.fit(v, rv[kv], w.clip_ratio)), kv
        assert np.all(np.diff(ks[kv]) > 0) and ks[kv][0] >= 0 and ks[kv][-1] <= 48


def test_library_lloyd_max_on_the_unit_gaussian():
    x = np.random.default_rng(1960).standard_normal(2_000_000)
    lv = hcb.lloyd_max(x, start=(-1.5, -0.5, 0.5, 1.5), max_iters=300)
    assert np.allclose(lv, [-1.510, -0.4528, 0.4528, 1.510], atol=6e-3)


def test_library_fit_on_uniform_values_is_the_uniform_optimum():
    # t uniform on [0, 3]: cells of width 3/4, centres 3/8 + 3k/4 = (6, 18, 30, 42) / 16
    t = (np.arange(600_000) + 0.5) * (3.0 / 600_000)
    assert list(hcb.to_sixteenths(hcb.lloyd_max(t, max_iters=500))) == [6, 18, 30, 42]
    assert list(hcb.to_sixteenths([0.0, 0.0, 0.0, 0.0])) == [0, 1, 2, 3]
    assert list(hcb.to_sixteenths([3.0, 3.0, 3.0, 3.0])) == [45, 46, 47, 48]
