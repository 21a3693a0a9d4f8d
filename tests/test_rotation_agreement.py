"""The library's host rotation builder and the oracle's must give the same bf16 R."""

import numpy as np
import pytest

import synth
from gpu_harness import bits_to_f64, rotations


@pytest.mark.parametrize("cfg", [1, 2, 5])
def test_library_rotation_equals_oracle_rotation(cfg):
    w = synth.workload(cfg)
    (rk_bits, rv_bits), (rk, rv) = rotations(w)
    assert rk_bits.shape == (w.n_kv_heads, 128, 128)
    assert np.array_equal(bits_to_f64(rk_bits), rk)
    assert np.array_equal(bits_to_f64(rv_bits), rv)
    # rounded R stays close to orthogonal (bf16 has 8 significant bits)
    for r in (rk[0], rv[0]):
        assert np.abs(r.T @ r - np.eye(128)).max() < 2e-2


def test_library_bf16_rounding_hand_cases():
    from bit_kv_cache_oscar_amd.rotation import bf16_bits_from_f64
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -40, -0.75, 2.0 ** -100])
    got = synth.bf16_value(bf16_bits_from_f64(x)).astype(np.float64)
    assert list(got) == [1.0, 1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -0.75, 2.0 ** -100]
