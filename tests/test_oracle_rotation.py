"""Pins for the oracle's rotation R = U * Hadamard * bit-reversal (CPU only)."""

import numpy as np
import pytest

from oracle import rotation as rot


def test_hadamard_small_orders_by_hand():
    s = 1 / np.sqrt(2)
    assert np.array_equal(rot.sylvester_hadamard(2), np.array([[s, s], [s, -s]]))
    h4 = 0.5 * np.array([[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]])
    assert np.allclose(rot.sylvester_hadamard(4), h4, atol=0, rtol=1e-15)


def test_hadamard_128_orthonormal_and_closed_form():
    h = rot.sylvester_hadamard(128)
    assert np.abs(h @ h.T - np.eye(128)).max() <= 1e-12
    assert np.array_equal(h, h.T)
    # Sylvester's closed form: H[i, j] = (-1)^popcount(i & j) / sqrt(n)
    i, j = np.meshgrid(np.arange(128), np.arange(128), indexing="ij")
    sign = np.array([[(-1) ** bin(a & b).count("1") for b in range(128)] for a in range(128)])
    assert np.array_equal(h * np.sqrt(128), sign.astype(float))
    del i, j


def test_bit_reverse_by_hand():
    assert [rot.bit_reverse(i, 7) for i in (0, 1, 2, 3, 5, 64, 127)] == [0, 64, 32, 96, 80, 1, 127]


def test_bit_reversal_is_an_involution_and_a_permutation():
    p = rot.bit_reversal_matrix(128)
    assert np.array_equal(p @ p, np.eye(128))
    assert np.array_equal(p.sum(0), np.ones(128)) and np.array_equal(p.sum(1), np.ones(128))


def test_eigenbasis_diagonal_closed_form():
    # Sigma diagonal with distinct entries: U is the permutation that sorts them descending
    d = np.array([3.0, 9.0, 1.0, 7.0])
    w, u = rot.eigenbasis(np.diag(d))
    assert np.array_equal(w, np.array([9.0, 7.0, 3.0, 1.0]))
    expect = np.zeros((4, 4))
    for col, row in enumerate([1, 3, 0, 2]):
        expect[row, col] = 1.0
    assert np.array_equal(u, expect)


def test_eigenbasis_residual_order_and_sign():
    a = np.random.default_rng(7).standard_normal((512, 128))
    sigma = a.T @ a
    w, u = rot.eigenbasis(sigma)
    assert np.all(np.diff(w) <= 0)
    assert np.abs(sigma @ u - u * w).max() <= 1e-10 * np.abs(sigma).max()
    assert np.abs(u.T @ u - np.eye(128)).max() <= 1e-12
    for j in range(128):
        k = int(np.argmax(np.abs(u[:, j])))
        assert u[k, j] > 0


def test_rotation_orthogonal_and_preserves_dot_products():
    a = np.random.default_rng(1).standard_normal((512, 128))
    r = rot.rotation_from_covariance(rot.gram_covariance(a))
    assert np.abs(r.T @ r - np.eye(128)).max() <= 1e-10
    g = np.random.default_rng(2)
    for _ in range(20):
        q, k = g.standard_normal(128) * 10, g.standard_normal(128) * 10
        assert abs(q @ k - (q @ r) @ (k @ r)) <= 1e-10 * np.linalg.norm(q) * np.linalg.norm(k)


def test_rotation_of_sorted_diagonal_is_hadamard_times_bit_reversal():
    # U = I, so R = H P, and (H P)[i, j] = H[i, rev(j)] = (-1)^popcount(i & rev(j)) / sqrt(128)
    sigma = np.diag(np.arange(128, 0, -1).astype(float))
    r = rot.rotation_from_covariance(sigma)
    expect = np.array([[(-1) ** bin(i & rot.bit_reverse(j, 7)).count("1") for j in range(128)]
                       for i in range(128)]) / np.sqrt(128)
    assert np.abs(r - expect).max() <= 1e-15


def test_key_covariance_is_psd_with_trace_equal_to_energy():
    q = np.random.default_rng(3).standard_normal((64, 4, 128))
    s = rot.key_covariance(q)
    assert np.allclose(s, s.T, rtol=0, atol=1e-9)
    assert np.linalg.eigvalsh(s).min() > -1e-9
    assert abs(np.trace(s) - (q ** 2).sum()) <= 1e-9 * (q ** 2).sum()


def test_value_covariance_constant_keys_gives_running_means():
    # all keys equal: causal softmax is uniform over j <= i, so S V holds running means
    g = np.random.default_rng(4)
    t = 40
    q = g.standard_normal((t, 2, 128))
    k = np.tile(g.standard_normal(128), (t, 1))
    v = g.standard_normal((t, 128))
    means = np.cumsum(v, axis=0) / np.arange(1, t + 1)[:, None]
    expect = 2 * sum(np.outer(means[i], means[i]) for i in range(t))
    got = rot.value_covariance(q, k, v, 0.125)
    assert np.abs(got - expect).max() <= 1e-10 * np.abs(expect).max()


def test_round_bf16_hand_cases():
    one = 1.0
    # bf16 keeps 8 significant bits: spacing 2^-7 just above 1
    assert rot.round_bf16(np.array([one + 2 ** -8]))[0] == 1.0                  # tie -> even
    assert rot.round_bf16(np.array([one + 3 * 2 ** -8]))[0] == 1.0 + 2 ** -6    # tie -> even
    assert rot.round_bf16(np.array([one + 2 ** -8 + 2 ** -40]))[0] == 1.0 + 2 ** -7
    assert rot.round_bf16(np.array([-(one + 2 ** -8 + 2 ** -40)]))[0] == -(1.0 + 2 ** -7)
    assert rot.round_bf16(np.array([0.0]))[0] == 0.0


def test_round_bf16_matches_torch_on_float32_values():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(5).standard_normal(20000).astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(rot.round_bf16(x), ref)
