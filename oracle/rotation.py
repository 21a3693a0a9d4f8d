"""Oracle: the fixed per-layer, per-KV-head rotation R = U * Hadamard * bit-reversal.

Source: the QbitAI article on OSCAR, section "OSCAR把旋转对准attention" (OSCAR aims the
rotation at attention): keys are rotated along the eigenvectors of the query covariance
Q^T Q, values along those of the score-weighted value covariance V^T S^T S V, both
estimated offline per layer and head; the final rotation is U * Hadamard * bit-reversal,
where U aligns attention-relevant directions, the Hadamard transform spreads outlier
energy and the bit-reversal balances the INT2 groups.

Readings taken where the text is silent:
  * vectors are rows and are rotated as y = x R (so U acts first); un-rotation is y R^T;
  * U's columns are Sigma's eigenvectors in descending eigenvalue order, each column's
    sign chosen so that its largest-magnitude entry is positive (first such entry on ties);
  * Hadamard is Sylvester's construction scaled by 1/sqrt(n); bit-reversal is the
    permutation matrix P[i, rev(i)] = 1 over log2(n) bits;
  * the rotation the kernels use is R rounded to bf16 (round to nearest, ties to even,
    in one step from fp64); both sides use those exact values everywhere.
"""

from __future__ import annotations

import numpy as np


def sylvester_hadamard(n: int) -> np.ndarray:
    """Orthonormal Hadamard matrix of order n (a power of two): H_1 = [1],
    H_2m = [[H_m, H_m], [H_m, -H_m]], then scaled by 1/sqrt(n)."""
    assert n >= 1 and n & (n - 1) == 0
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h / np.sqrt(n)


def bit_reverse(i: int, bits: int) -> int:
    r = 0
    for _ in range(bits):
        r = (r << 1) | (i & 1)
        i >>= 1
    return r


def bit_reversal_matrix(n: int) -> np.ndarray:
    """Permutation matrix with P[i, rev(i)] = 1, rev reversing the log2(n)-bit index."""
    bits = n.bit_length() - 1
    p = np.zeros((n, n))
    for i in range(n):
        p[i, bit_reverse(i, bits)] = 1.0
    return p


def eigenbasis(sigma: np.ndarray):
    """(eigenvalues descending, U) of a symmetric matrix, with the sign convention above."""
    w, u = np.linalg.eigh(sigma)
    order = np.argsort(-w, kind="stable")
    w, u = w[order], u[:, order].copy()
    for j in range(u.shape[1]):
        k = int(np.argmax(np.abs(u[:, j])))
        if u[k, j] < 0:
            u[:, j] = -u[:, j]
    return w, u


def rotation_from_covariance(sigma: np.ndarray) -> np.ndarray:
    """R = U H P in fp64."""
    n = sigma.shape[0]
    _, u = eigenbasis(sigma)
    return u @ sylvester_hadamard(n) @ bit_reversal_matrix(n)


def gram_covariance(a: np.ndarray) -> np.ndarray:
    """Sigma = A^T A."""
    return a.T @ a


def key_covariance(q_cal: np.ndarray) -> np.ndarray:
    """Query covariance for the keys of one KV head: sum over the group's query heads of
    Q_h^T Q_h; q_cal is [T, Gq, d]."""
    return sum(q_cal[:, h, :].T @ q_cal[:, h, :] for h in range(q_cal.shape[1]))


def causal_softmax_scores(q: np.ndarray, k: np.ndarray, sm_scale: float) -> np.ndarray:
    """S[i, j] = softmax_j(sm_scale * q_i . k_j) over j <= i."""
    t = q.shape[0]
    s = sm_scale * (q @ k.T)
    s[np.triu_indices(t, 1)] = -np.inf
    s = s - s.max(axis=1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=1, keepdims=True)


def value_covariance(q_cal: np.ndarray, k_cal: np.ndarray, v_cal: np.ndarray,
                     sm_scale: float) -> np.ndarray:
    """Score-weighted value covariance V^T S^T S V, summed over the group's query heads;
    S is each head's causal attention matrix on the calibration sequence."""
    total = np.zeros((v_cal.shape[1], v_cal.shape[1]))
    for h in range(q_cal.shape[1]):
        sv = causal_softmax_scores(q_cal[:, h, :], k_cal, sm_scale) @ v_cal
        total += sv.T @ sv
    return total


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp64 values rounded to the nearest bf16 value (8 significant bits, ties to even),
    in one rounding step. Values stay fp64. Normal-range inputs only."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                     # x = m * 2**e, 0.5 <= |m| < 1
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    return np.where(x == 0, 0.0, r)
