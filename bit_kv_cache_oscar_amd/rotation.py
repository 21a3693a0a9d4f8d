"""Host-side construction of OSCAR's per-head rotations (the offline step before the path).

OSCAR (QbitAI article, section on aiming the rotation at attention) estimates, offline
and per layer and head, the covariance that attention consumes: the query covariance
Q^T Q for keys and the score-weighted value covariance V^T S^T S V for values. The
rotation is R = U * Hadamard * bit-reversal with U the covariance's eigenvectors.

Here R is built in fp64 and rounded once to bf16, the form the kernels consume:
  * U: eigenvectors in descending eigenvalue order, each column signed so that its
    largest-magnitude entry is positive;
  * Hadamard: Sylvester order, orthonormal, applied to U's rows with a fast
    Walsh-Hadamard transform;
  * bit-reversal: column j of U H moves to column rev(j) (rev is an involution).
Rows are rotated as y = x R.
"""

from __future__ import annotations

import numpy as np

HEAD_DIM = 128


def fwht_rows(a: np.ndarray) -> np.ndarray:
    """Each row times the orthonormal Sylvester Hadamard matrix (butterflies, fp64)."""
    x = np.array(a, dtype=np.float64, copy=True)
    n = x.shape[-1]
    h = 1
    while h < n:
        x = x.reshape(*x.shape[:-1], n // (2 * h), 2, h)
        top = x[..., 0, :] + x[..., 1, :]
        bot = x[..., 0, :] - x[..., 1, :]
        x = np.stack([top, bot], axis=-2).reshape(*a.shape[:-1], n)
        h *= 2
    return x / np.sqrt(n)


def bit_reversed_indices(n: int) -> np.ndarray:
    bits = n.bit_length() - 1
    idx = np.arange(n)
    rev = np.zeros(n, dtype=np.int64)
    for b in range(bits):
        rev |= ((idx >> b) & 1) << (bits - 1 - b)
    return rev


def sorted_eigenvectors(sigma: np.ndarray) -> np.ndarray:
    w, u = np.linalg.eigh(np.asarray(sigma, dtype=np.float64))
    u = u[:, np.argsort(-w, kind="stable")]
    pivot = np.argmax(np.abs(u), axis=0)
    signs = np.where(u[pivot, np.arange(u.shape[1])] < 0, -1.0, 1.0)
    return u * signs


def rotation_fp64(sigma: np.ndarray) -> np.ndarray:
    """R = U H P for one covariance."""
    uh = fwht_rows(sorted_eigenvectors(sigma))
    rev = bit_reversed_indices(sigma.shape[0])
    r = np.empty_like(uh)
    r[:, rev] = uh
    return r


def bf16_bits_from_f64(x: np.ndarray) -> np.ndarray:
    """Nearest bf16 (ties to even) of fp64 values, rounded once; uint16 bits.
    Finite, normal-range inputs."""
    u = np.ascontiguousarray(x, dtype=np.float64).view(np.uint64)
    drop = np.uint64(45)                       # 52 - 7 fraction bits kept
    lsb = (u >> drop) & np.uint64(1)
    u = (u + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    f32 = u.view(np.float64).astype(np.float32)  # exact: 8 significant bits
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def query_covariance(q_cal: np.ndarray) -> np.ndarray:
    """Sum over the group's query heads of Q_h^T Q_h; q_cal [T, Gq, d]."""
    flat = np.asarray(q_cal, np.float64).reshape(-1, q_cal.shape[-1])
    return flat.T @ flat


def score_weighted_value_covariance(q_cal, k_cal, v_cal, sm_scale: float) -> np.ndarray:
    """Sum over the group's query heads of (S_h V)^T (S_h V), S_h the causal attention
    weights of head h on the calibration sequence."""
    t = k_cal.shape[0]
    mask = np.tril(np.ones((t, t), dtype=bool))
    out = np.zeros((v_cal.shape[1], v_cal.shape[1]))
    for h in range(q_cal.shape[1]):
        logits = np.where(mask, sm_scale * (q_cal[:, h, :] @ k_cal.T), -np.inf)
        logits -= logits.max(axis=1, keepdims=True)
        w = np.exp(logits)
        w /= w.sum(axis=1, keepdims=True)
        sv = w @ v_cal
        out += sv.T @ sv
    return out


def layer_rotations_from_calibration(calib, sm_scale: float):
    """(R_K bits, R_V bits) uint16 [Hkv, 128, 128] from per-KV-head calibration tuples
    (q [T, Gq, d], k [T, d], v [T, d])."""
    rk, rv = [], []
    for q, k, v in calib:
        rk.append(bf16_bits_from_f64(rotation_fp64(query_covariance(q))))
        rv.append(bf16_bits_from_f64(rotation_fp64(score_weighted_value_covariance(q, k, v, sm_scale))))
    return np.stack(rk), np.stack(rv)


def layer_rotations_from_gram(sources):
    """(R_K bits, R_V bits) with R_K = R_V from Sigma = A^T A per KV head."""
    r = np.stack([bf16_bits_from_f64(rotation_fp64(a.T @ a)) for a in sources])
    return r, r.copy()
