"""Oracle: decode attention over the three-segment pool, and the online-softmax merge.

Source: the QbitAI article on OSCAR, serving-path section: the token pool is a BF16
sink of 64 tokens, an INT2 history and a BF16 recent window of 256 tokens; at decode
the INT2 segment (unpack, scale/zero-point dequant, float accumulation) and the BF16
sink/recent segment are processed separately and joined by an online-softmax merge.

What one decode step computes for query head h of a request (kv = h // Gq, contiguous
GQA groups; reading):
  q_rot = q R_K[kv]
  window token i:   score_i = sm_scale * q . k_i              (k_i, v_i raw bf16)
  history token j:  score_j = sm_scale * q_rot . khat_j       (khat_j = dequantised, rotated basis)
  p = softmax over all scores together
  out = sum_i p_i v_i + (sum_j p_j vhat_j) R_V[kv]^T
Because R is orthogonal, q_rot . khat_j equals q . (khat_j R^T): attending in the
rotated basis is attending to the un-rotated dequantised keys.

The merge: a segment's partial is (m, l, acc) = (max score, sum exp(s - m),
sum exp(s - m) v); partials combine as M = max m_i, l = sum exp(m_i - M) l_i,
acc = sum exp(m_i - M) acc_i, and the output is acc / l. A segment with no tokens has
m = -inf, l = 0, acc = 0 and contributes nothing.
"""

from __future__ import annotations

import numpy as np

from . import codebook as _codebook
from . import groups as _groups
from .quant import dequantize


def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, sm_scale: float) -> np.ndarray:
    """Plain single-softmax attention of one query over rows k, v (fp64)."""
    s = sm_scale * (k @ q)
    p = np.exp(s - s.max())
    return (p @ v) / p.sum()


def partial(scores: np.ndarray, values: np.ndarray):
    """(m, l, acc) of one segment."""
    d = values.shape[1]
    if scores.size == 0:
        return -np.inf, 0.0, np.zeros(d)
    m = float(scores.max())
    p = np.exp(scores - m)
    return m, float(p.sum()), p @ values


def merge(parts):
    """Online-softmax merge of (m, l, acc) partials."""
    live = [p for p in parts if p[1] > 0.0]
    d = parts[0][2].shape[0]
    if not live:
        return -np.inf, 0.0, np.zeros(d)
    big = max(p[0] for p in live)
    l = sum(np.exp(p[0] - big) * p[1] for p in live)
    acc = sum(np.exp(p[0] - big) * p[2] for p in live)
    return big, float(l), acc


def finalize(part) -> np.ndarray:
    m, l, acc = part
    return acc / l if l > 0.0 else np.zeros_like(acc)


def head_inputs(hist, codebook=None):
    """Dequantised (khat, vhat) of one head's history tuple
    (k_codes, k_s16, k_z16, v_codes, v_s16, v_z16); with codebook = (K levels, V levels)
    in sixteenths, through those levels instead of the uniform ones. Scales and zero points
    of shape [n, n_g] (n_g > 1) are per group of 128 / n_g rotated dims (groups.py)."""
    kc, ks, kz, vc, vs, vz = hist
    if np.ndim(ks) == 2:
        if codebook is not None:
            raise ValueError("codebooks are defined for one group per vector")
        g = 128 // np.shape(ks)[1]
        return _groups.dequantize_grouped(kc, ks, kz, g), _groups.dequantize_grouped(vc, vs, vz, g)
    if codebook is not None:
        return _codebook.dequantize(kc, ks, kz, codebook[0]), _codebook.dequantize(vc, vs, vz, codebook[1])
    return dequantize(kc, ks, kz), dequantize(vc, vs, vz)


def decode_head(q, rot_k, rot_v, win_k, win_v, hist, sm_scale: float, codebook=None) -> np.ndarray:
    """Output of one query head: one softmax over window and history tokens together."""
    q = np.asarray(q, np.float64)
    q_rot = q @ rot_k
    khat, vhat = head_inputs(hist, codebook)
    s = np.concatenate([sm_scale * (np.asarray(win_k, np.float64) @ q), sm_scale * (khat @ q_rot)])
    if s.size == 0:
        return np.zeros(q.shape[0])
    p = np.exp(s - s.max())
    nw = win_k.shape[0]
    out = p[:nw] @ np.asarray(win_v, np.float64) + (p[nw:] @ vhat) @ rot_v.T
    return out / p.sum()


def decode(q, rot_k, rot_v, win_k, win_v, hists, sm_scale: float, codebooks=None) -> np.ndarray:
    """Outputs [Hq, 128] of one request.
    q [Hq,128]; rot_k, rot_v [Hkv,128,128]; win_k, win_v [Hkv, n_w, 128];
    hists[kv] = history tuple of KV head kv; codebooks[kv] = (K levels, V levels) in
    sixteenths for the codebook variant (None: the uniform levels)."""
    hq, hkv = q.shape[0], rot_k.shape[0]
    gq = hq // hkv
    out = np.zeros((hq, q.shape[1]))
    for h in range(hq):
        kv = h // gq
        out[h] = decode_head(q[h], rot_k[kv], rot_v[kv], win_k[kv], win_v[kv], hists[kv], sm_scale,
                             None if codebooks is None else codebooks[kv])
    return out


def decode_multi(q, rot_k, rot_v, win_k, win_v, hists, sm_scale: float, codebooks=None) -> np.ndarray:
    """Outputs [T, Hq, 128] of one request's T consecutive query tokens (q [T, Hq, 128]);
    codebooks as in decode() (None: the uniform levels).

    Reading (the pages name prefix-cache reuse; several query tokens over one compressed
    prefix, as in speculative verification or chunked prefill, is this library's reading):
    the T query tokens are the last T window tokens, so token t sits at window position
    n_w - T + t and attends to the whole history and to window slots [0, n_w - (T - 1 - t)),
    causal among the query tokens. T = 1 is decode()."""
    q = np.asarray(q, np.float64)
    n_tok, n_w = q.shape[0], np.asarray(win_k).shape[1]
    outs = []
    for t in range(n_tok):
        keep = max(0, n_w - (n_tok - 1 - t))
        outs.append(decode(q[t], rot_k, rot_v, np.asarray(win_k)[:, :keep], np.asarray(win_v)[:, :keep], hists,
                           sm_scale, codebooks))
    return np.stack(outs)


def history_partials(q, rot_k, hist, sm_scale: float, bounds):
    """INT2-segment partials of one query head over history ranges [a, b) (rotated
    basis, natural-log units)."""
    q_rot = np.asarray(q, np.float64) @ rot_k
    khat, vhat = head_inputs(hist)
    s = sm_scale * (khat @ q_rot)
    return [partial(s[a:b], vhat[a:b]) for a, b in bounds]


def window_partials(q, win_k, win_v, sm_scale: float, bounds):
    """BF16-segment partials of one query head over window ranges [a, b)."""
    q = np.asarray(q, np.float64)
    s = sm_scale * (np.asarray(win_k, np.float64) @ q)
    return [partial(s[a:b], np.asarray(win_v, np.float64)[a:b]) for a, b in bounds]


def merge_segments(hist_parts, win_parts, rot_v) -> np.ndarray:
    """Merge INT2 partials (rotated basis) and BF16 partials, un-rotating the INT2 side."""
    m_h, l_h, acc_h = merge(hist_parts)
    unrot = (m_h, l_h, acc_h @ rot_v.T)
    return finalize(merge([unrot, merge(win_parts)]))
