"""Seeded synthetic workloads for the OSCAR INT2 KV-cache decode and demotion path.

This module draws random numbers and lays out shapes; it holds none of the method's
arithmetic (no rotation, clipping, quantisation, packing or attention). It is the one
module that both sides use: the CPU oracle's tests and the GPU path's tests and
benchmark take their inputs from here, and each side then computes on its own.

Workloads follow the five layer shapes that the method is measured on (head_dim 128,
a BF16 sink of 64 tokens, an INT2 history, a BF16 recent window of 256 tokens, 64-token
pages). Values are N(0,1) with a few per-head outlier channels, rounded to bf16.

Token layout of one request with context length L (the decode step attends over all L):
  positions [0, 64)             sink, BF16 window slots [0, 64)
  positions [64, L-256)         history, INT2, history index j = position - 64
  positions [L-256, L)          recent, BF16 window slots [64, 320)
The last history token (position L-257) is the one the step demotes from the recent
window, so n_hist = L - 320 includes it.
"""

from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional, Tuple

import numpy as np

HEAD_DIM = 128
PAGE_TOKENS = 64
SINK_TOKENS = 64
RECENT_TOKENS = 256
WINDOW_TOKENS = SINK_TOKENS + RECENT_TOKENS
CALIB_TOKENS = 512
SHARED = 1 << 20  # request index used for the shared-prefix random stream

# random stream identifiers
_S_Q, _S_K, _S_V, _S_OUTLIER, _S_GRAM, _S_CALIB, _S_LEN, _S_PERM, _S_EXTRA = range(9)


def rng(seed: int, cfg: int, stream: int, *idx: int) -> np.random.Generator:
    """An independent PCG64 stream for (seed, config, stream, indices)."""
    return np.random.default_rng(np.random.SeedSequence([seed, cfg, stream, *idx]))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """float32 holding the bf16 value of `bits`."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    return bf16_value(bf16_bits(x))


@dataclass(frozen=True)
class Workload:
    cfg: int
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    ctx_lens: Tuple[int, ...]          # tokens the step attends over, per request
    capacity: int                      # largest context a request may reach (block-table width)
    shared_prefix: int = 0             # leading tokens common to every request
    permute_pages: bool = False        # physical pages in random order
    outlier_fixed: Optional[float] = 20.0   # outlier factor, or None for U[10, 30] per channel
    n_outliers: int = 4
    calib: str = "attention"           # "gram": Sigma = A^T A; "attention": Q/K/V calibration set
    clip_ratio: float = 0.9
    seed: int = 0

    @property
    def gq(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def sm_scale(self) -> float:
        return float(np.float32(1.0 / np.sqrt(HEAD_DIM)))

    def hist_len(self, b: int) -> int:
        return max(0, self.ctx_lens[b] - WINDOW_TOKENS)

    def win_len(self, b: int) -> int:
        return min(self.ctx_lens[b], WINDOW_TOKENS)

    @property
    def hist_lens(self) -> np.ndarray:
        return np.array([self.hist_len(b) for b in range(self.batch)], dtype=np.int32)

    @property
    def win_lens(self) -> np.ndarray:
        return np.array([self.win_len(b) for b in range(self.batch)], dtype=np.int32)

    @property
    def max_pages(self) -> int:
        return max(1, -(-max(0, self.capacity - WINDOW_TOKENS) // PAGE_TOKENS))

    @property
    def shared_pages(self) -> int:
        if self.batch < 2 or self.shared_prefix <= SINK_TOKENS:
            return 0
        return (self.shared_prefix - SINK_TOKENS) // PAGE_TOKENS

    def with_ctx(self, ctx_lens, capacity=None, shared_prefix=None) -> "Workload":
        ctx = tuple(int(c) for c in ctx_lens)
        cap = int(capacity) if capacity is not None else max(max(ctx), 1)
        sp = self.shared_prefix if shared_prefix is None else shared_prefix
        return replace(self, ctx_lens=ctx, batch=len(ctx), capacity=cap, shared_prefix=sp)


def workload(cfg: int, seed: int = 0) -> Workload:
    """The five layer shapes (1: tiny parity case; 2: 32K Qwen3-8B-like layer; 3: 100K
    context over randomly permuted pages; 4: batch 64 with a shared 4,096-token prefix;
    5: Qwen3-32B-like layer, batch 4 at 131,072 tokens)."""
    if cfg == 1:
        return Workload(1, "tiny-1kv-1q-1344ctx", 1, 1, 1, (SINK_TOKENS + 1024 + RECENT_TOKENS,),
                        SINK_TOKENS + 1024 + RECENT_TOKENS, outlier_fixed=20.0, calib="gram", seed=seed)
    if cfg == 2:
        return Workload(2, "qwen3-8b-layer-32k-b1", 1, 32, 8, (32768,), 32768,
                        outlier_fixed=None, seed=seed)
    if cfg == 3:
        return Workload(3, "qwen3-8b-layer-100k-b1-permuted", 1, 32, 8, (100000,), 100000,
                        permute_pages=True, outlier_fixed=20.0, seed=seed)
    if cfg == 4:
        g = rng(seed, 4, _S_LEN)
        lens = tuple(int(x) for x in g.integers(8192, 16384 + 1, size=64))
        return Workload(4, "qwen3-8b-layer-b64-8k16k-shared4k", 64, 32, 8, lens, 16384,
                        shared_prefix=4096, outlier_fixed=None, seed=seed)
    if cfg == 5:
        return Workload(5, "qwen3-32b-layer-128k-b4", 4, 64, 8, (131072,) * 4, 131072,
                        outlier_fixed=None, seed=seed)
    raise ValueError(f"unknown workload config {cfg}")


# ----------------------------------------------------------------------------------------
# outlier channels


def outliers(w: Workload, kv: int):
    """Per KV head: (kq_channels[4], k_factors[4], q_factors[Gq,4], v_channels[4], v_factors[4]).

    Keys and the query heads of that KV head's group share one channel set, so the large
    channels meet in q.k; values have an independent set."""
    g = rng(w.seed, w.cfg, _S_OUTLIER, kv)
    kq_ch = np.sort(g.choice(HEAD_DIM, w.n_outliers, replace=False))
    v_ch = np.sort(g.choice(HEAD_DIM, w.n_outliers, replace=False))

    def factors(shape):
        if w.outlier_fixed is not None:
            return np.full(shape, w.outlier_fixed, dtype=np.float32)
        return g.uniform(10.0, 30.0, size=shape).astype(np.float32)

    return kq_ch, factors(w.n_outliers), factors((w.gq, w.n_outliers)), v_ch, factors(w.n_outliers)


def _scaled(x: np.ndarray, ch: np.ndarray, f: np.ndarray) -> np.ndarray:
    x = x.copy()
    x[..., ch] *= f
    return x


def _normal(g: np.random.Generator, n: int) -> np.ndarray:
    return g.standard_normal((n, HEAD_DIM), dtype=np.float32)


# ----------------------------------------------------------------------------------------
# per-request data


ROW_CHUNK = 4096  # positions per independent random stream


def _rows(stream: int, w: Workload, who: int, kv: int, start: int, stop: int) -> np.ndarray:
    """N(0,1) float32 rows for absolute positions [start, stop) of stream `who`. Each block
    of ROW_CHUNK positions has its own generator, so any sub-range is cheap and identical
    however it is requested."""
    out = np.empty((stop - start, HEAD_DIM), np.float32)
    c = start // ROW_CHUNK
    while c * ROW_CHUNK < stop:
        lo, hi = c * ROW_CHUNK, (c + 1) * ROW_CHUNK
        blk = _normal(rng(w.seed, w.cfg, stream, who, kv, c), ROW_CHUNK)
        a, z = max(lo, start), min(hi, stop)
        out[a - start:z - start] = blk[a - lo:z - lo]
        c += 1
    return out


def kv_rows(w: Workload, b: int, kv: int, start: int = 0, stop: Optional[int] = None):
    """bf16-valued float32 K and V rows [stop-start, 128] for positions [start, stop) of
    request b, KV head kv. Positions below the shared prefix come from a stream common to
    all requests."""
    L = w.ctx_lens[b]
    stop = L if stop is None else stop
    assert 0 <= start <= stop <= L
    kq_ch, kf, _, v_ch, vf = outliers(w, kv)
    sp = w.shared_prefix if w.batch > 1 else 0
    parts_k, parts_v = [], []
    for lo, hi, who in ((0, sp, SHARED), (sp, L, b)):
        a, z = max(lo, start), min(hi, stop)
        if z <= a:
            continue
        parts_k.append(_scaled(_rows(_S_K, w, who, kv, a, z), kq_ch, kf))
        parts_v.append(_scaled(_rows(_S_V, w, who, kv, a, z), v_ch, vf))
    if not parts_k:
        e = np.zeros((0, HEAD_DIM), np.float32)
        return e, e.copy()
    return to_bf16_values(np.concatenate(parts_k)), to_bf16_values(np.concatenate(parts_v))


def query(w: Workload, b: int) -> np.ndarray:
    """bf16-valued float32 query [Hq, 128] of request b's decode step."""
    g = rng(w.seed, w.cfg, _S_Q, b)
    q = g.standard_normal((w.n_q_heads, HEAD_DIM), dtype=np.float32)
    for kv in range(w.n_kv_heads):
        kq_ch, _, qf, _, _ = outliers(w, kv)
        for i in range(w.gq):
            q[kv * w.gq + i, kq_ch] *= qf[i]
    return to_bf16_values(q)


def query_tokens(w: Workload, b: int, n_tok: int) -> np.ndarray:
    """bf16-valued float32 queries [n_tok, Hq, 128] of request b's last n_tok positions (a
    multi-query step); the last one is query(w, b), the others come from their own streams
    with the same per-head outlier channels."""
    out = np.empty((n_tok, w.n_q_heads, HEAD_DIM), np.float32)
    for t in range(n_tok):
        if t == n_tok - 1:
            out[t] = query(w, b)
            continue
        g = rng(w.seed, w.cfg, _S_Q, b, n_tok, t)
        q = g.standard_normal((w.n_q_heads, HEAD_DIM), dtype=np.float32)
        for kv in range(w.n_kv_heads):
            kq_ch, _, qf, _, _ = outliers(w, kv)
            for i in range(w.gq):
                q[kv * w.gq + i, kq_ch] *= qf[i]
        out[t] = to_bf16_values(q)
    return out


def window_rows(w: Workload, b: int, kv: int):
    """K and V [win_len, 128] of the BF16 window of request b: the sink then the recent
    tokens, in position order."""
    L = w.ctx_lens[b]
    k0, v0 = kv_rows(w, b, kv, 0, min(L, SINK_TOKENS))
    k1, v1 = kv_rows(w, b, kv, max(min(L, SINK_TOKENS), L - RECENT_TOKENS), L)
    return np.concatenate([k0, k1]), np.concatenate([v0, v1])


def history_rows(w: Workload, b: int, kv: int):
    """K and V [hist_len, 128] of request b's history (positions [64, L-256))."""
    n = w.hist_len(b)
    if n == 0:
        e = np.zeros((0, HEAD_DIM), np.float32)
        return e, e.copy()
    return kv_rows(w, b, kv, SINK_TOKENS, SINK_TOKENS + n)


# ----------------------------------------------------------------------------------------
# calibration inputs (the data a rotation is estimated from; the estimate itself is not here)


def gram_matrix_source(w: Workload, kv: int) -> np.ndarray:
    """A [512, 128] N(0,1), float64: the covariance source Sigma = A^T A of the tiny case."""
    return rng(w.seed, w.cfg, _S_GRAM, kv).standard_normal((CALIB_TOKENS, HEAD_DIM))


def calibration_set(w: Workload, kv: int):
    """A synthetic calibration sequence for one KV head: q [512, Gq, 128], k [512, 128],
    v [512, 128] (float64), with the same outlier model as the workload."""
    g = rng(w.seed, w.cfg, _S_CALIB, kv)
    kq_ch, kf, qf, v_ch, vf = outliers(w, kv)
    q = g.standard_normal((CALIB_TOKENS, w.gq, HEAD_DIM))
    for i in range(w.gq):
        q[:, i, kq_ch] *= qf[i]
    k = g.standard_normal((CALIB_TOKENS, HEAD_DIM))
    k[:, kq_ch] *= kf
    v = g.standard_normal((CALIB_TOKENS, HEAD_DIM))
    v[:, v_ch] *= vf
    return q, k, v


# ----------------------------------------------------------------------------------------
# paging


def block_table(w: Workload):
    """(table int32 [B, max_pages], n_physical_pages).

    Logical history page p of request b lives in physical page table[b, p]. Pages that
    hold the shared prefix are the same physical pages for every request. Unused entries
    are -1."""
    B, P = w.batch, w.max_pages
    table = np.full((B, P), -1, dtype=np.int64)
    nxt = 0
    shared = w.shared_pages
    shared_ids = np.arange(shared)
    nxt = shared
    for b in range(B):
        n = -(-w.hist_len(b) // PAGE_TOKENS)
        assert n <= P
        ns = min(shared, n)
        table[b, :ns] = shared_ids[:ns]
        table[b, ns:n] = np.arange(nxt, nxt + n - ns)
        nxt += n - ns
    n_phys = max(nxt, 1)
    if w.permute_pages:
        perm = rng(w.seed, w.cfg, _S_PERM).permutation(n_phys)
        m = table >= 0
        table[m] = perm[table[m]]
    return table.astype(np.int32), n_phys


def random_lengths(g: np.random.Generator, n: int, lo: int, hi: int) -> np.ndarray:
    return g.integers(lo, hi + 1, size=n)


def extra_rng(w: Workload, *idx: int) -> np.random.Generator:
    """A spare stream for test-specific draws (orders, sample indices)."""
    return rng(w.seed, w.cfg, _S_EXTRA, *idx)
