"""Oracle: the paged INT2 history layout (four 2-bit codes per byte).

Source: the QbitAI article on OSCAR, serving-path section: history is stored as INT2,
four 2-bit values packed into one byte, in a paged KV cache (the abstracts add that the
kernels keep paged KV-cache layouts and prefix caching). The byte layout inside a page
is not given anywhere; the one below is this library's, and the oracle packs into the
same layout so bytes compare directly.

A physical page holds 64 tokens of every KV head. Head h of page p starts at byte
(p * n_kv_heads + h) * 4608 and holds:
  [   0, 2048)  K codes. The 16 codes of slot t, dims 16w..16w+15, form one little-endian
                32-bit word; dim 16w + 4m + j sits in byte j of it at bits 2m..2m+1. The word
                of (slot t, w) is at byte 32 (16 (w // 2) + t // 4) + 8 (t % 4) + 4 (w % 2):
                the 32 bytes at 32 l hold, for l = 16 G + n, slots 4n..4n+3 and words 2G, 2G+1.
  [2048, 4096)  V codes. The 16 codes of dim d, slots 16u..16u+15, form one word; slot
                16u + 4m + j sits in byte j at bits 2m..2m+1. The word of (dim d, u) is at
                byte 2048 + 32 (16 u + d % 16) + 4 (d // 16).
  [4096, 4352)  K scale and zero point of slot t: fp16 s at 4096 + 4t, fp16 z at +2.
  [4352, 4608)  V scale and zero point of slot t, same form at 4352 + 4t.
History index j of a request lives in logical page j // 64, slot j % 64; the request's
block table maps logical pages to physical pages.
"""

from __future__ import annotations

import numpy as np

PAGE_TOKENS = 64
HEAD_DIM = 128
HEAD_BLOCK = 4608
K_CODES, V_CODES, K_META, V_META = 0, 2048, 4096, 4352


def k_word_offset(slot: int, w: int) -> int:
    """Byte offset of the word holding dims 16w..16w+15 of K slot `slot`."""
    return K_CODES + 32 * (16 * (w // 2) + slot // 4) + 8 * (slot % 4) + 4 * (w % 2)


def v_word_offset(dim: int, u: int) -> int:
    """Byte offset of the word holding slots 16u..16u+15 of V dim `dim`."""
    return V_CODES + 32 * (16 * u + dim % 16) + 4 * (dim // 16)


def k_code_position(slot: int, dim: int):
    """(byte offset within the head block, bit shift) of K code (slot, dim)."""
    w, r = divmod(dim, 16)
    m, j = divmod(r, 4)
    return k_word_offset(slot, w) + j, 2 * m


def v_code_position(slot: int, dim: int):
    """(byte offset within the head block, bit shift) of V code (slot, dim)."""
    u, r = divmod(slot, 16)
    m, j = divmod(r, 4)
    return v_word_offset(dim, u) + j, 2 * m


def _position_tables():
    kb = np.zeros((PAGE_TOKENS, HEAD_DIM), np.int64)
    ks = np.zeros_like(kb)
    vb = np.zeros_like(kb)
    vs = np.zeros_like(kb)
    for t in range(PAGE_TOKENS):
        for d in range(HEAD_DIM):
            kb[t, d], ks[t, d] = k_code_position(t, d)
            vb[t, d], vs[t, d] = v_code_position(t, d)
    return kb, ks, vb, vs


_KB, _KS, _VB, _VS = _position_tables()


def new_pool(n_pages: int, n_kv_heads: int) -> np.ndarray:
    return np.zeros((n_pages, n_kv_heads, HEAD_BLOCK), dtype=np.uint8)


def _put_code(block: np.ndarray, byte: np.ndarray, shift: np.ndarray, code: np.ndarray):
    # codes sharing a byte have different shifts: update one shift at a time
    for sh in np.unique(shift):
        sel = shift == sh
        cur = block[byte[sel]].astype(np.int64)
        cur &= ~(3 << int(sh))
        cur |= (code[sel].astype(np.int64) & 3) << int(sh)
        block[byte[sel]] = cur.astype(np.uint8)


def _put_meta(block: np.ndarray, offset: int, s16, z16):
    block[offset:offset + 2] = np.frombuffer(np.float16(s16).tobytes(), np.uint8)
    block[offset + 2:offset + 4] = np.frombuffer(np.float16(z16).tobytes(), np.uint8)


def write_token(pool: np.ndarray, page: int, slot: int, head: int,
                k_codes, k_s16, k_z16, v_codes, v_s16, v_z16):
    """Store one token's K and V codes and metadata for one head."""
    blk = pool[page, head]
    _put_code(blk, _KB[slot], _KS[slot], np.asarray(k_codes))
    _put_code(blk, _VB[slot], _VS[slot], np.asarray(v_codes))
    _put_meta(blk, K_META + 4 * slot, k_s16, k_z16)
    _put_meta(blk, V_META + 4 * slot, v_s16, v_z16)


def read_token(pool: np.ndarray, page: int, slot: int, head: int):
    """(k_codes[128], k_s16, k_z16, v_codes[128], v_s16, v_z16) of one token and head."""
    blk = pool[page, head].astype(np.int64)
    kc = (blk[_KB[slot]] >> _KS[slot]) & 3
    vc = (blk[_VB[slot]] >> _VS[slot]) & 3
    meta = pool[page, head]
    ks, kz = np.frombuffer(meta[K_META + 4 * slot:K_META + 4 * slot + 4].tobytes(), np.float16)
    vs, vz = np.frombuffer(meta[V_META + 4 * slot:V_META + 4 * slot + 4].tobytes(), np.float16)
    return kc.astype(np.uint8), ks, kz, vc.astype(np.uint8), vs, vz


def write_history(pool: np.ndarray, table_row: np.ndarray, head: int, start: int,
                  k_codes, k_s16, k_z16, v_codes, v_s16, v_z16):
    """Store history entries start, start+1, ... of one request and head."""
    for i in range(len(k_s16)):
        j = start + i
        write_token(pool, int(table_row[j // PAGE_TOKENS]), j % PAGE_TOKENS, head,
                    k_codes[i], k_s16[i], k_z16[i], v_codes[i], v_s16[i], v_z16[i])


def read_history(pool: np.ndarray, table_row: np.ndarray, head: int, n_hist: int):
    """All n_hist history entries of one request and head, in history order:
    (k_codes [n,128], k_s16 [n], k_z16 [n], v_codes [n,128], v_s16 [n], v_z16 [n])."""
    kc = np.zeros((n_hist, HEAD_DIM), np.uint8)
    vc = np.zeros((n_hist, HEAD_DIM), np.uint8)
    ks = np.zeros(n_hist, np.float16)
    kz = np.zeros_like(ks)
    vs = np.zeros_like(ks)
    vz = np.zeros_like(ks)
    for j in range(n_hist):
        kc[j], ks[j], kz[j], vc[j], vs[j], vz[j] = read_token(
            pool, int(table_row[j // PAGE_TOKENS]), j % PAGE_TOKENS, head)
    return kc, ks, kz, vc, vs, vz


def history_bytes_per_token_head() -> int:
    """Bytes one history token costs per KV head: K and V codes plus fp16 (s, z) each."""
    return 2 * (HEAD_DIM * 2 // 8) + 2 * 4


def bf16_bytes_per_token_head() -> int:
    return 2 * HEAD_DIM * 2


def pack_page(k_codes, k_s16, k_z16, v_codes, v_s16, v_z16) -> np.ndarray:
    """One head's 4608-byte block for a page of up to 64 tokens (missing slots zero).
    Codes [n,128] uint8, scales/zeros [n] float16."""
    n = len(k_s16)
    assert n <= PAGE_TOKENS
    blk = np.zeros(HEAD_BLOCK, dtype=np.uint8)
    kc = np.zeros((PAGE_TOKENS, HEAD_DIM), np.int64)
    vc = np.zeros((PAGE_TOKENS, HEAD_DIM), np.int64)
    kc[:n] = k_codes
    vc[:n] = v_codes
    for table_b, table_s, codes in ((_KB, _KS, kc), (_VB, _VS, vc)):
        for sh in (0, 2, 4, 6):
            sel = table_s == sh      # within one shift every byte appears once
            blk[table_b[sel]] |= (codes[sel] << sh).astype(np.uint8)
    meta = np.zeros((2, PAGE_TOKENS, 2), np.float16)
    meta[0, :n, 0], meta[0, :n, 1] = k_s16, k_z16
    meta[1, :n, 0], meta[1, :n, 1] = v_s16, v_z16
    blk[K_META:V_META] = meta[0].reshape(-1).view(np.uint8)
    blk[V_META:HEAD_BLOCK] = meta[1].reshape(-1).view(np.uint8)
    return blk


def unpack_page(blk: np.ndarray):
    """(k_codes [64,128], k_s16 [64], k_z16 [64], v_codes, v_s16, v_z16) of one block."""
    b = np.asarray(blk, dtype=np.uint8).astype(np.int64)
    kc = ((b[_KB] >> _KS) & 3).astype(np.uint8)
    vc = ((b[_VB] >> _VS) & 3).astype(np.uint8)
    km = np.asarray(blk[K_META:V_META], np.uint8).view(np.float16).reshape(PAGE_TOKENS, 2)
    vm = np.asarray(blk[V_META:HEAD_BLOCK], np.uint8).view(np.float16).reshape(PAGE_TOKENS, 2)
    return kc, km[:, 0].copy(), km[:, 1].copy(), vc, vm[:, 0].copy(), vm[:, 1].copy()


def pack_history(pool: np.ndarray, table_row: np.ndarray, head: int, hist):
    """Write a whole history (entries 0..n-1, page by page) of one request and head."""
    kc, ks, kz, vc, vs, vz = hist
    n = len(ks)
    for p in range(-(-n // PAGE_TOKENS)):
        a, z = p * PAGE_TOKENS, min(n, (p + 1) * PAGE_TOKENS)
        pool[int(table_row[p]), head] = pack_page(kc[a:z], ks[a:z], kz[a:z], vc[a:z], vs[a:z], vz[a:z])


def unpack_history(pool: np.ndarray, table_row: np.ndarray, head: int, n_hist: int):
    """Inverse of pack_history for the first n_hist entries."""
    parts = [unpack_page(pool[int(table_row[p]), head]) for p in range(-(-n_hist // PAGE_TOKENS))]
    if not parts:
        return read_history(pool, table_row, head, 0)
    return tuple(np.concatenate([pt[i] for pt in parts])[:n_hist] for i in range(6))
