"""Oracle: quantisation groups smaller than the head dimension (G = 32 or 64) and the page
layout that carries their scales and zero points.

Test infrastructure only: nothing outside tests/, the smoke check and the CPU baseline of
the benchmark may import this package.

Source: the QbitAI article on OSCAR, section on aiming the rotation at attention: the
bit-reversal in R = U * Hadamard * bit-reversal makes the INT2 groups more balanced, which
only matters when a group is shorter than the head dimension; the scale and zero point are
per group. Readings:

  * group g of a rotated vector y = x R is dims [g G, (g + 1) G) of y (contiguous in the
    rotated basis, that is after R's bit-reversal);
  * each group is quantised as quant.quantize_rows quantises a whole vector (clip of its own
    extremes, fp16 scale and zero point, round half to even, clamp to [0, 3]);
  * page layout per head block: the K and V codes exactly as for one group (bytes 0..4095),
    then the K (s16, z16) of slot t and group g at 4096 + 4 (n_g t + g), then the V pairs the
    same way after them: 4096 + 512 n_g bytes per head block (n_g = 128 / G).
"""

from __future__ import annotations

import numpy as np

from . import pages, quant

HEAD_DIM = 128


def n_groups(group: int) -> int:
    if group not in (32, 64, 128):
        raise ValueError("group size must be 32, 64 or 128")
    return HEAD_DIM // group


def quantize_rows_grouped(x, r, clip: float, group: int):
    """Demote rows x [N, 128] with rotation r and clip ratio `clip`, one scale and zero
    point per group of `group` rotated dims. Returns (codes uint8 [N, 128], s16 float16
    [N, n_g], z16 float16 [N, n_g], margin [N, 128]).

    Group g is quantised by quant.quantize_rows with the rotation's columns of group g
    repeated to fill 128 columns: its extremes are then those of the group alone, and each
    repeated column gets the same code, so the first G columns are the group's codes."""
    ng = n_groups(group)
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    n = x.shape[0]
    codes = np.zeros((n, HEAD_DIM), np.uint8)
    margin = np.zeros((n, HEAD_DIM))
    s16 = np.zeros((n, ng), np.float16)
    z16 = np.zeros((n, ng), np.float16)
    for g in range(ng):
        cols = np.arange(g * group, (g + 1) * group)
        rg = r[:, np.tile(cols, ng)]
        c, s, z, m = quant.quantize_rows(x, rg, clip)
        codes[:, cols] = c[:, :group]
        margin[:, cols] = m[:, :group]
        s16[:, g], z16[:, g] = s, z
    return codes, s16, z16, margin


def dequantize_grouped(codes, s16, z16, group: int) -> np.ndarray:
    """code * s16 + z16 with each dim's own group's scale and zero point (fp64, rotated basis)."""
    s = np.repeat(np.asarray(s16, np.float64), group, axis=-1)
    z = np.repeat(np.asarray(z16, np.float64), group, axis=-1)
    return np.asarray(codes, np.float64) * s + z


def head_block_bytes(group: int) -> int:
    return 4096 + 512 * n_groups(group)


def history_bytes_per_token_head(group: int) -> int:
    """K and V codes (32 B each) plus an fp16 (s, z) pair per group for each."""
    return 2 * 32 + 2 * 4 * n_groups(group)


def pack_page_grouped(k_codes, k_s16, k_z16, v_codes, v_s16, v_z16, group: int) -> np.ndarray:
    """One head's block for a page of up to 64 tokens (missing slots zero): codes [n, 128],
    scales and zero points [n, n_g]."""
    ng = n_groups(group)
    n = len(k_s16)
    base = pages.pack_page(k_codes, np.zeros(n, np.float16), np.zeros(n, np.float16), v_codes,
                           np.zeros(n, np.float16), np.zeros(n, np.float16))
    blk = np.zeros(head_block_bytes(group), np.uint8)
    blk[:4096] = base[:4096]
    meta = np.zeros((2, pages.PAGE_TOKENS, ng, 2), np.float16)
    meta[0, :n, :, 0], meta[0, :n, :, 1] = k_s16, k_z16
    meta[1, :n, :, 0], meta[1, :n, :, 1] = v_s16, v_z16
    blk[4096:4096 + 256 * ng] = meta[0].reshape(-1).view(np.uint8)
    blk[4096 + 256 * ng:] = meta[1].reshape(-1).view(np.uint8)
    return blk


def unpack_page_grouped(blk, group: int):
    """(k_codes [64, 128], k_s16 [64, n_g], k_z16, v_codes, v_s16, v_z16) of one block."""
    ng = n_groups(group)
    blk = np.asarray(blk, np.uint8)
    base = np.zeros(pages.HEAD_BLOCK, np.uint8)
    base[:4096] = blk[:4096]
    kc, _, _, vc, _, _ = pages.unpack_page(base)
    km = blk[4096:4096 + 256 * ng].view(np.float16).reshape(pages.PAGE_TOKENS, ng, 2)
    vm = blk[4096 + 256 * ng:].view(np.float16).reshape(pages.PAGE_TOKENS, ng, 2)
    return kc, km[..., 0].copy(), km[..., 1].copy(), vc, vm[..., 0].copy(), vm[..., 1].copy()
