"""Pins for the oracle's paged INT2 layout and byte accounting (CPU only)."""

import json
import os

import numpy as np

from oracle import pages

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "format_figures.json")


def test_code_positions_by_hand():
    # K: slot 0, dim 5 -> word w 0 (pair 0, odd 0) at 0, r 5 -> m 1, j 1 -> byte 1, bits 2..3
    assert pages.k_code_position(0, 5) == (1, 2)
    # K: slot 2, dim 127 -> w 7: 32 (16*3 + 0) + 8*2 + 4*1 = 1556; r 15 -> m 3, j 3
    assert pages.k_code_position(2, 127) == (1556 + 3, 6)
    # K: slot 13, dim 20 -> w 1: 32 (0 + 3) + 8*1 + 4 = 108; r 4 -> m 1, j 0
    assert pages.k_code_position(13, 20) == (108, 2)
    # V: slot 17, dim 3 -> u 1: 2048 + 32 (16 + 3) + 0 = 2656; r 1 -> m 0, j 1
    assert pages.v_code_position(17, 3) == (2656 + 1, 0)
    # V: slot 63, dim 127 -> u 3: 2048 + 32 (48 + 15) + 4*7 = 4092; r 15 -> m 3, j 3
    assert pages.v_code_position(63, 127) == (4092 + 3, 6)


def test_every_code_has_its_own_two_bits():
    seen = set()
    for t in range(64):
        for d in range(128):
            for b, s in (pages.k_code_position(t, d), pages.v_code_position(t, d)):
                key = (b, s)
                assert key not in seen
                seen.add(key)
    assert len(seen) == 2 * 64 * 128
    assert max(b for b, _ in seen) < pages.K_META


def _random_token(g):
    return (g.integers(0, 4, 128).astype(np.uint8), np.float16(g.uniform(0.01, 4)),
            np.float16(g.uniform(-20, 0)), g.integers(0, 4, 128).astype(np.uint8),
            np.float16(g.uniform(0.01, 4)), np.float16(g.uniform(-20, 0)))


def test_write_read_round_trip_with_overwrites():
    g = np.random.default_rng(0)
    pool = pages.new_pool(3, 2)
    pool[:] = g.integers(0, 256, pool.shape, dtype=np.uint8)   # stale bytes must be cleared
    truth = {}
    for _ in range(500):
        p, s, h = int(g.integers(3)), int(g.integers(64)), int(g.integers(2))
        tok = _random_token(g)
        pages.write_token(pool, p, s, h, *tok)
        truth[(p, s, h)] = tok
    for (p, s, h), tok in truth.items():
        got = pages.read_token(pool, p, s, h)
        for a, b in zip(got, tok):
            assert np.array_equal(np.asarray(a), np.asarray(b))


def test_word_unpack_gives_four_consecutive_codes():
    # the property the decode kernels rely on: (word >> 2m) & 0x03030303 holds, byte by
    # byte, the codes of four consecutive dims (K) or slots (V)
    g = np.random.default_rng(1)
    pool = pages.new_pool(1, 1)
    kc = g.integers(0, 4, (64, 128)).astype(np.uint8)
    vc = g.integers(0, 4, (64, 128)).astype(np.uint8)
    for t in range(64):
        pages.write_token(pool, 0, t, 0, kc[t], 1.0, 0.0, vc[t], 1.0, 0.0)
    blk = pool[0, 0]
    for t in (0, 9, 63):
        for w in range(8):
            o = pages.k_word_offset(t, w)
            word = int(blk[o:o + 4].view("<u4")[0])
            for m in range(4):
                b = ((word >> (2 * m)) & 0x03030303).to_bytes(4, "little")
                assert list(b) == list(kc[t, 16 * w + 4 * m:16 * w + 4 * m + 4])
    for d in (0, 77, 127):
        for u in range(4):
            o = pages.v_word_offset(d, u)
            word = int(blk[o:o + 4].view("<u4")[0])
            for m in range(4):
                b = ((word >> (2 * m)) & 0x03030303).to_bytes(4, "little")
                assert list(b) == list(vc[16 * u + 4 * m:16 * u + 4 * m + 4, d])


def test_lane_chunks_are_contiguous():
    # the decode pass reads, for lane l = 16 G + n, one 32-byte chunk of K words (slots
    # 4n..4n+3, words 2G and 2G+1) and one of V words (dims 16 dt + n for dt 0..7, word G)
    for G in range(4):
        for n in range(16):
            l = 16 * G + n
            k = [pages.k_word_offset(4 * n + nt, 2 * G + h) for nt in range(4) for h in range(2)]
            assert k == list(range(32 * l, 32 * l + 32, 4))
            v = [pages.v_word_offset(16 * dt + n, G) for dt in range(8)]
            assert v == list(range(2048 + 32 * l, 2048 + 32 * l + 32, 4))


def test_history_bytes_and_ratio_to_bf16():
    figs = json.load(open(GOLDEN))
    # codes alone: 4 per byte -> exactly 8x smaller than bf16 (16 bits per value)
    code_bytes = 128 // figs["codes_per_byte"]["value"]
    assert 2 * code_bytes * 8 == pages.bf16_bytes_per_token_head()
    assert pages.bf16_bytes_per_token_head() / (2 * code_bytes) == figs["history_memory_ratio_vs_bf16"]["value"]
    # with one fp16 scale and zero point per 128-value group: 72 B vs 512 B
    assert pages.history_bytes_per_token_head() == 72
    assert abs(512 / 72 - 7.111) < 1e-3
    assert pages.HEAD_BLOCK == 64 * 72


def test_bits_per_element_at_32k_matches_the_reported_figure():
    figs = json.load(open(GOLDEN))
    ctx = figs["bpe_qwen3_8b_aime25_32k"]["context_tokens"]
    window = figs["sink_tokens"]["value"] + figs["recent_tokens"]["value"]
    hist = ctx - window
    bits = (hist * pages.history_bytes_per_token_head() + window * pages.bf16_bytes_per_token_head()) * 8
    bpe = bits / (ctx * 2 * 128)
    assert abs(bpe - figs["bpe_qwen3_8b_aime25_32k"]["value"]) < 0.005
    # history alone is 2.25 bits per element
    assert pages.history_bytes_per_token_head() * 8 / 256 == 2.25


def test_history_round_trip_through_block_table():
    g = np.random.default_rng(2)
    pool = pages.new_pool(6, 1)
    table = np.array([4, 0, 5, 2])
    n = 150
    toks = [_random_token(g) for _ in range(n)]
    cols = list(zip(*toks))
    pages.write_history(pool, table, 0, 0, np.stack(cols[0]), np.array(cols[1]), np.array(cols[2]),
                        np.stack(cols[3]), np.array(cols[4]), np.array(cols[5]))
    back = pages.read_history(pool, table, 0, n)
    assert np.array_equal(back[0], np.stack(cols[0]))
    assert np.array_equal(back[3], np.stack(cols[3]))
    assert np.array_equal(back[1], np.array(cols[1]))
    # entries 64..127 went to physical page 0, 128.. to page 5; pages 1, 3 untouched
    assert not pool[1].any() and not pool[3].any()


def test_whole_page_packer_matches_token_writer():
    g = np.random.default_rng(3)
    toks = [_random_token(g) for _ in range(64)]
    cols = list(zip(*toks))
    hist = (np.stack(cols[0]), np.array(cols[1]), np.array(cols[2]),
            np.stack(cols[3]), np.array(cols[4]), np.array(cols[5]))
    for n in (64, 37, 1):
        pool = pages.new_pool(1, 1)
        for t in range(n):
            pages.write_token(pool, 0, t, 0, *[x[t] for x in hist])
        blk = pages.pack_page(*[x[:n] for x in hist])
        assert np.array_equal(blk, pool[0, 0])
        back = pages.unpack_page(blk)
        for a, b in zip(back, hist):
            assert np.array_equal(np.asarray(a)[:n], np.asarray(b)[:n])


def test_history_pack_unpack_through_table():
    g = np.random.default_rng(4)
    n = 200
    toks = [_random_token(g) for _ in range(n)]
    cols = list(zip(*toks))
    hist = (np.stack(cols[0]), np.array(cols[1]), np.array(cols[2]),
            np.stack(cols[3]), np.array(cols[4]), np.array(cols[5]))
    table = np.array([3, 1, 6, 0])
    pool = pages.new_pool(7, 2)
    pages.pack_history(pool, table, 1, hist)
    slow = pages.read_history(pool, table, 1, n)
    fast = pages.unpack_history(pool, table, 1, n)
    for a, b, c in zip(slow, fast, hist):
        assert np.array_equal(a, b) and np.array_equal(a, c)
    assert not pool[:, 0].any()
