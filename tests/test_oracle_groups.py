"""Pins for the oracle's quantisation groups shorter than the head dimension (CPU only):
reduction to the one-group scheme at G = 128, textbook per-group min-max INT2 under R = I,
independence of the groups, the page layout's metadata positions and round trip, the
bits-per-element figures, and attention over a losslessly quantised grouped history."""

import numpy as np
import pytest

from oracle import attention, groups, pages, quant
from oracle import groups as ogroups

import synth
from oracle.rotation import round_bf16, rotation_from_covariance

EYE = np.eye(128)


def test_one_group_is_the_plain_scheme():
    g = np.random.default_rng(1)
    r = round_bf16(rotation_from_covariance(np.diag(g.uniform(0.3, 3.0, 128))))
    x = round_bf16(g.standard_normal((40, 128)) * g.uniform(0.2, 3.0, (40, 1)))
    c1, s1, z1, m1 = quant.quantize_rows(x, r, 0.9)
    c2, s2, z2, m2 = groups.quantize_rows_grouped(x, r, 0.9, 128)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2[:, 0]) and np.array_equal(z1, z2[:, 0])
    assert np.array_equal(m1, m2)


@pytest.mark.parametrize("group", [32, 64])
def test_per_group_textbook_min_max(group):
    # R = I, c = 1: group g takes values b_g + s_g * {0, 1, 2, 3} with both ends present, so its
    # scale is s_g, its zero point b_g and its codes the multipliers
    ng = 128 // group
    g = np.random.default_rng(group)
    mult = g.integers(0, 4, (3, 128))
    mult[:, ::group] = 0
    mult[:, 1::group] = 3
    base = np.array([-4.0, 0.5, 2.0, -1.0])[:ng]
    step = np.array([0.5, 2.0, 0.25, 1.0])[:ng]
    x = np.repeat(base, group)[None] + mult * np.repeat(step, group)[None]
    codes, s16, z16, _ = groups.quantize_rows_grouped(x, EYE, 1.0, group)
    assert np.array_equal(codes, mult)
    assert np.array_equal(s16.astype(np.float64), np.tile(step, (3, 1)))
    assert np.array_equal(z16.astype(np.float64), np.tile(base, (3, 1)))
    assert np.array_equal(groups.dequantize_grouped(codes, s16, z16, group), x)


def test_groups_are_independent():
    g = np.random.default_rng(7)
    r = round_bf16(rotation_from_covariance(np.diag(g.uniform(0.3, 3.0, 128))))
    x = round_bf16(g.standard_normal((6, 128)))
    a = groups.quantize_rows_grouped(x, r, 0.9, 64)
    # changing the input changes y everywhere; compare against rows whose rotated values only
    # differ in group 1: under R = I change dims 64.. only
    y = round_bf16(g.standard_normal((6, 128)))
    y2 = y.copy()
    y2[:, 64:] = round_bf16(y2[:, 64:] * 3.0 + 1.0)
    b1 = groups.quantize_rows_grouped(y, EYE, 0.9, 64)
    b2 = groups.quantize_rows_grouped(y2, EYE, 0.9, 64)
    assert np.array_equal(b1[0][:, :64], b2[0][:, :64])
    assert np.array_equal(b1[1][:, 0], b2[1][:, 0]) and np.array_equal(b1[2][:, 0], b2[2][:, 0])
    assert not np.array_equal(b1[1][:, 1], b2[1][:, 1])
    assert a[1].shape == (6, 2)


@pytest.mark.parametrize("group", [32, 64, 128])
def test_page_layout_and_round_trip(group):
    ng = 128 // group
    g = np.random.default_rng(ng)
    n = 50
    kc = g.integers(0, 4, (n, 128)).astype(np.uint8)
    vc = g.integers(0, 4, (n, 128)).astype(np.uint8)
    ks = g.uniform(0.01, 2, (n, ng)).astype(np.float16)
    kz = g.uniform(-3, 0, (n, ng)).astype(np.float16)
    vs = g.uniform(0.01, 2, (n, ng)).astype(np.float16)
    vz = g.uniform(-3, 0, (n, ng)).astype(np.float16)
    blk = groups.pack_page_grouped(kc, ks, kz, vc, vs, vz, group)
    assert blk.size == groups.head_block_bytes(group) == 4096 + 512 * ng
    # hand-placed metadata: slot t, group j at 4096 + 4 (ng t + j); V after all K pairs
    t, j = 17, ng - 1
    at = 4096 + 4 * (ng * t + j)
    assert blk[at:at + 2].view(np.float16)[0] == ks[t, j] and blk[at + 2:at + 4].view(np.float16)[0] == kz[t, j]
    at = 4096 + 256 * ng + 4 * (ng * t + j)
    assert blk[at:at + 2].view(np.float16)[0] == vs[t, j]
    # codes sit where the one-group layout puts them
    assert np.array_equal(blk[:4096], pages.pack_page(kc, ks[:, 0], kz[:, 0], vc, vs[:, 0], vz[:, 0])[:4096])
    out = groups.unpack_page_grouped(blk, group)
    for got, want in zip(out, (kc, ks, kz, vc, vs, vz)):
        assert np.array_equal(got[:n], want)
        assert not np.any(got[n:].astype(np.float64))


def test_bits_per_element():
    # per token and KV head: 2 x 32 B of codes and an fp16 (s, z) pair per group for K and V,
    # over 2 x 128 elements: 2.25 bits at one group (the format the 2.28 / 2.38 BPE figures
    # fit), 2.5 at 64 and 3 at 32
    assert groups.history_bytes_per_token_head(128) == pages.history_bytes_per_token_head() == 72
    assert [groups.history_bytes_per_token_head(g) * 8 / 256 for g in (128, 64, 32)] == [2.25, 2.5, 3.0]


def test_attention_over_a_lossless_grouped_history():
    # histories whose groups hold exactly four levels dequantise exactly: the decode equals
    # plain softmax attention over the rotated-back rows
    g = np.random.default_rng(9)
    n = 12
    mult = g.integers(0, 4, (2, n, 128))
    mult[:, :, ::32] = 0
    mult[:, :, 1::32] = 3
    base = np.repeat(g.choice([-2.0, -1.0, 0.5], (2, n, 4)), 32, axis=-1)
    step = np.repeat(g.choice([0.25, 0.5, 1.0], (2, n, 4)), 32, axis=-1)
    y = base + mult * step  # rotated rows, R = I
    kc, ks, kz, _ = groups.quantize_rows_grouped(y[0], EYE, 1.0, 32)
    vc, vs, vz, _ = groups.quantize_rows_grouped(y[1], EYE, 1.0, 32)
    q = round_bf16(g.standard_normal(128))
    wk = round_bf16(g.standard_normal((3, 128)))
    wv = round_bf16(g.standard_normal((3, 128)))
    got = attention.decode_head(q, EYE, EYE, wk, wv, (kc, ks, kz, vc, vs, vz), 0.1)
    want = attention.softmax_attention(q, np.vstack([y[0], wk]), np.vstack([y[1], wv]), 0.1)
    assert np.allclose(got, want, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------------------
# What the bit reversal buys (QbitAI article on OSCAR, section on aiming the rotation at
# attention: the bit-reversal permutation makes the INT2 groups more even, so that no group
# is dominated by a few outlier channels; the accuracy section compares with a
# Hadamard-only rotation and with plain INT2). Measured on the oracle with the workloads'
# outlier rows, for R = U H P against U H (no bit reversal), H P (no eigenbasis) and I.

def _variants(w, kv):
    from oracle import rotation as orot

    q, k, v = synth.calibration_set(w, kv)
    h = orot.sylvester_hadamard(128)
    p = orot.bit_reversal_matrix(128)
    out = {}
    for name, sigma in (("K", orot.key_covariance(q)), ("V", orot.value_covariance(q, k, v, w.sm_scale))):
        _, u = orot.eigenbasis(sigma)
        out[name] = {"UHP": orot.round_bf16(u @ h @ p), "UH": orot.round_bf16(u @ h),
                     "HP": orot.round_bf16(h @ p), "I": np.eye(128)}
    return out


def _errors(x, r, clip, group, q=None):
    """(relative squared reconstruction error in the rotated basis, relative squared error of
    the attention logits q . k when q is given) of rows x under rotation r and group size."""
    from oracle import quant as oquant

    if group == 128:
        c, s, z, _ = oquant.quantize_rows(x, r, clip)
        yh = oquant.dequantize(c, s, z)
    else:
        c, s, z, _ = ogroups.quantize_rows_grouped(x, r, clip, group)
        yh = ogroups.dequantize_grouped(c, s, z, group)
    y = x @ r
    rec = float(np.sum((yh - y) ** 2) / np.sum(y ** 2))
    if q is None:
        return rec, None
    qr = q @ r
    ref = q @ x.T
    logit = float(np.sum((qr @ yh.T - ref) ** 2) / np.sum(ref ** 2))
    return rec, logit


@pytest.mark.parametrize("cfg,kv", [(2, 0), (5, 3)])
def test_bit_reversal_balances_the_groups(cfg, kv):
    """At one group per vector the bit reversal only reorders the group (U H P and U H give
    the same error); at groups of 64 and 32 rotated dims it lowers the reconstruction error
    and the key side's attention-logit error well below U H's; the eigenbasis matters too
    (U H P beats H P at every group size), and plain INT2 (R = I) is far worse."""
    w = synth.workload(cfg)
    rots = _variants(w, kv)
    hk, hv = synth.kv_rows(w, 0, kv, 64, 64 + 384)
    q = synth.query(w, 0).astype(np.float64)[kv * w.gq:(kv + 1) * w.gq]
    for name, x in (("K", hk.astype(np.float64)), ("V", hv.astype(np.float64))):
        for group in (128, 64, 32):
            err = {rn: _errors(x, r, w.clip_ratio, group, q if name == "K" else None)
                   for rn, r in rots[name].items()}
            rec = {k: v[0] for k, v in err.items()}
            what = f"cfg {cfg} kv {kv} {name} G {group}: {rec}"
            if group == 128:
                assert rec["UHP"] == pytest.approx(rec["UH"], rel=1e-9), what
            else:
                assert rec["UHP"] < (0.8 if group == 64 else 0.4) * rec["UH"], what
                if name == "K":
                    assert err["UHP"][1] < (0.8 if group == 64 else 0.4) * err["UH"][1], what
            assert rec["UHP"] < 0.95 * rec["HP"] and rec["UHP"] < 0.5 * rec["I"], what
