"""The C ABI without a GPU: the library loads, exports every declared symbol, and rejects
bad arguments on the host before any HIP call."""

import ctypes
import os
import re

import pytest

from bit_kv_cache_oscar_amd import _lib as L

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "oscar_kv.h")
FAKE = 0x10000  # never dereferenced: every call below fails validation first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("liboscar_kv.so is not built (run __graft_entry__.build())")
    return L.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(oscar_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert set(L._SIGNATURES) == set(names)


def test_helpers(lib):
    d = L.layer_desc(32, 8)
    assert L.oscar_version() >= 100
    assert L.oscar_check_desc(d) == L.OSCAR_OK
    assert L.oscar_page_bytes(d) == 8 * 4608
    assert L.oscar_window_tokens(d) == 320
    assert L.oscar_window_splits(d) == 5
    n, heads = 2 * 32 * 7, 2 * 32
    a256 = lambda x: -(-x // 256) * 256
    acc_off = a256(8 * n)
    ql_off = a256(acc_off + n * 512)
    qs_off = a256(ql_off + heads * 512)
    assert L.oscar_partials_bytes(d, 2, 7) == qs_off + heads * 32
    s = L.oscar_default_splits(d, 1, 32448)
    assert 1 <= s <= 507
    assert L.oscar_default_splits(d, 1, 0) == 1
    assert L.oscar_status_string(L.OSCAR_ERR_WORKSPACE) == "workspace too small"


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 64, L.OSCAR_ERR_UNSUPPORTED),
    ("group_size", 96, L.OSCAR_ERR_UNSUPPORTED),
    ("group_size", 16, L.OSCAR_ERR_UNSUPPORTED),
    ("page_tokens", 16, L.OSCAR_ERR_UNSUPPORTED),
    ("sink_tokens", 4, L.OSCAR_ERR_UNSUPPORTED),
    ("recent_tokens", 128, L.OSCAR_ERR_UNSUPPORTED),
    ("n_q_heads", 30, L.OSCAR_ERR_INVALID_ARG),
    ("n_q_heads", 8 * 32, L.OSCAR_ERR_UNSUPPORTED),
    ("n_kv_heads", 0, L.OSCAR_ERR_INVALID_ARG),
])
def test_bad_descriptors(lib, field, value, status):
    d = L.layer_desc(32, 8)
    setattr(d, field, value)
    assert L.oscar_check_desc(d) == status
    assert L.oscar_page_bytes(d) == 0
    assert L.oscar_last_error()
    st = lib.oscar_decode_int2(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 4, FAKE, 1, 0.08, 4, FAKE, 1 << 30, None)
    assert st == status


@pytest.mark.parametrize("group", [64, 32])
def test_grouped_descriptors(lib, group):
    """Groups of 64 and 32 dims: valid descriptors with larger pages; the one-group entry
    points refuse them, the grouped ones and the group-independent passes accept them."""
    d = L.layer_desc(32, 8, group)
    one = L.layer_desc(32, 8)
    assert L.oscar_check_desc(d) == L.OSCAR_OK
    assert L.oscar_page_bytes(d) == 8 * (4096 + 512 * (128 // group))
    assert L.oscar_partials_bytes(d, 2, 7) == L.oscar_partials_bytes(one, 2, 7)
    assert L.oscar_window_splits(d) == 5
    big = 1 << 40
    r = ctypes.byref(d)
    assert lib.oscar_decode_int2(r, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 1, 0.08, 4, FAKE, big, None) == \
        L.OSCAR_ERR_UNSUPPORTED
    assert lib.oscar_demote(r, FAKE, FAKE, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == L.OSCAR_ERR_UNSUPPORTED
    g = lib.oscar_decode_int2_grouped
    assert g(r, None, FAKE, FAKE, FAKE, 4, FAKE, 1, 0.08, 4, FAKE, big, None) == L.OSCAR_ERR_INVALID_ARG
    assert g(r, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 1, 0.08, 4, FAKE, big, None) == L.OSCAR_ERR_INVALID_ARG
    assert g(r, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 1, 0.08, 0, FAKE, big, None) == L.OSCAR_ERR_INVALID_ARG
    assert g(r, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 1, -1.0, 4, FAKE, big, None) == L.OSCAR_ERR_INVALID_ARG
    need = L.oscar_partials_bytes(d, 1, 4)
    assert g(r, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 1, 0.08, 4, FAKE, need - 1, None) == L.OSCAR_ERR_WORKSPACE
    assert g(r, FAKE + 8, FAKE, FAKE, FAKE, 4, FAKE, 1, 0.08, 4, FAKE, big, None) == L.OSCAR_ERR_INVALID_ARG
    assert g(r, FAKE, FAKE + 2, FAKE, FAKE, 4, FAKE, 1, 0.08, 4, FAKE, big, None) == L.OSCAR_ERR_INVALID_ARG
    assert "aligned" in L.oscar_last_error()
    dm = lib.oscar_demote_grouped
    assert dm(r, FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == L.OSCAR_OK
    assert dm(r, FAKE, FAKE, -1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == L.OSCAR_ERR_INVALID_ARG
    assert dm(r, FAKE, None, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == L.OSCAR_ERR_INVALID_ARG
    st = lib.oscar_decode_step_grouped
    args = [FAKE, FAKE, 0, None, None, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE, FAKE, 1, 0.08,
            4, FAKE]
    # the grouped step runs the one-group step's two launches: the same workspace
    wneed = L.oscar_decode_workspace_bytes(d, 1, 4)
    assert wneed == L.oscar_decode_workspace_bytes(one, 1, 4)
    assert st(r, *args, wneed - 1, FAKE, None) == L.OSCAR_ERR_WORKSPACE
    assert st(r, FAKE, FAKE, 2, None, FAKE, FAKE, FAKE, *args[7:], wneed, FAKE, None) == L.OSCAR_ERR_INVALID_ARG
    assert st(r, *args[:7], None, *args[8:], wneed, FAKE, None) == L.OSCAR_ERR_INVALID_ARG
    assert lib.oscar_decode_step(r, *args, big, FAKE, None) == L.OSCAR_ERR_UNSUPPORTED
    bad = L.layer_desc(32, 8, 48)
    assert dm(ctypes.byref(bad), FAKE, FAKE, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == \
        L.OSCAR_ERR_UNSUPPORTED


def test_null_desc(lib):
    assert lib.oscar_check_desc(None) == L.OSCAR_ERR_INVALID_ARG
    assert lib.oscar_merge(None, FAKE, 1, FAKE, FAKE, FAKE, 1, None) == L.OSCAR_ERR_INVALID_ARG


def test_decode_int2_argument_checks(lib):
    d = ctypes.byref(L.layer_desc(32, 8))
    call = lib.oscar_decode_int2
    big = 1 << 40
    assert call(d, None, FAKE, FAKE, FAKE, 4, FAKE, 1, 0.08, 4, FAKE, big, None) == L.OSCAR_ERR_INVALID_ARG
    assert call(d, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 0, 0.08, 4, FAKE, big, None) == L.OSCAR_ERR_INVALID_ARG
    assert call(d, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 1, 0.08, 0, FAKE, big, None) == L.OSCAR_ERR_INVALID_ARG
    assert call(d, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 1, 0.08, 4, FAKE, big, None) == L.OSCAR_ERR_INVALID_ARG
    assert call(d, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 1, -1.0, 4, FAKE, big, None) == L.OSCAR_ERR_INVALID_ARG
    assert call(d, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 1, float("nan"), 4, FAKE, big, None) == L.OSCAR_ERR_INVALID_ARG
    need = L.oscar_partials_bytes(L.layer_desc(32, 8), 1, 4)
    assert call(d, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 1, 0.08, 4, FAKE, need - 1, None) == L.OSCAR_ERR_WORKSPACE
    assert "workspace" in L.oscar_last_error()
    # at most 8192 pages per split: the pass's int32 value sums are bounded for that many
    assert call(d, FAKE, FAKE, FAKE, FAKE, 8193, FAKE, 1, 0.08, 1, FAKE, big, None) == L.OSCAR_ERR_UNSUPPORTED
    assert "pages per split" in L.oscar_last_error()


def test_default_splits_respect_the_pages_per_split_bound():
    d = L.layer_desc(32, 8)
    for batch in (1, 4, 64):
        for tokens in (2 ** 20, 2 ** 26, 2 ** 31 - 1):
            s = L.oscar_default_splits(d, batch, tokens)
            pages = -(-tokens // 64)
            assert 1 <= s <= 65535 and -(-pages // s) <= 8192, (batch, tokens, s)


def test_one_launch_step_sizes():
    """The one-launch step's split count keeps its grid (window items, one appended-token
    item per (request, KV head), history splits) at 240 workgroups or fewer, and the launch
    count follows from the grid fitting 256 workgroups."""
    d = L.layer_desc(32, 8)  # 5 window splits of 64 tokens (64 sink + 256 recent)
    # window items (two splits each) and the appended-token item, per KV head
    fixed = (L.oscar_window_splits(d) + 1) // 2 + 1
    for hist in (32448, 99680):
        s = L.oscar_decode_step_append_splits(d, 1, hist)
        assert fixed * 8 + s * 8 <= 240 < fixed * 8 + (s + 1) * 8
        assert L.oscar_decode_step_append_launches(d, 1, s) == 1
    # 256 workgroups still run at once; one more does not
    s_max = (256 - fixed * 8) // 8
    assert L.oscar_decode_step_append_launches(d, 1, s_max) == 1
    assert L.oscar_decode_step_append_launches(d, 1, s_max + 1) == 2
    # batch 4 of a 64-query-head layer: too many window items for one launch
    d5 = L.layer_desc(64, 8)
    s5 = L.oscar_decode_step_append_splits(d5, 4, 130752)
    assert L.oscar_decode_step_append_launches(d5, 4, s5) == 2
    assert L.oscar_decode_step_append_launches(d, 0, 4) == 0
    assert L.oscar_decode_step_append_launches(d, 1, 0) == 0


def test_one_launch_multi_sizes():
    """The multi-query decode's split count keeps its one-launch grid (window items and
    history splits, T x query heads per KV head over one or two head groups) within 240
    workgroups, falls back to the two-launch default when that grid cannot hold half the
    chip's units of history splits, and answers 1 for invalid arguments."""
    d = L.layer_desc(32, 8)
    fixed = (L.oscar_window_splits(d) + 1) // 2 + 1
    for t, groups in ((1, 1), (2, 1), (4, 2)):
        s = L.oscar_decode_multi_splits(d, 1, t, 32448)
        assert s == L.oscar_decode_step_append_splits(d, 1, 32448) or t > 1
        assert fixed * 8 + s * 8 * groups <= 240 < fixed * 8 + (s + 1) * 8 * groups
    # batch 4 of a 64-query-head layer with two tokens: the two-launch default
    d5 = L.layer_desc(64, 8)
    assert L.oscar_decode_multi_splits(d5, 4, 2, 130752) == L.oscar_default_splits(d5, 4, 130752)
    assert L.oscar_decode_multi_splits(d, 0, 2, 4096) == 1
    assert L.oscar_decode_multi_splits(d, 1, 0, 4096) == 1


def test_decode_bf16_and_merge_argument_checks(lib):
    desc = L.layer_desc(32, 8)
    d = ctypes.byref(desc)
    need = L.oscar_partials_bytes(desc, 2, 5)
    assert lib.oscar_decode_bf16(d, FAKE, FAKE, FAKE, FAKE, 2, 0.08, FAKE, need - 4, None) == L.OSCAR_ERR_WORKSPACE
    assert lib.oscar_decode_bf16(d, FAKE, None, FAKE, FAKE, 2, 0.08, FAKE, need, None) == L.OSCAR_ERR_INVALID_ARG
    assert lib.oscar_decode_bf16(d, FAKE, FAKE, FAKE, FAKE, -3, 0.08, FAKE, need, None) == L.OSCAR_ERR_INVALID_ARG
    assert lib.oscar_merge(d, FAKE, 0, FAKE, FAKE, FAKE, 2, None) == L.OSCAR_ERR_INVALID_ARG
    assert lib.oscar_merge(d, FAKE, 3, FAKE, None, FAKE, 2, None) == L.OSCAR_ERR_INVALID_ARG
    assert lib.oscar_merge(d, FAKE, 3, FAKE, FAKE, FAKE, 0, None) == L.OSCAR_ERR_INVALID_ARG


def test_demote_argument_checks(lib):
    d = ctypes.byref(L.layer_desc(32, 8))
    f = lib.oscar_demote
    assert f(d, FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == L.OSCAR_OK  # no-op
    assert f(d, FAKE, FAKE, -1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == L.OSCAR_ERR_INVALID_ARG
    assert f(d, FAKE, FAKE, 4, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == L.OSCAR_ERR_INVALID_ARG
    assert f(d, FAKE, FAKE, 4, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None) == L.OSCAR_ERR_INVALID_ARG
    assert f(d, FAKE, FAKE, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == L.OSCAR_ERR_INVALID_ARG


def test_decode_workspace_size():
    d = L.layer_desc(32, 8)
    a256 = lambda x: -(-x // 256) * 256
    # INT2 partials, window partials, then one 256-byte line per (request, KV head) arrival counter
    want = a256(L.oscar_partials_bytes(d, 3, 7)) + a256(L.oscar_partials_bytes(d, 3, 5)) + 3 * 8 * 256
    assert L.oscar_decode_workspace_bytes(d, 3, 7) == want
    bad = L.layer_desc(32, 8)
    bad.head_dim = 64
    assert L.oscar_decode_workspace_bytes(bad, 3, 7) == 0


def test_decode_step_argument_checks(lib):
    desc = L.layer_desc(32, 8)
    d = ctypes.byref(desc)
    need = L.oscar_decode_workspace_bytes(desc, 2, 4)
    step = lib.oscar_decode_step
    args = [FAKE, FAKE, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE, FAKE, 2, 0.08, 4,
            FAKE, need, FAKE, None]

    def call(over):
        a = list(args)
        for k, v in over.items():
            a[k] = v
        return step(d, *a)

    # argument positions after desc: 0 k_src, 2 n, 9 rot_v, 12 max_pages, 17 batch, 18 sm_scale,
    # 19 n_splits, 21 workspace_bytes, 22 out
    assert call({21: need - 1}) == L.OSCAR_ERR_WORKSPACE
    assert call({2: -1}) == L.OSCAR_ERR_INVALID_ARG
    assert call({0: None}) == L.OSCAR_ERR_INVALID_ARG        # demotion source missing with n > 0
    assert call({17: 0}) == L.OSCAR_ERR_INVALID_ARG
    assert call({19: 0}) == L.OSCAR_ERR_INVALID_ARG
    assert call({12: 0}) == L.OSCAR_ERR_INVALID_ARG
    assert call({12: 4 * 8192 + 1}) == L.OSCAR_ERR_UNSUPPORTED   # more than 8192 pages per split
    assert call({18: float("nan")}) == L.OSCAR_ERR_INVALID_ARG
    assert call({22: None}) == L.OSCAR_ERR_INVALID_ARG
    assert call({9: None}) == L.OSCAR_ERR_INVALID_ARG
    # n == 0 needs no demotion arguments; the remaining checks still apply
    assert call({2: 0, 0: None, 1: None, 3: None, 4: None, 5: None, 6: None, 21: need - 1}) == L.OSCAR_ERR_WORKSPACE
    att = lib.oscar_attend
    assert att(d, FAKE, FAKE, FAKE, 4, FAKE, 2, 4, FAKE, need - 1, FAKE, None) == L.OSCAR_ERR_WORKSPACE
    assert att(d, FAKE, FAKE, FAKE, 0, FAKE, 2, 4, FAKE, need, FAKE, None) == L.OSCAR_ERR_INVALID_ARG
    assert att(d, FAKE, FAKE, None, 4, FAKE, 2, 4, FAKE, need, FAKE, None) == L.OSCAR_ERR_INVALID_ARG
    prep = lib.oscar_prepare
    assert prep(d, FAKE, FAKE, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 0.08, 4, FAKE,
                need - 1, None) == L.OSCAR_ERR_WORKSPACE
    assert prep(d, FAKE, FAKE, 1, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 0.08, 4, FAKE,
                need, None) == L.OSCAR_ERR_INVALID_ARG


def test_python_binding_validates_shapes_before_the_library():
    torch = pytest.importorskip("torch")
    d = L.layer_desc(32, 8)
    cpu = torch.zeros(4, 8, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        L.oscar_demote(d, cpu, cpu, cpu, cpu, cpu, cpu, cpu, cpu, cpu)


def test_decode_multi_argument_checks(lib):
    desc = L.layer_desc(32, 8)  # 4 query heads per KV head: up to 4 query tokens
    d = ctypes.byref(desc)
    f = lib.oscar_decode_multi
    need = L.oscar_decode_workspace_bytes(desc, 2 * 4, 4)
    #       q, n_tokens, rot_k, rot_v, pool, table, max_pages, hist_len, k_win, v_win, win_len, batch,
    #       sm_scale, n_splits, workspace, bytes, out, stream
    args = [FAKE, 4, FAKE, FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE, FAKE, 2, 0.08, 4, FAKE, need, FAKE, None]

    def call(over):
        a = list(args)
        for k, v in over.items():
            a[k] = v
        return f(d, *a)

    assert call({15: need - 1}) == L.OSCAR_ERR_WORKSPACE
    assert call({1: 3}) == L.OSCAR_ERR_UNSUPPORTED       # not a power of two
    assert call({1: 8}) == L.OSCAR_ERR_UNSUPPORTED       # 8 x 4 virtual heads > 16
    assert call({1: 0}) == L.OSCAR_ERR_INVALID_ARG
    assert call({0: None}) == L.OSCAR_ERR_INVALID_ARG
    assert call({10: None}) == L.OSCAR_ERR_INVALID_ARG
    assert call({6: 0}) == L.OSCAR_ERR_INVALID_ARG
    assert call({12: 0.0}) == L.OSCAR_ERR_INVALID_ARG
    # one token needs the one-token workspace
    assert call({1: 1, 15: L.oscar_decode_workspace_bytes(desc, 2, 4) - 1}) == L.OSCAR_ERR_WORKSPACE


def test_codebook_entry_points_check_the_codebook_first(lib):
    desc = L.layer_desc(32, 8)
    d = ctypes.byref(desc)
    need = L.oscar_decode_workspace_bytes(desc, 2, 4)
    dem = lib.oscar_demote_codebook
    #            k, v, n, page, slot, rot_k, rot_v, clip_k, clip_v, codebook, pool, stream
    assert dem(d, FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None) == L.OSCAR_ERR_INVALID_ARG
    assert dem(d, FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 2, FAKE, None) == L.OSCAR_ERR_INVALID_ARG
    assert dem(d, FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == L.OSCAR_OK  # no-op
    assert dem(d, FAKE, FAKE, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == L.OSCAR_ERR_INVALID_ARG
    step = lib.oscar_decode_step_codebook
    # the oscar_decode_step arguments with the codebook inserted before the pool (position 10)
    args = [FAKE, FAKE, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE, FAKE, 2,
            0.08, 4, FAKE, need, FAKE, None]

    def call(over):
        a = list(args)
        for k, v in over.items():
            a[k] = v
        return step(d, *a)

    assert call({10: None}) == L.OSCAR_ERR_INVALID_ARG
    assert call({10: FAKE + 1}) == L.OSCAR_ERR_INVALID_ARG
    assert call({22: need - 1}) == L.OSCAR_ERR_WORKSPACE
    assert call({13: 4 * 8192 + 1}) == L.OSCAR_ERR_UNSUPPORTED
    dec = lib.oscar_decode_codebook
    #          q, rot_k, rot_v, codebook, pool, table, max_pages, hist, k_win, v_win, win_len, batch, sm, S, ws, bytes
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE, FAKE, 2, 0.08, 4, FAKE, need, FAKE, None]
    assert dec(d, *(base[:3] + [None] + base[4:])) == L.OSCAR_ERR_INVALID_ARG
    assert dec(d, *(base[:15] + [need - 1] + base[16:])) == L.OSCAR_ERR_WORKSPACE
    att = lib.oscar_attend_codebook
    assert att(d, FAKE, None, FAKE, FAKE, 4, FAKE, 2, 4, FAKE, need, FAKE, None) == L.OSCAR_ERR_INVALID_ARG
    assert att(d, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 2, 4, FAKE, need - 1, FAKE, None) == L.OSCAR_ERR_WORKSPACE
    prep = lib.oscar_prepare_codebook
    assert prep(d, FAKE, FAKE, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 2, 0.08, 4,
                FAKE, need, None) == L.OSCAR_ERR_INVALID_ARG
    assert prep(d, FAKE, FAKE, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 0.08, 4,
                FAKE, need - 1, None) == L.OSCAR_ERR_WORKSPACE


def test_calib_argument_checks(lib):
    desc = L.layer_desc(32, 8)
    d = ctypes.byref(desc)
    f = lib.oscar_calib_covariances
    need = L.oscar_calib_workspace_bytes(desc, 512)
    assert need == 512 * 32 * 128 * 4 + 32 * 8 * 128 * 128 * 4
    #         q, k, v, T, sm_scale, workspace, bytes, sigma_k, sigma_v, stream
    args = [FAKE, FAKE, FAKE, 512, 0.088, FAKE, need, FAKE, FAKE, None]

    def call(over):
        a = list(args)
        for k, v in over.items():
            a[k] = v
        return f(d, *a)

    assert call({6: need - 1}) == L.OSCAR_ERR_WORKSPACE
    assert call({3: 0}) == L.OSCAR_ERR_INVALID_ARG
    assert call({3: 65537}) == L.OSCAR_ERR_UNSUPPORTED
    assert call({4: 0.0}) == L.OSCAR_ERR_INVALID_ARG
    assert call({0: None}) == L.OSCAR_ERR_INVALID_ARG
    assert call({8: None}) == L.OSCAR_ERR_INVALID_ARG
    assert call({1: FAKE + 8}) == L.OSCAR_ERR_INVALID_ARG   # misaligned
    assert L.oscar_calib_workspace_bytes(desc, -1) == 0


def test_dense_bf16_argument_checks(lib):
    desc = L.layer_desc(32, 8)
    d = ctypes.byref(desc)
    f = lib.oscar_decode_dense_bf16
    need = L.oscar_dense_workspace_bytes(desc, 2, 4096)
    assert need == L.oscar_partials_bytes(desc, 2, 64)
    assert L.oscar_dense_workspace_bytes(desc, 2, 4000) == 0   # not a multiple of 64
    #         q, k, v, len, capacity, batch, sm_scale, workspace, bytes, out, stream
    args = [FAKE, FAKE, FAKE, FAKE, 4096, 2, 0.088, FAKE, need, FAKE, None]

    def call(over):
        a = list(args)
        for k, v in over.items():
            a[k] = v
        return f(d, *a)

    assert call({8: need - 1}) == L.OSCAR_ERR_WORKSPACE
    assert call({4: 4000}) == L.OSCAR_ERR_INVALID_ARG
    assert call({4: 0}) == L.OSCAR_ERR_INVALID_ARG
    assert call({4: 64 * 65536}) == L.OSCAR_ERR_UNSUPPORTED
    assert call({5: 0}) == L.OSCAR_ERR_INVALID_ARG
    assert call({3: None}) == L.OSCAR_ERR_INVALID_ARG
    assert call({6: -1.0}) == L.OSCAR_ERR_INVALID_ARG
