"""ctypes binding of liboscar_kv.so. Each function has the C entry point's name, checks
that the tensors match the descriptor (the C ABI cannot see tensor shapes), passes raw
device pointers and the current HIP stream, and raises OscarError on a non-zero status.
There is no fallback: if the library is missing, every call fails loudly."""

from __future__ import annotations

import ctypes
import functools
import os
from ctypes import POINTER, byref, c_float, c_int32, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liboscar_kv.so")

OSCAR_OK = 0
OSCAR_ERR_INVALID_ARG = 1
OSCAR_ERR_UNSUPPORTED = 2
OSCAR_ERR_WORKSPACE = 3
OSCAR_ERR_HIP = 4

HEAD_DIM = 128


class LayerDesc(ctypes.Structure):
    _fields_ = [
        ("head_dim", c_int32),
        ("group_size", c_int32),
        ("page_tokens", c_int32),
        ("n_q_heads", c_int32),
        ("n_kv_heads", c_int32),
        ("sink_tokens", c_int32),
        ("recent_tokens", c_int32),
    ]


def layer_desc(n_q_heads: int, n_kv_heads: int, group_size: int = 128) -> LayerDesc:
    return LayerDesc(128, group_size, 64, n_q_heads, n_kv_heads, 64, 256)


class OscarError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"liboscar_kv status {status}: {message}")
        self.status = status


_lib = None

_SIGNATURES = {
    "oscar_version": (c_int32, []),
    "oscar_status_string": (ctypes.c_char_p, [c_int32]),
    "oscar_last_error": (ctypes.c_char_p, []),
    "oscar_check_desc": (c_int32, [POINTER(LayerDesc)]),
    "oscar_page_bytes": (c_size_t, [POINTER(LayerDesc)]),
    "oscar_window_tokens": (c_int32, [POINTER(LayerDesc)]),
    "oscar_window_splits": (c_int32, [POINTER(LayerDesc)]),
    "oscar_partials_bytes": (c_size_t, [POINTER(LayerDesc), c_int32, c_int32]),
    "oscar_default_splits": (c_int32, [POINTER(LayerDesc), c_int32, c_int32]),
    "oscar_demote": (c_int32, [POINTER(LayerDesc), c_void_p, c_void_p, c_int32, c_void_p, c_void_p,
                               c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "oscar_demote_grouped": (c_int32, [POINTER(LayerDesc), c_void_p, c_void_p, c_int32, c_void_p, c_void_p,
                                       c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "oscar_decode_int2_grouped": (c_int32, [POINTER(LayerDesc), c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                                            c_void_p, c_int32, c_float, c_int32, c_void_p, c_size_t, c_void_p]),
    "oscar_decode_int2": (c_int32, [POINTER(LayerDesc), c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                                    c_void_p, c_int32, c_float, c_int32, c_void_p, c_size_t, c_void_p]),
    "oscar_decode_bf16": (c_int32, [POINTER(LayerDesc), c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                                    c_float, c_void_p, c_size_t, c_void_p]),
    "oscar_merge": (c_int32, [POINTER(LayerDesc), c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
                              c_int32, c_void_p]),
    "oscar_decode_workspace_bytes": (c_size_t, [POINTER(LayerDesc), c_int32, c_int32]),
    "oscar_decode_step": (c_int32, [POINTER(LayerDesc), c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
                                    c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_void_p,
                                    c_void_p, c_void_p, c_void_p, c_int32, c_float, c_int32, c_void_p, c_size_t,
                                    c_void_p, c_void_p]),
    "oscar_decode_step_append_workspace_bytes": (c_size_t, [POINTER(LayerDesc), c_int32, c_int32]),
    "oscar_decode_step_append_splits": (c_int32, [POINTER(LayerDesc), c_int32, c_int32]),
    "oscar_decode_step_append_launches": (c_int32, [POINTER(LayerDesc), c_int32, c_int32]),
    "oscar_decode_multi_splits": (c_int32, [POINTER(LayerDesc), c_int32, c_int32, c_int32]),
    "oscar_decode_step_append": (c_int32, [POINTER(LayerDesc), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                           c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p,
                                           c_void_p, c_void_p, c_int32, c_float, c_int32, c_void_p, c_size_t,
                                           c_void_p, c_void_p]),
    "oscar_decode_step_append_codebook": (c_int32, [POINTER(LayerDesc), c_void_p, c_void_p, c_void_p, c_void_p,
                                                    c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                                    c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_float,
                                                    c_int32, c_void_p, c_size_t, c_void_p, c_void_p]),
    "oscar_decode_step_noalloc_max_bytes": (c_size_t, []),
    "oscar_decode_step_noalloc": (c_int32, [POINTER(LayerDesc), c_void_p, c_void_p, c_int32, c_void_p, c_void_p,
                                            c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                            c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_float,
                                            c_int32, c_void_p, c_void_p]),
    "oscar_decode_step_grouped": (c_int32, [POINTER(LayerDesc), c_void_p, c_void_p, c_int32, c_void_p, c_void_p,
                                            c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                            c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_float, c_int32,
                                            c_void_p, c_size_t, c_void_p, c_void_p]),
    "oscar_decode": (c_int32, [POINTER(LayerDesc), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                               c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_float, c_int32, c_void_p, c_size_t,
                               c_void_p, c_void_p]),
    "oscar_decode_multi": (c_int32, [POINTER(LayerDesc), c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                     c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_float, c_int32,
                                     c_void_p, c_size_t, c_void_p, c_void_p]),
    "oscar_prepare": (c_int32, [POINTER(LayerDesc), c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
                                c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                c_int32, c_float, c_int32, c_void_p, c_size_t, c_void_p]),
    "oscar_attend": (c_int32, [POINTER(LayerDesc), c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_int32,
                               c_int32, c_void_p, c_size_t, c_void_p, c_void_p]),
    "oscar_dense_workspace_bytes": (c_size_t, [POINTER(LayerDesc), c_int32, c_int32]),
    "oscar_decode_dense_bf16": (c_int32, [POINTER(LayerDesc), c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                                          c_int32, c_float, c_void_p, c_size_t, c_void_p, c_void_p]),
    "oscar_calib_workspace_bytes": (c_size_t, [POINTER(LayerDesc), c_int32]),
    "oscar_calib_covariances": (c_int32, [POINTER(LayerDesc), c_void_p, c_void_p, c_void_p, c_int32, c_float,
                                          c_void_p, c_size_t, c_void_p, c_void_p, c_void_p]),
    "oscar_read_probe_words": (c_int32, []),
    "oscar_read_probe": (c_int32, [c_void_p, c_size_t, c_void_p, c_void_p]),
    # Lloyd-Max codebook variants: the entry point without the suffix with `codebook`
    # inserted before the pool
    "oscar_demote_codebook": (c_int32, [POINTER(LayerDesc), c_void_p, c_void_p, c_int32, c_void_p, c_void_p,
                                        c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "oscar_decode_step_codebook": (c_int32, [POINTER(LayerDesc), c_void_p, c_void_p, c_int32, c_void_p, c_void_p,
                                             c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                             c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                                             c_float, c_int32, c_void_p, c_size_t, c_void_p, c_void_p]),
    "oscar_decode_codebook": (c_int32, [POINTER(LayerDesc), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                        c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_float,
                                        c_int32, c_void_p, c_size_t, c_void_p, c_void_p]),
    "oscar_decode_multi_codebook": (c_int32, [POINTER(LayerDesc), c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
                                              c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                              c_int32, c_float, c_int32, c_void_p, c_size_t, c_void_p, c_void_p]),
    "oscar_prepare_codebook": (c_int32, [POINTER(LayerDesc), c_void_p, c_void_p, c_int32, c_void_p, c_void_p,
                                         c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                         c_void_p, c_void_p, c_void_p, c_int32, c_float, c_int32, c_void_p, c_size_t,
                                         c_void_p]),
    "oscar_attend_codebook": (c_int32, [POINTER(LayerDesc), c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                                        c_void_p, c_int32, c_int32, c_void_p, c_size_t, c_void_p, c_void_p]),
}


def lib():
    """The loaded library (loaded once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m bit_kv_cache_oscar_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status: int):
    if status != OSCAR_OK:
        raise OscarError(status, lib().oscar_last_error().decode())


def _run(prepare: bool, fn, *args):
    """fn(*args), its status checked. With `prepare`, that call is returned as a zero-argument
    callable instead: the arguments are validated and marshalled once, and each call of the
    callable is the C-ABI call alone (the tensors must stay alive and in place)."""
    if prepare:
        return functools.partial(_run, False, fn, *args)
    _check(fn(*args))


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return c_void_p(t)
    return c_void_p(t.data_ptr())


def _stream(stream):
    if isinstance(stream, int):
        return c_void_p(stream)
    import torch

    s = stream if stream is not None else torch.cuda.current_stream()
    return c_void_p(s.cuda_stream)


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _device16(t, name):
    import torch

    _need(t.is_cuda, f"{name} must be a device tensor")
    _need(t.dtype in (torch.bfloat16, torch.int16, torch.uint16, torch.float16), f"{name} must hold 16-bit values")
    _need(t.is_contiguous(), f"{name} must be contiguous")


def _device_i32(t, name, numel=None):
    import torch

    _need(t.is_cuda and t.dtype == torch.int32 and t.is_contiguous(), f"{name} must be a contiguous int32 device tensor")
    if numel is not None:
        _need(t.numel() >= numel, f"{name} holds {t.numel()} < {numel} entries")


def _check_codebook(desc: LayerDesc, codebook):
    """The Lloyd-Max variant's levels: uint8 [n_kv_heads, 2, 4] on the device (K, V)."""
    import torch

    _need(codebook.is_cuda and codebook.dtype == torch.uint8 and codebook.is_contiguous(),
          "codebook must be a contiguous uint8 device tensor")
    _need(codebook.numel() == desc.n_kv_heads * 8, "codebook must be [n_kv_heads, 2, 4]")


# ---------------------------------------------------------------------------------- helpers


def oscar_version() -> int:
    return lib().oscar_version()


def oscar_status_string(status: int) -> str:
    return lib().oscar_status_string(status).decode()


def oscar_last_error() -> str:
    return lib().oscar_last_error().decode()


def oscar_check_desc(desc: LayerDesc) -> int:
    return lib().oscar_check_desc(byref(desc))


def oscar_page_bytes(desc: LayerDesc) -> int:
    return lib().oscar_page_bytes(byref(desc))


def oscar_window_tokens(desc: LayerDesc) -> int:
    return lib().oscar_window_tokens(byref(desc))


def oscar_window_splits(desc: LayerDesc) -> int:
    return lib().oscar_window_splits(byref(desc))


def oscar_partials_bytes(desc: LayerDesc, batch: int, n_splits: int) -> int:
    return lib().oscar_partials_bytes(byref(desc), batch, n_splits)


def oscar_default_splits(desc: LayerDesc, batch: int, max_hist_len: int) -> int:
    return lib().oscar_default_splits(byref(desc), batch, max_hist_len)


def oscar_decode_workspace_bytes(desc: LayerDesc, batch: int, n_splits: int) -> int:
    return lib().oscar_decode_workspace_bytes(byref(desc), batch, n_splits)


# ------------------------------------------------------------------------------ entry points


def oscar_demote(desc: LayerDesc, k_src, v_src, dst_page, dst_slot, rot_k, rot_v, clip_k, clip_v, pool,
                 stream=None, codebook=None):
    """Demote n tokens (k_src/v_src [n, Hkv, 128] bf16) into (dst_page[i], dst_slot[i]).
    With `codebook` (uint8 [Hkv, 2, 4]) this is oscar_demote_codebook; with a desc of
    group_size 64 or 32, oscar_demote_grouped."""
    n = int(k_src.shape[0]) if k_src.dim() else 0
    hkv = desc.n_kv_heads
    _device16(k_src, "k_src")
    _device16(v_src, "v_src")
    _need(k_src.numel() == n * hkv * HEAD_DIM and v_src.numel() == n * hkv * HEAD_DIM,
          "k_src/v_src must be [n, n_kv_heads, 128]")
    _device_i32(dst_page, "dst_page", n)
    _device_i32(dst_slot, "dst_slot", n)
    for t, name in ((rot_k, "rot_k"), (rot_v, "rot_v")):
        _device16(t, name)
        _need(t.numel() == hkv * HEAD_DIM * HEAD_DIM, f"{name} must be [n_kv_heads, 128, 128]")
    for t, name in ((clip_k, "clip_k"), (clip_v, "clip_v")):
        _need(t.is_cuda and t.numel() == hkv and t.dtype.is_floating_point and t.element_size() == 4,
              f"{name} must be float32 [n_kv_heads] on the device")
    _need(pool.is_cuda and pool.is_contiguous(), "pool must be a contiguous device tensor")
    if desc.group_size != 128:
        _need(codebook is None, "codebooks are defined for one group per vector")
        _check(lib().oscar_demote_grouped(byref(desc), _ptr(k_src), _ptr(v_src), n, _ptr(dst_page), _ptr(dst_slot),
                                          _ptr(rot_k), _ptr(rot_v), _ptr(clip_k), _ptr(clip_v), _ptr(pool),
                                          _stream(stream)))
    elif codebook is None:
        _check(lib().oscar_demote(byref(desc), _ptr(k_src), _ptr(v_src), n, _ptr(dst_page), _ptr(dst_slot),
                                  _ptr(rot_k), _ptr(rot_v), _ptr(clip_k), _ptr(clip_v), _ptr(pool),
                                  _stream(stream)))
    else:
        _check_codebook(desc, codebook)
        _check(lib().oscar_demote_codebook(byref(desc), _ptr(k_src), _ptr(v_src), n, _ptr(dst_page),
                                           _ptr(dst_slot), _ptr(rot_k), _ptr(rot_v), _ptr(clip_k), _ptr(clip_v),
                                           _ptr(codebook), _ptr(pool), _stream(stream)))


def oscar_demote_codebook(desc: LayerDesc, k_src, v_src, dst_page, dst_slot, rot_k, rot_v, clip_k, clip_v, codebook,
                          pool, stream=None):
    """oscar_demote against the Lloyd-Max codebook (uint8 [Hkv, 2, 4], sixteenths of the scale)."""
    oscar_demote(desc, k_src, v_src, dst_page, dst_slot, rot_k, rot_v, clip_k, clip_v, pool, stream, codebook)


def oscar_decode_int2(desc: LayerDesc, q, rot_k, pool, block_table, hist_len, sm_scale: float, n_splits: int,
                      partials, stream=None, prepare=False):
    """INT2 history pass; q [B, Hq, 128] bf16, block_table [B, max_pages] int32,
    hist_len [B] int32; partials from oscar_partials_bytes(desc, B, n_splits). A desc with
    group_size 64 or 32 reads grouped pages (oscar_decode_int2_grouped)."""
    batch = int(q.shape[0])
    _device16(q, "q")
    _need(q.numel() == batch * desc.n_q_heads * HEAD_DIM, "q must be [batch, n_q_heads, 128]")
    _device16(rot_k, "rot_k")
    _need(rot_k.numel() == desc.n_kv_heads * HEAD_DIM * HEAD_DIM, "rot_k must be [n_kv_heads, 128, 128]")
    _need(block_table.dim() == 2 and block_table.shape[0] == batch, "block_table must be [batch, max_pages]")
    _device_i32(block_table, "block_table")
    _device_i32(hist_len, "hist_len", batch)
    _need(pool.is_cuda, "pool must be on the device")
    _need(partials.is_cuda and partials.is_contiguous(), "partials must be a contiguous device tensor")
    nbytes = partials.numel() * partials.element_size()
    fn = lib().oscar_decode_int2 if desc.group_size == 128 else lib().oscar_decode_int2_grouped
    return _run(prepare, fn, byref(desc), _ptr(q), _ptr(rot_k), _ptr(pool), _ptr(block_table),
                int(block_table.shape[1]), _ptr(hist_len), batch, float(sm_scale), int(n_splits), _ptr(partials),
                nbytes, _stream(stream))


def oscar_decode_bf16(desc: LayerDesc, q, k_win, v_win, win_len, sm_scale: float, win_partials, stream=None,
                      prepare=False):
    """BF16 window pass; k_win/v_win [B, Hkv, 320, 128] bf16, win_len [B] int32."""
    batch = int(q.shape[0])
    _device16(q, "q")
    _need(q.numel() == batch * desc.n_q_heads * HEAD_DIM, "q must be [batch, n_q_heads, 128]")
    w = desc.sink_tokens + desc.recent_tokens
    for t, name in ((k_win, "k_win"), (v_win, "v_win")):
        _device16(t, name)
        _need(t.numel() == batch * desc.n_kv_heads * w * HEAD_DIM, f"{name} must be [batch, n_kv_heads, {w}, 128]")
    _device_i32(win_len, "win_len", batch)
    _need(win_partials.is_cuda and win_partials.is_contiguous(), "win_partials must be a contiguous device tensor")
    nbytes = win_partials.numel() * win_partials.element_size()
    return _run(prepare, lib().oscar_decode_bf16, byref(desc), _ptr(q), _ptr(k_win), _ptr(v_win), _ptr(win_len),
                batch, float(sm_scale), _ptr(win_partials), nbytes, _stream(stream))


def oscar_dense_workspace_bytes(desc: LayerDesc, batch: int, capacity: int) -> int:
    return int(lib().oscar_dense_workspace_bytes(byref(desc), int(batch), int(capacity)))


def oscar_decode_dense_bf16(desc: LayerDesc, q, k, v, lens, sm_scale: float, workspace, out, stream=None):
    """Plain BF16 decode over a dense KV buffer (the uncompressed baseline): q [B, Hq, 128],
    k and v [B, Hkv, capacity, 128] bf16, lens int32 [B]; out [B, Hq, 128] float32."""
    import torch

    batch = int(q.shape[0])
    _device16(q, "q")
    _need(q.numel() == batch * desc.n_q_heads * HEAD_DIM, "q must be [batch, n_q_heads, 128]")
    _need(k.dim() == 4 and k.shape[0] == batch and k.shape[1] == desc.n_kv_heads and k.shape[3] == HEAD_DIM,
          "k must be [batch, n_kv_heads, capacity, 128]")
    cap = int(k.shape[2])
    for t, name in ((k, "k"), (v, "v")):
        _device16(t, name)
        _need(tuple(t.shape) == tuple(k.shape), f"{name} must be [batch, n_kv_heads, capacity, 128]")
    _device_i32(lens, "lens", batch)
    _need(workspace.is_cuda and workspace.is_contiguous(), "workspace must be a contiguous device tensor")
    _need(out.is_cuda and out.dtype == torch.float32 and out.is_contiguous()
          and out.numel() == batch * desc.n_q_heads * HEAD_DIM, "out must be float32 [batch, n_q_heads, 128]")
    _check(lib().oscar_decode_dense_bf16(byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(lens), cap, batch,
                                         float(sm_scale), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _ptr(out), _stream(stream)))


def oscar_calib_workspace_bytes(desc: LayerDesc, n_tokens: int) -> int:
    return int(lib().oscar_calib_workspace_bytes(byref(desc), int(n_tokens)))


def oscar_calib_covariances(desc: LayerDesc, q, k, v, sm_scale: float, workspace, sigma_k, sigma_v, stream=None):
    """Calibration covariances of one sequence: q [T, Hq, 128], k and v [T, Hkv, 128] bf16;
    sigma_k, sigma_v float32 [Hkv, 128, 128] outputs; workspace from
    oscar_calib_workspace_bytes(desc, T)."""
    import torch

    n_tok = int(q.shape[0])
    _device16(q, "q")
    _need(q.numel() == n_tok * desc.n_q_heads * HEAD_DIM, "q must be [T, n_q_heads, 128]")
    for t, name in ((k, "k"), (v, "v")):
        _device16(t, name)
        _need(t.numel() == n_tok * desc.n_kv_heads * HEAD_DIM, f"{name} must be [T, n_kv_heads, 128]")
    for t, name in ((sigma_k, "sigma_k"), (sigma_v, "sigma_v")):
        _need(t.is_cuda and t.dtype == torch.float32 and t.is_contiguous()
              and t.numel() == desc.n_kv_heads * HEAD_DIM * HEAD_DIM, f"{name} must be float32 [n_kv_heads, 128, 128]")
    _need(workspace.is_cuda and workspace.is_contiguous(), "workspace must be a contiguous device tensor")
    _check(lib().oscar_calib_covariances(byref(desc), _ptr(q), _ptr(k), _ptr(v), n_tok, float(sm_scale),
                                         _ptr(workspace), workspace.numel() * workspace.element_size(),
                                         _ptr(sigma_k), _ptr(sigma_v), _stream(stream)))


def oscar_read_probe(buf, out, stream=None):
    """Streaming read of the whole device tensor buf (a measurement helper); out: int32 device
    tensor of at least oscar_read_probe_words() entries."""
    import torch

    nbytes = buf.numel() * buf.element_size()
    _need(buf.is_cuda and buf.is_contiguous(), "buf must be a contiguous device tensor")
    _need(out.is_cuda and out.dtype == torch.int32 and out.numel() >= lib().oscar_read_probe_words(),
          "out must be an int32 device tensor of oscar_read_probe_words() entries")
    _check(lib().oscar_read_probe(_ptr(buf), nbytes, _ptr(out), _stream(stream)))


def oscar_merge(desc: LayerDesc, partials, n_splits: int, win_partials, rot_v, out, stream=None, prepare=False):
    """Join both segments into out [B, Hq, 128] float32."""
    import torch

    batch = int(out.shape[0])
    _need(out.is_cuda and out.dtype == torch.float32 and out.is_contiguous(), "out must be contiguous float32")
    _need(out.numel() == batch * desc.n_q_heads * HEAD_DIM, "out must be [batch, n_q_heads, 128]")
    _device16(rot_v, "rot_v")
    _need(rot_v.numel() == desc.n_kv_heads * HEAD_DIM * HEAD_DIM, "rot_v must be [n_kv_heads, 128, 128]")
    need = oscar_partials_bytes(desc, batch, n_splits)
    _need(partials.numel() * partials.element_size() >= need, "partials smaller than oscar_partials_bytes")
    wneed = oscar_partials_bytes(desc, batch, oscar_window_splits(desc))
    _need(win_partials.numel() * win_partials.element_size() >= wneed, "win_partials too small")
    return _run(prepare, lib().oscar_merge, byref(desc), _ptr(partials), int(n_splits), _ptr(win_partials),
                _ptr(rot_v), _ptr(out), batch, _stream(stream))


def _check_decode_args(desc: LayerDesc, q, rot_k, rot_v, pool, block_table, hist_len, k_win, v_win, win_len,
                       n_splits: int, workspace, out, n_tok: int = 1):
    import torch

    batch = int(q.shape[0])
    _device16(q, "q")
    shape = "[batch, n_q_heads, 128]" if n_tok == 1 else "[batch, T, n_q_heads, 128]"
    _need(q.numel() == batch * n_tok * desc.n_q_heads * HEAD_DIM, f"q must be {shape}")
    for t, name in ((rot_k, "rot_k"), (rot_v, "rot_v")):
        _device16(t, name)
        _need(t.numel() == desc.n_kv_heads * HEAD_DIM * HEAD_DIM, f"{name} must be [n_kv_heads, 128, 128]")
    _need(pool.is_cuda and pool.is_contiguous(), "pool must be a contiguous device tensor")
    _need(block_table.dim() == 2 and block_table.shape[0] == batch, "block_table must be [batch, max_pages]")
    _device_i32(block_table, "block_table")
    _device_i32(hist_len, "hist_len", batch)
    w = desc.sink_tokens + desc.recent_tokens
    for t, name in ((k_win, "k_win"), (v_win, "v_win")):
        _device16(t, name)
        _need(t.numel() == batch * desc.n_kv_heads * w * HEAD_DIM, f"{name} must be [batch, n_kv_heads, {w}, 128]")
    _device_i32(win_len, "win_len", batch)
    _need(workspace.is_cuda and workspace.is_contiguous(), "workspace must be a contiguous device tensor")
    _need(out.is_cuda and out.dtype == torch.float32 and out.is_contiguous(), "out must be contiguous float32")
    _need(out.numel() == batch * n_tok * desc.n_q_heads * HEAD_DIM, f"out must be {shape}")
    return batch, workspace.numel() * workspace.element_size()


def oscar_decode(desc: LayerDesc, q, rot_k, rot_v, pool, block_table, hist_len, k_win, v_win, win_len,
                 sm_scale: float, n_splits: int, workspace, out, stream=None, codebook=None):
    """Decode attention over the three segments in two launches; workspace from
    oscar_decode_workspace_bytes(desc, B, n_splits); out [B, Hq, 128] float32. With
    `codebook` this is oscar_decode_codebook."""
    batch, nbytes = _check_decode_args(desc, q, rot_k, rot_v, pool, block_table, hist_len, k_win, v_win, win_len,
                                       n_splits, workspace, out)
    rest = (_ptr(pool), _ptr(block_table), int(block_table.shape[1]), _ptr(hist_len), _ptr(k_win), _ptr(v_win),
            _ptr(win_len), batch, float(sm_scale), int(n_splits), _ptr(workspace), nbytes, _ptr(out), _stream(stream))
    if codebook is None:
        _check(lib().oscar_decode(byref(desc), _ptr(q), _ptr(rot_k), _ptr(rot_v), *rest))
    else:
        _check_codebook(desc, codebook)
        _check(lib().oscar_decode_codebook(byref(desc), _ptr(q), _ptr(rot_k), _ptr(rot_v), _ptr(codebook), *rest))


def oscar_decode_codebook(desc: LayerDesc, q, rot_k, rot_v, codebook, pool, block_table, hist_len, k_win, v_win,
                          win_len, sm_scale: float, n_splits: int, workspace, out, stream=None):
    """oscar_decode over a pool written with the Lloyd-Max codebook (uint8 [Hkv, 2, 4])."""
    oscar_decode(desc, q, rot_k, rot_v, pool, block_table, hist_len, k_win, v_win, win_len, sm_scale, n_splits,
                 workspace, out, stream, codebook)


def oscar_decode_multi(desc: LayerDesc, q, rot_k, rot_v, pool, block_table, hist_len, k_win, v_win, win_len,
                       sm_scale: float, n_splits: int, workspace, out, stream=None, codebook=None, prepare=False):
    """Decode attention for T query tokens per request (q [B, T, Hq, 128] bf16, out the same
    shape in float32; token t sees the window up to its own position), in one launch when the grid fits the chip
    at once (oscar_decode_multi_splits), else two; workspace from
    oscar_decode_workspace_bytes(desc, B * T, n_splits), zero-filled once before first use."""
    _need(q.dim() == 4 and q.shape[2] == desc.n_q_heads and q.shape[3] == HEAD_DIM, "q must be [batch, T, n_q_heads, 128]")
    n_tok = int(q.shape[1])
    batch, nbytes = _check_decode_args(desc, q, rot_k, rot_v, pool, block_table, hist_len, k_win, v_win, win_len,
                                       n_splits, workspace, out, n_tok)
    rest = (_ptr(pool), _ptr(block_table), int(block_table.shape[1]), _ptr(hist_len), _ptr(k_win), _ptr(v_win),
            _ptr(win_len), batch, float(sm_scale), int(n_splits), _ptr(workspace), nbytes, _ptr(out), _stream(stream))
    if codebook is None:
        return _run(prepare, lib().oscar_decode_multi, byref(desc), _ptr(q), n_tok, _ptr(rot_k), _ptr(rot_v), *rest)
    _check_codebook(desc, codebook)
    return _run(prepare, lib().oscar_decode_multi_codebook, byref(desc), _ptr(q), n_tok, _ptr(rot_k), _ptr(rot_v),
                _ptr(codebook), *rest)


def oscar_decode_multi_codebook(desc: LayerDesc, q, rot_k, rot_v, codebook, pool, block_table, hist_len, k_win, v_win,
                                win_len, sm_scale: float, n_splits: int, workspace, out, stream=None):
    """oscar_decode_multi over a pool written with the Lloyd-Max codebook (uint8 [Hkv, 2, 4])."""
    oscar_decode_multi(desc, q, rot_k, rot_v, pool, block_table, hist_len, k_win, v_win, win_len, sm_scale, n_splits,
                       workspace, out, stream, codebook)


def oscar_decode_step(desc: LayerDesc, k_src, v_src, dst_page, dst_slot, clip_k, clip_v, q, rot_k, rot_v, pool,
                      block_table, hist_len, k_win, v_win, win_len, sm_scale: float, n_splits: int, workspace, out,
                      stream=None, codebook=None, prepare=False):
    """Demote n tokens (k_src/v_src [n, Hkv, 128] bf16, n may be 0) and decode, in two launches.
    With `codebook` this is oscar_decode_step_codebook; with a desc of group_size 64 or 32,
    oscar_decode_step_grouped (four launches)."""
    batch, nbytes = _check_decode_args(desc, q, rot_k, rot_v, pool, block_table, hist_len, k_win, v_win, win_len,
                                       n_splits, workspace, out)
    n = int(k_src.shape[0]) if k_src is not None and k_src.dim() else 0
    if n:
        hkv = desc.n_kv_heads
        _device16(k_src, "k_src")
        _device16(v_src, "v_src")
        _need(k_src.numel() == n * hkv * HEAD_DIM and v_src.numel() == n * hkv * HEAD_DIM,
              "k_src/v_src must be [n, n_kv_heads, 128]")
        _device_i32(dst_page, "dst_page", n)
        _device_i32(dst_slot, "dst_slot", n)
        for t, name in ((clip_k, "clip_k"), (clip_v, "clip_v")):
            _need(t.is_cuda and t.numel() == hkv and t.dtype.is_floating_point and t.element_size() == 4,
                  f"{name} must be float32 [n_kv_heads] on the device")
    head = (_ptr(k_src) if n else None, _ptr(v_src) if n else None, n, _ptr(dst_page) if n else None,
            _ptr(dst_slot) if n else None, _ptr(clip_k) if n else None, _ptr(clip_v) if n else None, _ptr(q),
            _ptr(rot_k), _ptr(rot_v))
    rest = (_ptr(pool), _ptr(block_table), int(block_table.shape[1]), _ptr(hist_len), _ptr(k_win), _ptr(v_win),
            _ptr(win_len), batch, float(sm_scale), int(n_splits), _ptr(workspace), nbytes, _ptr(out), _stream(stream))
    if desc.group_size != 128:
        _need(codebook is None, "codebooks are defined for one group per vector")
        return _run(prepare, lib().oscar_decode_step_grouped, byref(desc), *head, *rest)
    if codebook is None:
        return _run(prepare, lib().oscar_decode_step, byref(desc), *head, *rest)
    _check_codebook(desc, codebook)
    return _run(prepare, lib().oscar_decode_step_codebook, byref(desc), *head, _ptr(codebook), *rest)


def oscar_decode_step_append_workspace_bytes(desc: LayerDesc, batch: int, n_splits: int) -> int:
    return int(lib().oscar_decode_step_append_workspace_bytes(byref(desc), int(batch), int(n_splits)))


def oscar_decode_step_append_splits(desc: LayerDesc, batch: int, max_hist_len: int) -> int:
    return int(lib().oscar_decode_step_append_splits(byref(desc), int(batch), int(max_hist_len)))


def oscar_decode_multi_splits(desc: LayerDesc, batch: int, n_tokens: int, max_hist_len: int) -> int:
    """Split count for oscar_decode_multi: one launch when its grid fits the chip at once."""
    return int(lib().oscar_decode_multi_splits(byref(desc), int(batch), int(n_tokens), int(max_hist_len)))


def oscar_decode_step_append_launches(desc: LayerDesc, batch: int, n_splits: int) -> int:
    """1 when oscar_decode_step_append runs in one launch for these sizes, 2 for prepare +
    attend, 0 for invalid arguments."""
    return int(lib().oscar_decode_step_append_launches(byref(desc), int(batch), int(n_splits)))


def oscar_decode_step_append(desc: LayerDesc, k_src, v_src, clip_k, clip_v, q, rot_k, rot_v, pool, block_table,
                             hist_len, k_win, v_win, win_len, sm_scale: float, n_splits: int, workspace, out,
                             stream=None, codebook=None, prepare=False):
    """One decode step in one launch: token b of k_src/v_src [batch, n_kv_heads, 128] bf16
    (None: nothing) becomes history token hist_len[b] - 1 of request b, then decode. The
    workspace's arrival counters must be zero before the first call (zero-fill it, and again
    when the batch or split count changes).
    With `prepare`, returns the call as a callable (see _run)."""
    _need(desc.group_size == 128, "the one-launch step reads one-group pages")
    batch = int(q.shape[0])
    _check_decode_args(desc, q, rot_k, rot_v, pool, block_table, hist_len, k_win, v_win, win_len, n_splits,
                       workspace, out)
    need = oscar_decode_step_append_workspace_bytes(desc, batch, n_splits)
    nbytes = workspace.numel() * workspace.element_size()
    _need(nbytes >= need, f"workspace holds {nbytes} bytes, needs {need}")
    app = k_src is not None
    if app:
        hkv = desc.n_kv_heads
        _device16(k_src, "k_src")
        _device16(v_src, "v_src")
        _need(k_src.numel() == batch * hkv * HEAD_DIM and v_src.numel() == batch * hkv * HEAD_DIM,
              "k_src/v_src must be [batch, n_kv_heads, 128]")
        for t, name in ((clip_k, "clip_k"), (clip_v, "clip_v")):
            _need(t.is_cuda and t.numel() == hkv and t.dtype.is_floating_point and t.element_size() == 4,
                  f"{name} must be float32 [n_kv_heads] on the device")
    head = (_ptr(k_src) if app else None, _ptr(v_src) if app else None, _ptr(clip_k) if app else None,
            _ptr(clip_v) if app else None, _ptr(q), _ptr(rot_k), _ptr(rot_v))
    rest = (_ptr(pool), _ptr(block_table), int(block_table.shape[1]), _ptr(hist_len), _ptr(k_win), _ptr(v_win),
            _ptr(win_len), batch, float(sm_scale), int(n_splits), _ptr(workspace), nbytes, _ptr(out), _stream(stream))
    if codebook is None:
        return _run(prepare, lib().oscar_decode_step_append, byref(desc), *head, *rest)
    _check_codebook(desc, codebook)
    return _run(prepare, lib().oscar_decode_step_append_codebook, byref(desc), *head, _ptr(codebook), *rest)


def oscar_decode_step_noalloc_max_bytes() -> int:
    return int(lib().oscar_decode_step_noalloc_max_bytes())


def oscar_decode_step_noalloc(desc: LayerDesc, k_src, v_src, dst_page, dst_slot, clip_k, clip_v, q, rot_k, rot_v,
                              pool, block_table, hist_len, k_win, v_win, win_len, sm_scale: float, n_splits: int,
                              out, stream=None):
    """oscar_decode_step with the library's static device workspace instead of a caller's
    (for callers that cannot allocate); uniform INT2 levels, one group per vector."""
    _need(desc.group_size == 128, "the no-allocation step reads one-group pages")
    batch = int(q.shape[0])
    _need(out.is_cuda and out.dtype.is_floating_point and out.element_size() == 4
          and out.numel() == batch * desc.n_q_heads * HEAD_DIM, "out must be float32 [batch, n_q_heads, 128]")
    n = int(k_src.shape[0]) if k_src is not None and k_src.dim() else 0
    if n:
        hkv = desc.n_kv_heads
        _device16(k_src, "k_src")
        _device16(v_src, "v_src")
        _need(k_src.numel() == n * hkv * HEAD_DIM and v_src.numel() == n * hkv * HEAD_DIM,
              "k_src/v_src must be [n, n_kv_heads, 128]")
        _device_i32(dst_page, "dst_page", n)
        _device_i32(dst_slot, "dst_slot", n)
    _check(lib().oscar_decode_step_noalloc(
        byref(desc), _ptr(k_src) if n else None, _ptr(v_src) if n else None, n, _ptr(dst_page) if n else None,
        _ptr(dst_slot) if n else None, _ptr(clip_k) if n else None, _ptr(clip_v) if n else None, _ptr(q),
        _ptr(rot_k), _ptr(rot_v), _ptr(pool), _ptr(block_table), int(block_table.shape[1]), _ptr(hist_len),
        _ptr(k_win), _ptr(v_win), _ptr(win_len), batch, float(sm_scale), int(n_splits), _ptr(out), _stream(stream)))


def oscar_decode_step_codebook(desc: LayerDesc, k_src, v_src, dst_page, dst_slot, clip_k, clip_v, q, rot_k, rot_v,
                               codebook, pool, block_table, hist_len, k_win, v_win, win_len, sm_scale: float,
                               n_splits: int, workspace, out, stream=None):
    """oscar_decode_step with the Lloyd-Max codebook (uint8 [Hkv, 2, 4]) for demotion and decode."""
    oscar_decode_step(desc, k_src, v_src, dst_page, dst_slot, clip_k, clip_v, q, rot_k, rot_v, pool, block_table,
                      hist_len, k_win, v_win, win_len, sm_scale, n_splits, workspace, out, stream, codebook)


def oscar_attend(desc: LayerDesc, rot_v, pool, block_table, hist_len, n_splits: int, workspace, out, stream=None,
                 codebook=None, prepare=False):
    """The second launch of oscar_decode_step alone (INT2 pass + merge into out). With
    `codebook` this is oscar_attend_codebook."""
    import torch

    batch = int(out.shape[0])
    _device16(rot_v, "rot_v")
    _need(rot_v.numel() == desc.n_kv_heads * HEAD_DIM * HEAD_DIM, "rot_v must be [n_kv_heads, 128, 128]")
    _need(pool.is_cuda and pool.is_contiguous(), "pool must be a contiguous device tensor")
    _need(block_table.dim() == 2 and block_table.shape[0] == batch, "block_table must be [batch, max_pages]")
    _device_i32(block_table, "block_table")
    _device_i32(hist_len, "hist_len", batch)
    _need(workspace.is_cuda and workspace.is_contiguous(), "workspace must be a contiguous device tensor")
    _need(out.is_cuda and out.dtype == torch.float32 and out.is_contiguous(), "out must be contiguous float32")
    _need(out.numel() == batch * desc.n_q_heads * HEAD_DIM, "out must be [batch, n_q_heads, 128]")
    rest = (_ptr(pool), _ptr(block_table), int(block_table.shape[1]), _ptr(hist_len), batch, int(n_splits),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out), _stream(stream))
    if codebook is None:
        return _run(prepare, lib().oscar_attend, byref(desc), _ptr(rot_v), *rest)
    _check_codebook(desc, codebook)
    return _run(prepare, lib().oscar_attend_codebook, byref(desc), _ptr(rot_v), _ptr(codebook), *rest)


def oscar_attend_codebook(desc: LayerDesc, rot_v, codebook, pool, block_table, hist_len, n_splits: int, workspace,
                          out, stream=None, prepare=False):
    """oscar_attend for a workspace that oscar_prepare_codebook prepared with the same codebook."""
    return oscar_attend(desc, rot_v, pool, block_table, hist_len, n_splits, workspace, out, stream, codebook,
                        prepare=prepare)


def oscar_prepare(desc: LayerDesc, k_src, v_src, dst_page, dst_slot, clip_k, clip_v, q, rot_k, rot_v, pool, k_win,
                  v_win, win_len, sm_scale: float, n_splits: int, workspace, stream=None, codebook=None):
    """The first launch of oscar_decode_step alone (demotion, window pass, query rotation).
    With `codebook` this is oscar_prepare_codebook."""
    batch = int(q.shape[0])
    _device16(q, "q")
    _need(q.numel() == batch * desc.n_q_heads * HEAD_DIM, "q must be [batch, n_q_heads, 128]")
    for t, name in ((rot_k, "rot_k"), (rot_v, "rot_v")):
        _device16(t, name)
        _need(t.numel() == desc.n_kv_heads * HEAD_DIM * HEAD_DIM, f"{name} must be [n_kv_heads, 128, 128]")
    w = desc.sink_tokens + desc.recent_tokens
    for t, name in ((k_win, "k_win"), (v_win, "v_win")):
        _device16(t, name)
        _need(t.numel() == batch * desc.n_kv_heads * w * HEAD_DIM, f"{name} must be [batch, n_kv_heads, {w}, 128]")
    _device_i32(win_len, "win_len", batch)
    _need(workspace.is_cuda and workspace.is_contiguous(), "workspace must be a contiguous device tensor")
    n = int(k_src.shape[0]) if k_src is not None and k_src.dim() else 0
    if n:
        hkv = desc.n_kv_heads
        _device16(k_src, "k_src")
        _device16(v_src, "v_src")
        _need(k_src.numel() == n * hkv * HEAD_DIM and v_src.numel() == n * hkv * HEAD_DIM,
              "k_src/v_src must be [n, n_kv_heads, 128]")
        _device_i32(dst_page, "dst_page", n)
        _device_i32(dst_slot, "dst_slot", n)
        for t, name in ((clip_k, "clip_k"), (clip_v, "clip_v")):
            _need(t.is_cuda and t.numel() == hkv and t.dtype.is_floating_point and t.element_size() == 4,
                  f"{name} must be float32 [n_kv_heads] on the device")
        _need(pool.is_cuda and pool.is_contiguous(), "pool must be a contiguous device tensor")
    head = (_ptr(k_src) if n else None, _ptr(v_src) if n else None, n, _ptr(dst_page) if n else None,
            _ptr(dst_slot) if n else None, _ptr(clip_k) if n else None, _ptr(clip_v) if n else None, _ptr(q),
            _ptr(rot_k), _ptr(rot_v))
    rest = (_ptr(pool), _ptr(k_win), _ptr(v_win), _ptr(win_len), batch, float(sm_scale), int(n_splits),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    if codebook is None:
        _check(lib().oscar_prepare(byref(desc), *head, *rest))
    else:
        _check_codebook(desc, codebook)
        _check(lib().oscar_prepare_codebook(byref(desc), *head, _ptr(codebook), *rest))


def oscar_prepare_codebook(desc: LayerDesc, k_src, v_src, dst_page, dst_slot, clip_k, clip_v, q, rot_k, rot_v,
                           codebook, pool, k_win, v_win, win_len, sm_scale: float, n_splits: int, workspace,
                           stream=None):
    """oscar_prepare with the Lloyd-Max codebook (uint8 [Hkv, 2, 4]) for demotion and the query data."""
    oscar_prepare(desc, k_src, v_src, dst_page, dst_slot, clip_k, clip_v, q, rot_k, rot_v, pool, k_win, v_win,
                  win_len, sm_scale, n_splits, workspace, stream, codebook)


def oscar_demote_grouped(desc: LayerDesc, k_src, v_src, dst_page, dst_slot, rot_k, rot_v, clip_k, clip_v, pool,
                         stream=None):
    """oscar_demote into grouped pages (desc.group_size 128, 64 or 32); arguments as oscar_demote."""
    n = int(k_src.shape[0]) if k_src.dim() else 0
    _device16(k_src, "k_src")
    _device16(v_src, "v_src")
    _need(k_src.numel() == n * desc.n_kv_heads * HEAD_DIM and v_src.numel() == k_src.numel(),
          "k_src/v_src must be [n, n_kv_heads, 128]")
    _device_i32(dst_page, "dst_page", n)
    _device_i32(dst_slot, "dst_slot", n)
    _need(pool.is_cuda and pool.is_contiguous(), "pool must be a contiguous device tensor")
    _check(lib().oscar_demote_grouped(byref(desc), _ptr(k_src), _ptr(v_src), n, _ptr(dst_page), _ptr(dst_slot),
                                      _ptr(rot_k), _ptr(rot_v), _ptr(clip_k), _ptr(clip_v), _ptr(pool),
                                      _stream(stream)))


def oscar_decode_int2_grouped(desc: LayerDesc, q, rot_k, pool, block_table, hist_len, sm_scale: float,
                              n_splits: int, partials, stream=None, prepare=False):
    """INT2 history pass over grouped pages (desc.group_size 128, 64 or 32); arguments as
    oscar_decode_int2."""
    batch = int(q.shape[0])
    _device16(q, "q")
    _need(q.numel() == batch * desc.n_q_heads * HEAD_DIM, "q must be [batch, n_q_heads, 128]")
    _need(block_table.dim() == 2 and block_table.shape[0] == batch, "block_table must be [batch, max_pages]")
    _device_i32(block_table, "block_table")
    _device_i32(hist_len, "hist_len", batch)
    _need(pool.is_cuda and partials.is_cuda and partials.is_contiguous(), "pool/partials must be device tensors")
    return _run(prepare, lib().oscar_decode_int2_grouped, byref(desc), _ptr(q), _ptr(rot_k), _ptr(pool),
                _ptr(block_table), int(block_table.shape[1]), _ptr(hist_len), batch, float(sm_scale), int(n_splits),
                _ptr(partials), partials.numel() * partials.element_size(), _stream(stream))


def oscar_decode_step_grouped(desc: LayerDesc, k_src, v_src, dst_page, dst_slot, clip_k, clip_v, q, rot_k, rot_v, pool,
                              block_table, hist_len, k_win, v_win, win_len, sm_scale: float, n_splits: int, workspace,
                              out, stream=None):
    """oscar_decode_step over grouped pages (desc.group_size 64 or 32)."""
    _need(desc.group_size in (64, 32), "oscar_decode_step_grouped takes a desc of group_size 64 or 32")
    oscar_decode_step(desc, k_src, v_src, dst_page, dst_slot, clip_k, clip_v, q, rot_k, rot_v, pool, block_table,
                      hist_len, k_win, v_win, win_len, sm_scale, n_splits, workspace, out, stream)
