"""One attention layer's three-segment KV pool on the GPU, driven through the C ABI.

Holds the device buffers a serving engine keeps per layer (INT2 page pool, block table,
history lengths, BF16 sink/recent window, per-head rotations and clip ratios) and the
partial-result workspaces, and calls the four entry points in the order a decode step
needs them: demote the oldest recent tokens, INT2 pass, BF16 pass, merge.
"""

from __future__ import annotations

import numpy as np
import torch

from . import _lib as L

HEAD_DIM = 128
PAGE_TOKENS = 64


def _bf16_tensor(bits_or_values, device) -> torch.Tensor:
    a = np.asarray(bits_or_values)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16).copy())
        return t.to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device).to(torch.bfloat16)


class LayerCache:
    def __init__(self, n_q_heads: int, n_kv_heads: int, batch: int, max_pages: int, n_pages: int,
                 device="cuda", group_size: int = 128):
        # group_size 64 or 32: grouped pages, read and written by demote() and decode() only
        self.desc = L.layer_desc(n_q_heads, n_kv_heads, group_size)
        st = L.oscar_check_desc(self.desc)
        if st != L.OSCAR_OK:
            raise L.OscarError(st, L.oscar_last_error())
        self.device = torch.device(device)
        self.batch = batch
        self.n_q, self.n_kv = n_q_heads, n_kv_heads
        self.window = L.oscar_window_tokens(self.desc)
        self.pool = torch.zeros(n_pages * L.oscar_page_bytes(self.desc), dtype=torch.uint8, device=self.device)
        self.block_table = torch.zeros((batch, max_pages), dtype=torch.int32, device=self.device)
        self.hist_len = torch.zeros(batch, dtype=torch.int32, device=self.device)
        self.k_win = torch.zeros((batch, n_kv_heads, self.window, HEAD_DIM), dtype=torch.bfloat16, device=self.device)
        self.v_win = torch.zeros_like(self.k_win)
        self.win_len = torch.zeros(batch, dtype=torch.int32, device=self.device)
        self.rot_k = torch.zeros((n_kv_heads, HEAD_DIM, HEAD_DIM), dtype=torch.bfloat16, device=self.device)
        self.rot_v = torch.zeros_like(self.rot_k)
        self.clip_k = torch.ones(n_kv_heads, dtype=torch.float32, device=self.device)
        self.clip_v = torch.ones_like(self.clip_k)
        self.out = torch.zeros((batch, n_q_heads, HEAD_DIM), dtype=torch.float32, device=self.device)
        self.n_splits = 1
        self.codebook = None  # Lloyd-Max variant: uint8 [Hkv, 2, 4] levels (None: uniform INT2)
        self._partials = None
        self._workspace = None
        self._append_ws_splits = None  # the split count the step workspace was zeroed for
        self._append_ws = None
        self.win_partials = torch.zeros(L.oscar_partials_bytes(self.desc, batch, L.oscar_window_splits(self.desc)),
                                        dtype=torch.uint8, device=self.device)

    # --------------------------------------------------------------------- setup helpers
    def set_rotations(self, rot_k_bits, rot_v_bits, clip_k, clip_v):
        self.rot_k.copy_(_bf16_tensor(rot_k_bits, self.device).reshape(self.rot_k.shape))
        self.rot_v.copy_(_bf16_tensor(rot_v_bits, self.device).reshape(self.rot_v.shape))
        self.clip_k.copy_(torch.as_tensor(np.asarray(clip_k, np.float32)).reshape(-1))
        self.clip_v.copy_(torch.as_tensor(np.asarray(clip_v, np.float32)).reshape(-1))

    def set_codebook(self, k_levels, v_levels):
        """Switch the layer to the Lloyd-Max codebook variant: k_levels/v_levels [Hkv, 4] are each
        head's four levels in sixteenths of the scale (strictly increasing, within [0, 48]).
        A pool is written and read with one codebook; None for both restores the uniform levels."""
        if k_levels is None and v_levels is None:
            self.codebook = None
            return
        k = np.asarray(k_levels, np.int64).reshape(self.n_kv, 4)
        v = np.asarray(v_levels, np.int64).reshape(self.n_kv, 4)
        for lv in (k, v):
            if np.any(lv < 0) or np.any(lv > 48) or np.any(np.diff(lv, axis=1) <= 0):
                raise ValueError("codebook levels must be strictly increasing within [0, 48]")
        cb = np.stack([k, v], axis=1).astype(np.uint8)
        self.codebook = torch.from_numpy(np.ascontiguousarray(cb)).to(self.device)

    def set_block_table(self, table: np.ndarray):
        t = torch.from_numpy(np.where(table < 0, 0, table).astype(np.int32))
        self.block_table.copy_(t)

    def set_hist_len(self, lens):
        self.hist_len.copy_(torch.as_tensor(np.asarray(lens, np.int32)))

    def set_window(self, b: int, kv: int, k_rows, v_rows):
        n = len(k_rows)
        self.k_win[b, kv, :n] = _bf16_tensor(k_rows, self.device)
        self.v_win[b, kv, :n] = _bf16_tensor(v_rows, self.device)

    def set_win_len(self, lens):
        self.win_len.copy_(torch.as_tensor(np.asarray(lens, np.int32)))

    def set_splits(self, n_splits: int):
        self.n_splits = int(n_splits)
        need = L.oscar_partials_bytes(self.desc, self.batch, self.n_splits)
        if self._partials is None or self._partials.numel() < need:
            self._partials = torch.zeros(need, dtype=torch.uint8, device=self.device)

    @property
    def workspace(self) -> torch.Tensor:
        """Workspace of the two-launch decode (no initialisation needed)."""
        need = L.oscar_decode_workspace_bytes(self.desc, self.batch, self.n_splits)
        if self._workspace is None or self._workspace.numel() < need:
            self._workspace = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self._workspace

    @property
    def append_workspace(self) -> torch.Tensor:
        """Workspace of the one-launch step, zero-filled when allocated and again when the
        split count changes: its arrival counters must start at zero (every call leaves them
        there), and they sit after the partials, whose size depends on the split count."""
        need = L.oscar_decode_step_append_workspace_bytes(self.desc, self.batch, self.n_splits)
        if self._append_ws is None or self._append_ws.numel() < need:
            self._append_ws = torch.zeros(need, dtype=torch.uint8, device=self.device)
            self._append_ws_splits = self.n_splits
        elif self._append_ws_splits != self.n_splits:
            self._append_ws.zero_()
            torch.cuda.current_stream(self.device).synchronize()  # before a launch on any stream
            self._append_ws_splits = self.n_splits
        return self._append_ws

    @property
    def partials(self) -> torch.Tensor:
        if self._partials is None:
            self.set_splits(self.n_splits)
        return self._partials

    # ------------------------------------------------------------------------ the path
    def demote(self, k_rows: torch.Tensor, v_rows: torch.Tensor, pages: torch.Tensor, slots: torch.Tensor,
               stream=None):
        """Demote tokens k_rows/v_rows [n, Hkv, 128] bf16 into (pages[i], slots[i])."""
        L.oscar_demote(self.desc, k_rows, v_rows, pages, slots, self.rot_k, self.rot_v, self.clip_k,
                       self.clip_v, self.pool, stream, self.codebook)

    def decode(self, q: torch.Tensor, sm_scale: float, stream=None, prepare=False):
        """Attention output [B, Hq, 128] float32 for queries q [B, Hq, 128] bf16, in three
        launches (INT2 pass, window pass, merge). With `prepare`, returns the three calls as one
        zero-argument callable (validated once)."""
        if self.codebook is not None:
            raise ValueError("the separate entry points read uniform INT2 levels; use decode_fused() or step()")
        calls = (L.oscar_decode_int2(self.desc, q, self.rot_k, self.pool, self.block_table, self.hist_len, sm_scale,
                                     self.n_splits, self.partials, stream, prepare=prepare),
                 L.oscar_decode_bf16(self.desc, q, self.k_win, self.v_win, self.win_len, sm_scale, self.win_partials,
                                     stream, prepare=prepare),
                 L.oscar_merge(self.desc, self.partials, self.n_splits, self.win_partials, self.rot_v, self.out,
                               stream, prepare=prepare))
        if prepare:
            def run():
                for c in calls:
                    c()
            return run
        return self.out

    def decode_fused(self, q: torch.Tensor, sm_scale: float, stream=None) -> torch.Tensor:
        """The same output as decode(), in two launches (oscar_decode)."""
        L.oscar_decode(self.desc, q, self.rot_k, self.rot_v, self.pool, self.block_table, self.hist_len,
                       self.k_win, self.v_win, self.win_len, sm_scale, self.n_splits, self.workspace, self.out,
                       stream, self.codebook)
        return self.out

    def step(self, k_rows, v_rows, pages, slots, q: torch.Tensor, sm_scale: float, stream=None, prepare=False):
        """Demote k_rows/v_rows [n, Hkv, 128] into (pages, slots), then decode q: one decode step in
        two launches (oscar_decode_step). hist_len must already count the demoted tokens. Returns
        out, or with `prepare` the call as a zero-argument callable (validated once)."""
        call = L.oscar_decode_step(self.desc, k_rows, v_rows, pages, slots, self.clip_k, self.clip_v, q, self.rot_k,
                                   self.rot_v, self.pool, self.block_table, self.hist_len, self.k_win, self.v_win,
                                   self.win_len, sm_scale, self.n_splits, self.workspace, self.out, stream,
                                   self.codebook, prepare=prepare)
        return call if prepare else self.out

    def step_append(self, k_rows, v_rows, q: torch.Tensor, sm_scale: float, stream=None, prepare=False):
        """One decode step in one launch (oscar_decode_step_append): k_rows/v_rows [B, Hkv, 128]
        (or None) become history token hist_len[b] - 1 of each request b, then decode q. Returns
        out, or with `prepare` the call as a zero-argument callable (validated once)."""
        call = L.oscar_decode_step_append(self.desc, k_rows, v_rows, self.clip_k, self.clip_v, q, self.rot_k,
                                          self.rot_v, self.pool, self.block_table, self.hist_len, self.k_win,
                                          self.v_win, self.win_len, sm_scale, self.n_splits, self.append_workspace,
                                          self.out, stream, self.codebook, prepare=prepare)
        return call if prepare else self.out
