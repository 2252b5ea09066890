"""Device buffers and call sequences for one decode step and one chunked-prefill call.

This module only allocates device memory (through torch) and calls the C
entry points in order; all arithmetic runs in libmla.so.

Decode step (one query token per sequence):
    mla_absorb_query -> mla_decode_partial -> mla_combine -> mla_out_proj
or, with the work-balanced split over ``n_units`` workgroups:
    mla_absorb_query -> mla_decode_partial_balanced -> mla_combine_balanced -> mla_out_proj
and, with ``fused=True``, the merge and the value projection as one call
(mla_combine_out_proj / mla_combine_out_proj_balanced; z is then not written).
Chunked prefill (q_len query tokens per sequence):
    mla_absorb_query -> mla_prefill_chunk -> mla_out_proj
Multi-token verify (q_len query tokens per sequence, as batch * q_len decode rows):
    mla_verify_rows -> mla_absorb_query -> mla_decode_partial_balanced -> mla_combine_balanced
    -> mla_out_proj
Any of these sequences can be captured once in a HIP graph and replayed (CapturedStep).
"""

from __future__ import annotations

import numpy as np
import torch

from . import _lib as L


def to_device(x: np.ndarray, device) -> torch.Tensor:
    """Host array -> device tensor.  uint16 arrays are bfloat16 bit patterns; a tensor already on
    the device is used as it is."""
    if isinstance(x, torch.Tensor):
        return x.to(device)
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(x).to(device)


def _torch_dtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def q_hat_dtype(dtype: str):
    """Storage of the absorbed query: IEEE binary16 on the bf16 path, float32 otherwise."""
    return torch.float16 if dtype == "bf16" else torch.float32


def compute_units(device=None) -> int:
    """Compute units of the device (one balanced-split unit each)."""
    return int(torch.cuda.get_device_properties(torch.device(device or "cuda:0")).multi_processor_count)


def balanced_units(lens, n_cu: int, min_tiles: int = 4) -> int:
    """Units of the balanced split for a batch: one per compute unit, fewer when that would leave
    a unit less than `min_tiles` tiles (MLA_BALANCED_TILE tokens each) of cache to read."""
    lens = np.asarray(lens, dtype=np.int64)
    tiles = int(np.sum((lens + L.MLA_BALANCED_TILE - 1) // L.MLA_BALANCED_TILE))
    return max(1, min(int(n_cu), L.MLA_BALANCED_MAX_UNITS, -(-tiles // min_tiles)))


def partials_workspace(d: L.MlaDims, slots: int, device, nbytes: int | None = None):
    """A split-K workspace of `slots` partial slots (or `nbytes` bytes) and its two views:
    o_part float [slots, H, d_c] and lse_part float [slots, H] (the layout of include/mla.h)."""
    need = L.mla_partials_bytes(d, slots)
    nbytes = need if nbytes is None else int(nbytes)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
    off = L.mla_partials_lse_offset(d, slots)
    H, dc = d.n_heads, d.d_c
    o_part = ws[:slots * H * dc * 4].view(torch.float32).view(slots, H, dc)
    lse_part = ws[off:off + slots * H * 4].view(torch.float32).view(slots, H)
    return ws, nbytes, o_part, lse_part


def dims_for(w, flags: int = 0) -> L.MlaDims:
    return L.dims(w.n_heads, w.d_c, w.d_r, w.d_k, w.d_v, dtype=L.MLA_BF16 if w.dtype == "bf16" else L.MLA_F32,
                  rope_base=w.rope_base, sm_scale=0.0, flags=flags)


class DecodeStep:
    """All device buffers of one batched decode step; ``run()`` enqueues the four calls.

    ``split_tokens`` > 0 selects fixed chunks of that many tokens; ``n_units`` selects the
    work-balanced split instead (``split_tokens`` is then ignored).
    """

    def __init__(self, inp: dict, split_tokens: int = 0, device="cuda:0", flags: int = 0,
                 max_len: int | None = None, n_units: int | None = None, fused: bool = False):
        w = inp["workload"]
        self.w = w
        self.device = torch.device(device)
        self.d = dims_for(w, flags)
        dev = self.device
        self.q_c = to_device(inp["q_c"], dev)
        self.q_r = to_device(inp["q_r"], dev)
        self.w_uk = to_device(inp["w_uk"], dev)
        self.w_uv = to_device(inp["w_uv"], dev)
        self.pool = to_device(inp["pool"], dev)
        self.page_table = to_device(inp["page_table"], dev)
        self.lens = to_device(inp["lens"].astype(np.int32), dev)
        self.pos = to_device(inp["pos"].astype(np.int32), dev)
        self.B = int(inp["lens"].shape[0])
        self.max_len = int(inp["lens"].max()) if max_len is None else int(max_len)
        H, W = w.n_heads, w.d_c + w.d_r
        self.n_units = None if n_units is None else int(n_units)
        if self.n_units is not None:
            self.split_tokens = 0
            self.S = L.mla_balanced_num_slots(self.B, self.n_units)
            slots = self.S
        else:
            self.split_tokens = int(split_tokens)
            self.S = L.mla_decode_num_splits(self.max_len, self.split_tokens)
            slots = self.B * self.S
        td = _torch_dtype(w.dtype)
        self.q_hat = torch.empty((self.B, H, W), dtype=q_hat_dtype(w.dtype), device=dev)
        self.ws, self.ws_bytes, o_part, lse_part = partials_workspace(self.d, slots, dev)
        if self.n_units is None:  # slot b * S + i: chunk i of sequence b
            o_part = o_part.view(self.B, self.S, H, w.d_c)
            lse_part = lse_part.view(self.B, self.S, H)
        self.o_part, self.lse_part = o_part, lse_part
        self.z = torch.empty((self.B, H, w.d_c), dtype=torch.float32, device=dev)
        self.lse = torch.empty((self.B, H), dtype=torch.float32, device=dev)
        self.out = torch.empty((self.B, H, w.d_v), dtype=torch.float32, device=dev)
        self.c = L.cache(self.pool, self.page_table, self.lens)
        self.fused = bool(fused) and L.mla_combine_out_proj_supported(self.d)

    def uses_mfma(self) -> bool:
        return L.mla_decode_uses_mfma(self.d, self.c, self.split_tokens)

    def absorb(self, stream=None):
        L.mla_absorb_query(self.d, self.q_c, self.q_r, self.w_uk, self.pos, self.B, self.q_hat, stream)

    def attend(self, stream=None):
        if self.n_units is not None:
            L.mla_decode_partial_balanced(self.d, self.c, self.q_hat, self.n_units, self.ws, self.ws_bytes, stream)
        else:
            L.mla_decode_partial(self.d, self.c, self.q_hat, self.max_len, self.split_tokens, self.ws, self.ws_bytes,
                                 stream)

    def combine(self, stream=None):
        if self.n_units is not None:
            L.mla_combine_balanced(self.d, self.c, self.n_units, self.ws, self.ws_bytes, self.z, self.lse, stream)
        else:
            L.mla_combine(self.d, self.B, self.S, self.ws, self.ws_bytes, self.z, self.lse, stream)

    def out_proj(self, stream=None):
        L.mla_out_proj(self.d, self.z, self.w_uv, self.B, self.out, stream)

    def combine_out_proj(self, stream=None):
        """Merge and value projection in one call (out and lse; z is not written)."""
        if self.n_units is not None:
            L.mla_combine_out_proj_balanced(self.d, self.c, self.n_units, self.ws, self.ws_bytes, self.w_uv, self.out,
                                            self.lse, stream)
        else:
            L.mla_combine_out_proj(self.d, self.B, self.S, self.ws, self.ws_bytes, self.w_uv, self.out, self.lse,
                                   stream)

    def finish(self, stream=None):
        """Everything after the split-K decode: the fused call, or mla_combine* then mla_out_proj."""
        if self.fused:
            self.combine_out_proj(stream)
        else:
            self.combine(stream)
            self.out_proj(stream)

    def run(self, stream=None):
        self.absorb(stream)
        self.attend(stream)
        self.finish(stream)


class PrefillStep:
    """Device buffers of one chunked-prefill call; ``run()`` enqueues absorb, prefill, out_proj."""

    def __init__(self, inp: dict, device="cuda:0", flags: int = 0):
        w = inp["workload"]
        self.w = w
        self.device = torch.device(device)
        self.d = dims_for(w, flags)
        dev = self.device
        self.q_c = to_device(inp["q_c"], dev)
        self.q_r = to_device(inp["q_r"], dev)
        self.w_uk = to_device(inp["w_uk"], dev)
        self.w_uv = to_device(inp["w_uv"], dev)
        self.pool = to_device(inp["pool"], dev)
        self.page_table = to_device(inp["page_table"], dev)
        self.lens = to_device(inp["lens"].astype(np.int32), dev)
        self.q_start = to_device(inp["q_start"].astype(np.int32), dev)
        B, Sq = inp["q_c"].shape[0], inp["q_c"].shape[1]
        self.B, self.Sq = int(B), int(Sq)
        pos = (inp["q_start"][:, None] + np.arange(Sq)[None, :]).astype(np.int32).reshape(-1)
        self.pos = to_device(pos, dev)
        H, W = w.n_heads, w.d_c + w.d_r
        td = _torch_dtype(w.dtype)
        self.q_hat = torch.empty((self.B, self.Sq, H, W), dtype=q_hat_dtype(w.dtype), device=dev)
        self.z = torch.empty((self.B, self.Sq, H, w.d_c), dtype=torch.float32, device=dev)
        self.lse = torch.empty((self.B, self.Sq, H), dtype=torch.float32, device=dev)
        self.out = torch.empty((self.B, self.Sq, H, w.d_v), dtype=torch.float32, device=dev)
        self.c = L.cache(self.pool, self.page_table, self.lens)

    def uses_mfma(self) -> bool:
        return L.mla_prefill_uses_mfma(self.d, self.c)

    def absorb(self, stream=None):
        L.mla_absorb_query(self.d, self.q_c, self.q_r, self.w_uk, self.pos, self.B * self.Sq, self.q_hat, stream)

    def attend(self, stream=None):
        L.mla_prefill_chunk(self.d, self.c, self.q_hat, self.Sq, self.q_start, self.z, self.lse, stream)

    def out_proj(self, stream=None):
        L.mla_out_proj(self.d, self.z, self.w_uv, self.B * self.Sq, self.out, stream)

    def run(self, stream=None):
        self.absorb(stream)
        self.attend(stream)
        self.out_proj(stream)


class VerifyStep:
    """Device buffers of one multi-token verify call on the decode path: query i of sequence b
    becomes decode row b * q_len + i over its own prefix (mla_verify_rows writes the rows' page
    table, lengths and positions), then the work-balanced decode over ``n_units`` workgroups with
    the q_len rows of a sequence as one row group (mla_decode_partial_grouped: the draft rows of a
    sequence read its pages side by side), or the plain balanced split when ``grouped`` is false.
    ``n_units`` is rounded down to a multiple of q_len for the grouped split.
    Same inputs and outputs as PrefillStep (``out`` [B, q_len, H, d_v], ``lse`` [B, q_len, H])."""

    def __init__(self, inp: dict, device="cuda:0", n_units: int = 256, flags: int = 0, grouped: bool = True,
                 fused: bool = False):
        w = inp["workload"]
        self.w = w
        self.device = torch.device(device)
        self.d = dims_for(w, flags)
        dev = self.device
        self.q_c = to_device(inp["q_c"], dev)
        self.q_r = to_device(inp["q_r"], dev)
        self.w_uk = to_device(inp["w_uk"], dev)
        self.w_uv = to_device(inp["w_uv"], dev)
        self.pool = to_device(inp["pool"], dev)
        self.page_table = to_device(inp["page_table"], dev)
        self.lens = to_device(inp["lens"].astype(np.int32), dev)
        self.q_start = to_device(inp["q_start"].astype(np.int32), dev)
        self.B, self.Sq = int(inp["q_c"].shape[0]), int(inp["q_c"].shape[1])
        R = self.B * self.Sq
        H, W = w.n_heads, w.d_c + w.d_r
        self.group = self.Sq if grouped and int(n_units) >= self.Sq else 1
        self.n_units = int(n_units) // self.group * self.group
        max_pages = int(self.page_table.shape[1])
        self.row_table = torch.empty((R, max_pages), dtype=torch.int32, device=dev)
        self.row_lens = torch.empty((R,), dtype=torch.int32, device=dev)
        self.row_pos = torch.empty((R,), dtype=torch.int32, device=dev)
        self.S = L.mla_balanced_num_slots(R, self.n_units)
        td = _torch_dtype(w.dtype)
        self.q_hat = torch.empty((R, H, W), dtype=q_hat_dtype(w.dtype), device=dev)
        self.ws, self.ws_bytes, self.o_part, self.lse_part = partials_workspace(self.d, self.S, dev)
        self.z = torch.empty((self.B, self.Sq, H, w.d_c), dtype=torch.float32, device=dev)
        self.lse = torch.empty((self.B, self.Sq, H), dtype=torch.float32, device=dev)
        self.out = torch.empty((self.B, self.Sq, H, w.d_v), dtype=torch.float32, device=dev)
        self.c = L.cache(self.pool, self.page_table, self.lens)
        self.rc = L.cache(self.pool, self.row_table, self.row_lens, batch=R, page_size=int(self.pool.shape[1]),
                          max_pages=max_pages, num_pages=int(self.pool.shape[0]))
        self.fused = bool(fused) and L.mla_combine_out_proj_supported(self.d)

    def rows(self, stream=None):
        L.mla_verify_rows(self.c, self.q_start, self.Sq, self.row_table, self.row_lens, self.row_pos, stream)

    def absorb(self, stream=None):
        L.mla_absorb_query(self.d, self.q_c, self.q_r, self.w_uk, self.row_pos, self.B * self.Sq, self.q_hat, stream)

    def attend(self, stream=None):
        L.mla_decode_partial_grouped(self.d, self.rc, self.q_hat, self.n_units, self.group, self.ws, self.ws_bytes,
                                     stream)

    def combine(self, stream=None):
        L.mla_combine_grouped(self.d, self.rc, self.n_units, self.group, self.ws, self.ws_bytes, self.z, self.lse,
                              stream)

    def out_proj(self, stream=None):
        L.mla_out_proj(self.d, self.z, self.w_uv, self.B * self.Sq, self.out, stream)

    def combine_out_proj(self, stream=None):
        L.mla_combine_out_proj_grouped(self.d, self.rc, self.n_units, self.group, self.ws, self.ws_bytes, self.w_uv,
                                       self.out, self.lse, stream)

    def finish(self, stream=None):
        if self.fused:
            self.combine_out_proj(stream)
        else:
            self.combine(stream)
            self.out_proj(stream)

    def run(self, stream=None):
        self.rows(stream)
        self.absorb(stream)
        self.attend(stream)
        self.finish(stream)


class PrefillUnabsorbedStep:
    """Device buffers of one unabsorbed chunked-prefill call; ``run()`` enqueues the per-head
    decompression of the cached latents, then causal attention over the decompressed keys and
    values (output in the value space, like PrefillStep.out)."""

    def __init__(self, inp: dict, device="cuda:0", max_len: int | None = None):
        w = inp["workload"]
        self.w = w
        self.device = torch.device(device)
        self.d = dims_for(w)
        dev = self.device
        self.q_c = to_device(inp["q_c"], dev)
        self.q_r = to_device(inp["q_r"], dev)
        self.w_uk = to_device(inp["w_uk"], dev)
        self.w_uv = to_device(inp["w_uv"], dev)
        self.pool = to_device(inp["pool"], dev)
        self.page_table = to_device(inp["page_table"], dev)
        self.lens = to_device(inp["lens"].astype(np.int32), dev)
        self.q_start = to_device(inp["q_start"].astype(np.int32), dev)
        self.B, self.Sq = int(inp["q_c"].shape[0]), int(inp["q_c"].shape[1])
        self.max_len = int(max_len or max(1, int(np.max(inp["lens"]))))
        H = w.n_heads
        self.k = torch.empty((self.B, H, self.max_len, w.d_k), dtype=torch.float16, device=dev)
        self.v = torch.empty((self.B, H, self.max_len, w.d_v), dtype=torch.float16, device=dev)
        self.k_r = torch.empty((self.B, self.max_len, w.d_r), dtype=torch.float16, device=dev)
        self.lse = torch.empty((self.B, self.Sq, H), dtype=torch.float32, device=dev)
        self.out = torch.empty((self.B, self.Sq, H, w.d_v), dtype=torch.float32, device=dev)
        self.c = L.cache(self.pool, self.page_table, self.lens)

    def supported(self) -> bool:
        return L.mla_prefill_unabsorbed_supported(self.d)

    def decompress(self, stream=None):
        L.mla_decompress_kv(self.d, self.c, self.max_len, self.w_uk, self.w_uv, self.k, self.v, self.k_r, stream)

    def attend(self, stream=None):
        L.mla_prefill_unabsorbed(self.d, self.c, self.max_len, self.q_c, self.q_r, self.q_start, self.Sq, self.k,
                                 self.v, self.k_r, self.out, self.lse, stream)

    def run(self, stream=None):
        self.decompress(stream)
        self.attend(stream)


class CapturedStep:
    """One call sequence of a step object captured in a HIP graph and replayed.

    The graph holds the step's own kernel launches on its own buffers (no allocation, no memset,
    no synchronisation happens inside the entry points), so a replay is the same work as
    ``step.run()`` with one host launch instead of one per kernel.  Inputs are read at every
    replay: write new values into the step's input tensors in place between replays.  The
    step's tensors must stay alive as long as the graph.
    """

    def __init__(self, step, warmup: int = 2):
        self.step = step
        side = torch.cuda.Stream()  # default priority
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(warmup):
                step.run()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            step.run()
        torch.cuda.synchronize()

    def run(self):
        self.graph.replay()
