"""ctypes binding over libmla.so: argument marshalling only.

Each function has the name and argument order of the C entry point in
include/mla.h.  Tensor arguments may be torch tensors (their device address is
passed) or plain integers holding device addresses.  Every step of the
computation runs in the HIP kernels of libmla.so; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmla.so")

MLA_OK = 0
MLA_ERR_NULL = 1
MLA_ERR_SHAPE = 2
MLA_ERR_DTYPE = 3
MLA_ERR_ALIGN = 4
MLA_ERR_UNSUPPORTED = 5
MLA_ERR_HIP = 6
MLA_ERR_WORKSPACE = 7

MLA_F32 = 0
MLA_BF16 = 1
MLA_FLAG_FORCE_GENERIC = 1
MLA_FLAG_CACHE_FP8 = 2
MLA_FP8_ROW_BYTES = 656
MLA_NOALLOC_SCRATCH_BYTES = 8 << 20

# Balanced split-K constants (include/mla.h)
MLA_BALANCED_TILE = 32
MLA_BALANCED_SEG_COST = 8
MLA_BALANCED_MAX_UNITS = 2048


class MlaDims(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("d_c", ctypes.c_int32), ("d_r", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32), ("rope_base", ctypes.c_float),
                ("sm_scale", ctypes.c_float), ("dtype", ctypes.c_int32), ("flags", ctypes.c_int32)]


class MlaCache(ctypes.Structure):
    _fields_ = [("pool", ctypes.c_void_p), ("page_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("page_size", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("num_pages", ctypes.c_int32)]


class MlaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_lib = None

_VP, _I32, _F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
_PD, _PC = ctypes.POINTER(MlaDims), ctypes.POINTER(MlaCache)

_SIGNATURES = {
    "mla_status_str": (ctypes.c_char_p, [_I32]),
    "mla_absorb_query": (_I32, [_PD, _VP, _VP, _VP, _VP, _I32, _VP, _VP]),
    "mla_decode_num_splits": (_I32, [_I32, _I32]),
    "mla_decode_uses_mfma": (_I32, [_PD, _PC, _I32]),
    "mla_prefill_uses_mfma": (_I32, [_PD, _PC]),
    "mla_partials_lse_offset": (ctypes.c_size_t, [_PD, _I32]),
    "mla_partials_bytes": (ctypes.c_size_t, [_PD, _I32]),
    "mla_decode_workspace_bytes": (ctypes.c_size_t, [_PD, _PC, _I32, _I32]),
    "mla_decode_partial": (_I32, [_PD, _PC, _VP, _I32, _I32, _VP, ctypes.c_size_t, _VP]),
    "mla_combine": (_I32, [_PD, _I32, _I32, _VP, ctypes.c_size_t, _VP, _VP, _VP]),
    "mla_balanced_num_slots": (_I32, [_I32, _I32]),
    "mla_decode_balanced_workspace_bytes": (ctypes.c_size_t, [_PD, _PC, _I32]),
    "mla_decode_partial_balanced": (_I32, [_PD, _PC, _VP, _I32, _VP, ctypes.c_size_t, _VP]),
    "mla_combine_balanced": (_I32, [_PD, _PC, _I32, _VP, ctypes.c_size_t, _VP, _VP, _VP]),
    "mla_decode_partial_grouped": (_I32, [_PD, _PC, _VP, _I32, _I32, _VP, ctypes.c_size_t, _VP]),
    "mla_combine_grouped": (_I32, [_PD, _PC, _I32, _I32, _VP, ctypes.c_size_t, _VP, _VP, _VP]),
    "mla_out_proj": (_I32, [_PD, _VP, _VP, _I32, _VP, _VP]),
    "mla_combine_out_proj_supported": (_I32, [_PD]),
    "mla_combine_out_proj": (_I32, [_PD, _I32, _I32, _VP, ctypes.c_size_t, _VP, _VP, _VP, _VP]),
    "mla_combine_out_proj_balanced": (_I32, [_PD, _PC, _I32, _VP, ctypes.c_size_t, _VP, _VP, _VP, _VP]),
    "mla_combine_out_proj_grouped": (_I32, [_PD, _PC, _I32, _I32, _VP, ctypes.c_size_t, _VP, _VP, _VP, _VP]),
    "mla_prefill_chunk": (_I32, [_PD, _PC, _VP, _I32, _VP, _VP, _VP, _VP]),
    "mla_project_query": (_I32, [_PD, _I32, _I32, _VP, _VP, _VP, _VP, _I32, _VP, _VP, _VP]),
    "mla_decompress_kv": (_I32, [_PD, _PC, _I32, _VP, _VP, _VP, _VP, _VP, _VP]),
    "mla_prefill_unabsorbed": (_I32, [_PD, _PC, _I32, _VP, _VP, _VP, _I32, _VP, _VP, _VP, _VP, _VP, _VP]),
    "mla_prefill_unabsorbed_supported": (_I32, [_PD]),
    "mla_kv_append_workspace_bytes": (ctypes.c_size_t, [_PD, _I32, _I32]),
    "mla_kv_append": (_I32, [_PD, _PC, _I32, _VP, _VP, _VP, _VP, _VP, _I32, _F32, _VP, ctypes.c_size_t, _VP]),
    "mla_kv_append_noalloc": (_I32, [_PD, _PC, _I32, _VP, _VP, _VP, _VP, _VP, _I32, _F32, _VP]),
    "mla_verify_rows": (_I32, [_PC, _VP, _I32, _VP, _VP, _VP, _VP]),
    "mla_quantize_rows_fp8": (_I32, [_PD, _VP, ctypes.c_int64, _VP, _VP]),
    "mla_precompose_query": (_I32, [_PD, _I32, _VP, _VP, _VP, _VP, _VP]),
    "mla_precompose_out": (_I32, [_PD, _I32, _VP, _VP, _VP, _VP]),
    "mla_absorb_query_precomposed_workspace_bytes": (ctypes.c_size_t, [_PD, _I32, _I32]),
    "mla_absorb_query_precomposed": (_I32, [_PD, _I32, _VP, _VP, _VP, _I32, _VP, _VP, ctypes.c_size_t, _VP]),
    "mla_out_proj_fused_workspace_bytes": (ctypes.c_size_t, [_PD, _I32, _I32]),
    "mla_out_proj_fused": (_I32, [_PD, _I32, _VP, _VP, _I32, _VP, _VP, ctypes.c_size_t, _VP]),
    "mla_output_projection_workspace_bytes": (ctypes.c_size_t, [_PD, _I32, _I32]),
    "mla_output_projection": (_I32, [_PD, _I32, _VP, _VP, _I32, _VP, _VP, ctypes.c_size_t, _VP]),
}


def library() -> ctypes.CDLL:
    """Load libmla.so (built in-tree by mla_latent_kv_31_amd.build).  Raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m mla_latent_kv_31_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _addr(x) -> int | None:
    """Device address of a tensor argument (None -> NULL)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        if not x.is_cuda:
            raise ValueError("libmla takes device tensors; got a host tensor")
        if not x.is_contiguous():
            raise ValueError("libmla takes contiguous tensors")
        return x.data_ptr()
    raise TypeError(f"cannot pass {type(x).__name__} as a device pointer")


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, what: str) -> None:
    if status != MLA_OK:
        msg = library().mla_status_str(status).decode()
        raise MlaError(status, f"{what}: {msg}")


def dims(n_heads, d_c, d_r, d_k, d_v, dtype=MLA_BF16, rope_base=10000.0, sm_scale=0.0, flags=0) -> MlaDims:
    return MlaDims(n_heads, d_c, d_r, d_k, d_v, rope_base, sm_scale, dtype, flags)


def cache(pool, page_table, seq_lens, batch=None, page_size=None, max_pages=None, num_pages=None) -> MlaCache:
    """Describe a paged cache.  Sizes default to the tensor shapes (pool [P, page, W],
    page_table [B, max_pages])."""
    if batch is None:
        batch = page_table.shape[0]
    if max_pages is None:
        max_pages = page_table.shape[1]
    if page_size is None:
        page_size = pool.shape[1]
    if num_pages is None:
        num_pages = pool.shape[0]
    return MlaCache(_addr(pool), _addr(page_table), _addr(seq_lens), batch, page_size, max_pages, num_pages)


def mla_status_str(status: int) -> str:
    return library().mla_status_str(status).decode()


def mla_decode_num_splits(max_len: int, split_tokens: int) -> int:
    return library().mla_decode_num_splits(max_len, split_tokens)


def mla_decode_uses_mfma(d: MlaDims, c: MlaCache, split_tokens: int) -> bool:
    return bool(library().mla_decode_uses_mfma(ctypes.byref(d), ctypes.byref(c), split_tokens))


def mla_prefill_uses_mfma(d: MlaDims, c: MlaCache) -> bool:
    return bool(library().mla_prefill_uses_mfma(ctypes.byref(d), ctypes.byref(c)))


def mla_absorb_query(d: MlaDims, q_c, q_r, w_uk, pos, rows: int, q_hat, stream=None) -> None:
    _check(library().mla_absorb_query(ctypes.byref(d), _addr(q_c), _addr(q_r), _addr(w_uk), _addr(pos), rows,
                                      _addr(q_hat), _stream(stream)), "mla_absorb_query")


def mla_partials_lse_offset(d: MlaDims, slots: int) -> int:
    return int(library().mla_partials_lse_offset(ctypes.byref(d), slots))


def mla_partials_bytes(d: MlaDims, slots: int) -> int:
    return int(library().mla_partials_bytes(ctypes.byref(d), slots))


def mla_decode_workspace_bytes(d: MlaDims, c: MlaCache, max_len: int, split_tokens: int) -> int:
    return int(library().mla_decode_workspace_bytes(ctypes.byref(d), ctypes.byref(c), max_len, split_tokens))


def mla_decode_partial(d: MlaDims, c: MlaCache, q_hat, max_len: int, split_tokens: int, workspace,
                       workspace_bytes: int, stream=None) -> None:
    _check(library().mla_decode_partial(ctypes.byref(d), ctypes.byref(c), _addr(q_hat), max_len, split_tokens,
                                        _addr(workspace), workspace_bytes, _stream(stream)), "mla_decode_partial")


def mla_combine(d: MlaDims, batch: int, n_splits: int, workspace, workspace_bytes: int, z, lse=None,
                stream=None) -> None:
    _check(library().mla_combine(ctypes.byref(d), batch, n_splits, _addr(workspace), workspace_bytes, _addr(z),
                                 _addr(lse), _stream(stream)), "mla_combine")


def mla_balanced_num_slots(batch: int, n_units: int) -> int:
    return library().mla_balanced_num_slots(batch, n_units)


def mla_decode_balanced_workspace_bytes(d: MlaDims, c: MlaCache, n_units: int) -> int:
    return int(library().mla_decode_balanced_workspace_bytes(ctypes.byref(d), ctypes.byref(c), n_units))


def mla_decode_partial_balanced(d: MlaDims, c: MlaCache, q_hat, n_units: int, workspace, workspace_bytes: int,
                                stream=None) -> None:
    _check(library().mla_decode_partial_balanced(ctypes.byref(d), ctypes.byref(c), _addr(q_hat), n_units,
                                                 _addr(workspace), workspace_bytes, _stream(stream)),
           "mla_decode_partial_balanced")


def mla_combine_balanced(d: MlaDims, c: MlaCache, n_units: int, workspace, workspace_bytes: int, z, lse=None,
                         stream=None) -> None:
    _check(library().mla_combine_balanced(ctypes.byref(d), ctypes.byref(c), n_units, _addr(workspace),
                                          workspace_bytes, _addr(z), _addr(lse), _stream(stream)),
           "mla_combine_balanced")


def mla_decode_partial_grouped(d: MlaDims, c: MlaCache, q_hat, n_units: int, row_group: int, workspace,
                               workspace_bytes: int, stream=None) -> None:
    _check(library().mla_decode_partial_grouped(ctypes.byref(d), ctypes.byref(c), _addr(q_hat), n_units, row_group,
                                                _addr(workspace), workspace_bytes, _stream(stream)),
           "mla_decode_partial_grouped")


def mla_combine_grouped(d: MlaDims, c: MlaCache, n_units: int, row_group: int, workspace, workspace_bytes: int, z,
                        lse=None, stream=None) -> None:
    _check(library().mla_combine_grouped(ctypes.byref(d), ctypes.byref(c), n_units, row_group, _addr(workspace),
                                         workspace_bytes, _addr(z), _addr(lse), _stream(stream)),
           "mla_combine_grouped")


def mla_out_proj(d: MlaDims, z, w_uv, rows: int, out, stream=None) -> None:
    _check(library().mla_out_proj(ctypes.byref(d), _addr(z), _addr(w_uv), rows, _addr(out), _stream(stream)),
           "mla_out_proj")


def mla_combine_out_proj_supported(d: MlaDims) -> bool:
    return bool(library().mla_combine_out_proj_supported(ctypes.byref(d)))


def mla_combine_out_proj(d: MlaDims, batch: int, n_splits: int, workspace, workspace_bytes: int, w_uv, out,
                         lse=None, stream=None) -> None:
    _check(library().mla_combine_out_proj(ctypes.byref(d), batch, n_splits, _addr(workspace), workspace_bytes,
                                          _addr(w_uv), _addr(out), _addr(lse), _stream(stream)),
           "mla_combine_out_proj")


def mla_combine_out_proj_balanced(d: MlaDims, c: MlaCache, n_units: int, workspace, workspace_bytes: int, w_uv, out,
                                  lse=None, stream=None) -> None:
    _check(library().mla_combine_out_proj_balanced(ctypes.byref(d), ctypes.byref(c), n_units, _addr(workspace),
                                                   workspace_bytes, _addr(w_uv), _addr(out), _addr(lse),
                                                   _stream(stream)), "mla_combine_out_proj_balanced")


def mla_combine_out_proj_grouped(d: MlaDims, c: MlaCache, n_units: int, row_group: int, workspace,
                                 workspace_bytes: int, w_uv, out, lse=None, stream=None) -> None:
    _check(library().mla_combine_out_proj_grouped(ctypes.byref(d), ctypes.byref(c), n_units, row_group,
                                                  _addr(workspace), workspace_bytes, _addr(w_uv), _addr(out),
                                                  _addr(lse), _stream(stream)), "mla_combine_out_proj_grouped")


def mla_prefill_chunk(d: MlaDims, c: MlaCache, q_hat, q_len: int, q_start, z, lse=None, stream=None) -> None:
    _check(library().mla_prefill_chunk(ctypes.byref(d), ctypes.byref(c), _addr(q_hat), q_len, _addr(q_start),
                                       _addr(z), _addr(lse), _stream(stream)), "mla_prefill_chunk")


def mla_project_query(d: MlaDims, d_model: int, d_cq: int, h, w_dq, w_uq, w_qr, rows: int, q_c, q_r,
                      stream=None) -> None:
    _check(library().mla_project_query(ctypes.byref(d), d_model, d_cq, _addr(h), _addr(w_dq), _addr(w_uq),
                                       _addr(w_qr), rows, _addr(q_c), _addr(q_r), _stream(stream)),
           "mla_project_query")


def mla_decompress_kv(d: MlaDims, c: MlaCache, max_len: int, w_uk, w_uv, k, v, k_r, stream=None) -> None:
    _check(library().mla_decompress_kv(ctypes.byref(d), ctypes.byref(c), max_len, _addr(w_uk), _addr(w_uv),
                                       _addr(k), _addr(v), _addr(k_r), _stream(stream)), "mla_decompress_kv")


def mla_prefill_unabsorbed(d: MlaDims, c: MlaCache, max_len: int, q_c, q_r, q_start, q_len: int, k, v, k_r, out,
                           lse=None, stream=None) -> None:
    _check(library().mla_prefill_unabsorbed(ctypes.byref(d), ctypes.byref(c), max_len, _addr(q_c), _addr(q_r),
                                            _addr(q_start), q_len, _addr(k), _addr(v), _addr(k_r), _addr(out),
                                            _addr(lse), _stream(stream)), "mla_prefill_unabsorbed")


def mla_prefill_unabsorbed_supported(d: MlaDims) -> bool:
    return bool(library().mla_prefill_unabsorbed_supported(ctypes.byref(d)))


def mla_precompose_query(d: MlaDims, d_cq: int, w_uq, w_uk, w_qr, w_qcat, stream=None) -> None:
    _check(library().mla_precompose_query(ctypes.byref(d), d_cq, _addr(w_uq), _addr(w_uk), _addr(w_qr),
                                          _addr(w_qcat), _stream(stream)), "mla_precompose_query")


def mla_precompose_out(d: MlaDims, d_model: int, w_uv, w_o, w_uvo, stream=None) -> None:
    _check(library().mla_precompose_out(ctypes.byref(d), d_model, _addr(w_uv), _addr(w_o), _addr(w_uvo),
                                        _stream(stream)), "mla_precompose_out")


def mla_absorb_query_precomposed_workspace_bytes(d: MlaDims, d_cq: int, rows: int) -> int:
    return int(library().mla_absorb_query_precomposed_workspace_bytes(ctypes.byref(d), d_cq, rows))


def mla_absorb_query_precomposed(d: MlaDims, d_cq: int, c_q, w_qcat, pos, rows: int, q_hat, workspace,
                                 workspace_bytes: int, stream=None) -> None:
    _check(library().mla_absorb_query_precomposed(ctypes.byref(d), d_cq, _addr(c_q), _addr(w_qcat), _addr(pos), rows,
                                                  _addr(q_hat), _addr(workspace), workspace_bytes, _stream(stream)),
           "mla_absorb_query_precomposed")


def mla_out_proj_fused_workspace_bytes(d: MlaDims, d_model: int, rows: int) -> int:
    return int(library().mla_out_proj_fused_workspace_bytes(ctypes.byref(d), d_model, rows))


def mla_out_proj_fused(d: MlaDims, d_model: int, z, w_uvo, rows: int, out, workspace, workspace_bytes: int,
                       stream=None) -> None:
    _check(library().mla_out_proj_fused(ctypes.byref(d), d_model, _addr(z), _addr(w_uvo), rows, _addr(out),
                                        _addr(workspace), workspace_bytes, _stream(stream)), "mla_out_proj_fused")


def mla_output_projection_workspace_bytes(d: MlaDims, d_model: int, rows: int) -> int:
    return int(library().mla_output_projection_workspace_bytes(ctypes.byref(d), d_model, rows))


def mla_output_projection(d: MlaDims, d_model: int, o, w_o, rows: int, out, workspace, workspace_bytes: int,
                          stream=None) -> None:
    _check(library().mla_output_projection(ctypes.byref(d), d_model, _addr(o), _addr(w_o), rows, _addr(out),
                                           _addr(workspace), workspace_bytes, _stream(stream)), "mla_output_projection")


def mla_quantize_rows_fp8(d: MlaDims, src, rows: int, dst, stream=None) -> None:
    _check(library().mla_quantize_rows_fp8(ctypes.byref(d), _addr(src), rows, _addr(dst), _stream(stream)),
           "mla_quantize_rows_fp8")


def mla_verify_rows(c: MlaCache, q_start, q_len: int, row_table, row_lens, row_pos=None, stream=None) -> None:
    _check(library().mla_verify_rows(ctypes.byref(c), _addr(q_start), q_len, _addr(row_table), _addr(row_lens),
                                     _addr(row_pos), _stream(stream)), "mla_verify_rows")


def mla_kv_append_workspace_bytes(d: MlaDims, d_model: int, rows: int) -> int:
    return int(library().mla_kv_append_workspace_bytes(ctypes.byref(d), d_model, rows))


def mla_kv_append(d: MlaDims, c: MlaCache, d_model: int, h, w_dkv, w_kr, seq_ids, positions, rows: int,
                  rms_eps: float = 0.0, workspace=None, workspace_bytes: int = 0, stream=None) -> None:
    _check(library().mla_kv_append(ctypes.byref(d), ctypes.byref(c), d_model, _addr(h), _addr(w_dkv), _addr(w_kr),
                                   _addr(seq_ids), _addr(positions), rows, rms_eps, _addr(workspace),
                                   workspace_bytes, _stream(stream)),
           "mla_kv_append")


def mla_kv_append_noalloc(d: MlaDims, c: MlaCache, d_model: int, h, w_dkv, w_kr, seq_ids, positions, rows: int,
                          rms_eps: float = 0.0, stream=None) -> None:
    _check(library().mla_kv_append_noalloc(ctypes.byref(d), ctypes.byref(c), d_model, _addr(h), _addr(w_dkv),
                                           _addr(w_kr), _addr(seq_ids), _addr(positions), rows, rms_eps,
                                           _stream(stream)),
           "mla_kv_append_noalloc")
