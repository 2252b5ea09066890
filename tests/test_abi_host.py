"""C-ABI checks that need no GPU: the library loads, exports every declared symbol, and
rejects bad arguments on the host before any HIP call (no compute call is made here)."""

import ctypes
import os
import re
import subprocess

import pytest

import mla_latent_kv_31_amd as M
from mla_latent_kv_31_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")

# Fake, 16-byte aligned device addresses: validation never dereferences them, and every call
# below fails validation (or has an empty size) before anything is launched.
A = 0x7F0000000000
B_ = A + 0x100000
U = A + 4  # misaligned


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(mla_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 10, names
    lib = M.library()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in mla.h but not exported"
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (mla_\w+)", out))
    assert set(names) <= exported
    assert set(_lib._SIGNATURES) == set(names), "binding signatures and header disagree"


def test_status_strings_and_splits():
    for s in range(8):
        assert M.mla_status_str(s).startswith("MLA_")
    assert M.mla_decode_num_splits(131072, 512) == 256
    assert M.mla_decode_num_splits(4096, 256) == 16
    assert M.mla_decode_num_splits(4097, 256) == 17
    assert M.mla_decode_num_splits(0, 64) == 1
    assert M.mla_decode_num_splits(10, 0) == -1


def _dims(**kw):
    base = dict(n_heads=128, d_c=512, d_r=64, d_k=128, d_v=128, dtype=M.MLA_BF16)
    base.update(kw)
    return M.dims(**base)


def _cache(**kw):
    base = dict(pool=A, page_table=A, seq_lens=A, batch=4, page_size=64, max_pages=2048, num_pages=8192)
    base.update(kw)
    return M.MlaCache(base["pool"], base["page_table"], base["seq_lens"], base["batch"], base["page_size"],
                      base["max_pages"], base["num_pages"])


def _status(fn, *args):
    return getattr(M.library(), fn)(*args)


def _absorb(d, q_c=A, q_r=A, w=A, pos=A, rows=1, q_hat=B_):
    return _status("mla_absorb_query", ctypes.byref(d) if d is not None else None, q_c, q_r, w, pos, rows, q_hat, None)


BIG = 1 << 40  # a workspace size that passes every size check


def _decode(d, c, q_hat=A, max_len=131072, split=512, ws=B_, nbytes=BIG):
    return _status("mla_decode_partial", ctypes.byref(d), ctypes.byref(c) if c is not None else None, q_hat,
                   max_len, split, ws, nbytes, None)


def test_absorb_validation():
    assert _absorb(None) == M.MLA_ERR_NULL
    assert _absorb(_dims(dtype=7)) == M.MLA_ERR_DTYPE
    assert _absorb(_dims(d_r=3)) == M.MLA_ERR_SHAPE
    assert _absorb(_dims(n_heads=0)) == M.MLA_ERR_SHAPE
    assert _absorb(_dims(d_c=-1)) == M.MLA_ERR_SHAPE
    assert _absorb(_dims(sm_scale=-1.0)) == M.MLA_ERR_SHAPE
    assert _absorb(_dims(rope_base=0.0)) == M.MLA_ERR_SHAPE
    assert _absorb(_dims(d_c=4096)) == M.MLA_ERR_UNSUPPORTED
    assert _absorb(_dims(), q_c=None) == M.MLA_ERR_NULL
    assert _absorb(_dims(), q_hat=None) == M.MLA_ERR_NULL
    assert _absorb(_dims(), w=U) == M.MLA_ERR_ALIGN
    assert _absorb(_dims(), rows=-1) == M.MLA_ERR_SHAPE
    assert _absorb(_dims(), rows=0) == M.MLA_OK  # empty input: nothing to launch
    assert _absorb(_dims(d_r=0), q_r=None, rows=0) == M.MLA_OK


def test_decode_validation():
    d = _dims()
    assert _decode(d, None) == M.MLA_ERR_NULL
    assert _decode(d, _cache(pool=0)) == M.MLA_ERR_NULL
    assert _decode(d, _cache(page_table=U)) == M.MLA_ERR_ALIGN
    assert _decode(d, _cache(page_size=0)) == M.MLA_ERR_SHAPE
    assert _decode(d, _cache(), split=100) == M.MLA_ERR_SHAPE      # not a multiple of the page size
    assert _decode(d, _cache(), split=0) == M.MLA_ERR_SHAPE
    assert _decode(d, _cache(), max_len=2048 * 64 + 1) == M.MLA_ERR_SHAPE  # beyond the page table
    assert _decode(d, _cache(), max_len=-1) == M.MLA_ERR_SHAPE
    assert _decode(d, _cache(), ws=U) == M.MLA_ERR_ALIGN
    assert _decode(d, _cache(), ws=None) == M.MLA_ERR_NULL
    assert _decode(d, _cache(batch=0)) == M.MLA_OK               # empty batch
    assert _decode(d, _cache(batch=70000)) == M.MLA_ERR_UNSUPPORTED


def test_other_entry_points_validation():
    lib = M.library()
    d = _dims()
    c = _cache()
    assert lib.mla_combine(ctypes.byref(d), 4, 0, A, BIG, A, None, None) == M.MLA_ERR_SHAPE
    assert lib.mla_combine(ctypes.byref(d), 4, 256, A, BIG, None, None, None) == M.MLA_ERR_NULL
    assert lib.mla_combine(ctypes.byref(d), 4, 256, A, BIG, A, U, None) == M.MLA_ERR_ALIGN
    assert lib.mla_combine(ctypes.byref(d), 4, 256, None, BIG, A, None, None) == M.MLA_ERR_NULL
    assert lib.mla_combine(ctypes.byref(d), 0, 256, A, 0, A, None, None) == M.MLA_OK
    assert lib.mla_out_proj(ctypes.byref(d), A, None, 4, A, None) == M.MLA_ERR_NULL
    assert lib.mla_out_proj(ctypes.byref(d), A, A, -2, A, None) == M.MLA_ERR_SHAPE
    assert lib.mla_out_proj(ctypes.byref(d), A, A, 0, A, None) == M.MLA_OK
    assert lib.mla_prefill_chunk(ctypes.byref(d), ctypes.byref(c), A, -1, A, A, None, None) == M.MLA_ERR_SHAPE
    assert lib.mla_prefill_chunk(ctypes.byref(d), ctypes.byref(c), A, 512, None, A, None, None) == M.MLA_ERR_NULL
    assert lib.mla_prefill_chunk(ctypes.byref(d), ctypes.byref(c), A, 0, A, A, None, None) == M.MLA_OK
    assert lib.mla_project_query(ctypes.byref(d), 0, 3, A, A, A, A, 1, A, A, None) == M.MLA_ERR_SHAPE
    assert lib.mla_project_query(ctypes.byref(d), 8, 3, A, A, A, None, 1, A, A, None) == M.MLA_ERR_NULL
    assert lib.mla_kv_append(ctypes.byref(d), ctypes.byref(c), 8, A, A, A, A, None, 1, 0.0, None, 0,
                             None) == M.MLA_ERR_NULL
    assert lib.mla_kv_append(ctypes.byref(d), ctypes.byref(c), 8, A, A, A, A, A, 0, 0.0, None, 0, None) == M.MLA_OK


def test_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    d = _dims()
    x = torch.zeros(16)
    with pytest.raises(ValueError):
        M.mla_out_proj(d, x, x, 1, x, stream=0)


def test_balanced_validation():
    lib = M.library()
    d = _dims()
    assert M.mla_balanced_num_slots(64, 256) == 319
    assert M.mla_balanced_num_slots(0, 256) == 0
    assert M.mla_balanced_num_slots(4, 0) == -1
    assert M.mla_balanced_num_slots(4, M.MLA_BALANCED_MAX_UNITS + 1) == -1

    def dec(c, n=256, q=A, ws=B_, nbytes=BIG):
        return lib.mla_decode_partial_balanced(ctypes.byref(d), ctypes.byref(c), q, n, ws, nbytes, None)

    def comb(c, n=256, z=A, lse=None):
        return lib.mla_combine_balanced(ctypes.byref(d), ctypes.byref(c), n, A, BIG, z, lse, None)

    assert dec(_cache(), n=0) == M.MLA_ERR_SHAPE
    assert dec(_cache(), n=M.MLA_BALANCED_MAX_UNITS + 1) == M.MLA_ERR_UNSUPPORTED
    assert dec(_cache(), q=None) == M.MLA_ERR_NULL
    assert dec(_cache(), ws=U) == M.MLA_ERR_ALIGN
    assert dec(_cache(seq_lens=0)) == M.MLA_ERR_NULL
    assert dec(_cache(batch=0)) == M.MLA_OK
    # device-side cost sums must stay inside int32
    assert dec(_cache(batch=65535, max_pages=1 << 16, page_size=64)) == M.MLA_ERR_UNSUPPORTED
    assert comb(_cache(), n=0) == M.MLA_ERR_SHAPE
    assert comb(_cache(), z=None) == M.MLA_ERR_NULL
    assert comb(_cache(), lse=U) == M.MLA_ERR_ALIGN
    assert comb(_cache(batch=0)) == M.MLA_OK


def test_grouped_validation():
    """Row groups must be >= 1 and divide both the batch and the unit count; the workspace is the
    plain balanced split's."""
    lib = M.library()
    d = _dims()

    def dec(c, n=256, g=4, nbytes=BIG):
        return lib.mla_decode_partial_grouped(ctypes.byref(d), ctypes.byref(c), A, n, g, B_, nbytes, None)

    def comb(c, n=256, g=4, nbytes=BIG):
        return lib.mla_combine_grouped(ctypes.byref(d), ctypes.byref(c), n, g, A, nbytes, A, None, None)

    for fn in (dec, comb):
        assert fn(_cache(), g=0) == M.MLA_ERR_SHAPE
        assert fn(_cache(), g=-4) == M.MLA_ERR_SHAPE
        assert fn(_cache(batch=6), g=4) == M.MLA_ERR_SHAPE      # 4 does not divide the batch
        assert fn(_cache(batch=8), n=254, g=4) == M.MLA_ERR_SHAPE  # nor the units
        assert fn(_cache(), n=0) == M.MLA_ERR_SHAPE
        assert fn(_cache(batch=0)) == M.MLA_OK
    need = M.mla_decode_balanced_workspace_bytes(d, _cache(), 256)
    assert dec(_cache(), nbytes=need - 1) == M.MLA_ERR_WORKSPACE
    assert comb(_cache(), nbytes=need - 1) == M.MLA_ERR_WORKSPACE


def test_kv_append_workspace_validation():
    """The MFMA cache write needs a caller workspace of the advertised size; other shapes need none."""
    lib = M.library()
    d = _dims()
    need = M.mla_kv_append_workspace_bytes(d, 4096, 64)
    assert need == 16 * 64 * 576 * 4  # 16 K splits for a 64-row decode batch
    assert M.mla_kv_append_workspace_bytes(d, 4096, 1024) == 2 * 1024 * 576 * 4
    assert M.mla_kv_append_workspace_bytes(d, 4000, 64) == 0  # d_model not a multiple of 256: generic
    assert M.mla_kv_append_workspace_bytes(_dims(dtype=M.MLA_F32), 4096, 64) == 0
    assert M.mla_kv_append_workspace_bytes(_dims(flags=M.MLA_FLAG_FORCE_GENERIC), 4096, 64) == 0
    assert M.mla_kv_append_workspace_bytes(d, 4096, 0) == 0

    def call(ws=A, nbytes=need, rows=64):
        return lib.mla_kv_append(ctypes.byref(d), ctypes.byref(_cache()), 4096, A, A, A, A, A, rows, 1e-6, ws,
                                 nbytes, None)

    assert call(ws=None) == M.MLA_ERR_NULL
    assert call(nbytes=need - 4) == M.MLA_ERR_WORKSPACE
    assert call(ws=U) == M.MLA_ERR_ALIGN
    assert call(rows=0, ws=None, nbytes=0) == M.MLA_OK


def test_kv_append_noalloc_validation():
    """The allocation-free cache write refuses, before any launch, a call whose split-K partial
    products would not fit its fixed scratch: rows > 3640 at any d_model (at most 1,820 rows take
    more than one split, and one split of 3,641 rows of 576 floats exceeds 8 MiB)."""
    lib = M.library()
    d = _dims()
    assert M.MLA_NOALLOC_SCRATCH_BYTES == 8 << 20

    def call(rows, d_model=4096, dd=d, ptr=A):
        return lib.mla_kv_append_noalloc(ctypes.byref(dd), ctypes.byref(_cache()), d_model, ptr, A, A, A, A, rows,
                                         1e-6, None)

    for dm in (4096, 7168, 16384):
        for rows in (1, 64, 1024, 1821, 3640):
            assert M.mla_kv_append_workspace_bytes(d, dm, rows) <= M.MLA_NOALLOC_SCRATCH_BYTES, (dm, rows)
        assert M.mla_kv_append_workspace_bytes(d, dm, 3641) > M.MLA_NOALLOC_SCRATCH_BYTES
        assert call(3641, dm) == M.MLA_ERR_WORKSPACE
    assert call(0) == M.MLA_OK
    assert call(-1) == M.MLA_ERR_SHAPE
    assert call(64, ptr=None) == M.MLA_ERR_NULL
    # fp8 rows need the MFMA path; f32 takes the generic kernel, which uses no scratch
    assert call(64, d_model=4000, dd=_dims(flags=M.MLA_FLAG_CACHE_FP8)) == M.MLA_ERR_UNSUPPORTED


def test_verify_rows_validation():
    lib = M.library()
    c = _cache()

    def call(cache=c, q_start=A, q_len=4, table=B_, lens=B_, pos=None):
        return lib.mla_verify_rows(ctypes.byref(cache) if cache is not None else None, q_start, q_len, table, lens,
                                   pos, None)

    assert call(cache=None) == M.MLA_ERR_NULL
    assert call(q_start=None) == M.MLA_ERR_NULL
    assert call(table=None) == M.MLA_ERR_NULL
    assert call(lens=U) == M.MLA_ERR_ALIGN
    assert call(pos=U) == M.MLA_ERR_ALIGN
    assert call(q_len=-1) == M.MLA_ERR_SHAPE
    assert call(cache=_cache(batch=20000), q_len=4) == M.MLA_ERR_UNSUPPORTED  # 80,000 rows
    assert call(q_len=0) == M.MLA_OK
    assert call(cache=_cache(batch=0)) == M.MLA_OK


def test_fp8_flag_validation():
    """FP8 cache rows: the quantiser's argument checks, and the flag refused where no FP8 kernel
    exists (generic kernels forced, other shapes, the unabsorbed prefill), all before any launch."""
    lib = M.library()
    d = _dims()
    assert M.MLA_FP8_ROW_BYTES == 656
    assert lib.mla_quantize_rows_fp8(ctypes.byref(d), None, 4, B_, None) == M.MLA_ERR_NULL
    assert lib.mla_quantize_rows_fp8(ctypes.byref(d), A, 4, U, None) == M.MLA_ERR_ALIGN
    assert lib.mla_quantize_rows_fp8(ctypes.byref(d), A, -1, B_, None) == M.MLA_ERR_SHAPE
    assert lib.mla_quantize_rows_fp8(ctypes.byref(_dims(d_c=256)), A, 4, B_, None) == M.MLA_ERR_UNSUPPORTED
    assert lib.mla_quantize_rows_fp8(ctypes.byref(_dims(dtype=M.MLA_F32)), A, 4, B_, None) == M.MLA_ERR_UNSUPPORTED
    assert lib.mla_quantize_rows_fp8(ctypes.byref(d), A, 0, B_, None) == M.MLA_OK
    assert lib.mla_quantize_rows_fp8(ctypes.byref(d), A, 4 * 0x7FFFFFFF + 1, B_, None) == M.MLA_ERR_UNSUPPORTED
    f8g = _dims(flags=M.MLA_FLAG_CACHE_FP8 | M.MLA_FLAG_FORCE_GENERIC)
    f8s = _dims(flags=M.MLA_FLAG_CACHE_FP8, n_heads=64)
    c = _cache()
    for dd in (f8g, f8s):
        assert _decode(dd, c) == M.MLA_ERR_UNSUPPORTED
        assert lib.mla_decode_partial_balanced(ctypes.byref(dd), ctypes.byref(c), A, 256, B_, BIG,
                                               None) == M.MLA_ERR_UNSUPPORTED
        assert lib.mla_prefill_chunk(ctypes.byref(dd), ctypes.byref(c), A, 4, A, B_, None,
                                     None) == M.MLA_ERR_UNSUPPORTED
    f8 = _dims(flags=M.MLA_FLAG_CACHE_FP8)
    assert lib.mla_decompress_kv(ctypes.byref(f8), ctypes.byref(c), 64, A, A, B_, B_, B_, None) == M.MLA_ERR_UNSUPPORTED
    assert lib.mla_kv_append(ctypes.byref(_dims(flags=M.MLA_FLAG_CACHE_FP8 | M.MLA_FLAG_FORCE_GENERIC)),
                             ctypes.byref(c), 4096, A, A, A, A, A, 4, 1e-6, A, 1 << 20, None) == M.MLA_ERR_UNSUPPORTED


def test_split_k_workspace_sizes_and_rejection():
    """The split-K workspace: its advertised size is the partials' closed form (o_part float
    [slots, H, d_c], then lse_part float [slots, H] at a 256-byte boundary), and every decode or
    combine call given one byte less returns MLA_ERR_WORKSPACE before anything is launched."""
    lib = M.library()
    d = _dims()
    H, dc = 128, 512

    def closed(slots):
        o = slots * H * dc * 4
        return -(-o // 256) * 256 + slots * H * 4

    assert M.mla_partials_bytes(d, 3) == closed(3)
    assert M.mla_partials_lse_offset(d, 3) == 3 * H * dc * 4
    odd = _dims(n_heads=3, d_c=5)
    assert M.mla_partials_lse_offset(odd, 1) == 256 and M.mla_partials_bytes(odd, 1) == 256 + 12
    assert M.mla_partials_bytes(d, -1) == 0
    c = _cache()  # batch 4
    need = M.mla_decode_workspace_bytes(d, c, 131072, 512)
    assert need == closed(4 * 256)
    assert M.mla_decode_workspace_bytes(d, c, 131072, 0) == 0
    assert M.mla_decode_workspace_bytes(d, c, 4097, 256) == closed(4 * 17)
    need_b = M.mla_decode_balanced_workspace_bytes(d, c, 256)
    assert need_b == closed(256 + 4 - 1)
    assert M.mla_decode_balanced_workspace_bytes(d, c, 0) == 0
    assert _decode(d, c, nbytes=need - 1) == M.MLA_ERR_WORKSPACE
    assert lib.mla_combine(ctypes.byref(d), 4, 256, A, need - 1, A, None, None) == M.MLA_ERR_WORKSPACE
    assert lib.mla_decode_partial_balanced(ctypes.byref(d), ctypes.byref(c), A, 256, A, need_b - 1,
                                           None) == M.MLA_ERR_WORKSPACE
    assert lib.mla_combine_balanced(ctypes.byref(d), ctypes.byref(c), 256, A, need_b - 1, A, None,
                                    None) == M.MLA_ERR_WORKSPACE
    # an empty batch needs no partial bytes
    assert _decode(d, _cache(batch=0), nbytes=0) == M.MLA_OK
    assert M.mla_decode_balanced_workspace_bytes(d, _cache(batch=0), 256) == 0


def test_combine_out_proj_validation():
    """The fused merge + value projection: supported only for the bf16 V3 shape, and rejected on
    the host like the two calls it replaces (sizes, NULLs, alignment, short workspace)."""
    lib = M.library()
    d = _dims()
    c = _cache()
    assert M.mla_combine_out_proj_supported(d)
    assert not M.mla_combine_out_proj_supported(_dims(dtype=M.MLA_F32))
    assert not M.mla_combine_out_proj_supported(_dims(d_c=256))
    assert not M.mla_combine_out_proj_supported(_dims(flags=M.MLA_FLAG_FORCE_GENERIC))

    def fixed(dd=d, batch=4, n=256, ws=A, nbytes=BIG, w=A, out=A, lse=None):
        return lib.mla_combine_out_proj(ctypes.byref(dd), batch, n, ws, nbytes, w, out, lse, None)

    def grouped(cc=c, n=256, g=1, ws=A, nbytes=BIG, w=A, out=A, lse=None, dd=d):
        return lib.mla_combine_out_proj_grouped(ctypes.byref(dd), ctypes.byref(cc), n, g, ws, nbytes, w, out, lse,
                                                None)

    assert fixed(n=0) == M.MLA_ERR_SHAPE
    assert fixed(batch=-1) == M.MLA_ERR_SHAPE
    assert fixed(batch=70000) == M.MLA_ERR_UNSUPPORTED
    assert fixed(dd=_dims(dtype=M.MLA_F32)) == M.MLA_ERR_UNSUPPORTED
    assert fixed(w=None) == M.MLA_ERR_NULL
    assert fixed(out=U) == M.MLA_ERR_ALIGN
    assert fixed(lse=U) == M.MLA_ERR_ALIGN
    assert fixed(ws=None) == M.MLA_ERR_NULL
    need = M.mla_partials_bytes(d, 4 * 256)
    assert fixed(nbytes=need - 1) == M.MLA_ERR_WORKSPACE
    assert fixed(batch=0, nbytes=0) == M.MLA_OK
    assert grouped(n=0) == M.MLA_ERR_SHAPE
    assert grouped(g=3) == M.MLA_ERR_SHAPE              # does not divide batch 4
    assert grouped(cc=_cache(page_size=0)) == M.MLA_ERR_SHAPE
    assert grouped(dd=_dims(d_v=64)) == M.MLA_ERR_UNSUPPORTED
    assert grouped(w=None) == M.MLA_ERR_NULL
    need = M.mla_decode_balanced_workspace_bytes(d, c, 256)
    assert grouped(nbytes=need - 1) == M.MLA_ERR_WORKSPACE
    assert lib.mla_combine_out_proj_balanced(ctypes.byref(d), ctypes.byref(c), 256, A, need - 1, A, A, None,
                                             None) == M.MLA_ERR_WORKSPACE
    assert grouped(cc=_cache(batch=0), nbytes=0) == M.MLA_OK
