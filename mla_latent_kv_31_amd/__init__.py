"""MI355X-native weight-absorbed MLA over a latent cache.

The computation lives in libmla.so (hand-written HIP for gfx950, C ABI in
include/mla.h).  This package is its Python binding: the functions below have
the names and argument order of the C entry points and only marshal arguments.
"""

from ._lib import (  # noqa: F401
    LIB_PATH,
    MLA_BALANCED_MAX_UNITS,
    MLA_BALANCED_SEG_COST,
    MLA_BALANCED_TILE,
    MLA_BF16,
    MLA_ERR_ALIGN,
    MLA_ERR_DTYPE,
    MLA_ERR_HIP,
    MLA_ERR_NULL,
    MLA_ERR_SHAPE,
    MLA_ERR_UNSUPPORTED,
    MLA_F32,
    MLA_FLAG_FORCE_GENERIC,
    MLA_OK,
    MlaCache,
    MlaDims,
    MlaError,
    cache,
    dims,
    library,
    mla_absorb_query,
    mla_balanced_num_slots,
    mla_combine,
    mla_combine_balanced,
    mla_decode_num_splits,
    mla_decode_partial,
    mla_decode_partial_balanced,
    mla_decode_uses_mfma,
    mla_decompress_kv,
    mla_kv_append,
    mla_kv_append_workspace_bytes,
    mla_out_proj,
    mla_prefill_chunk,
    mla_prefill_uses_mfma,
    mla_prefill_unabsorbed,
    mla_prefill_unabsorbed_supported,
    mla_project_query,
    mla_status_str,
)
