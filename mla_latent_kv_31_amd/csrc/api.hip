// C ABI of libmla: argument validation and kernel dispatch.  Every check here runs on the host
// before any HIP call, so a rejected call has no side effects.

#include <math.h>
#include <stdint.h>

#include "launch.h"
#include "mla.h"

namespace mla {
namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

mla_status check_dims(const mla_dims* dims, Dims* out) {
  if (!dims) return MLA_ERR_NULL;
  if (dims->dtype != MLA_F32 && dims->dtype != MLA_BF16) return MLA_ERR_DTYPE;
  if (dims->n_heads < 1 || dims->d_c < 1 || dims->d_r < 0 || (dims->d_r & 1) || dims->d_k < 1 || dims->d_v < 1)
    return MLA_ERR_SHAPE;
  if (dims->n_heads > 65535) return MLA_ERR_UNSUPPORTED;
  if (!(dims->sm_scale >= 0.f) || !isfinite(dims->sm_scale)) return MLA_ERR_SHAPE;
  if (dims->d_r > 0 && !(dims->rope_base > 0.f && isfinite(dims->rope_base))) return MLA_ERR_SHAPE;
  if (dims->d_c > kGenericMaxDc || dims->d_c + dims->d_r > kGenericMaxRow || dims->d_k > kGenericMaxDk ||
      dims->d_v > 4096)
    return MLA_ERR_UNSUPPORTED;
  out->H = dims->n_heads;
  out->dc = dims->d_c;
  out->dr = dims->d_r;
  out->dk = dims->d_k;
  out->dv = dims->d_v;
  out->rope_base = dims->rope_base;
  out->sm_scale = dims->sm_scale > 0.f ? dims->sm_scale : 1.0f / sqrtf(float(dims->d_k + dims->d_r));
  out->dtype = dims->dtype;
  return MLA_OK;
}

mla_status check_cache(const mla_cache* cache, Cache* out) {
  if (!cache) return MLA_ERR_NULL;
  if (!cache->pool || !cache->page_table || !cache->seq_lens) return MLA_ERR_NULL;
  if (!aligned16(cache->pool) || !aligned16(cache->page_table) || !aligned16(cache->seq_lens)) return MLA_ERR_ALIGN;
  if (cache->batch < 0 || cache->page_size < 1 || cache->max_pages < 1 || cache->num_pages < 1)
    return MLA_ERR_SHAPE;
  if (cache->batch > 65535) return MLA_ERR_UNSUPPORTED;
  out->pool = cache->pool;
  out->page_table = cache->page_table;
  out->seq_lens = cache->seq_lens;
  out->batch = cache->batch;
  out->page_size = cache->page_size;
  out->max_pages = cache->max_pages;
  out->num_pages = cache->num_pages;
  return MLA_OK;
}

// The balanced split counts costs in int32 on the device: keep the total well inside its range.
mla_status check_balanced(const Cache& c, int n_units) {
  if (n_units < 1) return MLA_ERR_SHAPE;
  if (n_units > MLA_BALANCED_MAX_UNITS) return MLA_ERR_UNSUPPORTED;
  const int64_t per_seq = int64_t(c.max_pages) * c.page_size / MLA_BALANCED_TILE + 1 + MLA_BALANCED_SEG_COST;
  if (int64_t(c.batch) * per_seq >= (int64_t(1) << 31) - (int64_t(1) << 12)) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

// Row groups of the balanced split: G consecutive rows per group, G dividing batch and n_units.
mla_status check_group(const Cache& c, int n_units, int group) {
  if (group < 1 || c.batch % group != 0 || n_units % group != 0) return MLA_ERR_SHAPE;
  return MLA_OK;
}

mla_status ptr_ok(const void* p) {
  if (!p) return MLA_ERR_NULL;
  return aligned16(p) ? MLA_OK : MLA_ERR_ALIGN;
}

mla_status hip_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

// Split-K workspace layout: o_part float [slots, H, d_c] at byte 0, lse_part float [slots, H] at the
// o_part size rounded up to 256 bytes.
size_t partials_lse_offset(const Dims& d, int64_t slots) {
  const size_t o = size_t(slots) * size_t(d.H) * size_t(d.dc) * sizeof(float);
  return (o + 255) & ~size_t(255);
}
size_t partials_bytes(const Dims& d, int64_t slots) {
  return partials_lse_offset(d, slots) + size_t(slots) * size_t(d.H) * sizeof(float);
}

// The partials of a checked workspace.
struct Partials {
  float* o;
  float* lse;
};
mla_status check_workspace(const Dims& d, int64_t slots, const void* ws, size_t ws_bytes, Partials* out) {
  if (!ws) return MLA_ERR_NULL;
  if (!aligned16(ws)) return MLA_ERR_ALIGN;
  if (ws_bytes < partials_bytes(d, slots)) return MLA_ERR_WORKSPACE;
  unsigned char* base = static_cast<unsigned char*>(const_cast<void*>(ws));
  out->o = reinterpret_cast<float*>(base);
  out->lse = reinterpret_cast<float*>(base + partials_lse_offset(d, slots));
  return MLA_OK;
}

bool cache_fp8(const mla_dims* dims) { return (dims->flags & MLA_FLAG_CACHE_FP8) != 0; }
bool generic_forced(const mla_dims* dims) { return (dims->flags & MLA_FLAG_FORCE_GENERIC) != 0; }

#define MLA_TRY(expr)                 \
  do {                                \
    mla_status _st = (expr);          \
    if (_st != MLA_OK) return _st;    \
  } while (0)

}  // namespace
}  // namespace mla

using namespace mla;

extern "C" {

const char* mla_status_str(mla_status s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL: return "MLA_ERR_NULL: a required pointer is NULL";
    case MLA_ERR_SHAPE: return "MLA_ERR_SHAPE: a size or dimension is out of range or inconsistent";
    case MLA_ERR_DTYPE: return "MLA_ERR_DTYPE: unknown dtype code";
    case MLA_ERR_ALIGN: return "MLA_ERR_ALIGN: a device pointer is not 16-byte aligned";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: well-formed but beyond the implemented limits";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: a HIP runtime call or kernel launch failed";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: the workspace is smaller than the call needs";
  }
  return "unknown mla_status";
}

int32_t mla_decode_num_splits(int32_t max_len, int32_t split_tokens) {
  if (split_tokens < 1 || max_len < 0) return -1;
  const int64_t s = (int64_t(max_len) + split_tokens - 1) / split_tokens;
  return int32_t(s < 1 ? 1 : s);
}

int32_t mla_decode_uses_mfma(const mla_dims* dims, const mla_cache* cache, int32_t split_tokens) {
  Dims d;
  Cache c;
  if (check_dims(dims, &d) != MLA_OK || check_cache(cache, &c) != MLA_OK) return 0;
  if (dims->flags & MLA_FLAG_FORCE_GENERIC) return 0;
  return decode_mfma_supported(d, c, split_tokens) ? 1 : 0;
}

int32_t mla_prefill_uses_mfma(const mla_dims* dims, const mla_cache* cache) {
  Dims d;
  Cache c;
  if (check_dims(dims, &d) != MLA_OK || check_cache(cache, &c) != MLA_OK) return 0;
  if (dims->flags & MLA_FLAG_FORCE_GENERIC) return 0;
  return prefill_mfma_supported(d, c) ? 1 : 0;
}

mla_status mla_absorb_query(const mla_dims* dims, const void* q_c, const void* q_r, const void* w_uk,
                            const int32_t* pos, int32_t rows, void* q_hat, void* stream) {
  Dims d;
  MLA_TRY(check_dims(dims, &d));
  if (rows < 0) return MLA_ERR_SHAPE;
  MLA_TRY(ptr_ok(q_c));
  if (d.dr > 0) MLA_TRY(ptr_ok(q_r));
  MLA_TRY(ptr_ok(w_uk));
  MLA_TRY(ptr_ok(pos));
  MLA_TRY(ptr_ok(q_hat));
  if (rows == 0) return MLA_OK;
  if (!(dims->flags & MLA_FLAG_FORCE_GENERIC) && proj_mfma_supported(d) && rows <= 65535 * 64)
    return hip_status(launch_absorb_mfma(d, q_c, q_r, w_uk, pos, rows, q_hat, (hipStream_t)stream));
  return hip_status(launch_absorb_generic(d, q_c, q_r, w_uk, pos, rows, q_hat, (hipStream_t)stream));
}

size_t mla_partials_lse_offset(const mla_dims* dims, int32_t slots) {
  Dims d;
  if (check_dims(dims, &d) != MLA_OK || slots < 0) return 0;
  return partials_lse_offset(d, slots);
}

size_t mla_partials_bytes(const mla_dims* dims, int32_t slots) {
  Dims d;
  if (check_dims(dims, &d) != MLA_OK || slots < 0) return 0;
  return partials_bytes(d, slots);
}

size_t mla_decode_workspace_bytes(const mla_dims* dims, const mla_cache* cache, int32_t max_len,
                                  int32_t split_tokens) {
  Dims d;
  Cache c;
  if (check_dims(dims, &d) != MLA_OK || check_cache(cache, &c) != MLA_OK) return 0;
  if (split_tokens < 1 || max_len < 0) return 0;
  return partials_bytes(d, int64_t(c.batch) * mla_decode_num_splits(max_len, split_tokens));
}

mla_status mla_decode_partial(const mla_dims* dims, const mla_cache* cache, const void* q_hat, int32_t max_len,
                              int32_t split_tokens, void* workspace, size_t workspace_bytes, void* stream) {
  Dims d;
  Cache c;
  Partials p;
  MLA_TRY(check_dims(dims, &d));
  MLA_TRY(check_cache(cache, &c));
  MLA_TRY(ptr_ok(q_hat));
  if (split_tokens < 1 || split_tokens % c.page_size != 0) return MLA_ERR_SHAPE;
  if (max_len < 0 || int64_t(max_len) > int64_t(c.max_pages) * c.page_size) return MLA_ERR_SHAPE;
  const int S = mla_decode_num_splits(max_len, split_tokens);
  MLA_TRY(check_workspace(d, int64_t(c.batch) * S, workspace, workspace_bytes, &p));
  const bool mfma = !generic_forced(dims) && decode_mfma_supported(d, c, split_tokens);
  if (cache_fp8(dims) && !mfma) return MLA_ERR_UNSUPPORTED;
  if (c.batch == 0) return MLA_OK;
  if (mfma)
    return hip_status(launch_decode_mfma(d, c, q_hat, S, split_tokens, p.o, p.lse, (hipStream_t)stream,
                                         cache_fp8(dims)));
  return hip_status(launch_decode_generic(d, c, q_hat, S, split_tokens, p.o, p.lse, (hipStream_t)stream));
}

mla_status mla_combine(const mla_dims* dims, int32_t batch, int32_t n_splits, const void* workspace,
                       size_t workspace_bytes, float* z, float* lse, void* stream) {
  Dims d;
  Partials p;
  MLA_TRY(check_dims(dims, &d));
  if (batch < 0 || n_splits < 1) return MLA_ERR_SHAPE;
  if (batch > 65535) return MLA_ERR_UNSUPPORTED;
  MLA_TRY(check_workspace(d, int64_t(batch) * n_splits, workspace, workspace_bytes, &p));
  MLA_TRY(ptr_ok(z));
  if (lse && !(reinterpret_cast<uintptr_t>(lse) % 16 == 0)) return MLA_ERR_ALIGN;
  if (batch == 0) return MLA_OK;
  if (!(dims->flags & MLA_FLAG_FORCE_GENERIC) && combine_fast_supported(d, n_splits))
    return hip_status(launch_combine_fast(d, batch, n_splits, p.o, p.lse, z, lse, (hipStream_t)stream));
  return hip_status(launch_combine_generic(d, batch, n_splits, p.o, p.lse, z, lse, (hipStream_t)stream));
}

int32_t mla_balanced_num_slots(int32_t batch, int32_t n_units) {
  if (batch < 0 || n_units < 1 || n_units > MLA_BALANCED_MAX_UNITS) return -1;
  return batch == 0 ? 0 : n_units + batch - 1;
}

size_t mla_decode_balanced_workspace_bytes(const mla_dims* dims, const mla_cache* cache, int32_t n_units) {
  Dims d;
  Cache c;
  if (check_dims(dims, &d) != MLA_OK || check_cache(cache, &c) != MLA_OK) return 0;
  const int32_t slots = mla_balanced_num_slots(c.batch, n_units);
  return slots < 0 ? 0 : partials_bytes(d, slots);
}

mla_status mla_decode_partial_grouped(const mla_dims* dims, const mla_cache* cache, const void* q_hat,
                                      int32_t n_units, int32_t row_group, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  Dims d;
  Cache c;
  Partials p;
  MLA_TRY(check_dims(dims, &d));
  MLA_TRY(check_cache(cache, &c));
  MLA_TRY(check_balanced(c, n_units));
  MLA_TRY(check_group(c, n_units, row_group));
  MLA_TRY(ptr_ok(q_hat));
  MLA_TRY(check_workspace(d, mla_balanced_num_slots(c.batch, n_units), workspace, workspace_bytes, &p));
  const bool mfma = !generic_forced(dims) && decode_mfma_supported(d, c, 0);
  if (cache_fp8(dims) && !mfma) return MLA_ERR_UNSUPPORTED;
  if (c.batch == 0) return MLA_OK;
  if (mfma)
    return hip_status(launch_decode_mfma_balanced(d, c, q_hat, n_units, row_group, p.o, p.lse, (hipStream_t)stream,
                                                  cache_fp8(dims)));
  return hip_status(launch_decode_generic_balanced(d, c, q_hat, n_units, row_group, p.o, p.lse, (hipStream_t)stream));
}

mla_status mla_decode_partial_balanced(const mla_dims* dims, const mla_cache* cache, const void* q_hat,
                                       int32_t n_units, void* workspace, size_t workspace_bytes, void* stream) {
  return mla_decode_partial_grouped(dims, cache, q_hat, n_units, 1, workspace, workspace_bytes, stream);
}

mla_status mla_combine_grouped(const mla_dims* dims, const mla_cache* cache, int32_t n_units, int32_t row_group,
                               const void* workspace, size_t workspace_bytes, float* z, float* lse, void* stream) {
  Dims d;
  Cache c;
  Partials p;
  MLA_TRY(check_dims(dims, &d));
  MLA_TRY(check_cache(cache, &c));
  MLA_TRY(check_balanced(c, n_units));
  MLA_TRY(check_group(c, n_units, row_group));
  MLA_TRY(check_workspace(d, mla_balanced_num_slots(c.batch, n_units), workspace, workspace_bytes, &p));
  MLA_TRY(ptr_ok(z));
  if (lse && !(reinterpret_cast<uintptr_t>(lse) % 16 == 0)) return MLA_ERR_ALIGN;
  if (c.batch == 0) return MLA_OK;
  if (!(dims->flags & MLA_FLAG_FORCE_GENERIC) && combine_fast_supported(d, n_units))
    return hip_status(
        launch_combine_fast_balanced(d, c, n_units, row_group, p.o, p.lse, z, lse, (hipStream_t)stream));
  return hip_status(
      launch_combine_generic_balanced(d, c, n_units, row_group, p.o, p.lse, z, lse, (hipStream_t)stream));
}

mla_status mla_combine_balanced(const mla_dims* dims, const mla_cache* cache, int32_t n_units,
                                const void* workspace, size_t workspace_bytes, float* z, float* lse, void* stream) {
  return mla_combine_grouped(dims, cache, n_units, 1, workspace, workspace_bytes, z, lse, stream);
}

mla_status mla_out_proj(const mla_dims* dims, const float* z, const void* w_uv, int32_t rows, float* out,
                        void* stream) {
  Dims d;
  MLA_TRY(check_dims(dims, &d));
  if (rows < 0) return MLA_ERR_SHAPE;
  if (rows > 65535) return MLA_ERR_UNSUPPORTED;
  MLA_TRY(ptr_ok(z));
  MLA_TRY(ptr_ok(w_uv));
  MLA_TRY(ptr_ok(out));
  if (rows == 0) return MLA_OK;
  if (!(dims->flags & MLA_FLAG_FORCE_GENERIC) && proj_mfma_supported(d))
    return hip_status(launch_out_proj_mfma(d, z, w_uv, rows, out, (hipStream_t)stream));
  return hip_status(launch_out_proj_generic(d, z, w_uv, rows, out, (hipStream_t)stream));
}

int32_t mla_combine_out_proj_supported(const mla_dims* dims) {
  Dims d;
  if (check_dims(dims, &d) != MLA_OK || generic_forced(dims)) return 0;
  return proj_mfma_supported(d) ? 1 : 0;
}

mla_status mla_combine_out_proj(const mla_dims* dims, int32_t batch, int32_t n_splits, const void* workspace,
                                size_t workspace_bytes, const void* w_uv, float* out, float* lse, void* stream) {
  Dims d;
  Partials p;
  MLA_TRY(check_dims(dims, &d));
  if (batch < 0 || n_splits < 1) return MLA_ERR_SHAPE;
  if (batch > 65535) return MLA_ERR_UNSUPPORTED;
  if (!mla_combine_out_proj_supported(dims)) return MLA_ERR_UNSUPPORTED;
  MLA_TRY(check_workspace(d, int64_t(batch) * n_splits, workspace, workspace_bytes, &p));
  MLA_TRY(ptr_ok(w_uv));
  MLA_TRY(ptr_ok(out));
  if (lse && !(reinterpret_cast<uintptr_t>(lse) % 16 == 0)) return MLA_ERR_ALIGN;
  if (batch == 0) return MLA_OK;
  return hip_status(
      launch_combine_out_proj(d, nullptr, batch, n_splits, 1, p.o, p.lse, w_uv, out, lse, (hipStream_t)stream));
}

mla_status mla_combine_out_proj_grouped(const mla_dims* dims, const mla_cache* cache, int32_t n_units,
                                        int32_t row_group, const void* workspace, size_t workspace_bytes,
                                        const void* w_uv, float* out, float* lse, void* stream) {
  Dims d;
  Cache c;
  Partials p;
  MLA_TRY(check_dims(dims, &d));
  MLA_TRY(check_cache(cache, &c));
  MLA_TRY(check_balanced(c, n_units));
  MLA_TRY(check_group(c, n_units, row_group));
  if (!mla_combine_out_proj_supported(dims)) return MLA_ERR_UNSUPPORTED;
  MLA_TRY(check_workspace(d, mla_balanced_num_slots(c.batch, n_units), workspace, workspace_bytes, &p));
  MLA_TRY(ptr_ok(w_uv));
  MLA_TRY(ptr_ok(out));
  if (lse && !(reinterpret_cast<uintptr_t>(lse) % 16 == 0)) return MLA_ERR_ALIGN;
  if (c.batch == 0) return MLA_OK;
  return hip_status(launch_combine_out_proj(d, &c, c.batch, n_units, row_group, p.o, p.lse, w_uv, out, lse,
                                            (hipStream_t)stream));
}

mla_status mla_combine_out_proj_balanced(const mla_dims* dims, const mla_cache* cache, int32_t n_units,
                                         const void* workspace, size_t workspace_bytes, const void* w_uv, float* out,
                                         float* lse, void* stream) {
  return mla_combine_out_proj_grouped(dims, cache, n_units, 1, workspace, workspace_bytes, w_uv, out, lse, stream);
}

mla_status mla_prefill_chunk(const mla_dims* dims, const mla_cache* cache, const void* q_hat, int32_t q_len,
                             const int32_t* q_start, float* z, float* lse, void* stream) {
  Dims d;
  Cache c;
  MLA_TRY(check_dims(dims, &d));
  MLA_TRY(check_cache(cache, &c));
  if (q_len < 0) return MLA_ERR_SHAPE;
  MLA_TRY(ptr_ok(q_hat));
  MLA_TRY(ptr_ok(q_start));
  MLA_TRY(ptr_ok(z));
  if (lse && !(reinterpret_cast<uintptr_t>(lse) % 16 == 0)) return MLA_ERR_ALIGN;
  const bool mfma = !generic_forced(dims) && prefill_mfma_supported(d, c);
  if (cache_fp8(dims) && !mfma) return MLA_ERR_UNSUPPORTED;
  if (c.batch == 0 || q_len == 0) return MLA_OK;
  if (int64_t(c.batch) * q_len > (int64_t(1) << 31) - 1) return MLA_ERR_UNSUPPORTED;
  if (mfma)
    return hip_status(launch_prefill_mfma(d, c, q_hat, q_len, q_start, z, lse, (hipStream_t)stream, cache_fp8(dims)));
  return hip_status(launch_prefill_generic(d, c, q_hat, q_len, q_start, z, lse, (hipStream_t)stream));
}

mla_status mla_project_query(const mla_dims* dims, int32_t d_model, int32_t d_cq, const void* h, const void* w_dq,
                             const void* w_uq, const void* w_qr, int32_t rows, void* q_c, void* q_r, void* stream) {
  Dims d;
  MLA_TRY(check_dims(dims, &d));
  if (d_model < 1 || d_cq < 1 || rows < 0) return MLA_ERR_SHAPE;
  if (d_model + d_cq > 8192) return MLA_ERR_UNSUPPORTED;
  MLA_TRY(ptr_ok(h));
  MLA_TRY(ptr_ok(w_dq));
  MLA_TRY(ptr_ok(w_uq));
  MLA_TRY(ptr_ok(q_c));
  if (d.dr > 0) {
    MLA_TRY(ptr_ok(w_qr));
    MLA_TRY(ptr_ok(q_r));
  }
  if (rows == 0) return MLA_OK;
  return hip_status(launch_project_query(d, d_model, d_cq, h, w_dq, w_uq, w_qr, rows, q_c, q_r, (hipStream_t)stream));
}

int32_t mla_prefill_unabsorbed_supported(const mla_dims* dims) {
  Dims d;
  return check_dims(dims, &d) == MLA_OK && prefill_unabsorbed_supported(d) ? 1 : 0;
}

mla_status mla_decompress_kv(const mla_dims* dims, const mla_cache* cache, int32_t max_len, const void* w_uk,
                             const void* w_uv, void* k, void* v, void* k_r, void* stream) {
  Dims d;
  Cache c;
  MLA_TRY(check_dims(dims, &d));
  MLA_TRY(check_cache(cache, &c));
  if (!prefill_unabsorbed_supported(d) || cache_fp8(dims)) return MLA_ERR_UNSUPPORTED;
  if (max_len < 1) return MLA_ERR_SHAPE;
  if (int64_t(c.batch) * d.H * int64_t(max_len) * d.dk > (int64_t(1) << 40)) return MLA_ERR_UNSUPPORTED;
  MLA_TRY(ptr_ok(w_uk));
  MLA_TRY(ptr_ok(w_uv));
  MLA_TRY(ptr_ok(k));
  MLA_TRY(ptr_ok(v));
  MLA_TRY(ptr_ok(k_r));
  if (c.batch == 0) return MLA_OK;
  return hip_status(launch_decompress_kv(d, c, max_len, w_uk, w_uv, k, v, k_r, (hipStream_t)stream));
}

mla_status mla_prefill_unabsorbed(const mla_dims* dims, const mla_cache* cache, int32_t max_len, const void* q_c,
                                  const void* q_r, const int32_t* q_start, int32_t q_len, const void* k,
                                  const void* v, const void* k_r, float* out, float* lse, void* stream) {
  Dims d;
  Cache c;
  MLA_TRY(check_dims(dims, &d));
  MLA_TRY(check_cache(cache, &c));
  if (!prefill_unabsorbed_supported(d) || cache_fp8(dims)) return MLA_ERR_UNSUPPORTED;
  if (max_len < 1 || q_len < 0) return MLA_ERR_SHAPE;
  if (int64_t(c.batch) * d.H * int64_t(max_len) * d.dk > (int64_t(1) << 40)) return MLA_ERR_UNSUPPORTED;
  MLA_TRY(ptr_ok(q_c));
  MLA_TRY(ptr_ok(q_r));
  MLA_TRY(ptr_ok(q_start));
  MLA_TRY(ptr_ok(k));
  MLA_TRY(ptr_ok(v));
  MLA_TRY(ptr_ok(k_r));
  MLA_TRY(ptr_ok(out));
  if (lse && !(reinterpret_cast<uintptr_t>(lse) % 16 == 0)) return MLA_ERR_ALIGN;
  if (c.batch == 0 || q_len == 0) return MLA_OK;
  return hip_status(launch_attend_unabsorbed(d, c, max_len, q_c, q_r, q_start, q_len, k, v, k_r, out, lse,
                                             (hipStream_t)stream));
}

static bool kv_append_uses_mfma(const mla_dims* dims, const Dims& d, int32_t d_model) {
  return !(dims->flags & MLA_FLAG_FORCE_GENERIC) && kv_append_mfma_supported(d, d_model);
}

size_t mla_kv_append_workspace_bytes(const mla_dims* dims, int32_t d_model, int32_t rows) {
  Dims d;
  if (check_dims(dims, &d) != MLA_OK || d_model < 1 || rows < 1) return 0;
  return kv_append_uses_mfma(dims, d, d_model) ? kv_append_mfma_workspace(d_model, rows) : 0;
}

mla_status mla_kv_append(const mla_dims* dims, const mla_cache* cache, int32_t d_model, const void* h,
                         const void* w_dkv, const void* w_kr, const int32_t* seq_ids, const int32_t* positions,
                         int32_t rows, float rms_eps, float* workspace, size_t workspace_bytes, void* stream) {
  Dims d;
  Cache c;
  MLA_TRY(check_dims(dims, &d));
  MLA_TRY(check_cache(cache, &c));
  if (d_model < 1 || rows < 0 || !(rms_eps == rms_eps)) return MLA_ERR_SHAPE;
  const bool mfma = kv_append_uses_mfma(dims, d, d_model);
  if (cache_fp8(dims) && !mfma) return MLA_ERR_UNSUPPORTED;
  if (!mfma && d_model + d.dc + d.dr > 8192) return MLA_ERR_UNSUPPORTED;
  if (mfma && int64_t(rows) * d_model > (int64_t(1) << 31) - 1) return MLA_ERR_UNSUPPORTED;
  MLA_TRY(ptr_ok(h));
  MLA_TRY(ptr_ok(w_dkv));
  if (d.dr > 0) MLA_TRY(ptr_ok(w_kr));
  MLA_TRY(ptr_ok(seq_ids));
  MLA_TRY(ptr_ok(positions));
  if (rows == 0) return MLA_OK;
  if (mfma) {
    MLA_TRY(ptr_ok(workspace));
    if (workspace_bytes < kv_append_mfma_workspace(d_model, rows)) return MLA_ERR_WORKSPACE;
    return hip_status(launch_kv_append_mfma(d, c, d_model, h, w_dkv, w_kr, seq_ids, positions, rows, rms_eps,
                                            workspace, (hipStream_t)stream, cache_fp8(dims)));
  }
  return hip_status(
      launch_kv_append(d, c, d_model, h, w_dkv, w_kr, seq_ids, positions, rows, rms_eps, (hipStream_t)stream));
}

mla_status mla_kv_append_noalloc(const mla_dims* dims, const mla_cache* cache, int32_t d_model, const void* h,
                                 const void* w_dkv, const void* w_kr, const int32_t* seq_ids,
                                 const int32_t* positions, int32_t rows, float rms_eps, void* stream) {
  Dims d;
  Cache c;
  MLA_TRY(check_dims(dims, &d));
  MLA_TRY(check_cache(cache, &c));
  if (d_model < 1 || rows < 0 || !(rms_eps == rms_eps)) return MLA_ERR_SHAPE;
  const bool mfma = kv_append_uses_mfma(dims, d, d_model);
  if (cache_fp8(dims) && !mfma) return MLA_ERR_UNSUPPORTED;
  if (!mfma && d_model + d.dc + d.dr > 8192) return MLA_ERR_UNSUPPORTED;
  if (mfma && int64_t(rows) * d_model > (int64_t(1) << 31) - 1) return MLA_ERR_UNSUPPORTED;
  MLA_TRY(ptr_ok(h));
  MLA_TRY(ptr_ok(w_dkv));
  if (d.dr > 0) MLA_TRY(ptr_ok(w_kr));
  MLA_TRY(ptr_ok(seq_ids));
  MLA_TRY(ptr_ok(positions));
  if (rows == 0) return MLA_OK;
  if (mfma) {
    if (kv_append_mfma_workspace(d_model, rows) > kNoAllocScratchBytes) return MLA_ERR_WORKSPACE;
    float* scratch = nullptr;
    MLA_TRY(hip_status(kv_append_noalloc_scratch(&scratch)));
    return hip_status(launch_kv_append_mfma(d, c, d_model, h, w_dkv, w_kr, seq_ids, positions, rows, rms_eps,
                                            scratch, (hipStream_t)stream, cache_fp8(dims)));
  }
  return hip_status(
      launch_kv_append(d, c, d_model, h, w_dkv, w_kr, seq_ids, positions, rows, rms_eps, (hipStream_t)stream));
}

static bool precomposed_dims(const mla_dims* dims, Dims* d) {
  return check_dims(dims, d) == MLA_OK && precomposed_supported(*d);
}

mla_status mla_precompose_query(const mla_dims* dims, int32_t d_cq, const void* w_uq, const void* w_uk,
                                const void* w_qr, void* w_qcat, void* stream) {
  Dims d;
  MLA_TRY(check_dims(dims, &d));
  if (!precomposed_supported(d)) return MLA_ERR_UNSUPPORTED;
  if (d_cq < 64 || d_cq % 64 != 0) return MLA_ERR_SHAPE;
  MLA_TRY(ptr_ok(w_uq));
  MLA_TRY(ptr_ok(w_uk));
  MLA_TRY(ptr_ok(w_qr));
  MLA_TRY(ptr_ok(w_qcat));
  return hip_status(launch_precompose_query(d, d_cq, w_uq, w_uk, w_qr, w_qcat, (hipStream_t)stream));
}

mla_status mla_precompose_out(const mla_dims* dims, int32_t d_model, const void* w_uv, const void* w_o, void* w_uvo,
                              void* stream) {
  Dims d;
  MLA_TRY(check_dims(dims, &d));
  if (!precomposed_supported(d)) return MLA_ERR_UNSUPPORTED;
  if (d_model < 128 || d_model % 128 != 0) return MLA_ERR_SHAPE;
  if (d_model > 65536) return MLA_ERR_UNSUPPORTED;
  MLA_TRY(ptr_ok(w_uv));
  MLA_TRY(ptr_ok(w_o));
  MLA_TRY(ptr_ok(w_uvo));
  return hip_status(launch_precompose_out(d, d_model, w_uv, w_o, w_uvo, (hipStream_t)stream));
}

size_t mla_absorb_query_precomposed_workspace_bytes(const mla_dims* dims, int32_t d_cq, int32_t rows) {
  Dims d;
  if (!precomposed_dims(dims, &d) || d_cq < 64 || d_cq % 64 != 0 || rows < 1) return 0;
  return absorb_precomposed_workspace(d, d_cq, rows);
}

mla_status mla_absorb_query_precomposed(const mla_dims* dims, int32_t d_cq, const void* c_q, const void* w_qcat,
                                        const int32_t* pos, int32_t rows, void* q_hat, float* workspace,
                                        size_t workspace_bytes, void* stream) {
  Dims d;
  MLA_TRY(check_dims(dims, &d));
  if (!precomposed_supported(d)) return MLA_ERR_UNSUPPORTED;
  if (d_cq < 64 || d_cq % 64 != 0 || rows < 0) return MLA_ERR_SHAPE;
  if (int64_t(rows) > 65535 * 64) return MLA_ERR_UNSUPPORTED;
  MLA_TRY(ptr_ok(c_q));
  MLA_TRY(ptr_ok(w_qcat));
  MLA_TRY(ptr_ok(pos));
  MLA_TRY(ptr_ok(q_hat));
  if (rows == 0) return MLA_OK;
  MLA_TRY(ptr_ok(workspace));
  if (workspace_bytes < absorb_precomposed_workspace(d, d_cq, rows)) return MLA_ERR_WORKSPACE;
  return hip_status(launch_absorb_precomposed(d, d_cq, c_q, w_qcat, pos, rows, q_hat, workspace, (hipStream_t)stream));
}

size_t mla_out_proj_fused_workspace_bytes(const mla_dims* dims, int32_t d_model, int32_t rows) {
  Dims d;
  if (!precomposed_dims(dims, &d) || d_model < 128 || d_model % 128 != 0 || rows < 1) return 0;
  return out_fused_workspace(d, d_model, rows);
}

mla_status mla_out_proj_fused(const mla_dims* dims, int32_t d_model, const float* z, const void* w_uvo, int32_t rows,
                              float* out, float* workspace, size_t workspace_bytes, void* stream) {
  Dims d;
  MLA_TRY(check_dims(dims, &d));
  if (!precomposed_supported(d)) return MLA_ERR_UNSUPPORTED;
  if (d_model < 128 || d_model % 128 != 0 || rows < 0) return MLA_ERR_SHAPE;
  if (d_model > 65536 || int64_t(rows) > 65535 * 64) return MLA_ERR_UNSUPPORTED;
  MLA_TRY(ptr_ok(z));
  MLA_TRY(ptr_ok(w_uvo));
  MLA_TRY(ptr_ok(out));
  if (rows == 0) return MLA_OK;
  MLA_TRY(ptr_ok(workspace));
  if (workspace_bytes < out_fused_workspace(d, d_model, rows)) return MLA_ERR_WORKSPACE;
  return hip_status(launch_out_fused(d, d_model, z, w_uvo, rows, out, workspace, (hipStream_t)stream));
}

size_t mla_output_projection_workspace_bytes(const mla_dims* dims, int32_t d_model, int32_t rows) {
  Dims d;
  if (!precomposed_dims(dims, &d) || d_model < 128 || d_model % 128 != 0 || rows < 1) return 0;
  if ((int64_t(d.H) * d.dv) % 64 != 0) return 0;
  return output_projection_workspace(d, d_model, rows);
}

mla_status mla_output_projection(const mla_dims* dims, int32_t d_model, const float* o, const void* w_o, int32_t rows,
                                 float* out, float* workspace, size_t workspace_bytes, void* stream) {
  Dims d;
  MLA_TRY(check_dims(dims, &d));
  if (!precomposed_supported(d) || (int64_t(d.H) * d.dv) % 64 != 0) return MLA_ERR_UNSUPPORTED;
  if (d_model < 128 || d_model % 128 != 0 || rows < 0) return MLA_ERR_SHAPE;
  if (d_model > 65536 || int64_t(rows) > 65535 * 64) return MLA_ERR_UNSUPPORTED;
  MLA_TRY(ptr_ok(o));
  MLA_TRY(ptr_ok(w_o));
  MLA_TRY(ptr_ok(out));
  if (rows == 0) return MLA_OK;
  MLA_TRY(ptr_ok(workspace));
  if (workspace_bytes < output_projection_workspace(d, d_model, rows)) return MLA_ERR_WORKSPACE;
  return hip_status(launch_output_projection(d, d_model, o, w_o, rows, out, workspace, (hipStream_t)stream));
}

mla_status mla_quantize_rows_fp8(const mla_dims* dims, const void* src, int64_t rows, void* dst, void* stream) {
  Dims d;
  MLA_TRY(check_dims(dims, &d));
  if (d.dtype != MLA_BF16 || d.dc != 512 || d.dr != 64) return MLA_ERR_UNSUPPORTED;
  if (rows < 0) return MLA_ERR_SHAPE;
  if (rows > int64_t(4) * 0x7fffffff) return MLA_ERR_UNSUPPORTED;  // four rows per workgroup, 2^31 - 1 workgroups
  MLA_TRY(ptr_ok(src));
  MLA_TRY(ptr_ok(dst));
  if (rows == 0) return MLA_OK;
  return hip_status(launch_quantize_rows_fp8(src, rows, dst, (hipStream_t)stream));
}

mla_status mla_verify_rows(const mla_cache* cache, const int32_t* q_start, int32_t q_len, int32_t* row_table,
                           int32_t* row_lens, int32_t* row_pos, void* stream) {
  Cache c;
  MLA_TRY(check_cache(cache, &c));
  if (q_len < 0) return MLA_ERR_SHAPE;
  if (int64_t(c.batch) * q_len > 65535) return MLA_ERR_UNSUPPORTED;
  MLA_TRY(ptr_ok(q_start));
  MLA_TRY(ptr_ok(row_table));
  MLA_TRY(ptr_ok(row_lens));
  if (row_pos && !aligned16(row_pos)) return MLA_ERR_ALIGN;
  if (c.batch == 0 || q_len == 0) return MLA_OK;
  return hip_status(launch_verify_rows(c, q_start, q_len, row_table, row_lens, row_pos, (hipStream_t)stream));
}

}  // extern "C"
