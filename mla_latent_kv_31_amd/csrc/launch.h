// Host-side launchers behind the C ABI.  Arguments are already validated by api.hip;
// each launcher returns the HIP status of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla.h"

namespace mla {

struct Dims {
  int H, dc, dr, dk, dv;
  float rope_base, sm_scale;
  int dtype;
  __host__ __device__ int W() const { return dc + dr; }
};

struct Cache {
  const void* pool;
  const int32_t* page_table;
  const int32_t* seq_lens;
  int batch, page_size, max_pages, num_pages;
};

// ---- dimension-generic kernels (any sizes within the documented limits; fp32 or bf16)
constexpr int kGenericMaxDc = 1024;   // latent width handled by the generic decode/combine
constexpr int kGenericMaxRow = 2048;  // d_c + d_r
constexpr int kGenericMaxDk = 1024;

// ---- bf16 MFMA decode for the DeepSeek-V3 shape (128 heads, d_c 512, d_r 64, 32-token tiles).
// split_tokens == 0 asks about the balanced split.
bool decode_mfma_supported(const Dims& d, const Cache& c, int split_tokens);
hipError_t launch_decode_mfma(const Dims& d, const Cache& c, const void* q_hat, int n_splits, int split_tokens,
                              float* o_part, float* lse_part, hipStream_t s, bool fp8 = false);
// balanced split over n_units units with row groups of `group` rows (schedule.h; 1: plain split)
hipError_t launch_decode_mfma_balanced(const Dims& d, const Cache& c, const void* q_hat, int n_units, int group,
                                       float* o_part, float* lse_part, hipStream_t s, bool fp8 = false);
// chunked prefill on the same kernel: one workgroup per query row over its causal key range
bool prefill_mfma_supported(const Dims& d, const Cache& c);
hipError_t launch_prefill_mfma(const Dims& d, const Cache& c, const void* q_hat, int q_len, const int32_t* q_start,
                               float* z, float* lse, hipStream_t s, bool fp8 = false);

// ---- bf16 MFMA per-head projections (d_c 512, d_k = d_v = 128) and the vectorised combine
bool proj_mfma_supported(const Dims& d);
hipError_t launch_absorb_mfma(const Dims& d, const void* q_c, const void* q_r, const void* w_uk, const int32_t* pos,
                              int rows, void* q_hat, hipStream_t s);
hipError_t launch_out_proj_mfma(const Dims& d, const float* z, const void* w_uv, int rows, float* out,
                                hipStream_t s);
bool combine_fast_supported(const Dims& d, int n_splits);
hipError_t launch_combine_fast(const Dims& d, int batch, int n_splits, const float* o_part, const float* lse_part,
                               float* z, float* lse, hipStream_t s);
hipError_t launch_combine_fast_balanced(const Dims& d, const Cache& c, int n_units, int group, const float* o_part,
                                        const float* lse_part, float* z, float* lse, hipStream_t s);
// split-K merge fused with the value projection (proj_mfma.hip; proj_mfma_supported shapes): c is the
// cache of the balanced split (S = n_units, row groups of `group`), or NULL for the fixed split
// (S = n_splits)
hipError_t launch_combine_out_proj(const Dims& d, const Cache* c, int batch, int S, int group, const float* o_part,
                                   const float* lse_part, const void* w_uv, float* out, float* lse, hipStream_t s);

hipError_t launch_absorb_generic(const Dims& d, const void* q_c, const void* q_r, const void* w_uk,
                                 const int32_t* pos, int rows, void* q_hat, hipStream_t s);
hipError_t launch_decode_generic(const Dims& d, const Cache& c, const void* q_hat, int n_splits,
                                 int split_tokens, float* o_part, float* lse_part, hipStream_t s);
hipError_t launch_prefill_generic(const Dims& d, const Cache& c, const void* q_hat, int q_len,
                                  const int32_t* q_start, float* z, float* lse, hipStream_t s);
hipError_t launch_combine_generic(const Dims& d, int batch, int n_splits, const float* o_part,
                                  const float* lse_part, float* z, float* lse, hipStream_t s);
hipError_t launch_decode_generic_balanced(const Dims& d, const Cache& c, const void* q_hat, int n_units, int group,
                                          float* o_part, float* lse_part, hipStream_t s);
hipError_t launch_combine_generic_balanced(const Dims& d, const Cache& c, int n_units, int group,
                                           const float* o_part, const float* lse_part, float* z, float* lse,
                                           hipStream_t s);
hipError_t launch_out_proj_generic(const Dims& d, const float* z, const void* w_uv, int rows, float* out,
                                   hipStream_t s);
hipError_t launch_project_query(const Dims& d, int d_model, int d_cq, const void* h, const void* w_dq,
                                const void* w_uq, const void* w_qr, int rows, void* q_c, void* q_r,
                                hipStream_t s);
// ---- unabsorbed chunked prefill for the DeepSeek-V3 shape (bf16, 128 heads, 512 / 64 / 128)
bool prefill_unabsorbed_supported(const Dims& d);
hipError_t launch_decompress_kv(const Dims& d, const Cache& c, int max_len, const void* w_uk, const void* w_uv,
                                void* k_out, void* v_out, void* kr_out, hipStream_t s);
hipError_t launch_attend_unabsorbed(const Dims& d, const Cache& c, int max_len, const void* q_c, const void* q_r,
                                    const int32_t* q_start, int q_len, const void* k, const void* v, const void* kr,
                                    float* out, float* lse, hipStream_t s);

// ---- bf16 MFMA cache write for the DeepSeek-V3 latent shape (d_c 512, d_r 64, d_model % 256 == 0)
bool kv_append_mfma_supported(const Dims& d, int d_model);
size_t kv_append_mfma_workspace(int d_model, int rows);
hipError_t launch_kv_append_mfma(const Dims& d, const Cache& c, int d_model, const void* h, const void* w_dkv,
                                 const void* w_kr, const int32_t* seq_ids, const int32_t* positions, int rows,
                                 float rms_eps, float* workspace, hipStream_t s, bool fp8 = false);
// The allocation-free variant's fixed scratch (kv_append_mfma.hip): its device address on the
// current device (looked up once per device).
constexpr size_t kNoAllocScratchBytes = MLA_NOALLOC_SCRATCH_BYTES;
hipError_t kv_append_noalloc_scratch(float** ptr);
hipError_t launch_kv_append(const Dims& d, const Cache& c, int d_model, const void* h, const void* w_dkv,
                            const void* w_kr, const int32_t* seq_ids, const int32_t* positions, int rows,
                            float rms_eps, hipStream_t s);

// bf16 cache rows [rows, 576] -> FP8 cache rows [rows, 656 bytes] (fp8_quantize.hip).
hipError_t launch_quantize_rows_fp8(const void* src, int64_t rows, void* dst, hipStream_t stream);

// Precomposed weights (precomposed.hip).
bool precomposed_supported(const Dims& d);
size_t absorb_precomposed_workspace(const Dims& d, int d_cq, int rows);
size_t out_fused_workspace(const Dims& d, int d_model, int rows);
size_t output_projection_workspace(const Dims& d, int d_model, int rows);
hipError_t launch_precompose_query(const Dims& d, int d_cq, const void* w_uq, const void* w_uk, const void* w_qr,
                                   void* w_qcat, hipStream_t s);
hipError_t launch_precompose_out(const Dims& d, int d_model, const void* w_uv, const void* w_o, void* w_uvo,
                                 hipStream_t s);
hipError_t launch_absorb_precomposed(const Dims& d, int d_cq, const void* c_q, const void* w_qcat, const int32_t* pos,
                                     int rows, void* q_hat, float* workspace, hipStream_t s);
hipError_t launch_out_fused(const Dims& d, int d_model, const float* z, const void* w_uvo, int rows, float* out,
                            float* workspace, hipStream_t s);
hipError_t launch_output_projection(const Dims& d, int d_model, const float* o, const void* w_o, int rows, float* out,
                                    float* workspace, hipStream_t s);

// Multi-token verify rows for the decode path (verify_rows.hip).
hipError_t launch_verify_rows(const Cache& c, const int32_t* q_start, int q_len, int32_t* row_table,
                              int32_t* row_lens, int32_t* row_pos, hipStream_t stream);

}  // namespace mla
