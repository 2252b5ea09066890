/*
 * libmla -- weight-absorbed Multi-Head Latent Attention over a latent cache, for gfx950.
 *
 * Pages defining the operations (cited by title and section):
 *   [molayo] "Multi-Head Latent Attention (MLA)" (molayo1419.me)
 *   [ase]    "MLA의 계산: KV를 펼치지 않고 Attention하기" (ai-systems-engineering.com)
 *   [huny]   "DeepSeek Multi-Head Latent Attention(MLA) 아키텍처 해부 ..." (blog.huny.dev)
 *
 * Common rules for every entry point
 *   - Device pointers are plain device addresses owned by the caller.  The library allocates
 *     nothing, keeps no state between calls and retains no pointer after a call returns.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL selects the null stream).
 *     No call allocates, synchronises or enqueues a memset or copy: only kernel launches go
 *     on the stream, so any sequence of calls can be captured in a HIP graph and replayed.
 *   - Host-visible arguments are validated before anything is launched; a failed check returns
 *     an MLA_ERR_* code and touches no device memory.  A failed launch returns MLA_ERR_HIP.
 *     Faults during execution surface at the caller's next synchronisation.
 *   - Device-resident values (seq_lens, page_table, positions) are trusted: out-of-range
 *     values are undefined behaviour.  Cache slots past a sequence's length may hold any bits,
 *     NaN included; results never depend on them.
 *   - Every device pointer must be 16-byte aligned (MLA_ERR_ALIGN otherwise).
 *   - Outputs are overwritten, never accumulated into.  Entry points are thread-safe.
 *   - Tensors are dense row-major in the index order written next to them.
 *   - Values of type "dtype" are float32 (MLA_F32) or bfloat16 bit patterns (MLA_BF16) as
 *     selected by mla_dims.dtype; arithmetic accumulates in float32.
 *   - The absorbed query q_hat is float32 for MLA_F32 and IEEE binary16 for MLA_BF16: the score
 *     products run in binary16 on the bf16 path (the bf16 cache values convert to binary16
 *     exactly over the latents' range), whose 11 significant bits keep the score error of a
 *     576-long dot product well inside the bf16 output tolerance.  Its values must stay within
 *     +-65504 (scores of that size are far outside any softmax's useful range).
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,        /* a required pointer is NULL */
  MLA_ERR_SHAPE = 2,       /* a size or dimension is out of range or inconsistent */
  MLA_ERR_DTYPE = 3,       /* unknown dtype code */
  MLA_ERR_ALIGN = 4,       /* a device pointer is not 16-byte aligned */
  MLA_ERR_UNSUPPORTED = 5, /* well-formed but beyond what the kernels implement */
  MLA_ERR_HIP = 6,         /* a HIP runtime call or a kernel launch failed */
  MLA_ERR_WORKSPACE = 7    /* a caller-provided workspace is smaller than the call needs */
} mla_status;

typedef enum { MLA_F32 = 0, MLA_BF16 = 1 } mla_dtype;

/* Flags for mla_dims.flags. */
#define MLA_FLAG_FORCE_GENERIC 1 /* use the dimension-generic kernels even where a tuned one exists */
/* The cache pool holds FP8 rows (row N1; [huny] section 5, FP8 mixed-precision item: E4M3 on the
 * 512-wide latent with a per-token scale).  Row of MLA_FP8_ROW_BYTES bytes:
 *   bytes   0..511  E4M3 codes of c / 2^e (OCP 8-bit E4M3: bias 7, subnormals m * 2^-9, largest
 *                   finite 448; nearest-even), e the smallest integer with max|c| <= 448 * 2^e
 *   bytes 512..639  the 64 rotary values k^R, bf16, unchanged
 *   bytes 640..643  the scale 2^e as a float32;  bytes 644..655 zero
 * The cache then holds code value x 2^e, exact in bf16, and every kernel reads those values.
 * Honoured by mla_decode_partial(_balanced, _grouped), mla_prefill_chunk (through the MFMA kernels for
 * d_c 512, d_r 64, 128 heads) and mla_kv_append (its MFMA path); elsewhere, or for other shapes,
 * the calls return MLA_ERR_UNSUPPORTED.  Latent rows whose largest magnitude is below 2^-110 are
 * outside the supported range (their scale would leave the float32 normal range). */
#define MLA_FLAG_CACHE_FP8 2
#define MLA_FP8_ROW_BYTES 656

/* Model dimensions shared by every call.
 * Cached row of one token: [c^KV (d_c) | k^R (d_r)], k^R already rotated at its position and
 * shared by all heads ([huny] section 2, decoupled-RoPE principle; [ase] Fig. 1 caption). */
typedef struct {
  int32_t n_heads;  /* H */
  int32_t d_c;      /* latent width */
  int32_t d_r;      /* rotary width of the position query/key (even, may be 0) */
  int32_t d_k;      /* content query/key width per head */
  int32_t d_v;      /* value width per head */
  float rope_base;  /* RoPE base; inverse frequencies base^(-2i/d_r) on interleaved pairs */
  float sm_scale;   /* softmax scale; 0 selects 1/sqrt(d_k + d_r) ([ase] scale remark, Fig. 2) */
  int32_t dtype;    /* mla_dtype of queries, weights and cache rows (q_hat: see above) */
  int32_t flags;    /* MLA_FLAG_* */
} mla_dims;

/* A paged latent cache ([molayo] key concept 5: a page table holding latent rows).
 * Token t of sequence b lives at pool[page_table[b*max_pages + t/page_size]][t % page_size].
 * A contiguous cache is the identity page table. */
typedef struct {
  const void* pool;          /* device, dtype [num_pages, page_size, d_c + d_r] */
  const int32_t* page_table; /* device [batch, max_pages]; entries past a sequence's pages unused */
  const int32_t* seq_lens;   /* device [batch]; valid tokens per sequence, current token included */
  int32_t batch;
  int32_t page_size;
  int32_t max_pages;
  int32_t num_pages;
} mla_cache;

/* Human-readable name of a status code (static storage). */
const char* mla_status_str(mla_status s);

/* Absorbed query ([ase] "Key 투영을 Query 쪽으로 옮기기", Fig. 3 equation; [ase] Fig. 1 for the
 * rotated position query; [molayo] key concept 1):
 *   q_hat[r,h,:] = [ q_c[r,h,:] . W_UK[h]^T  |  RoPE_{pos[r]}(q_r[r,h,:]) ] * (sm_scale * log2(e))
 * The product with log2(e) makes later scores base-2 logits; lse outputs stay natural-log.
 *   q_c   device dtype [rows, H, d_k]
 *   q_r   device dtype [rows, H, d_r]   (unrotated; may be NULL when d_r == 0)
 *   w_uk  device dtype [H, d_c, d_k]
 *   pos   device int32 [rows]           absolute position of each query row
 *   q_hat device [rows, H, d_c + d_r]  (output; float32, or binary16 for MLA_BF16)             */
mla_status mla_absorb_query(const mla_dims* dims, const void* q_c, const void* q_r, const void* w_uk,
                            const int32_t* pos, int32_t rows, void* q_hat, void* stream);

/* Number of split-K chunks per sequence: ceil(max_len / split_tokens), at least 1. */
int32_t mla_decode_num_splits(int32_t max_len, int32_t split_tokens);

/* Nonzero when mla_decode_partial / mla_prefill_chunk take the MFMA kernels for these arguments
 * (split_tokens == 0 asks about mla_decode_partial_balanced). */
int32_t mla_decode_uses_mfma(const mla_dims* dims, const mla_cache* cache, int32_t split_tokens);
int32_t mla_prefill_uses_mfma(const mla_dims* dims, const mla_cache* cache);

/* Split-K workspace.  The split-K decode calls write one partial result per (segment, head) into a
 * caller-provided workspace that the combine calls then read.  A workspace of `slots` partial
 * slots holds
 *   o_part   float [slots, H, d_c]   at byte 0
 *   lse_part float [slots, H]        at byte mla_partials_lse_offset(dims, slots)
 *                                    (the o_part bytes rounded up to a multiple of 256)
 * and spans mla_partials_bytes(dims, slots) bytes.  Both return 0 for invalid arguments.
 * The split into pieces and the merge are not on the pages; they are an exact rewrite of the
 * one-pass softmax of [ase] Fig. 2 (see mla_combine).  A serving system sizes the workspace once
 * ([molayo] key concept 5: a page table of latents served by custom attention kernels). */
size_t mla_partials_lse_offset(const mla_dims* dims, int32_t slots);
size_t mla_partials_bytes(const mla_dims* dims, int32_t slots);

/* Workspace bytes mla_decode_partial needs for these arguments: mla_partials_bytes for
 * batch * mla_decode_num_splits(max_len, split_tokens) slots (0 for invalid arguments). */
size_t mla_decode_workspace_bytes(const mla_dims* dims, const mla_cache* cache, int32_t max_len,
                                  int32_t split_tokens);

/* Split-K decode over the latent cache, one query token per sequence (the newest, at position
 * seq_lens[b]-1).  Chunk i of sequence b covers tokens [i*split_tokens, (i+1)*split_tokens)
 * intersected with [0, seq_lens[b]).  For each chunk and head it writes the chunk-local softmax
 * result into slot b*S + i of the workspace ([ase] Fig. 2 scores over the 576-wide concatenation;
 * Fig. 4: the weighted latent z = a.C, the rotary part is never summed):
 *   o_part[b*S+i,h,:] = sum_t softmax_t(s) c_t  (normalised within the chunk)
 *   lse_part[b*S+i,h] = ln sum_t exp(s_t)        with s_t = q_hat . row_t / log2(e)
 * An empty chunk writes lse_part = -inf and may leave its o_part row untouched: the combine gives
 * it zero weight and never reads it.
 *   q_hat    device [batch, H, d_c + d_r]   (as written by mla_absorb_query)
 *   max_len  host bound >= every seq_lens[b]; sets S = mla_decode_num_splits(max_len, split_tokens)
 *   split_tokens  > 0 and a multiple of cache->page_size
 *   workspace      device, workspace_bytes long, 16-byte aligned
 *   workspace_bytes  MLA_ERR_WORKSPACE (before any launch) when below
 *                  mla_decode_workspace_bytes(dims, cache, max_len, split_tokens)              */
mla_status mla_decode_partial(const mla_dims* dims, const mla_cache* cache, const void* q_hat,
                              int32_t max_len, int32_t split_tokens, void* workspace, size_t workspace_bytes,
                              void* stream);

/* Log-sum-exp merge of split-K partials: LSE = ln sum_i exp(lse_i),
 * z = sum_i exp(lse_i - LSE) o_i.  Over any split this equals the single-pass softmax of
 * [ase] Fig. 2.  All chunks empty gives z = 0 and lse = -inf.
 *   workspace  device, partials of batch * n_splits slots in the layout above, slot b*n_splits + i
 *              holding chunk i of sequence b (as mla_decode_partial writes them)
 *   workspace_bytes  MLA_ERR_WORKSPACE when below mla_partials_bytes(dims, batch * n_splits)
 *   z        device float [batch, H, d_c]       (output; float32 for either dtype: the weighted
 *                                                 latent keeps its precision into mla_out_proj)
 *   lse      device float [batch, H] or NULL   (output)                                          */
mla_status mla_combine(const mla_dims* dims, int32_t batch, int32_t n_splits, const void* workspace,
                       size_t workspace_bytes, float* z, float* lse, void* stream);

/* Work-balanced split-K ([ase] Fig. 2 softmax over all cached positions, evaluated piecewise and
 * merged as in mla_combine).  Fixed-size chunks leave most of the GPU idle on ragged batches; this
 * variant splits the whole batch into n_units pieces of equal cost, so one launch of n_units
 * workgroups (one per compute unit) finishes together.  The split is a pure function of seq_lens:
 *   len_b   = min(max(seq_lens[b], 0), max_pages * page_size)
 *   tiles_b = ceil(len_b / MLA_BALANCED_TILE)
 *   cost_b  = tiles_b > 0 ? tiles_b + MLA_BALANCED_SEG_COST : 0,   C_b = cost_0 + ... + cost_{b-1}
 *   q       = ceil(C_batch / n_units)
 * Unit w owns cost positions [w*q, (w+1)*q); sequence b's tiles sit at positions
 * C_b + MLA_BALANCED_SEG_COST + k, k = 0 .. tiles_b-1 (the leading positions price the fixed cost
 * of a segment).  Segment (w, b) = the tiles of b in unit w, i.e. tokens
 * [MLA_BALANCED_TILE*k0, min(MLA_BALANCED_TILE*k1, len_b)); when non-empty its partial goes to
 * slot w + b, distinct for distinct non-empty segments.  Slots of empty segments are not written. */
#define MLA_BALANCED_TILE 32
#define MLA_BALANCED_SEG_COST 8
#define MLA_BALANCED_MAX_UNITS 2048

/* Number of partial slots of the balanced split: n_units + batch - 1 (-1 on bad arguments). */
int32_t mla_balanced_num_slots(int32_t batch, int32_t n_units);

/* Workspace bytes mla_decode_partial_balanced needs: mla_partials_bytes for
 * mla_balanced_num_slots(batch, n_units) slots (0 for invalid arguments). */
size_t mla_decode_balanced_workspace_bytes(const mla_dims* dims, const mla_cache* cache, int32_t n_units);

/* Balanced split-K decode: writes, for every non-empty segment (w, b) and head h, the same
 * chunk-local pair as mla_decode_partial over the segment's tokens into slot w + b:
 *   o_part[w+b,h,:]  (normalised),  lse_part[w+b,h]  (natural log)
 *   n_units  1 .. MLA_BALANCED_MAX_UNITS
 *   workspace, workspace_bytes  as for mla_decode_partial; MLA_ERR_WORKSPACE when below
 *            mla_decode_balanced_workspace_bytes(dims, cache, n_units)
 * MLA_ERR_UNSUPPORTED when batch * (max_pages*page_size / MLA_BALANCED_TILE + 9) >= 2^31 - 2^12. */
mla_status mla_decode_partial_balanced(const mla_dims* dims, const mla_cache* cache, const void* q_hat,
                                       int32_t n_units, void* workspace, size_t workspace_bytes, void* stream);

/* Merge of the balanced partials: for every sequence, the log-sum-exp merge of mla_combine over
 * the slots of its non-empty segments (none: z = 0, lse = -inf).  cache supplies seq_lens, batch,
 * page_size and max_pages (pool and page_table are not read but must be valid pointers).
 *   workspace, workspace_bytes  as written by mla_decode_partial_balanced with the same n_units
 *   z   device float [batch, H, d_c]   (output)
 *   lse device float [batch, H] or NULL (output)                                                  */
mla_status mla_combine_balanced(const mla_dims* dims, const mla_cache* cache, int32_t n_units,
                                const void* workspace, size_t workspace_bytes, float* z, float* lse, void* stream);

/* Balanced split with row groups, for the draft rows of a multi-token verify step ([molayo] key
 * concept 5, speculative decoding; [ase] causal-mask remark after Fig. 2): batch rows in
 * batch / row_group groups of row_group consecutive rows that read the same sequence's keys,
 * each up to its own seq_lens entry (the rows mla_verify_rows writes).  The split above runs
 * over groups, a group costing like its longest row, with n_units / row_group group-units;
 * unit row_group*w + i runs row i of every group segment (w, g), clamped to that row's tokens,
 * and writes its partial to slot row_group*(w + g) + i.  The row_group units of a group-unit
 * read the same pages side by side (and share an L2), so the cache is fetched about once per
 * group.  Results equal those of the plain balanced split up to the order of summation
 * (different segment boundaries); row_group = 1 is mla_decode_partial_balanced.
 *   row_group  >= 1, dividing both batch and n_units (MLA_ERR_SHAPE otherwise)
 *   workspace, workspace_bytes  as for mla_decode_partial_balanced (the same size suffices)
 * mla_combine_grouped merges what mla_decode_partial_grouped wrote with the same n_units and
 * row_group, as mla_combine_balanced does for the plain split. */
mla_status mla_decode_partial_grouped(const mla_dims* dims, const mla_cache* cache, const void* q_hat,
                                      int32_t n_units, int32_t row_group, void* workspace, size_t workspace_bytes,
                                      void* stream);
mla_status mla_combine_grouped(const mla_dims* dims, const mla_cache* cache, int32_t n_units, int32_t row_group,
                               const void* workspace, size_t workspace_bytes, float* z, float* lse, void* stream);

/* Value up-projection applied once after the weighted sum ([ase] "Value 투영을 가중합 뒤로
 * 옮기기", Fig. 4 equation; [huny] section 2, value absorption):
 *   out[r,h,:] = z[r,h,:] . W_UV[h]
 *   z    device float [rows, H, d_c]
 *   w_uv device dtype [H, d_c, d_v]
 *   out  device float [rows, H, d_v]   (output)                                                  */
mla_status mla_out_proj(const mla_dims* dims, const float* z, const void* w_uv, int32_t rows, float* out,
                        void* stream);

/* Split-K merge and value projection in one call: for every row b and head h,
 *   out[b,h,:] = (sum_i exp(lse_i - LSE) o_i) . W_UV[h],   LSE = ln sum_i exp(lse_i)
 * over the slots i of row b, i.e. mla_combine* followed by mla_out_proj ([ase] Fig. 2 softmax
 * merged piecewise, then the Fig. 4 value projection applied once after the weighted sum), with
 * the merged latent z kept on chip instead of written and read back.  Results equal those of the
 * two calls up to the order of floating-point summation.  A row with no key gives out = 0,
 * lse = -inf.  Only the DeepSeek-V3 shape in bf16 is implemented (d_c 512, d_k = d_v 128, d_r a
 * multiple of 8 up to 64): mla_combine_out_proj_supported(dims) says whether dims qualify (0 also
 * for invalid dims or MLA_FLAG_FORCE_GENERIC); otherwise every variant returns
 * MLA_ERR_UNSUPPORTED and the caller runs the two calls.
 *   workspace, workspace_bytes  the partials as mla_decode_partial (mla_combine_out_proj: batch,
 *            n_splits) or mla_decode_partial_balanced / _grouped (same n_units, row_group) wrote
 *            them; MLA_ERR_WORKSPACE when below the size the matching merge call requires
 *   w_uv     device bf16 [H, d_c, d_v]
 *   out      device float [batch, H, d_v]   (output)
 *   lse      device float [batch, H] or NULL (output, natural log)                              */
int32_t mla_combine_out_proj_supported(const mla_dims* dims);
mla_status mla_combine_out_proj(const mla_dims* dims, int32_t batch, int32_t n_splits, const void* workspace,
                                size_t workspace_bytes, const void* w_uv, float* out, float* lse, void* stream);
mla_status mla_combine_out_proj_balanced(const mla_dims* dims, const mla_cache* cache, int32_t n_units,
                                         const void* workspace, size_t workspace_bytes, const void* w_uv, float* out,
                                         float* lse, void* stream);
mla_status mla_combine_out_proj_grouped(const mla_dims* dims, const mla_cache* cache, int32_t n_units,
                                        int32_t row_group, const void* workspace, size_t workspace_bytes,
                                        const void* w_uv, float* out, float* lse, void* stream);

/* Causal multi-query attention for a chunk of new tokens whose rows are already in the cache
 * ([ase] causal-mask remark after Fig. 2; [molayo] chunked prefill).  Query i of sequence b sits
 * at absolute position q_start[b] + i and reads tokens t <= q_start[b] + i, t < seq_lens[b].
 *   q_hat   device [batch, q_len, H, d_c + d_r]  (as written by mla_absorb_query)
 *   q_start device int32 [batch]
 *   z       device float [batch, q_len, H, d_c]   (output, normalised)
 *   lse     device float [batch, q_len, H] or NULL (output, natural log)                         */
mla_status mla_prefill_chunk(const mla_dims* dims, const mla_cache* cache, const void* q_hat, int32_t q_len,
                             const int32_t* q_start, float* z, float* lse, void* stream);

/* Unabsorbed chunked prefill (row N4), the other path for a chunk of new queries: for long chunks
 * the per-pair work of plain attention (2 * (d_k + d_r) + 2 * d_v flops) is far below the absorbed
 * path's (2 * (d_c + d_r) + 2 * d_c), once every cached latent is decompressed per head
 * ([molayo] formal definition and chunked-prefill note; [ase] Fig. 3 and Fig. 4 left-hand sides).
 * Only the DeepSeek-V3 shape in bf16 (H 128, d_c 512, d_r 64, d_k = d_v 128) is implemented;
 * other dims give MLA_ERR_UNSUPPORTED (the absorbed mla_prefill_chunk handles every shape).
 *
 * Step 1, decompression: for t < seq_lens[b],
 *   k[b,h,t,:] = c_t . W_UK[h],  v[b,h,t,:] = c_t . W_UV[h],  k_r[b,t,:] = k^R_t (copied)
 *   w_uk, w_uv  device bf16 [H, d_c, d_k] / [H, d_c, d_v]
 *   k, v        device binary16 (fp16) [batch, H, max_len, d_k] / [.., d_v]   (outputs, fp32 sums
 *               rounded once; rows t >= seq_lens[b] are not written)
 *   k_r         device binary16 [batch, max_len, d_r]                          (output)
 *   max_len     host bound >= every seq_lens[b]
 * The intermediates are binary16 rather than bf16 for three more significand bits at the same
 * MFMA rate; their magnitudes must stay below 65504 (K and V of RMS-normalised latents are
 * orders of magnitude below it).                                                               */
mla_status mla_decompress_kv(const mla_dims* dims, const mla_cache* cache, int32_t max_len, const void* w_uk,
                             const void* w_uv, void* k, void* v, void* k_r, void* stream);

/* Step 2, causal attention over the decompressed keys and values: query i of sequence b sits at
 * absolute position p = q_start[b] + i and reads keys t <= p, t < seq_lens[b]:
 *   s_t = (q_c[b,i,h,:] . k[b,h,t,:] + RoPE_p(q_r[b,i,h,:]) . k_r[b,t,:]) * sm_scale
 *   out[b,i,h,:] = sum_t softmax_t(s) v[b,h,t,:];  lse[b,i,h] = ln sum_t exp(s_t)
 * This is the output of mla_prefill_chunk followed by mla_out_proj, up to rounding (the
 * associativity behind absorption).  No visible key gives out = 0, lse = -inf.
 *   q_c, q_r  device bf16 [batch, q_len, H, d_k] / [.., d_r]  (q_r unrotated)
 *   q_start   device int32 [batch]
 *   k, v, k_r as written by mla_decompress_kv with the same max_len
 *   out       device float [batch, q_len, H, d_v];  lse device float [batch, q_len, H] or NULL   */
mla_status mla_prefill_unabsorbed(const mla_dims* dims, const mla_cache* cache, int32_t max_len, const void* q_c,
                                  const void* q_r, const int32_t* q_start, int32_t q_len, const void* k,
                                  const void* v, const void* k_r, float* out, float* lse, void* stream);
/* Nonzero when the unabsorbed prefill supports these dims. */
int32_t mla_prefill_unabsorbed_supported(const mla_dims* dims);

/* bf16 cache rows -> FP8 cache rows (MLA_FLAG_CACHE_FP8 layout), row by row; the scale of each row
 * comes from its own 512 latent values.  src device bf16 [rows, 576]; dst device bytes
 * [rows, MLA_FP8_ROW_BYTES].  Only d_c 512, d_r 64 in bf16, at most 4 * (2^31 - 1) rows (else
 * MLA_ERR_UNSUPPORTED).  Rows holding
 * non-finite values give unspecified codes (never read: slots past a sequence's length). */
mla_status mla_quantize_rows_fp8(const mla_dims* dims, const void* src, int64_t rows, void* dst, void* stream);

/* ---- Precomposed weights (row N2): products of consecutive projections taken once, offline
 * ([molayo] formal definition, the absorbed weight W_UQ[h] . W_UK[h]^T; [ase] section on
 * multiplying consecutive projections ahead of time, query and value sides; [huny] section 2,
 * output-projection fusion).  bf16 dims with d_c 512, d_r 64 only (else MLA_ERR_UNSUPPORTED).
 *
 * mla_precompose_query: w_qcat[q, h, :] = [ (W_UQ[h] . W_UK[h]^T)[q, :] | W_QR[h][q, :] ], one bf16
 * rounding of float32 sums.  w_uq bf16 [H, d_cq, d_k]; w_uk [H, d_c, d_k]; w_qr [H, d_cq, d_r];
 * w_qcat bf16 [d_cq, H, d_c + d_r] (output).  d_cq a multiple of 64.                           */
mla_status mla_precompose_query(const mla_dims* dims, int32_t d_cq, const void* w_uq, const void* w_uk,
                                const void* w_qr, void* w_qcat, void* stream);
/* mla_precompose_out: w_uvo[h] = W_UV[h] . W_O[h] with W_O[h] the d_v rows h*d_v .. of W_O.
 * w_uv bf16 [H, d_c, d_v]; w_o bf16 [H * d_v, d_model]; w_uvo bf16 [H, d_c, d_model] (output).
 * d_model a multiple of 128. */
mla_status mla_precompose_out(const mla_dims* dims, int32_t d_model, const void* w_uv, const void* w_o, void* w_uvo,
                              void* stream);
/* The absorbed query straight from the query latent: q_hat[r, h, :] = [c_q[r] . W_absorbed[h] |
 * RoPE_pos[r](c_q[r] . W_QR[h])] * sm_scale * log2(e), rounded to binary16 once (the layout and
 * scaling of mla_absorb_query).  c_q bf16 [rows, d_cq]; w_qcat from mla_precompose_query; pos
 * device int32 [rows]; q_hat binary16 [rows, H, d_c + d_r].  workspace: device float32 scratch of at
 * least mla_absorb_query_precomposed_workspace_bytes bytes (caller-owned, overwritten; smaller:
 * MLA_ERR_WORKSPACE). */
size_t mla_absorb_query_precomposed_workspace_bytes(const mla_dims* dims, int32_t d_cq, int32_t rows);
mla_status mla_absorb_query_precomposed(const mla_dims* dims, int32_t d_cq, const void* c_q, const void* w_qcat,
                                        const int32_t* pos, int32_t rows, void* q_hat, float* workspace,
                                        size_t workspace_bytes, void* stream);
/* The layer output straight from the weighted latents: out[r, :] = sum_h z[r, h, :] . w_uvo[h].
 * z float32 [rows, H, d_c] (mla_combine's output, as float32 through bf16 hi + lo parts);
 * w_uvo from mla_precompose_out; out float32 [rows, d_model]; workspace as above. */
size_t mla_out_proj_fused_workspace_bytes(const mla_dims* dims, int32_t d_model, int32_t rows);
mla_status mla_out_proj_fused(const mla_dims* dims, int32_t d_model, const float* z, const void* w_uvo, int32_t rows,
                              float* out, float* workspace, size_t workspace_bytes, void* stream);
/* The unfused counterpart's last step, the output projection of the per-head outputs:
 * out[r, :] = o[r, :, :] (heads concatenated) . W_O.  o float32 [rows, H, d_v]; w_o bf16
 * [H * d_v, d_model]; out float32 [rows, d_model]; workspace as above. */
size_t mla_output_projection_workspace_bytes(const mla_dims* dims, int32_t d_model, int32_t rows);
mla_status mla_output_projection(const mla_dims* dims, int32_t d_model, const float* o, const void* w_o, int32_t rows,
                                 float* out, float* workspace, size_t workspace_bytes, void* stream);

/* Multi-token verify (row N4, speculative decoding) through the split-K decode path.  Query i of
 * sequence b sits at position q_start[b] + i and reads keys t <= q_start[b] + i, t < seq_lens[b]
 * (the causal rule of a chunk, [ase] causal-mask remark after Fig. 2).  Each such query is a decode
 * query over its own prefix, so a verify step is decode over batch * q_len rows; this call writes
 * the rows' description, for row r = b * q_len + i:
 *   row_table  device int32 [batch * q_len, max_pages]: a copy of page_table row b   (output)
 *   row_lens   device int32 [batch * q_len]: clamp(q_start[b] + i + 1, 0, seq_lens[b])  (output)
 *   row_pos    device int32 [batch * q_len] or NULL: q_start[b] + i, the rotary position (output)
 *   q_start    device int32 [batch]
 * The rows then form the cache {pool, row_table, row_lens, batch * q_len, page_size, max_pages,
 * num_pages} for mla_absorb_query (positions row_pos), mla_decode_partial_balanced,
 * mla_combine_balanced and mla_out_proj, whose outputs are those of mla_prefill_chunk on the same
 * queries up to rounding.  batch * q_len must not exceed 65535 (MLA_ERR_UNSUPPORTED).  */
mla_status mla_verify_rows(const mla_cache* cache, const int32_t* q_start, int32_t q_len, int32_t* row_table,
                           int32_t* row_lens, int32_t* row_pos, void* stream);

/* Query side of one layer ([ase] "현재 토큰의 Query 만들기", Fig. 1; [molayo] query compression):
 *   c^Q = h . W_DQ;  q_c[r,h,:] = c^Q . W_UQ[h];  q_r[r,h,:] = c^Q . W_QR[h]  (unrotated)
 *   h    device dtype [rows, d_model];  w_dq dtype [d_model, d_cq]
 *   w_uq dtype [H, d_cq, d_k];  w_qr dtype [H, d_cq, d_r]
 *   q_c  dtype [rows, H, d_k], q_r dtype [rows, H, d_r]   (outputs)                              */
mla_status mla_project_query(const mla_dims* dims, int32_t d_model, int32_t d_cq, const void* h,
                             const void* w_dq, const void* w_uq, const void* w_qr, int32_t rows,
                             void* q_c, void* q_r, void* stream);

/* Cache write for new tokens ([molayo] formal definition, compression; [huny] section 2,
 * decoupled RoPE; [ase] Fig. 1 note on the latent norm):
 *   c = h . W_DKV, optionally RMS-normalised (unit gain) when rms_eps > 0:
 *       c / sqrt(mean(c^2) + rms_eps) over the d_c latent values;
 *   k^R = RoPE_{pos}(h . W_KR); row [c | k^R] stored at token `positions[r]` of sequence
 *   `seq_ids[r]` through the page table of `cache` (cache->pool is written; no other row is).
 *   h device dtype [rows, d_model]; w_dkv dtype [d_model, d_c]; w_kr dtype [d_model, d_r]
 *   seq_ids, positions device int32 [rows]; two rows must not name the same token.
 *   workspace: device fp32 scratch of at least mla_kv_append_workspace_bytes(dims, d_model, rows)
 *   bytes, owned by the caller, contents ignored and overwritten (NULL allowed when that size
 *   is 0).  A smaller workspace_bytes gives MLA_ERR_WORKSPACE.
 * bf16 with d_c 512, d_r 64 and d_model a multiple of 256 runs on MFMA (a split-K product into
 * the workspace, then one wave per row for the norm, the rotation and the store); every other
 * shape runs the generic kernel, which needs no workspace. */
size_t mla_kv_append_workspace_bytes(const mla_dims* dims, int32_t d_model, int32_t rows);
mla_status mla_kv_append(const mla_dims* dims, const mla_cache* cache, int32_t d_model, const void* h,
                         const void* w_dkv, const void* w_kr, const int32_t* seq_ids,
                         const int32_t* positions, int32_t rows, float rms_eps, float* workspace,
                         size_t workspace_bytes, void* stream);

/* Allocation-free cache write, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): mla_kv_append with the
 * split-K partial products in a fixed scratch array of MLA_NOALLOC_SCRATCH_BYTES that the library
 * holds on every GPU it runs on until the process ends, instead of a caller workspace.  Arguments,
 * results and errors are those of mla_kv_append; a call whose partial products would exceed the
 * scratch (mla_kv_append_workspace_bytes(dims, d_model, rows) > MLA_NOALLOC_SCRATCH_BYTES, which
 * holds exactly when rows > 3640, whatever d_model) returns MLA_ERR_WORKSPACE before anything is
 * launched.  Shapes that take the generic kernel use no scratch and have no such limit.
 * Every call on one GPU uses that GPU's one scratch array: calls that overlap on a GPU (concurrent
 * streams, or threads without ordering between their streams) race and must not be issued.  The
 * scratch needs no clearing (each call overwrites what it reads).  The first call on each device
 * looks up the array's device address (no allocation); make one call before capturing a graph that
 * contains this one. */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
mla_status mla_kv_append_noalloc(const mla_dims* dims, const mla_cache* cache, int32_t d_model, const void* h,
                                 const void* w_dkv, const void* w_kr, const int32_t* seq_ids,
                                 const int32_t* positions, int32_t rows, float rms_eps, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
