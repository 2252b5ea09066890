// Unabsorbed chunked prefill on bf16 MFMA (gfx950), DeepSeek-V3 shape (128 heads, d_c 512,
// d_r 64, d_k = d_v = 128).
//
// For a chunk of Sq new queries per sequence the absorbed path pays 2 * (576 + 512) flops per
// (query head, key) pair.  Decompressing every cached latent once per chunk into per-head keys
// and values ([molayo] formal definition: K_h = C W_UK[h], V_h = C W_UV[h]) costs 2 * 2 * 512 * 128
// flops per (token, head) and leaves 2 * (192 + 128) per pair: plain multi-head attention with a
// 192-wide score (content part plus the shared rotary key, [ase] Fig. 2) and a 128-wide value.
// Both per-head projections of the absorbed path disappear as well.  Two launches:
//
// decompress_kv_kernel: per (128 tokens of a sequence, head), out^T = W^T . C^T for the head's
// W_UK and W_UV (256 output columns, K = 512) with v_mfma_f32_32x32x16_bf16.  The latent rows come
// through the page table straight from the pool as the B operand (16 bytes per lane); the weight
// slice is staged in LDS 32 rows at a time (double-buffered) and read with ds_read_b64_tr_b16.
// Results go through LDS and out as whole 256-byte rows of K and V ([b][h][t][128] bf16); the
// head-0 workgroups also copy the rotary keys to kr ([b][t][64] bf16).
//
// attend_unabsorbed_kernel: per (128 queries, head, sequence), four waves of 32 queries.  Keys and
// values stream through LDS in 32-token tiles (double-buffered, staged through registers).  Scores
// are computed transposed, S^T = [K | k^R] . Q^T (tokens on M, queries on N, 12 k-steps), so every
// lane holds 16 scores of one query and the softmax stays in the lane plus one v_permlane32_swap.
// Online softmax with a running maximum; the accumulator is rescaled only when a maximum moved.
// The weighted sum is accumulated transposed, O^T += V^T . P^T, with V^T from transposing reads in
// the token order of the score layout.  Output o [b][q][h][128] float32 and lse [b][q][h].

#include <math.h>

#include "common.h"
#include "launch.h"

namespace mla {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kH = 128, kDc = 512, kDr = 64, kW = kDc + kDr, kDk = 128;
constexpr int kRowB = kDk * 2;  // 256 bytes: one K or V row

__device__ __forceinline__ bf16x8 lds16(const lds_u8* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(p);
}
__device__ __forceinline__ bf16x8 tr_pair(const lds_u8* p0, const lds_u8* p1) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p0);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p1);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// ------------------------------------------------------------------------------- decompression
constexpr int kDcTok = 128;                  // tokens per workgroup (4 waves x 32)
constexpr int kDcJ = 32;                     // weight rows staged per chunk
constexpr int kDcRowB = 2 * kRowB;           // a staged weight row: 128 W_UK + 128 W_UV columns
constexpr int kDcChunkB = kDcJ * kDcRowB;    // 16 KiB
constexpr int kDcOutRow = 2 * kRowB + 16;     // staged output row (K | V) + padding against bank conflicts
constexpr int kDcOutB = kDcTok * kDcOutRow;    // 66 KiB output staging

// 16-byte chunk c (0..31) of staged weight row r sits at c ^ 4*(r & 3): the transposing reads of
// 4 rows x 4 chunks by 32 lanes then cover 16 distinct bank groups.
__device__ __forceinline__ int dc_swz(int r, int c) { return c ^ ((r & 3) << 2); }

__global__ __launch_bounds__(256) void decompress_kv_kernel(Cache c, int max_len, const uint16_t* __restrict__ w_uk,
                                                            const uint16_t* __restrict__ w_uv,
                                                            uint16_t* __restrict__ k_out,
                                                            uint16_t* __restrict__ v_out,
                                                            uint16_t* __restrict__ kr_out) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kDcOutB];  // 2 weight chunks, then the output
  lds_u8* const lbase = (lds_u8*)smem;
  const int tb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int len = min(c.seq_lens[b], c.max_pages * c.page_size);
  const int t0 = tb * kDcTok;
  if (t0 >= len) return;  // uniform
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, hi = lane >> 5, g = lane >> 4, ii = lane & 15;
  const uint16_t* pool = static_cast<const uint16_t*>(c.pool);

  // B operand: latent row of token t0 + 32*wave + lane%32 (clamped inside the sequence)
  const int tok = min(t0 + 32 * wave + (lane & 31), len - 1);
  const uint16_t* crow = pool + row_index(c.page_table, c.max_pages, c.page_size, b, tok) * kW + 8 * hi;

  // staging: chunk k covers weight rows j = 32k .. 32k+31; thread t moves 16-byte pieces
  // p = t + 256x (x < 4): row p / 32, piece p % 32 (pieces 0..15 from W_UK, 16..31 from W_UV)
  u32x4 st[4];
  auto load_w = [&](int k) {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int p = threadIdx.x + 256 * x, r = p >> 5, q = p & 31;
      const uint16_t* src = (q < 16 ? w_uk : w_uv) + (size_t(h) * kDc + 32 * k + r) * kDk + 8 * (q & 15);
      st[x] = *reinterpret_cast<const u32x4*>(src);
    }
  };
  auto store_w = [&](int buf) {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int p = threadIdx.x + 256 * x, r = p >> 5, q = p & 31;
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(lbase + buf * kDcChunkB + r * kDcRowB +
                                                                  16 * dc_swz(r, q)) = st[x];
    }
  };
  // A operand of output block ob (0..3: K columns 32ob.., 4..7: V) at k-step s of a chunk: group g
  // addresses rows 8*(g/2) + (lane%16)/4 (+4 for the second read), columns 32ob + 16(g%2) + 4(lane%4)
  auto a_op = [&](int buf, int s, int ob) {
    const int r = 16 * s + 8 * (g >> 1) + (ii >> 2);
    const int col = 32 * ob + 16 * (g & 1) + 4 * (ii & 3);
    const lds_u8* base = lbase + buf * kDcChunkB;
    const lds_u8* p0 = base + r * kDcRowB + 16 * dc_swz(r, col >> 3) + 2 * (col & 7);
    const lds_u8* p1 = base + (r + 4) * kDcRowB + 16 * dc_swz(r + 4, col >> 3) + 2 * (col & 7);
    return tr_pair(p0, p1);
  };

  f32x16 acc[8];
#pragma unroll
  for (int ob = 0; ob < 8; ++ob)
#pragma unroll
    for (int x = 0; x < 16; ++x) acc[ob][x] = 0.f;

  constexpr int kChunks = kDc / kDcJ;  // 16
  bf16x8 bcur[2], bnxt[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) bcur[s] = *reinterpret_cast<const bf16x8*>(crow + 16 * s);
  load_w(0);
  store_w(0);
  __syncthreads();
  for (int k = 0; k < kChunks; ++k) {
    const int buf = k & 1;
    const int kn = min(k + 1, kChunks - 1);  // unconditional loads keep the wait counts exact
#pragma unroll
    for (int s = 0; s < 2; ++s) bnxt[s] = *reinterpret_cast<const bf16x8*>(crow + 32 * kn + 16 * s);
    load_w(kn);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int ob = 0; ob < 8; ++ob)
        acc[ob] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_op(buf, s, ob), bcur[s], acc[ob], 0, 0, 0);
    if (k + 1 < kChunks) store_w(buf ^ 1);  // that buffer was last read before the previous barrier
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 2; ++s) bcur[s] = bnxt[s];
  }

  // D layout: lane holds token lane%32 of the wave and columns 32ob + 8(x/4) + 4hi + x%4.  Stage
  // [128 tokens][K row | V row] in LDS (the weight chunks are done), then write whole rows.
  {
    lds_u8* const orow = lbase + (32 * wave + (lane & 31)) * kDcOutRow;
#pragma unroll
    for (int ob = 0; ob < 8; ++ob)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = 32 * ob + 8 * q + 4 * hi;  // 0..255 across K | V
        u32x2 v;
        v[0] = uint32_t(f32_to_bf16(acc[ob][4 * q])) | (uint32_t(f32_to_bf16(acc[ob][4 * q + 1])) << 16);
        v[1] = uint32_t(f32_to_bf16(acc[ob][4 * q + 2])) | (uint32_t(f32_to_bf16(acc[ob][4 * q + 3])) << 16);
        *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(orow + 2 * col) = v;
      }
  }
  __syncthreads();
  const int ntok = min(kDcTok, len - t0);
  const size_t obase = (size_t(b) * kH + h) * max_len + t0;
  for (int idx = threadIdx.x; idx < ntok * 32; idx += 256) {  // 32 pieces of 16 B per token
    const int t = idx >> 5, q = idx & 31;
    const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(lbase + t * kDcOutRow + 16 * q);
    uint16_t* dst = (q < 16 ? k_out : v_out) + (obase + t) * kDk + 8 * (q & 15);
    *reinterpret_cast<u32x4*>(dst) = v;
  }
  if (h == 0) {  // rotary keys of these tokens: 8 pieces of 16 B per token
    for (int idx = threadIdx.x; idx < ntok * 8; idx += 256) {
      const int t = idx >> 3, q = idx & 7;
      const uint16_t* src = pool + row_index(c.page_table, c.max_pages, c.page_size, b, t0 + t) * kW + kDc + 8 * q;
      *reinterpret_cast<u32x4*>(kr_out + (size_t(b) * max_len + t0 + t) * kDr + 8 * q) =
          *reinterpret_cast<const u32x4*>(src);
    }
  }
}

// ------------------------------------------------------------------------------- attention
constexpr int kAtQ = 128;                    // queries per workgroup (4 waves x 32)
constexpr int kAtT = 32;                     // tokens per tile
constexpr int kTileKB = kAtT * kRowB;        // 8 KiB of K
constexpr int kTileRB = kAtT * kDr * 2;      // 4 KiB of k^R
constexpr int kTileB = 2 * kTileKB + kTileRB;  // K | V | k^R: 20 KiB
constexpr int kAtPieces = kTileB / 16 / 256;   // 5 x 16 B per thread

// K and V rows: 16-byte chunk c (0..15) of row r at c ^ f(r), f(r) = ((r & 3) << 2) | ((r >> 2) & 3):
// 16 consecutive rows at one logical chunk (score reads) and 4 rows x 4 chunks (transposing reads)
// hit 16 distinct bank groups.  k^R rows (8 chunks, 128 B): chunk c of row r at c ^ ((r >> 1) & 7).
__device__ __forceinline__ int kv_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int kr_swz(int r) { return (r >> 1) & 7; }

struct RopeTab {
  double v[kDr / 2];
};

__global__ __launch_bounds__(256) void attend_unabsorbed_kernel(
    const int32_t* __restrict__ seq_lens, int cap, int max_len, const uint16_t* __restrict__ q_c,
    const uint16_t* __restrict__ q_r, const int32_t* __restrict__ q_start, int q_len, float qscale, RopeTab rope,
    const uint16_t* __restrict__ k_in, const uint16_t* __restrict__ v_in, const uint16_t* __restrict__ kr_in,
    float* __restrict__ out, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kTileB];  // 40 KiB
  lds_u8* const lbase = (lds_u8*)smem;
  const int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, hi = lane >> 5, g = lane >> 4, ii = lane & 15;
  const int len = min(seq_lens[b], cap);
  const int qs = q_start[b];
  const int q0 = kAtQ * qb;  // first query of the workgroup (chunk index)
  if (q0 >= q_len) return;
  const int qi = q0 + 32 * wave + (lane & 31);  // this lane's query (chunk index)
  const bool qvalid = qi < q_len;
  const int qpos = qs + min(qi, q_len - 1);     // its absolute position
  // keys visible to the workgroup: t < min(len, qs + q0 + 128); to this wave: < min(len, qs + q0w + 32)
  const int t_end = min(len, max(qs + min(q0 + kAtQ, q_len), 0));
  const int ntiles = (t_end + kAtT - 1) / kAtT;

  // ---- Q^T operand (B of the score MFMA): query qi, k = 16ks + 8hi .. +7; the content part is
  // q_c as stored (exact), the rotary part is rotated here at qpos and rounded to bf16 once; the
  // scale sm_scale*log2(e) is applied to the float scores instead
  bf16x8 qf[12];
  {
    const size_t qrow = (size_t(b) * q_len + min(qi, q_len - 1)) * kH + h;
    const uint16_t* qcp = q_c + qrow * kDk + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qcp + 16 * ks);
    const uint16_t* qrp = q_r + qrow * kDr + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qrp + 16 * ks);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        // rotary pair 8ks + 4hi + k; two uniform table reads and a select (a per-lane index into
        // the kernel argument would be one memory load per use)
        const double ang = double(qpos) * (hi ? rope.v[8 * ks + 4 + k] : rope.v[8 * ks + k]);
        const double rd = ang - 6.283185307179586 * rint(ang * 0.15915494309189535);
        float sn, cs;
        sincosf(float(rd), &sn, &cs);
        const float x1 = bf16_to_f32(uint16_t(v[k] & 0xffffu)), x2 = bf16_to_f32(uint16_t(v[k] >> 16));
        qf[8 + ks][2 * k] = (__bf16)(x1 * cs - x2 * sn);
        qf[8 + ks][2 * k + 1] = (__bf16)(x1 * sn + x2 * cs);
      }
    }
  }

  // ---- tile staging: thread t moves 16-byte pieces p = t + 256x (x < 5) of the 20 KiB tile
  // (pieces 0..511 K, 512..1023 V, 1024..1279 k^R), swizzled into LDS
  const size_t kvbase = (size_t(b) * kH + h) * max_len;
  u32x4 st[kAtPieces];
  // rows past the sequence end are loaded from a valid row and replaced by zeros: their buffer
  // memory may hold anything, and 0 x NaN would reach the weighted sum
  auto load_tile = [&](int j) {
    const int tt0 = kAtT * j;
#pragma unroll
    for (int x = 0; x < kAtPieces; ++x) {
      const int p = threadIdx.x + 256 * x;
      const uint16_t* src;
      int r;
      if (p < 1024) {
        r = (p & 511) >> 4;
        const int q = p & 15;
        src = (p < 512 ? k_in : v_in) + (kvbase + min(tt0 + r, len - 1)) * kDk + 8 * q;
      } else {
        r = (p - 1024) >> 3;
        const int q = p & 7;
        src = kr_in + (size_t(b) * max_len + min(tt0 + r, len - 1)) * kDr + 8 * q;
      }
      const u32x4 v = *reinterpret_cast<const u32x4*>(src);
      st[x] = tt0 + r < len ? v : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_tile = [&](int buf) {
    lds_u8* const tb = lbase + buf * kTileB;
#pragma unroll
    for (int x = 0; x < kAtPieces; ++x) {
      const int p = threadIdx.x + 256 * x;
      int off;
      if (p < 1024) {
        const int r = (p & 511) >> 4, q = p & 15;
        off = (p < 512 ? 0 : kTileKB) + r * kRowB + 16 * (q ^ kv_swz(r));
      } else {
        const int r = (p - 1024) >> 3, q = p & 7;
        off = 2 * kTileKB + r * (kDr * 2) + 16 * (q ^ kr_swz(r));
      }
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(tb + off) = st[x];
    }
  };
  // score A operand (rows = tokens): row lane%32, logical chunk 2ks + hi
  const int sr = lane & 31;
  auto s_op = [&](const lds_u8* tb, int ks) -> bf16x8 {
    if (ks < 8) return lds16(tb + sr * kRowB + 16 * ((2 * ks + hi) ^ kv_swz(sr)));
    return lds16(tb + 2 * kTileKB + sr * (kDr * 2) + 16 * ((2 * (ks - 8) + hi) ^ kr_swz(sr)));
  };
  // weighted-sum A operand V^T for value block db, k-step s: tokens 16s + 4*(g/2) + (lane%16)/4 and
  // +8, value columns 32db + 16(g%2) + 4(lane%4) .. +3 (the token order of the score layout)
  auto v_op = [&](const lds_u8* tb, int s, int db) -> bf16x8 {
    const int r = 16 * s + 4 * (g >> 1) + (ii >> 2);
    const int col = 32 * db + 16 * (g & 1) + 4 * (ii & 3);
    const lds_u8* vb = tb + kTileKB;
    return tr_pair(vb + r * kRowB + 16 * ((col >> 3) ^ kv_swz(r)) + 2 * (col & 7),
                   vb + (r + 8) * kRowB + 16 * ((col >> 3) ^ kv_swz(r + 8)) + 2 * (col & 7));
  };

  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int x = 0; x < 16; ++x) acc[db][x] = 0.f;
  float m_run = -INFINITY, l_lane = 0.f;
  const int wq_last = qs + min(q0 + 32 * wave + 31, q_len - 1);  // the wave's last query position

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    load_tile(min(j + 1, ntiles - 1));  // unconditional: exact wait counts
    __builtin_amdgcn_sched_barrier(0);
    const lds_u8* const tb = lbase + buf * kTileB;
    const int tt0 = kAtT * j;
    if (tt0 <= wq_last) {  // the wave sees some token of this tile (uniform)
      f32x16 s;
#pragma unroll
      for (int x = 0; x < 16; ++x) s[x] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 12; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(s_op(tb, ks), qf[ks], s, 0, 0, 0);
#pragma unroll
      for (int x = 0; x < 16; ++x) s[x] *= qscale;  // base-2 logits
      // mask: tokens past the query's position or the sequence end
      if (tt0 + kAtT - 1 > qs + q0 + 32 * wave || tt0 + kAtT > len) {
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const int t = tt0 + 8 * (x >> 2) + 4 * hi + (x & 3);
          if (t > qpos || t >= len) s[x] = -INFINITY;
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int x = 0; x < 16; ++x) mx = fmaxf(mx, s[x]);
      {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
      }
      const float m_new = fmaxf(m_run, mx);
      if (__builtin_amdgcn_ballot_w64(m_new > m_run) != 0) {  // some maximum moved: rescale
        // (lanes whose maximum stayed, -inf included when no key is visible yet, keep factor 1)
        const float alpha = m_new > m_run ? fast_exp2(m_run - m_new) : 1.f;
        l_lane *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int x = 0; x < 16; ++x) acc[db][x] *= alpha;
        m_run = m_new;
      }
      float p[16], tsum = 0.f;
      const float m_use = m_run == -INFINITY ? 0.f : m_run;  // a query with no visible key yet
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        p[x] = fast_exp2(s[x] - m_use);
        tsum += p[x];
      }
      l_lane += tsum;
      bf16x8 pb0, pb1;
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        pb0[x] = (__bf16)p[x];
        pb1[x] = (__bf16)p[8 + x];
      }
#pragma unroll
      for (int sk = 0; sk < 2; ++sk)
#pragma unroll
        for (int db = 0; db < 4; ++db)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_op(tb, sk, db), sk ? pb1 : pb0, acc[db], 0, 0, 0);
    }
    if (j + 1 < ntiles) store_tile(buf ^ 1);  // that buffer was last read before the previous barrier
    __syncthreads();
  }

  // ---- normalise and write: lane holds query qi, values 32db + 8(x/4) + 4hi + x%4
  const float l_tot = [&] {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_lane), __float_as_uint(l_lane), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }();
  if (!qvalid) return;
  const bool empty = !(l_tot > 0.f);  // no visible key
  const float inv = empty ? 0.f : 1.f / l_tot;
  float* o = out + ((size_t(b) * q_len + qi) * kH + h) * kDk + 4 * hi;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<f32x4*>(o + 32 * db + 8 * q) =
          f32x4{acc[db][4 * q] * inv, acc[db][4 * q + 1] * inv, acc[db][4 * q + 2] * inv, acc[db][4 * q + 3] * inv};
  if (lse && hi == 0) lse[(size_t(b) * q_len + qi) * kH + h] = empty ? -INFINITY : (m_run + log2f(l_tot)) * kLn2;
}

}  // namespace

bool prefill_unabsorbed_supported(const Dims& d) {
  return d.dtype == MLA_BF16 && d.H == kH && d.dc == kDc && d.dr == kDr && d.dk == kDk && d.dv == kDk;
}

hipError_t launch_decompress_kv(const Dims& d, const Cache& c, int max_len, const void* w_uk, const void* w_uv,
                                void* k_out, void* v_out, void* kr_out, hipStream_t s) {
  (void)d;
  const dim3 grid((max_len + kDcTok - 1) / kDcTok, kH, c.batch);
  decompress_kv_kernel<<<grid, 256, 0, s>>>(c, max_len, static_cast<const uint16_t*>(w_uk),
                                            static_cast<const uint16_t*>(w_uv), static_cast<uint16_t*>(k_out),
                                            static_cast<uint16_t*>(v_out), static_cast<uint16_t*>(kr_out));
  return hipGetLastError();
}

hipError_t launch_attend_unabsorbed(const Dims& d, const Cache& c, int max_len, const void* q_c, const void* q_r,
                                    const int32_t* q_start, int q_len, const void* k, const void* v, const void* kr,
                                    float* out, float* lse, hipStream_t s) {
  RopeTab rope;
  for (int i = 0; i < kDr / 2; ++i) rope.v[i] = pow(double(d.rope_base), -2.0 * i / kDr);
  const float qscale = d.sm_scale * kLog2e;
  const dim3 grid((q_len + kAtQ - 1) / kAtQ, kH, c.batch);
  attend_unabsorbed_kernel<<<grid, 256, 0, s>>>(c.seq_lens, c.max_pages * c.page_size, max_len,
                                                static_cast<const uint16_t*>(q_c), static_cast<const uint16_t*>(q_r),
                                                q_start, q_len, qscale, rope, static_cast<const uint16_t*>(k),
                                                static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(kr), out,
                                                lse);
  return hipGetLastError();
}

}  // namespace mla
