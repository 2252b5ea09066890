// Unabsorbed chunked prefill on MFMA (gfx950), DeepSeek-V3 shape (128 heads, d_c 512, d_r 64,
// d_k = d_v = 128).
//
// For a chunk of Sq new queries per sequence the absorbed path pays 2 * (576 + 512) flops per
// (query head, key) pair.  Decompressing every cached latent once per chunk into per-head keys
// and values ([molayo] formal definition: K_h = C W_UK[h], V_h = C W_UV[h]) costs 2 * 2 * 512 * 128
// flops per (token, head) and leaves 2 * (192 + 128) per pair: plain multi-head attention with a
// 192-wide score (content part plus the shared rotary key, [ase] Fig. 2) and a 128-wide value.
// Both per-head projections of the absorbed path disappear as well.
//
// Precision: the decompression multiplies the bf16 cache and weights exactly as stored; what it
// produces (K, V, and the copied k^R) is kept in binary16, which carries three more significand
// bits than bf16 at the same MFMA rate, and the attention runs on binary16 MFMAs with the query
// and the probabilities in binary16 too.  Every rounding of the path is then 2^-11 relative
// instead of 2^-8.  Binary16 holds magnitudes up to 65504; K and V of RMS-normalised latents stay
// orders of magnitude below that.  Two launches:
//
// decompress_kv_kernel: per (128 tokens of a sequence, head), out^T = W^T . C^T for the head's
// W_UK and W_UV (256 output columns, K = 512) with v_mfma_f32_32x32x16_bf16.  K is walked in 16
// chunks of 32: each chunk's 32 W_UK and 32 W_UV rows and the matching 64 bytes of the 128 tokens'
// latent rows (through the page table) stream into LDS by direct global-to-LDS transfers, two
// chunks in flight while one is multiplied.  The weights are read with ds_read_b64_tr_b16 as the
// A operand, the latents row-wise as the B operand.
// Results go through LDS and out as whole 256-byte rows of K and V ([b][h][t][128] binary16);
// the head-0 workgroups also copy the rotary keys to kr ([b][t][64] binary16).
//
// attend_unabsorbed_kernel: per (128 queries, head, sequence), four waves of 32 queries.  Keys and
// values stream into LDS in 32-token tiles through direct global-to-LDS transfers, three tiles in
// flight.  Scores are computed transposed, S^T = [K | k^R] . Q^T (tokens on M, queries on N, 12 k-steps), so every
// lane holds 16 scores of one query and the softmax stays in the lane plus one v_permlane32_swap.
// Online softmax against a per-query reference that may trail the running maximum by up to 8
// (base 2): probabilities are taken times 2^7 relative to it (at most 2^15, inside binary16), and
// the accumulator is rescaled only when some query's maximum climbs further, behind a branch that
// is uniform over the wave and after the first tiles rarely taken.
// The weighted sum is accumulated transposed, O^T += V^T . P^T, with V^T from transposing reads in
// the token order of the score layout.  Output o [b][q][h][128] float32 and lse [b][q][h].

#include <math.h>

#include "common.h"
#include "launch.h"

namespace mla {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
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
__device__ __forceinline__ f16x8 lds16h(const lds_u8* p) { return __builtin_bit_cast(f16x8, lds16(p)); }
__device__ __forceinline__ f16x8 tr_pair_h(const lds_u8* p0, const lds_u8* p1) {
  return __builtin_bit_cast(f16x8, tr_pair(p0, p1));
}
// binary16 bits of a float, round to nearest even
__device__ __forceinline__ uint32_t f16_bits(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }

// One 16-byte-per-lane transfer from global memory straight into LDS at M0 + 16 * lane, waited for
// with explicit vmcnt waits (the compiler does not see that it writes LDS).
__device__ __forceinline__ void dma16(uint32_t lds_dst, uint32_t voff, const void* gbase) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_dst), "v"(voff), "s"(gbase) : "memory");
}
// The same with a full 64-bit address per lane (for rows anywhere in a cache pool of any size).
__device__ __forceinline__ void dma16_at(uint32_t lds_dst, const void* src) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_dst), "v"(src) : "memory");
}

// ------------------------------------------------------------------------------- decompression
constexpr int kDcTok = 128;                    // tokens per workgroup (4 waves x 32)
constexpr int kDcJ = 32;                       // weight rows per chunk
constexpr int kDcChunks = kDc / kDcJ;          // 16
constexpr int kDcWB = 2 * kDcJ * kRowB;        // 16 KiB: 32 W_UK rows | 32 W_UV rows
constexpr int kDcCB = kDcTok * kDcJ * 2;        // 8 KiB: the 128 tokens' latents over the chunk's 32 j
constexpr int kDcChunkB = kDcWB + kDcCB;        // 24 KiB
constexpr int kDcBuf = 3;                       // chunk buffers: one in use, two in flight
constexpr int kDcXfer = kDcChunkB / 1024 / 4;   // 6 one-KiB transfers per wave per chunk
constexpr int kDcOutRow = 2 * kRowB + 16;      // staged output row (K | V) + padding against bank conflicts
constexpr int kDcOutB = kDcTok * kDcOutRow;    // 66 KiB output staging (reuses the chunk buffers)
constexpr int kDcLds = kDcOutB > kDcBuf * kDcChunkB ? kDcOutB : kDcBuf * kDcChunkB;

// 256-byte rows (K, V, staged weights): 16-byte chunk c of row r at c ^ f(r),
// f(r) = ((r & 3) << 2) | ((r >> 2) & 3): 16 consecutive rows at one logical chunk (row-wise reads)
// and 4 rows x 4 chunks (transposing reads) hit 16 distinct bank groups.  128-byte k^R rows: chunk
// c of row r at c ^ ((r >> 1) & 7).
// Workgroups are dispatched round-robin over the 8 XCDs, each with its own L2.  The per_group
// workgroups of group grp all run on XCD grp % 8 (linear id 8k + grp % 8), so the data they share
// (a head's weights, a sequence-head's keys and values) is fetched from HBM once, not once per XCD.
__device__ __forceinline__ bool xcd_group_map(int per_group, int groups, int& grp, int& inner) {
  const int id = blockIdx.x, k = id >> 3;
  grp = (k / per_group) * 8 + (id & 7);
  inner = k % per_group;
  return grp < groups;
}
__host__ inline unsigned xcd_group_grid(int per_group, int groups) {
  return unsigned(8 * ((groups + 7) / 8) * per_group);
}

__device__ __forceinline__ int kv_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int kr_swz(int r) { return (r >> 1) & 7; }

__global__ __launch_bounds__(256, 2) void decompress_kv_kernel(Cache c, int max_len, const uint16_t* __restrict__ w_uk,
                                                               const uint16_t* __restrict__ w_uv,
                                                               uint16_t* __restrict__ k_out,
                                                               uint16_t* __restrict__ v_out,
                                                               uint16_t* __restrict__ kr_out) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kDcLds];
  lds_u8* const lbase = (lds_u8*)smem;
  // group = head (its W_UK and W_UV slices), members = (sequence, 128-token block)
  const int ntb = (max_len + kDcTok - 1) / kDcTok;
  int h, inner;
  if (!xcd_group_map(ntb * c.batch, kH, h, inner)) return;
  const int tb = inner % ntb, b = inner / ntb;
  const int len = min(c.seq_lens[b], c.max_pages * c.page_size);
  const int t0 = tb * kDcTok;
  if (t0 >= len) return;  // uniform
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, hi = lane >> 5, g = lane >> 4, ii = lane & 15;
  const uint16_t* pool = static_cast<const uint16_t*>(c.pool);

  // chunk transfers of 1 KiB, six per wave.  Weight transfers T = 4*wave + x (x < 4): T < 8 W_UK
  // rows 32k + 4T .., else W_UV rows 32k + 4(T-8) .. (256 B each, lane L fills LDS chunk L%16 of
  // row L/16).  Latent transfers u = 2*wave + (x-4) (x = 4, 5): tokens 16u .. 16u+15 over
  // j = 32k .. 32k+31 (64 B per token, lane L fills chunk L%4 of token row L/4), so a wave fetches
  // the latents of its own 32 tokens.  Latent rows come through the page table (clamped inside the
  // sequence); each lane keeps the pool offsets of its two token rows.
  const uint32_t lds0 = uint32_t(reinterpret_cast<uintptr_t>(lbase));
  const uint16_t* const ukh = w_uk + size_t(h) * kDc * kDk;
  const uint16_t* const uvh = w_uv + size_t(h) * kDc * kDk;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const uint16_t* crow[2];  // the token rows of this lane's latent transfers, at its chunk
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int r = 16 * (2 * wv + u) + (lane >> 2), cc = (lane & 3) ^ ((r >> 2) & 3);
    crow[u] = pool + row_index(c.page_table, c.max_pages, c.page_size, b, min(t0 + r, len - 1)) * kW + 8 * cc;
  }
  auto dma_chunk = [&](int k, int buf) {
    const uint32_t dst = lds0 + uint32_t(buf * kDcChunkB);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int T = 4 * wv + x;
      const int r = 4 * (T & 7) + (lane >> 4), cc = (lane & 15) ^ kv_swz(r);
      dma16(dst + uint32_t(T * 1024), uint32_t((kDcJ * k + r) * kRowB + 16 * cc), T < 8 ? ukh : uvh);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) dma16_at(dst + uint32_t(kDcWB + (2 * wv + u) * 1024), crow[u] + kDcJ * k);
  };
  // B operand: latents of token 32*tb + lane%32 at j = 16s + 8hi of the chunk (64-byte token rows,
  // chunk c of row r at c ^ ((r >> 2) & 3))
  auto b_op = [&](int buf, int s, int tb) {
    const int r = 32 * tb + (lane & 31);
    return lds16(lbase + buf * kDcChunkB + kDcWB + r * 64 + 16 * ((2 * s + hi) ^ ((r >> 2) & 3)));
  };
  // A operand of output block ob (0..3: K columns 32ob.., 4..7: V) at k-step s of a chunk: group g
  // addresses rows 16s + 8(g/2) + (lane%16)/4 (+4 for the second read), columns 32(ob%4) + 16(g%2)
  // + 4(lane%4) of the K or V half
  auto a_op = [&](int buf, int s, int ob) {
    const int r = 16 * s + 8 * (g >> 1) + (ii >> 2);
    const int col = 32 * (ob & 3) + 16 * (g & 1) + 4 * (ii & 3);
    const lds_u8* base = lbase + buf * kDcChunkB + (ob >> 2) * (kDcJ * kRowB);  // K or V half
    const lds_u8* p0 = base + r * kRowB + 16 * ((col >> 3) ^ kv_swz(r)) + 2 * (col & 7);
    const lds_u8* p1 = base + (r + 4) * kRowB + 16 * ((col >> 3) ^ kv_swz(r + 4)) + 2 * (col & 7);
    return tr_pair(p0, p1);
  };

  // wave w owns output blocks 2w and 2w+1 (K columns for w < 2, V columns beyond) for all four
  // 32-token blocks: each weight operand read from LDS feeds four MFMAs, each latent operand two
  f32x16 acc[8];  // [2 * 0 + tb] and [4 + tb]: blocks 2w and 2w+1 of token block tb
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int x = 0; x < 16; ++x) acc[a][x] = 0.f;

  // chunks k and k+1 in flight while chunk k is multiplied; every iteration issues the same
  // transfers (past the end they repeat the last chunk into the free buffer), so one wait count
  // fits all
#pragma unroll
  for (int k = 0; k < kDcBuf - 1; ++k) dma_chunk(k, k);
  for (int k = 0; k < kDcChunks; ++k) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kDcXfer) : "memory");  // chunk k landed (own part)
    __syncthreads();  // every wave's part landed; the buffer of chunk k-1 is free
    dma_chunk(min(k + kDcBuf - 1, kDcChunks - 1), (k + kDcBuf - 1) % kDcBuf);
    const int buf = k % kDcBuf;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 bq[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) bq[tb] = b_op(buf, s, tb);
#pragma unroll
      for (int obl = 0; obl < 2; ++obl) {
        const bf16x8 aw = a_op(buf, s, 2 * wave + obl);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
          acc[4 * obl + tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw, bq[tb], acc[4 * obl + tb], 0, 0, 0);
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();  // every wave is done with the chunk buffers and no transfer is in flight

  // D layout: lane holds token 32tb + lane%32 and columns 32ob + 8(x/4) + 4hi + x%4.  Stage
  // [128 tokens][K row | V row] in LDS, then write whole rows.
#pragma unroll
  for (int obl = 0; obl < 2; ++obl)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      lds_u8* const orow = lbase + (32 * tb + (lane & 31)) * kDcOutRow;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = 32 * (2 * wave + obl) + 8 * q + 4 * hi;  // 0..255 across K | V
        const f32x16& a = acc[4 * obl + tb];
        u32x2 v;
        v[0] = f16_bits(a[4 * q]) | (f16_bits(a[4 * q + 1]) << 16);
        v[1] = f16_bits(a[4 * q + 2]) | (f16_bits(a[4 * q + 3]) << 16);
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
  if (h == 0) {  // rotary keys of these tokens, bf16 -> binary16: 8 pieces of 8 values per token
    for (int idx = threadIdx.x; idx < ntok * 8; idx += 256) {
      const int t = idx >> 3, q = idx & 7;
      const uint16_t* src = pool + row_index(c.page_table, c.max_pages, c.page_size, b, t0 + t) * kW + kDc + 8 * q;
      const u32x4 x = *reinterpret_cast<const u32x4*>(src);
      u32x4 y;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        y[k] = f16_bits(__uint_as_float(x[k] << 16)) | (f16_bits(__uint_as_float(x[k] & 0xffff0000u)) << 16);
      *reinterpret_cast<u32x4*>(kr_out + (size_t(b) * max_len + t0 + t) * kDr + 8 * q) = y;
    }
  }
}

// ------------------------------------------------------------------------------- attention
constexpr int kAtQ = 128;                    // queries per workgroup (4 waves x 32)
constexpr int kAtT = 32;                     // tokens per tile
constexpr int kTileKB = kAtT * kRowB;        // 8 KiB of K
constexpr int kTileRB = kAtT * kDr * 2;      // 4 KiB of k^R
constexpr int kTileB = 2 * kTileKB + kTileRB;  // K | V | k^R: 20 KiB
constexpr int kAtBuf = 4;                      // LDS tile buffers: one in use, three in flight
constexpr int kAtXfer = kTileB / 1024 / 4;     // 5 one-KiB transfers per wave per tile
constexpr float kPShift = 7.f;                 // log2 of the probability scale
constexpr float kLag = 8.f;                     // the reference may trail a query's maximum by this much

// K, V and k^R tile rows use the swizzles of the decompression section above.

struct RopeTab {
  double v[kDr / 2];
};

__global__ __launch_bounds__(256, 2) void attend_unabsorbed_kernel(
    int batch, const int32_t* __restrict__ seq_lens, int cap, int max_len, const uint16_t* __restrict__ q_c,
    const uint16_t* __restrict__ q_r, const int32_t* __restrict__ q_start, int q_len, float qscale, RopeTab rope,
    const uint16_t* __restrict__ k_in, const uint16_t* __restrict__ v_in, const uint16_t* __restrict__ kr_in,
    float* __restrict__ out, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kAtBuf * kTileB];  // 80 KiB
  lds_u8* const lbase = (lds_u8*)smem;
  // group = (sequence, head) (its keys and values), members = 128-query blocks
  int grp, qb;
  if (!xcd_group_map((q_len + kAtQ - 1) / kAtQ, batch * kH, grp, qb)) return;
  const int h = grp % kH, b = grp / kH;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, hi = lane >> 5, g = lane >> 4, ii = lane & 15;
  // workgroup- and wave-uniform values kept in scalar registers, so that the tile loop and its
  // per-tile decisions stay scalar branches instead of masked vector code
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int len = __builtin_amdgcn_readfirstlane(min(seq_lens[b], cap));
  const int qs = __builtin_amdgcn_readfirstlane(q_start[b]);
  const int q0 = kAtQ * qb;  // first query of the workgroup (chunk index)
  if (q0 >= q_len) return;
  const int qi = q0 + 32 * wave + (lane & 31);  // this lane's query (chunk index)
  const bool qvalid = qi < q_len;
  const int qpos = qs + min(qi, q_len - 1);     // its absolute position
  // keys visible to the workgroup: t < min(len, qs + q0 + 128); to this wave: < min(len, qs + q0w + 32)
  const int t_end = min(len, max(qs + min(q0 + kAtQ, q_len), 0));
  const int ntiles = (t_end + kAtT - 1) / kAtT;

  // ---- Q^T operand (B of the score MFMA): query qi, k = 16ks + 8hi .. +7, in binary16; the
  // content part is q_c as stored (bf16 values from 2^-17 to 65504 are binary16 values), the rotary
  // part is rotated here at qpos and rounded once; the scale sm_scale*log2(e) is applied to the
  // float scores instead
  f16x8 qf[12];
  {
    const size_t qrow = (size_t(b) * q_len + min(qi, q_len - 1)) * kH + h;
    const uint16_t* qcp = q_c + qrow * kDk + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(qcp + 16 * ks);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        qf[ks][2 * k] = (_Float16)__uint_as_float(x[k] << 16);
        qf[ks][2 * k + 1] = (_Float16)__uint_as_float(x[k] & 0xffff0000u);
      }
    }
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
        qf[8 + ks][2 * k] = (_Float16)(x1 * cs - x2 * sn);
        qf[8 + ks][2 * k + 1] = (_Float16)(x1 * sn + x2 * cs);
      }
    }
  }

  // ---- tile transfers: transfer T = 5*wave + x (x < 5) of a tile moves 1 KiB: T < 8 K rows
  // 4T..4T+3, T < 16 V rows 4(T-8).., else k^R rows 8(T-16)..+7.  Lane L fills LDS chunk L of the
  // transfer; the global chunk it reads is the one the swizzle places there.  Rows past the
  // sequence end copy row len-1 (finite; their scores are masked, so their weight is 0).
  const uint16_t* const kbase = k_in + (size_t(b) * kH + h) * max_len * kDk;
  const uint16_t* const vbase = v_in + (size_t(b) * kH + h) * max_len * kDk;
  const uint16_t* const rbase = kr_in + size_t(b) * max_len * kDr;
  const uint32_t lds0 = uint32_t(reinterpret_cast<uintptr_t>(lbase));
  auto dma_tile = [&](int j, int buf) {  // tile j into LDS buffer buf
    const int tt0 = kAtT * j;
    const uint32_t dst = lds0 + uint32_t(buf * kTileB);
#pragma unroll
    for (int x = 0; x < kAtXfer; ++x) {
      const int T = kAtXfer * __builtin_amdgcn_readfirstlane(wave) + x;
      if (T < 16) {
        const int r = 4 * (T & 7) + (lane >> 4), c = (lane & 15) ^ kv_swz(r);
        const uint32_t voff = uint32_t(min(tt0 + r, len - 1) * kRowB + 16 * c);
        dma16(dst + uint32_t(T * 1024), voff, T < 8 ? kbase : vbase);
      } else {
        const int r = 8 * (T - 16) + (lane >> 3), c = (lane & 7) ^ kr_swz(r);
        const uint32_t voff = uint32_t(min(tt0 + r, len - 1) * (kDr * 2) + 16 * c);
        dma16(dst + uint32_t(T * 1024), voff, rbase);
      }
    }
  };
  // score A operand (rows = tokens): row lane%32, logical chunk 2ks + hi
  const int sr = lane & 31;
  auto s_op = [&](const lds_u8* tb, int ks) -> f16x8 {
    if (ks < 8) return lds16h(tb + sr * kRowB + 16 * ((2 * ks + hi) ^ kv_swz(sr)));
    return lds16h(tb + 2 * kTileKB + sr * (kDr * 2) + 16 * ((2 * (ks - 8) + hi) ^ kr_swz(sr)));
  };
  // weighted-sum A operand V^T for value block db, k-step s: tokens 16s + 4*(g/2) + (lane%16)/4 and
  // +8, value columns 32db + 16(g%2) + 4(lane%4) .. +3 (the token order of the score layout)
  auto v_op = [&](const lds_u8* tb, int s, int db) -> f16x8 {
    const int r = 16 * s + 4 * (g >> 1) + (ii >> 2);
    const int col = 32 * db + 16 * (g & 1) + 4 * (ii & 3);
    const lds_u8* vb = tb + kTileKB;
    return tr_pair_h(vb + r * kRowB + 16 * ((col >> 3) ^ kv_swz(r)) + 2 * (col & 7),
                     vb + (r + 8) * kRowB + 16 * ((col >> 3) ^ kv_swz(r + 8)) + 2 * (col & 7));
  };

  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int x = 0; x < 16; ++x) acc[db][x] = 0.f;
  float m_run = -INFINITY, l_lane = 0.f;

  // tiles 0..2 in flight before the loop; past the last tile the transfers repeat it (into a
  // buffer nobody reads), which keeps every wait count uniform
  if (ntiles > 0) {
#pragma unroll
    for (int k = 0; k < kAtBuf - 1; ++k) dma_tile(min(k, ntiles - 1), k);
  }
  for (int j = 0; j < ntiles; ++j) {
    // own transfers of tile j done (tiles j+1, j+2 may fly); the barrier makes every wave's part
    // visible and frees the buffer of tile j-1 for tile j+3
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kAtXfer) : "memory");
    __syncthreads();
    dma_tile(min(j + kAtBuf - 1, ntiles - 1), (j + kAtBuf - 1) % kAtBuf);
    const lds_u8* const tb = lbase + (j % kAtBuf) * kTileB;
    const int tt0 = kAtT * j;
    // Every wave scores every tile: tiles past a wave's last query are fully masked (weight 0).
    // Skipping them behind a branch made the compiler copy the accumulators and the softmax
    // state at every loop edge, which cost more than the few masked tiles of the diagonal block.
    {
      f32x16 s;
#pragma unroll
      for (int x = 0; x < 16; ++x) s[x] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 12; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_f16(s_op(tb, ks), qf[ks], s, 0, 0, 0);
#pragma unroll
      for (int x = 0; x < 16; ++x) s[x] *= qscale;  // base-2 logits
      // mask: tokens past the query's position or the sequence end
      if (tt0 + kAtT - 1 > qs + q0 + 32 * wv || tt0 + kAtT > len) {
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
      // the reference m_run moves (and the running sums are rescaled by exp2(old - new)) only
      // where a query's maximum climbs more than kLag above it, which after the first tiles is
      // rare: the rescale is skipped when no lane of the wave needs it (a uniform branch), and
      // inside it the factor is 1 for the other lanes (-inf: no key visible yet)
      const float m_new = fmaxf(m_run, mx);
      const bool move = m_new > m_run + kLag;
      if (__builtin_amdgcn_ballot_w64(move)) {
        const float alpha = move ? fast_exp2(m_run - m_new) : 1.f;
        l_lane *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int x = 0; x < 16; ++x) acc[db][x] *= alpha;
        m_run = move ? m_new : m_run;
      }
      // probabilities times 2^kPShift relative to the reference: at most 2^(kPShift + kLag) =
      // 2^15, inside binary16, and weights far below the maximum stay normal numbers; the factor
      // cancels in out and is taken off lse
      float p[16], tsum = 0.f;
      const float m_use = (m_run == -INFINITY ? 0.f : m_run) - kPShift;  // (no visible key yet: 0)
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        p[x] = fast_exp2(s[x] - m_use);
        tsum += p[x];
      }
      l_lane += tsum;
      f16x8 pb0, pb1;
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        pb0[x] = (_Float16)p[x];
        pb1[x] = (_Float16)p[8 + x];
      }
#pragma unroll
      for (int sk = 0; sk < 2; ++sk)
#pragma unroll
        for (int db = 0; db < 4; ++db)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(v_op(tb, sk, db), sk ? pb1 : pb0, acc[db], 0, 0, 0);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no transfer outlives the workgroup

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
  if (lse && hi == 0)
    lse[(size_t(b) * q_len + qi) * kH + h] = empty ? -INFINITY : (m_run + (log2f(l_tot) - kPShift)) * kLn2;
}

}  // namespace

bool prefill_unabsorbed_supported(const Dims& d) {
  return d.dtype == MLA_BF16 && d.H == kH && d.dc == kDc && d.dr == kDr && d.dk == kDk && d.dv == kDk;
}

hipError_t launch_decompress_kv(const Dims& d, const Cache& c, int max_len, const void* w_uk, const void* w_uv,
                                void* k_out, void* v_out, void* kr_out, hipStream_t s) {
  (void)d;
  const int ntb = (max_len + kDcTok - 1) / kDcTok;
  decompress_kv_kernel<<<dim3(xcd_group_grid(ntb * c.batch, kH)), 256, 0, s>>>(c, max_len, static_cast<const uint16_t*>(w_uk),
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
  const dim3 grid(xcd_group_grid((q_len + kAtQ - 1) / kAtQ, c.batch * kH));
  attend_unabsorbed_kernel<<<grid, 256, 0, s>>>(c.batch, c.seq_lens, c.max_pages * c.page_size, max_len,
                                                static_cast<const uint16_t*>(q_c), static_cast<const uint16_t*>(q_r),
                                                q_start, q_len, qscale, rope, static_cast<const uint16_t*>(k),
                                                static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(kr), out,
                                                lse);
  return hipGetLastError();
}

}  // namespace mla
