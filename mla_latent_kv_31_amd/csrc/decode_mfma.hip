// Split-K flash-decode over the latent cache on bf16 MFMA (gfx950), DeepSeek-V3 shape:
// 128 heads, rows of 576 values = [c^KV (512) | k^R (64)], bf16 cache and q_hat, fp32 accumulate.
//
// One workgroup per (chunk, sequence); four waves, wave w owns heads 32w..32w+31 for the whole
// chunk.  All 128 heads read the same cached rows, so each 64-token tile (73,728 B) is fetched
// from HBM once per workgroup, straight into LDS with 16-byte global_load_lds transfers, double
// buffered so the next tile streams in while the current one is consumed.
//
// Scores ([ase] Fig. 2: content dot plus position dot over the concatenated row) are computed
// transposed, S^T = tile . q_hat^T, with v_mfma_f32_32x32x16_bf16: tokens on M, heads on N, so
// every lane holds the 16 scores of one head and the softmax max/sum stay inside the lane plus
// one v_permlane32_swap between the two lane halves.  The weighted latent sum ([ase] Fig. 4,
// z = a.C, rotary columns never summed) is accumulated transposed as well, O^T += C^T . P^T,
// with the 512 latent columns on M (16 blocks of 32) and heads on N: the per-head rescale of
// the accumulator is again a per-lane scalar.  C^T operands come from ds_read_b64_tr_b16, the
// gfx950 transposing LDS read, so the row-major tile needs no reshuffle.  The token order inside
// each 16-wide MFMA k-step follows the score layout; both operands use the same order.
//
// LDS tile layout: a latent region (64 rows x 1,024 B) followed by a rotary region (64 rows x
// 128 B); inside each 128-byte block the 16-byte chunks are XOR-swizzled by (row & 7), which
// spreads both the score reads (32 rows x 32 B) and the transposing reads (8 rows x 64 B)
// evenly over the banks.  One 1 KiB latent row is exactly one wave-wide 16-byte transfer.
//
// The tile transfers are issued with inline global_load_lds_dwordx4 and waited for explicitly
// (s_waitcnt vmcnt(0) + barrier at the top of each tile): the compiler cannot see that the
// transfer in flight targets the other buffer and would otherwise wait for it before every
// LDS read.  M0 carries the LDS destination; this kernel has no other M0 user.
//
// Softmax uses base-2 logits (q_hat carries sm_scale*log2 e) with a lazily updated reference
// maximum: the accumulator is rescaled only when the running maximum grows by more than
// 2^8, so probabilities stay <= 256 (exact enough in bf16/fp32) and the rescale of the
// 256-register accumulator is rare.

#include <math.h>

#include "common.h"
#include "launch.h"

namespace mla {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

constexpr int kH = 128, kDc = 512, kW = 576;
constexpr int kRowB = kW * 2;                    // 1,152 bytes per cached row
constexpr int kTile = 64;                        // tokens per tile
constexpr int kTileB = kTile * kRowB;            // 73,728 bytes
constexpr int kLatB = kDc * 2;                   // 1,024 latent bytes per row
constexpr int kRopeB = kRowB - kLatB;            // 128 rotary bytes per row
constexpr int kRopeOff = kTile * kLatB;          // rotary region offset inside a tile buffer
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kKSteps = kW / 16;                 // 36 score k-steps
constexpr int kMBlk = kDc / 32;                  // 16 accumulator blocks
constexpr float kRescaleThreshold = 8.0f;

__device__ __forceinline__ float lane_swap_max(float v) {
  // v_permlane32_swap(v, v): lanes < 32 receive the upper half in .y, lanes >= 32 the lower
  // half in .x; the max of both is the max over the lane pair (l, l^32).
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float lane_swap_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// acc *= alpha on an accumulator block that lives in AGPRs, without exposing a VALU use of the
// accumulator to the register allocator (which would otherwise move every loop-carried
// accumulator to VGPRs): read, multiply and write back one AGPR at a time in inline asm.
__device__ __forceinline__ void scale_acc(f32x16& v, float alpha) {
  float e0 = v[0], e1 = v[1], e2 = v[2], e3 = v[3], e4 = v[4], e5 = v[5], e6 = v[6], e7 = v[7];
  float e8 = v[8], e9 = v[9], e10 = v[10], e11 = v[11], e12 = v[12], e13 = v[13], e14 = v[14], e15 = v[15];
  float t;
#define MLA_SCALE_ONE(n) "v_accvgpr_read_b32 %16, %" #n "\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %" #n ", %16\n\t"
  asm volatile(MLA_SCALE_ONE(0) MLA_SCALE_ONE(1) MLA_SCALE_ONE(2) MLA_SCALE_ONE(3) MLA_SCALE_ONE(4) MLA_SCALE_ONE(5)
               MLA_SCALE_ONE(6) MLA_SCALE_ONE(7) MLA_SCALE_ONE(8) MLA_SCALE_ONE(9) MLA_SCALE_ONE(10)
               MLA_SCALE_ONE(11) MLA_SCALE_ONE(12) MLA_SCALE_ONE(13) MLA_SCALE_ONE(14) MLA_SCALE_ONE(15)
               : "+a"(e0), "+a"(e1), "+a"(e2), "+a"(e3), "+a"(e4), "+a"(e5), "+a"(e6), "+a"(e7), "+a"(e8),
                 "+a"(e9), "+a"(e10), "+a"(e11), "+a"(e12), "+a"(e13), "+a"(e14), "+a"(e15), "=&v"(t)
               : "v"(alpha));
#undef MLA_SCALE_ONE
  v = f32x16{e0, e1, e2, e3, e4, e5, e6, e7, e8, e9, e10, e11, e12, e13, e14, e15};
}

__device__ __forceinline__ bf16x8 pack8(const float* p) {
  bf16x8 r;
#pragma unroll
  for (int x = 0; x < 8; ++x) r[x] = (__bf16)p[x];
  return r;
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_mfma_kernel(const uint16_t* __restrict__ pool, const int32_t* __restrict__ page_table,
                        const int32_t* __restrict__ seq_lens, int max_pages, int page_size,
                        const uint16_t* __restrict__ q_hat, int n_splits, int split_tokens,
                        float* __restrict__ o_part, float* __restrict__ lse_part) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kTileB];
  lds_u8* const lbase = (lds_u8*)smem;

  const int chunk = blockIdx.x, b = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int hi = lane >> 5;
  const int head = wave * 32 + (lane & 31);
  const int len = min(seq_lens[b], max_pages * page_size);  // never index past the page table
  const int t0 = chunk * split_tokens;
  const int t1 = min(t0 + split_tokens, len);
  const size_t orow = (size_t(b) * n_splits + chunk) * kH + head;

  if (t0 >= t1) {  // empty chunk: zero partial, lse = -inf (uniform over the block)
    float4* op = reinterpret_cast<float4*>(o_part + orow * kDc) + hi * (kDc / 8);
#pragma unroll 4
    for (int x = 0; x < kDc / 8; ++x) op[x] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (hi == 0) lse_part[orow] = -INFINITY;
    return;
  }
  const int ntiles = (t1 - t0 + kTile - 1) / kTile;

  // ---- tile loader.  Transfer n < 64 fills latent row n; transfers 64..71 fill rotary rows
  // 8m..8m+7 (m = n - 64).  Lane L writes LDS chunk L of the transfer's 1 KiB; the global chunk
  // it reads is the one that the XOR swizzle places there.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t lat_off[2] = {
      uint32_t(16 * ((lane & ~7) | ((lane ^ (wave_u)) & 7))),
      uint32_t(16 * ((lane & ~7) | ((lane ^ (4 + wave_u)) & 7)))};
  const uint32_t rope_off = uint32_t((lane >> 3) * kRowB + kLatB + 16 * ((lane ^ (lane >> 3)) & 7));
  const uint32_t lds0 = uint32_t(reinterpret_cast<uintptr_t>(lbase));
  auto issue_tile = [&](int k, int buf) {
    const int tok = t0 + k * kTile;
    const int pg = page_table[size_t(b) * max_pages + tok / page_size];
    const unsigned char* g =
        reinterpret_cast<const unsigned char*>(pool + (size_t(pg) * page_size + (tok % page_size)) * kW);
    const uint32_t dst = lds0 + uint32_t(buf * kTileB);
#pragma unroll
    for (int x = 0; x < kTile / kWaves; ++x) {  // 16 latent rows per wave
      const int n = 4 * x + wave_u;
      const unsigned char* gr = g + size_t(n) * kRowB;
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                   :: "s"(dst + uint32_t(n * kLatB)), "v"(lat_off[x & 1]), "s"(gr) : "memory");
    }
#pragma unroll
    for (int x = 0; x < 2; ++x) {  // two blocks of 8 rotary rows per wave
      const int m = 4 * x + wave_u;
      const unsigned char* gr = g + size_t(8 * m) * kRowB;
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                   :: "s"(dst + uint32_t(kRopeOff + m * 1024)), "v"(rope_off), "s"(gr) : "memory");
    }
  };

  issue_tile(0, 0);

  // ---- this wave's 32 heads of q_hat, as the B operand of S^T = tile . q_hat^T
  bf16x8 qf[kKSteps];
  {
    const uint16_t* qrow = q_hat + (size_t(b) * kH + head) * kW + 8 * hi;
#pragma unroll
    for (int k = 0; k < kKSteps; ++k) qf[k] = *reinterpret_cast<const bf16x8*>(qrow + 16 * k);
  }
  // Drain these loads here, where the compiler can see it: otherwise its waits for them land
  // inside the tile loop and would also stall on the tile transfers issued there.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  // ---- per-lane LDS offsets
  // score reads: row 32*blk + (lane&31), logical chunk 2k + hi (latent) or 2(k-32) + hi (rotary)
  int qk_off[4], qr_off[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    qk_off[kk] = (lane & 31) * kLatB + 16 * (((2 * kk + hi) ^ lane) & 7);
    qr_off[kk] = kRopeOff + (lane & 31) * kRopeB + 16 * (((2 * kk + hi) ^ lane) & 7);
  }
  // transposing reads: lane group g = lane/16 reads rows r0 = 4*(g/2) + (lane%16)/4 (+16a, +8),
  // columns 32*mb + 16*(g%2) + 4*(lane%4) .. +3
  const int g = lane >> 4, ii = lane & 15, qq = ii & 3;
  const int r0 = 4 * (g >> 1) + (ii >> 2);
  int pv_off[2];
#pragma unroll
  for (int m1 = 0; m1 < 2; ++m1)
    pv_off[m1] = r0 * kLatB + 16 * ((4 * m1 + 2 * (g & 1) + (qq >> 1)) ^ r0) + 8 * (qq & 1);

  f32x16 acc[kMBlk];
#pragma unroll
  for (int mb = 0; mb < kMBlk; ++mb)
#pragma unroll
    for (int x = 0; x < 16; ++x) acc[mb][x] = 0.f;
  float m_run = -INFINITY, l_lane = 0.f;
  bool started = false;

  for (int k = 0; k < ntiles; ++k) {
    const int buf = k & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's part of tile k has landed
    __syncthreads();                      // every wave's part has landed; tile k-1 fully consumed
    if (k + 1 < ntiles) issue_tile(k + 1, buf ^ 1);
    lds_u8* const tb = lbase + buf * kTileB;
    const int nvalid = min(kTile, t1 - (t0 + k * kTile));
    if (nvalid < kTile) {  // tail tile: latent rows past the sequence end read as zeros
      typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
      const u32x4 zero = {0u, 0u, 0u, 0u};
      for (int x = threadIdx.x; x < (kTile - nvalid) * (kLatB / 16); x += kThreads)
        *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(tb + nvalid * kLatB + 16 * x) = zero;
      __syncthreads();
    }

    // ---- 32-token blocks: scores, online softmax, weighted latent sum
    const int nblk = (nvalid + 31) >> 5;
    for (int blk = 0; blk < nblk; ++blk) {
      lds_u8* const lat = tb + blk * 32 * kLatB;
      lds_u8* const rope = tb + blk * 32 * kRopeB;
      auto a_src = [&](int kk) -> const lds_u8* {
        return kk < kDc / 16 ? lat + 128 * (kk >> 2) + qk_off[kk & 3] : rope + qr_off[kk & 3];
      };
      auto lds16 = [](const lds_u8* p) {
        return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(p);
      };
      // S^T[token, head] = tile . q_hat^T, K = 576 in 36 steps, operand loads kept 3 steps ahead
      f32x16 sacc;
#pragma unroll
      for (int x = 0; x < 16; ++x) sacc[x] = 0.f;
      bf16x8 ab[4];
      ab[0] = lds16(a_src(0));
      ab[1] = lds16(a_src(1));
      ab[2] = lds16(a_src(2));
#pragma unroll
      for (int kk = 0; kk < kKSteps; ++kk) {
        if (kk + 3 < kKSteps) ab[(kk + 3) & 3] = lds16(a_src(kk + 3));
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab[kk & 3], qf[kk], sacc, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }

      // online softmax (base-2 logits); lane = one head, the lane pair (l, l^32) shares it
      if (32 * blk + 32 > nvalid) {
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const int tok = 32 * blk + 8 * (x >> 2) + 4 * hi + (x & 3);
          if (tok >= nvalid) sacc[x] = -INFINITY;
        }
      }
      float mx = sacc[0];
#pragma unroll
      for (int x = 1; x < 16; ++x) mx = fmaxf(mx, sacc[x]);
      mx = lane_swap_max(mx);
      const bool grow = mx > m_run + kRescaleThreshold;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float alpha = grow ? fast_exp2(m_run - mx) : 1.f;
        if (started) {
#pragma unroll
          for (int mb = 0; mb < kMBlk; ++mb) scale_acc(acc[mb], alpha);
        }
        l_lane *= alpha;
        m_run = grow ? mx : m_run;
      }
      started = true;
      float pr[16];
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        pr[x] = fast_exp2(sacc[x] - m_run);
        l_lane += pr[x];
      }
      const bf16x8 pb0 = pack8(&pr[0]);
      const bf16x8 pb1 = pack8(&pr[8]);

      // O^T[col, head] += C^T[col, token] . P^T[token, head]: 2 k-steps x 16 column blocks
      auto tr_src = [&](int i) -> const lds_u8* {  // i = 16 * kstep + mb
        return lat + 16 * (i >> 4) * kLatB + 128 * ((i & 15) >> 1) + pv_off[i & 1];
      };
      auto tr8 = [](const lds_u8* p0) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p0);
        const i16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(p0 + 8 * kLatB));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      bf16x8 cb[4];
      cb[0] = tr8(tr_src(0));
      cb[1] = tr8(tr_src(1));
      cb[2] = tr8(tr_src(2));
#pragma unroll
      for (int i = 0; i < 2 * kMBlk; ++i) {
        if (i + 3 < 2 * kMBlk) cb[(i + 3) & 3] = tr8(tr_src(i + 3));
        acc[i & 15] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cb[i & 3], (i < kMBlk) ? pb0 : pb1, acc[i & 15],
                                                              0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // ---- normalise and write the chunk's partial
  const float l_tot = lane_swap_sum(l_lane);
  const float inv = 1.f / l_tot;
  float* op = o_part + orow * kDc + 4 * hi;
#pragma unroll
  for (int mb = 0; mb < kMBlk; ++mb) {
    const f32x16 v = acc[mb] * inv;
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4)
      *reinterpret_cast<float4*>(op + 32 * mb + 8 * j4) = make_float4(v[4 * j4], v[4 * j4 + 1], v[4 * j4 + 2], v[4 * j4 + 3]);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (hi == 0) lse_part[orow] = (m_run + log2f(l_tot)) * kLn2;
}

}  // namespace

bool decode_mfma_supported(const Dims& d, const Cache& c, int split_tokens) {
  return d.dtype == MLA_BF16 && d.H == kH && d.dc == kDc && d.dr == kW - kDc && c.page_size % kTile == 0 &&
         split_tokens % kTile == 0;
}

hipError_t launch_decode_mfma(const Dims& d, const Cache& c, const void* q_hat, int n_splits, int split_tokens,
                              float* o_part, float* lse_part, hipStream_t s) {
  (void)d;
  decode_mfma_kernel<<<dim3(n_splits, c.batch), kThreads, 0, s>>>(
      static_cast<const uint16_t*>(c.pool), c.page_table, c.seq_lens, c.max_pages, c.page_size,
      static_cast<const uint16_t*>(q_hat), n_splits, split_tokens, o_part, lse_part);
  return hipGetLastError();
}

}  // namespace mla
