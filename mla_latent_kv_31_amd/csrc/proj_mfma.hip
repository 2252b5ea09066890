// Per-head projections on bf16 MFMA (gfx950): the absorbed query and the value up-projection.
//
// mla_absorb_query ([ase] "Key 투영을 Query 쪽으로 옮기기", Fig. 3 equation):
//   q_hat[r,h,j] = (sum_k q_c[r,h,k] W_UK[h,j,k]) * qscale,  j < d_c
//   q_hat[r,h,d_c+2i, d_c+2i+1] = rotation of (q_r[r,h,2i], q_r[r,h,2i+1]) by pos[r]*base^(-2i/d_r), * qscale
// (q_hat stored in IEEE binary16), computed transposed, q_hat^T = W_UK[h] . q_c^T, so that W_UK
// rows (contiguous over k) are the A operand and query rows (contiguous over k) the B operand, both
// straight from global memory, and the output tile is assembled in LDS and written as whole rows.  One workgroup per (head, 64
// query rows), all workgroups of a head on one XCD.
//
// mla_out_proj ([ase] "Value 투영을 가중합 뒤로 옮기기", Fig. 4 equation):
//   out[r,h,v] = sum_j z[r,h,j] W_UV[h,j,v]
// computed as out^T = W_UV[h]^T . z^T.  The contraction runs over j, the row index of W_UV, so
// the A operand comes from W_UV staged in LDS through the transposing ds_read_b64_tr_b16; the
// four waves of a workgroup split j.  Up to 256 rows: one workgroup per (head, 64 value columns,
// 32 or 64 rows); beyond that one workgroup per (head, 64 value columns) streams every row slice.
// z is float32: it is split into bf16 hi + lo parts and both are multiplied (two MFMAs), which
// keeps the product at float32-level accuracy.
//
// mla_combine_out_proj (+ _balanced, _grouped): the split-K log-sum-exp merge and the value
// projection in one kernel, out = (sum_i exp(lse_i - LSE) o_i) . W_UV[h], with the same product as
// mla_out_proj and the merged latent kept in registers.

#include <math.h>

#include "common.h"
#include "launch.h"
#include "schedule.h"

namespace mla {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kDc = 512, kDk = 128, kDv = 128;
constexpr int kMaxDr = 64;   // the absorb output tile: 64 rows x (512 + 64) bf16 = 72 KiB of LDS

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

// ---------------------------------------------------------------------------------------- absorb

// Workgroups are dispatched round-robin over the 8 XCDs, each with its own L2.  All workgroups of
// head h are placed on XCD h % 8 (linear id = 8k + h % 8), so the operands they share (the head's
// weight slices, the query rows of a row slice) are fetched from HBM once per head and then hit
// that XCD's L2.  `per_head` workgroups per head, numbered `inner`.
__device__ __forceinline__ bool xcd_head_map(int per_head, int H, int& h, int& inner) {
  const int id = blockIdx.x, k = id >> 3;
  h = (k / per_head) * 8 + (id & 7);
  inner = k % per_head;
  return h < H;
}
__host__ inline int xcd_grid(int per_head, int H) { return 8 * ((H + 7) / 8) * per_head; }

// One workgroup per (head h, 32 * RB query rows); 4 waves, wave w computes latent columns
// [128w, 128w + 128) in four 32-column MFMA blocks, the RB row blocks sharing every A operand
// (RB = 1 for small batches, so that a decode step still spreads over every compute unit).
// The 64 x (d_c + d_r) bf16 output tile, rotary columns included, is assembled in LDS and then
// written as whole contiguous rows of q_hat (64 x 16 B per store instruction).
// RoPE inverse frequencies base^(-2i/d_r), computed on the host in double (kernel argument).
struct RopeFreq {
  double v[kMaxDr / 2];
};

template <int RB, int CS>
__global__ __launch_bounds__(256) void absorb_mfma_kernel(int H, int R, int dr, RopeFreq inv_freq, float qscale,
                                                          const uint16_t* __restrict__ q_c,
                                                          const uint16_t* __restrict__ q_r,
                                                          const uint16_t* __restrict__ w_uk,
                                                          const int32_t* __restrict__ pos, uint16_t* __restrict__ q_hat) {
  __shared__ __attribute__((aligned(16))) unsigned char ab_smem[32 * RB * (kDc + kMaxDr + 8) * 2];
  constexpr int kRows = 32 * RB;
  constexpr int kJB = 4 / CS;             // 32-column blocks per wave
  constexpr int kPartCols = kDc / CS;     // latent columns per workgroup
  const int slices = (R + kRows - 1) / kRows;
  int h, inner;
  if (!xcd_head_map(slices * CS, H, h, inner)) return;
  const int rs = inner / CS, part = inner % CS;
  const bool do_rope = part == 0;         // the first column part also rotates q_R (uniform)
  const int r0 = kRows * rs, nrows = min(kRows, R - r0);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, hi = lane >> 5;
  const int W = kDc + dr;
  const int TW = W + 8;  // LDS row stride: 16 bytes of padding spread the rows over the banks
  typedef __attribute__((address_space(3))) uint16_t lds_u16;
  typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
  lds_u16* const tile = (lds_u16*)ab_smem;
  __shared__ double freq[kMaxDr / 2];  // per-lane indexing of the kernel argument would be a load per use

  // B operands: both row blocks of q_c, loaded once
  bf16x8 bq[RB][kDk / 16];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = r0 + 32 * rb + (lane & 31);
    const uint16_t* qrow = q_c + (size_t(r < R ? r : 0) * H + h) * kDk + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < kDk / 16; ++ks) bq[rb][ks] = r < R ? load_bf16x8(qrow + 16 * ks) : bf16x8{};
  }
  // rotary inputs: thread t handles (row, 4 pairs) items t and t + 256 (at most RB of them), loaded
  // here with everything else so that the workgroup waits for memory once
  const int quads = dr / 8;  // dr is a multiple of 8 here
  u32x4 rin[RB];
  int rpos[RB];
#pragma unroll
  for (int t = 0; t < RB; ++t) {
    const int idx = threadIdx.x + 256 * t, rr = idx / max(quads, 1), qd = idx - rr * max(quads, 1);
    const bool ok = do_rope && idx < nrows * quads;
    const int r = ok ? r0 + rr : r0;
    rin[t] = ok ? *reinterpret_cast<const u32x4*>(q_r + (size_t(r) * H + h) * dr + 8 * qd) : u32x4{0u, 0u, 0u, 0u};
    rpos[t] = ok ? pos[r] : 0;
  }
  double fr = 0.0;  // the frequency table entry this thread stages in LDS
  if (threadIdx.x < kMaxDr / 2) fr = inv_freq.v[threadIdx.x];
  // A operands of this wave's column blocks (latent columns col0 .. col0 + 32 kJB), loaded together
  // with the B operands so that the wave waits for memory once
  const int col0 = kPartCols * part + 32 * kJB * wave;
  const uint16_t* wbase = w_uk + (size_t(h) * kDc + col0 + (lane & 31)) * kDk + 8 * hi;
  bf16x8 a[kJB][kDk / 16];
#pragma unroll
  for (int jb = 0; jb < kJB; ++jb)
#pragma unroll
    for (int ks = 0; ks < kDk / 16; ++ks) a[jb][ks] = load_bf16x8(wbase + size_t(32 * jb) * kDk + 16 * ks);
  // an empty asm that reads every loaded value: the compiler would otherwise move loads next to
  // their uses and put several memory latencies in a row on the critical path
#pragma unroll
  for (int jb = 0; jb < kJB; ++jb)
#pragma unroll
    for (int ks = 0; ks < kDk / 16; ++ks) asm volatile("" : "+v"(a[jb][ks]));
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int ks = 0; ks < kDk / 16; ++ks) asm volatile("" : "+v"(bq[rb][ks]));
    asm volatile("" : "+v"(rin[rb]), "+v"(rpos[rb]));
  }
#pragma unroll
  for (int jb = 0; jb < kJB; ++jb) {
    f32x16 acc[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int x = 0; x < 16; ++x) acc[rb][x] = 0.f;
#pragma unroll
    for (int ks = 0; ks < kDk / 16; ++ks)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[jb][ks], bq[rb][ks], acc[rb], 0, 0, 0);
    // D layout: lane holds row 32rb + lane%32 and columns j = col0 + 32jb + 8g + 4hi + 0..3
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      lds_u16* trow = tile + (32 * rb + (lane & 31)) * TW + col0 + 32 * jb + 4 * hi;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 v;
        v[0] = uint32_t(f32_to_f16(acc[rb][4 * g] * qscale)) |
               (uint32_t(f32_to_f16(acc[rb][4 * g + 1] * qscale)) << 16);
        v[1] = uint32_t(f32_to_f16(acc[rb][4 * g + 2] * qscale)) |
               (uint32_t(f32_to_f16(acc[rb][4 * g + 3] * qscale)) << 16);
        *(lds_u32x2*)(trow + 8 * g) = v;
      }
    }
  }
  if (threadIdx.x < kMaxDr / 2) freq[threadIdx.x] = fr;
  __syncthreads();  // the frequency table is visible to every wave
  // rotary columns
#pragma unroll
  for (int t = 0; t < RB; ++t) {
    const int idx = threadIdx.x + 256 * t;
    if (!do_rope || idx >= nrows * quads) break;
    const int rr = idx / quads, qd = idx - rr * quads;
    const u32x4 in = rin[t];
    const double p = double(rpos[t]);
    u32x4 outv;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = 4 * qd + k;
      // angle in double, reduced to [-pi, pi] before the float32 sine/cosine
      const double ang = p * freq[i];
      const double red = ang - 6.283185307179586 * rint(ang * 0.15915494309189535);
      float sn, cs;
      sincosf(float(red), &sn, &cs);
      const float x1 = bf16_to_f32(uint16_t(in[k] & 0xffffu)), x2 = bf16_to_f32(uint16_t(in[k] >> 16));
      outv[k] = uint32_t(f32_to_f16((x1 * cs - x2 * sn) * qscale)) |
                (uint32_t(f32_to_f16((x1 * sn + x2 * cs) * qscale)) << 16);
    }
    *(lds_u32x4*)(tile + rr * TW + kDc + 8 * qd) = outv;
  }
  __syncthreads();
  // write the tile: row rr of the workgroup is q_hat[(r0 + rr) * H + h], this part's latent columns
  // and (first part) the rotary columns
  const int lat_chunks = kPartCols / 8, chunks = lat_chunks + (do_rope ? dr / 8 : 0);
  for (int idx = threadIdx.x; idx < nrows * chunks; idx += blockDim.x) {
    const int rr = idx / chunks, cc = idx % chunks;
    const int c = cc < lat_chunks ? kPartCols / 8 * part + cc : kDc / 8 + (cc - lat_chunks);
    const u32x4 v = *(const lds_u32x4*)(tile + rr * TW + 8 * c);
    *reinterpret_cast<u32x4*>(q_hat + (size_t(r0 + rr) * H + h) * W + 8 * c) = v;
  }
}

// ---------------------------------------------------------------------------------------- out_proj
constexpr int kOpCols = 64;                    // v columns per workgroup
constexpr int kOpRowB = kOpCols * 2;           // 128 bytes per W row slice in LDS
constexpr int kOpJ = kDc / 4;                  // j rows (contraction) per wave
constexpr int kOpWaveB = kOpJ * kOpRowB;       // 16 KiB: a wave's W slice, later its partial sums

// LDS place of 16-byte chunk c (0..7) of W row j: rows j and j+2 sit half a row apart, so that
// the 4-row x 64-byte transposing reads cover all 64 banks.
__device__ __forceinline__ int op_chunk(int j, int c) { return c ^ (((j >> 1) & 1) << 2); }

// z[r][j .. j+7] as a bf16 hi + lo pair (zero for rows past the end)
__device__ __forceinline__ void split_hilo(f32x4 z0, f32x4 z1, bool valid, bf16x8& zh, bf16x8& zl) {
  const float zv[8] = {z0[0], z0[1], z0[2], z0[3], z1[0], z1[1], z1[2], z1[3]};
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    const float v = valid ? zv[x] : 0.f;
    zh[x] = (__bf16)v;
    zl[x] = (__bf16)(v - float(zh[x]));
  }
}

// One workgroup per (head, 64 value columns, 32 * RB rows), a head's workgroups on its XCD so that
// the two column halves of a row slice read the same z rows from that XCD's L2.  The contraction
// over j = 0..511 is split across the 4 waves (128 j each).  Every wave issues all its loads at
// once, its W_UV rows (staged in its own 16 KiB of LDS, which no other wave reads) and its z
// pieces (16 bytes per lane per k-step and row block), so that a workgroup waits for memory once.
// The waves' partial sums then meet in LDS: wave w adds up accumulator w of all four.
template <int RB>
__global__ __launch_bounds__(256) void out_proj_mfma_kernel(int H, int R, const float* __restrict__ z,
                                                            const uint16_t* __restrict__ w_uv,
                                                            float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[4 * kOpWaveB];
  constexpr int kHalves = kDv / kOpCols;
  constexpr int kRows = 32 * RB;
  const int slices = (R + kRows - 1) / kRows;
  int h, inner;
  if (!xcd_head_map(kHalves * slices, H, h, inner)) return;
  const int v0 = kOpCols * (inner % kHalves), r0 = kRows * (inner / kHalves);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, hi = lane >> 5, g = lane >> 4, ii = lane & 15;
  const int j0 = kOpJ * wave;
  lds_u8* const lw = (lds_u8*)smem + wave * kOpWaveB;

  // W_UV[h][j0 .. j0+127][v0 .. v0+63]: 128 rows x 8 chunks of 16 B, 16 per lane
  constexpr int kPer = kOpJ * 8 / 64;
  u32x4 wv[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int c = lane + 64 * k, j = c >> 3, ch = c & 7;
    wv[k] = *reinterpret_cast<const u32x4*>(w_uv + (size_t(h) * kDc + j0 + j) * kDv + v0 + 8 * ch);
  }
  // z pieces: row r0 + 32rb + lane%32, j = j0 + 16ks + 8hi .. +7
  f32x4 zr[RB][kOpJ / 16][2];
  bool valid[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = r0 + 32 * rb + (lane & 31);
    valid[rb] = r < R;
    const float* zp = z + (size_t(valid[rb] ? r : 0) * H + h) * kDc + j0 + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < kOpJ / 16; ++ks) {
      zr[rb][ks][0] = *reinterpret_cast<const f32x4*>(zp + 16 * ks);
      zr[rb][ks][1] = *reinterpret_cast<const f32x4*>(zp + 16 * ks + 4);
    }
  }
  // an empty asm that reads every loaded value keeps the compiler from sinking loads towards their
  // uses (which would put one memory latency per k-step on the critical path)
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int ks = 0; ks < kOpJ / 16; ++ks) asm volatile("" : "+v"(zr[rb][ks][0]), "+v"(zr[rb][ks][1]));
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int c = lane + 64 * k, j = c >> 3, ch = c & 7;
    *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(lw + j * kOpRowB + 16 * op_chunk(j, ch)) = wv[k];
  }
  // (a wave reads only what it wrote itself: LDS operations of one wave complete in order)

  // out^T[v][r] = W_UV^T[v][j] . z^T[j][r]; A operand by transposing reads: lane group g covers
  // j rows 8*(g/2) + (lane%16)/4 (+4 for the second read), v columns 32vb + 16(g%2) + 4(lane%4)
  f32x16 acc[2][RB];
#pragma unroll
  for (int vb = 0; vb < 2; ++vb)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int x = 0; x < 16; ++x) acc[vb][rb][x] = 0.f;
#pragma unroll
  for (int ks = 0; ks < kOpJ / 16; ++ks) {
    bf16x8 zh[RB], zl[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) split_hilo(zr[rb][ks][0], zr[rb][ks][1], valid[rb], zh[rb], zl[rb]);
#pragma unroll
    for (int vb = 0; vb < 2; ++vb) {
      const int jr = 16 * ks + 8 * (g >> 1) + (ii >> 2), ccol = 32 * vb + 16 * (g & 1) + 4 * (ii & 3);
      const lds_u8* p0 = lw + jr * kOpRowB + 16 * op_chunk(jr, ccol >> 3) + 2 * (ccol & 7);
      const lds_u8* p1 = lw + (jr + 4) * kOpRowB + 16 * op_chunk(jr + 4, ccol >> 3) + 2 * (ccol & 7);
      const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p0);
      const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p1);
      const bf16x8 aw = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        acc[vb][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw, zh[rb], acc[vb][rb], 0, 0, 0);
        acc[vb][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw, zl[rb], acc[vb][rb], 0, 0, 0);
      }
    }
  }

  // partial sums into this wave's LDS (its W slice is no longer read), then wave w finishes
  // accumulator w (vb = w % 2, rb = w / 2) from all four waves
  typedef __attribute__((address_space(3))) f32x4 lds_f4;
#pragma unroll
  for (int vb = 0; vb < 2; ++vb)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(lds_f4*)(lw + ((2 * rb + vb) * 4 + q) * 1024 + 16 * lane) =
            f32x4{acc[vb][rb][4 * q], acc[vb][rb][4 * q + 1], acc[vb][rb][4 * q + 2], acc[vb][rb][4 * q + 3]};
  __syncthreads();
  if (wave >= 2 * RB) return;
  const int vb = wave & 1, rb = wave >> 1;
  const int r = r0 + 32 * rb + (lane & 31);
  if (r >= R) return;
  float* o = out + (size_t(r) * H + h) * kDv + v0 + 32 * vb + 4 * hi;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < 4; ++w) sum += *(const lds_f4*)((lds_u8*)smem + w * kOpWaveB + (wave * 4 + q) * 1024 + 16 * lane);
    // D layout: lane holds row lane%32, v = 8q + 4hi + 0..3 of the 32-column block
    *reinterpret_cast<f32x4*>(o + 8 * q) = sum;
  }
}

// Large row counts (prefill chunks): one workgroup per (head, 64 value columns) streams every row
// slice of 32 through a W_UV slice staged once.  Each wave owns 128 of the 512 j (its W rows in
// its own LDS) and keeps the z pieces of the next slice in flight while it multiplies the current
// one; the four partial sums of a slice meet in one of two LDS buffers and waves 0 and 1 finish
// the two 32-column halves.  z is read once per column half, the second time from the XCD's L2.
constexpr int kOpPartB = 4 * 2 * 16 * 64 * 4;  // partial sums of one slice: 4 waves x 8 KiB

__global__ __launch_bounds__(256) void out_proj_stream_kernel(int H, int R, const float* __restrict__ z,
                                                              const uint16_t* __restrict__ w_uv,
                                                              float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[4 * kOpWaveB + 2 * kOpPartB];  // 128 KiB
  constexpr int kHalves = kDv / kOpCols;
  int h, inner;
  if (!xcd_head_map(kHalves, H, h, inner)) return;
  const int v0 = kOpCols * inner;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, hi = lane >> 5, g = lane >> 4, ii = lane & 15;
  const int j0 = kOpJ * wave;
  lds_u8* const lw = (lds_u8*)smem + wave * kOpWaveB;
  lds_u8* const lpart = (lds_u8*)smem + 4 * kOpWaveB;
  typedef __attribute__((address_space(3))) f32x4 lds_f4;

  constexpr int kPer = kOpJ * 8 / 64;
  u32x4 wv[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int c = lane + 64 * k, j = c >> 3, ch = c & 7;
    wv[k] = *reinterpret_cast<const u32x4*>(w_uv + (size_t(h) * kDc + j0 + j) * kDv + v0 + 8 * ch);
  }
  const int slices = (R + 31) / 32;
  auto load_z = [&](f32x4 (&zr)[kOpJ / 16][2], int s) {
    const int r = 32 * s + (lane & 31);
    const float* zp = z + (size_t(r < R ? r : 0) * H + h) * kDc + j0 + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < kOpJ / 16; ++ks) {
      zr[ks][0] = *reinterpret_cast<const f32x4*>(zp + 16 * ks);
      zr[ks][1] = *reinterpret_cast<const f32x4*>(zp + 16 * ks + 4);
    }
  };
  f32x4 za[kOpJ / 16][2], zb[kOpJ / 16][2];
  load_z(za, 0);
  // wait for the first slice here, together with the W_UV slice (an empty asm that reads the
  // values), rather than letting the compiler move these loads behind the LDS staging
#pragma unroll
  for (int ks = 0; ks < kOpJ / 16; ++ks) asm volatile("" : "+v"(za[ks][0]), "+v"(za[ks][1]));
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int c = lane + 64 * k, j = c >> 3, ch = c & 7;
    *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(lw + j * kOpRowB + 16 * op_chunk(j, ch)) = wv[k];
  }

  // one slice: multiply the z pieces in `zc` (slice s) while those of slice s+1 load into `zn`.
  // The loads are unconditional (past the end they repeat the last slice) so that the in-order
  // wait counts only ever wait for the slice being multiplied.  `buf` alternates the partial-sum
  // buffers.
  auto slice = [&](f32x4 (&zc)[kOpJ / 16][2], f32x4 (&zn)[kOpJ / 16][2], int s, int buf) {
    load_z(zn, min(s + 1, slices - 1));
    __builtin_amdgcn_sched_barrier(0);  // issue them before the multiplications, not after
    const bool valid = 32 * s + (lane & 31) < R;
    f32x16 acc[2];
#pragma unroll
    for (int vb = 0; vb < 2; ++vb)
#pragma unroll
      for (int x = 0; x < 16; ++x) acc[vb][x] = 0.f;
#pragma unroll
    for (int ks = 0; ks < kOpJ / 16; ++ks) {
      bf16x8 zh, zl;
      split_hilo(zc[ks][0], zc[ks][1], valid, zh, zl);
#pragma unroll
      for (int vb = 0; vb < 2; ++vb) {
        const int jr = 16 * ks + 8 * (g >> 1) + (ii >> 2), ccol = 32 * vb + 16 * (g & 1) + 4 * (ii & 3);
        const lds_u8* p0 = lw + jr * kOpRowB + 16 * op_chunk(jr, ccol >> 3) + 2 * (ccol & 7);
        const lds_u8* p1 = lw + (jr + 4) * kOpRowB + 16 * op_chunk(jr + 4, ccol >> 3) + 2 * (ccol & 7);
        const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p0);
        const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p1);
        const bf16x8 aw = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw, zh, acc[vb], 0, 0, 0);
        acc[vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw, zl, acc[vb], 0, 0, 0);
      }
    }
    lds_u8* const part = lpart + buf * kOpPartB;
#pragma unroll
    for (int vb = 0; vb < 2; ++vb)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(lds_f4*)(part + ((wave * 2 + vb) * 4 + q) * 1024 + 16 * lane) =
            f32x4{acc[vb][4 * q], acc[vb][4 * q + 1], acc[vb][4 * q + 2], acc[vb][4 * q + 3]};
    // every partial of this slice written; the other buffer, used by the slice before, fully read
    __syncthreads();
    if (wave < 2) {
      const int r = 32 * s + (lane & 31);
      if (r < R) {
        float* o = out + (size_t(r) * H + h) * kDv + v0 + 32 * wave + 4 * hi;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int w = 0; w < 4; ++w) sum += *(const lds_f4*)(part + ((w * 2 + wave) * 4 + q) * 1024 + 16 * lane);
          *reinterpret_cast<f32x4*>(o + 8 * q) = sum;
        }
      }
    }
  };
  // slices in pairs; an odd count repeats the last slice, which stores the same rows again
  for (int s = 0; s < slices; s += 2) {
    slice(za, zb, s, 0);
    slice(zb, za, min(s + 1, slices - 1), 1);
  }
}

// ------------------------------------------------------------------- split-K merge + out_proj
// out[b,h,:] = (sum_i exp(lse_i - LSE) o_i) . W_UV[h], LSE = ln sum_i exp(lse_i), over the split-K
// slots i of row b ([ase] Fig. 2 softmax merged piecewise, then the Fig. 4 value projection): the
// merge of mla_combine_* and the product of mla_out_proj in one pass, so that the merged latent z
// never goes through memory.  One workgroup of eight waves per (head h, 32 rows), all 128 value
// columns; the workgroups of a head sit on its XCD, which fetches W_UV[h] from HBM once.  Wave w
// owns the contraction slice j = 64w .. 64w + 63: its W_UV rows (16 KiB) stream into its own LDS
// by direct global-to-LDS transfers while the wave merges, for row r0 + lane % 32, the 32 values
// z[j0 + 16ks + 8hi .. +7] (ks = 0..3) over that row's slots, four slots' loads in flight (the
// first four issued together with the log-sum-exp loads, before the weights are known).  The
// merged values are split into bf16 hi + lo parts and multiplied as in out_proj; the eight
// slices' sums meet in LDS.  Slots of zero weight (empty chunks, never written) are loaded but
// dropped by a select, so whatever bits they hold never reach the output.
constexpr int kCpRows = 32;                 // rows per workgroup
constexpr int kCpWaves = 8;
constexpr int kCpJ = kDc / kCpWaves;        // 64 contraction rows per wave
constexpr int kCpKs = kCpJ / 16;            // 4 MFMA k-steps per wave
constexpr int kCpSlots = 3;                 // slots per load round
constexpr int kCpRowB = kDv * 2;            // 256 bytes: one W_UV row in LDS
constexpr int kCpWaveB = kCpJ * kCpRowB;    // 16 KiB: a wave's W_UV rows, later its partial sums

// LDS chunk position of 16-byte chunk c of W_UV row j (j taken within a wave's rows): the
// 4-row x 32-byte transposing reads then fall into four different 32-byte bank groups.
__device__ __forceinline__ int cp_chunk(int j, int c) { return c ^ (2 * (j & 3)); }

__device__ __forceinline__ void cp_dma16(uint32_t lds_dst, uint32_t voff, const unsigned char* gbase) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_dst), "v"(voff), "s"(gbase)
               : "memory");
}

// kBalanced: S = n_units and `group` the row-group size of the balanced split (schedule.h);
// otherwise S = n_splits and row b's slots are b*S .. b*S+S-1.
template <bool kBalanced>
__global__ __launch_bounds__(64 * kCpWaves) void combine_out_proj_kernel(
    int H, int S, int group, const int32_t* __restrict__ seq_lens, int batch, int cap,
    const float* __restrict__ o_part, const float* __restrict__ lse_part, const uint16_t* __restrict__ w_uv,
    float* __restrict__ out, float* __restrict__ lse_out) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kCpWaves * kCpWaveB];  // 128 KiB
  int h, inner;
  if (!xcd_head_map((batch + kCpRows - 1) / kCpRows, H, h, inner)) return;
  // the wave index as a wave-uniform value: the transfer addresses below live in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, hi = lane >> 5, g = lane >> 4, ii = lane & 15;
  const int j0 = kCpJ * wave;
  lds_u8* const lw = (lds_u8*)smem + wave * kCpWaveB;

  // ---- the slots of row r: base, base + step, ... (count of them)
  const int r = kCpRows * inner + (lane & 31);
  const bool valid = r < batch;
  const int b = valid ? r : batch - 1;
  int base = b * S, count = valid ? S : 0, step = 1;
  if constexpr (kBalanced) {
    const int n_groups = batch / group, grp = b / group, gi = b - grp * group;
    const int tiles = sched_tiles(sched_len(seq_lens[b], cap));  // this row's own tiles
    // cost prefix of this lane's group and the total cost, in one wave-wide scan over the groups
    int total = 0, cb = 0;
    for (int c0 = 0; c0 < n_groups; c0 += 64) {
      const int i = c0 + lane;
      const int c = i < n_groups ? sched_cost(sched_group_len(seq_lens, i, group, cap)) : 0;
      int incl = c;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
      }
      const int src = grp - c0;
      const int ex = __shfl(incl - c, src & 63, 64);
      if (src >= 0 && src < 64) cb = total + ex;
      total += __shfl(incl, 63, 64);
    }
    base = 0;
    count = 0;
    if (valid && tiles > 0) {
      int w0, w1;
      sched_units(cb, tiles, sched_quota(total, S / group), w0, w1);
      base = sched_slot(w0, grp, group, gi);
      count = w1 - w0 + 1;
      step = group;
    }
  }
  int maxc = count;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) maxc = max(maxc, __shfl_xor(maxc, o, 64));
  const float* lp = lse_part + size_t(base) * H + h;
  const size_t lstride = size_t(step) * H;
  const float* op = o_part + (size_t(base) * H + h) * kDc + j0 + 8 * hi;
  const size_t ostride = size_t(step) * H * kDc;

  // one round: the lse and z pieces of slots s0 .. s0 + kCpSlots - 1 (clamped to the row's last
  // slot, so that every load stays inside the row's own slots)
  f32x4 x[kCpSlots][kCpKs][2];
  float xl[kCpSlots];
  auto load_round = [&](int s0) {
#pragma unroll
    for (int k = 0; k < kCpSlots; ++k) {
      const int s = min(s0 + k, max(count - 1, 0));
      xl[k] = lp[s * lstride];
      const float* p = op + s * ostride;
#pragma unroll
      for (int ks = 0; ks < kCpKs; ++ks) {
        x[k][ks][0] = *reinterpret_cast<const f32x4*>(p + 16 * ks);
        x[k][ks][1] = *reinterpret_cast<const f32x4*>(p + 16 * ks + 4);
      }
    }
  };
  load_round(0);

  // ---- this wave's W_UV rows, in flight while the slots are merged: 16 transfers of four 256-byte
  // rows; lane L fills LDS chunk L % 16 of row 4t + L / 16 with the global chunk cp_chunk places there
  {
    const unsigned char* src = reinterpret_cast<const unsigned char*>(w_uv + (size_t(h) * kDc + j0) * kDv);
    const uint32_t dst = uint32_t(reinterpret_cast<uintptr_t>(lw));
    const uint32_t voff = uint32_t(kCpRowB * g + 16 * cp_chunk(g, ii));
#pragma unroll
    for (int t = 0; t < kCpJ / 4; ++t) cp_dma16(dst + 1024u * t, voff, src + size_t(1024) * t);
  }

  // ---- log-sum-exp weights of the row's slots (the first eight loaded at once)
  constexpr int kL = 8;
  float lv[kL];
#pragma unroll
  for (int k = 0; k < kL; ++k) lv[k] = k < count ? lp[k * lstride] : -INFINITY;
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < kL; ++k) mx = fmaxf(mx, lv[k]);
  for (int s = kL; s < count; ++s) mx = fmaxf(mx, lp[s * lstride]);
  float tot = 0.f;
  if (mx != -INFINITY) {
#pragma unroll
    for (int k = 0; k < kL; ++k) tot += k < count ? expf(lv[k] - mx) : 0.f;
    for (int s = kL; s < count; ++s) tot += expf(lp[s * lstride] - mx);
  }
  const float inv = mx != -INFINITY ? 1.f / tot : 0.f;
  if (lse_out && wave == 0 && hi == 0 && valid)
    lse_out[size_t(r) * H + h] = mx != -INFINITY ? mx + logf(tot) : -INFINITY;

  // ---- z pieces of this row and contraction slice, merged over the slots
  f32x4 za[kCpKs][2];
#pragma unroll
  for (int ks = 0; ks < kCpKs; ++ks) za[ks][0] = za[ks][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0;;) {
#pragma unroll
    for (int k = 0; k < kCpSlots; ++k) {
      const float wk = s0 + k < count && mx != -INFINITY ? expf(xl[k] - mx) * inv : 0.f;
      const bool use = wk != 0.f;
#pragma unroll
      for (int ks = 0; ks < kCpKs; ++ks)
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int q = 0; q < 4; ++q) za[ks][e][q] = use ? fmaf(wk, x[k][ks][e][q], za[ks][e][q]) : za[ks][e][q];
    }
    s0 += kCpSlots;
    if (s0 >= maxc) break;
    load_round(s0);
  }

  // ---- out^T[v][r] = W_UV^T[v][j] . z^T[j][r] over this wave's slice, as in out_proj
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's W_UV rows have landed
  f32x16 acc[4];
#pragma unroll
  for (int vb = 0; vb < 4; ++vb)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[vb][e] = 0.f;
#pragma unroll
  for (int ks = 0; ks < kCpKs; ++ks) {
    bf16x8 zh, zl;
    split_hilo(za[ks][0], za[ks][1], true, zh, zl);
#pragma unroll
    for (int vb = 0; vb < 4; ++vb) {
      const int jr = 16 * ks + 8 * (g >> 1) + (ii >> 2), ccol = 32 * vb + 16 * (g & 1) + 4 * (ii & 3);
      const lds_u8* p0 = lw + jr * kCpRowB + 16 * cp_chunk(jr, ccol >> 3) + 2 * (ccol & 7);
      const lds_u8* p1 = lw + (jr + 4) * kCpRowB + 16 * cp_chunk(jr + 4, ccol >> 3) + 2 * (ccol & 7);
      const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p0);
      const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p1);
      const bf16x8 aw = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
      acc[vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw, zh, acc[vb], 0, 0, 0);
      acc[vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw, zl, acc[vb], 0, 0, 0);
    }
  }

  // ---- the eight slices' sums meet in LDS, each wave's in its own (no longer read) W_UV rows;
  // wave w < 4 finishes value block w
  typedef __attribute__((address_space(3))) f32x4 lds_f4;
#pragma unroll
  for (int vb = 0; vb < 4; ++vb)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *(lds_f4*)(lw + (vb * 4 + q) * 1024 + 16 * lane) =
          f32x4{acc[vb][4 * q], acc[vb][4 * q + 1], acc[vb][4 * q + 2], acc[vb][4 * q + 3]};
  __syncthreads();
  if (wave >= 4 || !valid) return;
  float* o = out + (size_t(r) * H + h) * kDv + 32 * wave + 4 * hi;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kCpWaves; ++w)
      sum += *(const lds_f4*)((lds_u8*)smem + w * kCpWaveB + (wave * 4 + q) * 1024 + 16 * lane);
    // D layout: lane holds row lane % 32, v = 8q + 4hi + 0..3 of the 32-column block
    *reinterpret_cast<f32x4*>(o + 8 * q) = sum;
  }
}

}  // namespace

bool proj_mfma_supported(const Dims& d) {
  // the LDS output tile of the absorb kernel holds 64 rows of d_c + d_r <= 576 values
  return d.dtype == MLA_BF16 && d.dc == kDc && d.dk == kDk && d.dv == kDv && d.dr % 8 == 0 && d.dr <= kMaxDr;
}

hipError_t launch_absorb_mfma(const Dims& d, const void* q_c, const void* q_r, const void* w_uk, const int32_t* pos,
                              int rows, void* q_hat, hipStream_t s) {
  const float qscale = d.sm_scale * kLog2e;
  const uint16_t *qc = static_cast<const uint16_t*>(q_c), *qr = static_cast<const uint16_t*>(q_r);
  const uint16_t* wk = static_cast<const uint16_t*>(w_uk);
  RopeFreq inv{};
  for (int i = 0; i < d.dr / 2; ++i) inv.v[i] = pow(double(d.rope_base), -2.0 * i / d.dr);
  if (rows <= 4 * 32)  // small batch: 32-row workgroups, the latent columns split in two halves
    absorb_mfma_kernel<1, 2><<<dim3(xcd_grid(2 * ((rows + 31) / 32), d.H)), 256, 0, s>>>(
        d.H, rows, d.dr, inv, qscale, qc, qr, wk, pos, static_cast<uint16_t*>(q_hat));
  else
    absorb_mfma_kernel<2, 1><<<dim3(xcd_grid((rows + 63) / 64, d.H)), 256, 0, s>>>(
        d.H, rows, d.dr, inv, qscale, qc, qr, wk, pos, static_cast<uint16_t*>(q_hat));
  return hipGetLastError();
}

hipError_t launch_out_proj_mfma(const Dims& d, const float* z, const void* w_uv, int rows, float* out,
                                hipStream_t s) {
  constexpr int kHalves = kDv / kOpCols;
  if (rows <= 4 * 32)  // small batch: 32-row workgroups, so that a decode step fills the chip
    out_proj_mfma_kernel<1><<<dim3(xcd_grid(kHalves * ((rows + 31) / 32), d.H)), 256, 0, s>>>(
        d.H, rows, z, static_cast<const uint16_t*>(w_uv), out);
  else if (rows <= 8 * 32)
    out_proj_mfma_kernel<2><<<dim3(xcd_grid(kHalves * ((rows + 63) / 64), d.H)), 256, 0, s>>>(
        d.H, rows, z, static_cast<const uint16_t*>(w_uv), out);
  else  // prefill chunks: one streaming workgroup per (head, column half)
    out_proj_stream_kernel<<<dim3(xcd_grid(kHalves, d.H)), 256, 0, s>>>(d.H, rows, z,
                                                                        static_cast<const uint16_t*>(w_uv), out);
  return hipGetLastError();
}

hipError_t launch_combine_out_proj(const Dims& d, const Cache* c, int batch, int S, int group, const float* o_part,
                                   const float* lse_part, const void* w_uv, float* out, float* lse, hipStream_t s) {
  const dim3 grid(xcd_grid((batch + kCpRows - 1) / kCpRows, d.H));
  const uint16_t* w = static_cast<const uint16_t*>(w_uv);
  if (c)
    combine_out_proj_kernel<true><<<grid, 64 * kCpWaves, 0, s>>>(d.H, S, group, c->seq_lens, batch,
                                                      c->max_pages * c->page_size, o_part, lse_part, w, out, lse);
  else
    combine_out_proj_kernel<false><<<grid, 64 * kCpWaves, 0, s>>>(d.H, S, 1, nullptr, batch, 0, o_part, lse_part, w, out, lse);
  return hipGetLastError();
}

}  // namespace mla
