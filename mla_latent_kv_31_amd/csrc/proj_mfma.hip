// Per-head projections on bf16 MFMA (gfx950): the absorbed query and the value up-projection.
//
// mla_absorb_query ([ase] "Key 투영을 Query 쪽으로 옮기기", Fig. 3 equation):
//   q_hat[r,h,j] = (sum_k q_c[r,h,k] W_UK[h,j,k]) * qscale,  j < d_c
//   q_hat[r,h,d_c+2i, d_c+2i+1] = rotation of (q_r[r,h,2i], q_r[r,h,2i+1]) by pos[r]*base^(-2i/d_r), * qscale
// computed transposed, q_hat^T = W_UK[h] . q_c^T, so that W_UK rows (contiguous over k) are the
// A operand and query rows (contiguous over k) the B operand, both straight from global memory,
// and the output tile is assembled in LDS and written as whole rows.  One workgroup per (head, 64
// query rows), all workgroups of a head on one XCD.
//
// mla_out_proj ([ase] "Value 투영을 가중합 뒤로 옮기기", Fig. 4 equation):
//   out[r,h,v] = sum_j z[r,h,j] W_UV[h,j,v]
// computed as out^T = W_UV[h]^T . z^T.  The contraction runs over j, the row index of W_UV, so
// the workgroup stages its 512 x 64 slice of W_UV in LDS and reads the A operand with the
// transposing ds_read_b64_tr_b16; one workgroup per (head, 64 value columns, 128 rows).  z is float32: it is split into bf16 hi + lo parts and both are
// multiplied (two MFMAs), which keeps the product at float32-level accuracy.

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
template <int RB>
__global__ __launch_bounds__(256) void absorb_mfma_kernel(int H, int R, int dr, float rope_base, float qscale,
                                                          const uint16_t* __restrict__ q_c,
                                                          const uint16_t* __restrict__ q_r,
                                                          const uint16_t* __restrict__ w_uk,
                                                          const int32_t* __restrict__ pos, uint16_t* __restrict__ q_hat) {
  __shared__ __attribute__((aligned(16))) unsigned char ab_smem[32 * RB * (kDc + kMaxDr + 8) * 2 + kMaxDr / 2 * 8];
  constexpr int kRows = 32 * RB;
  const int slices = (R + kRows - 1) / kRows;
  int h, rs;
  if (!xcd_head_map(slices, H, h, rs)) return;
  const int r0 = kRows * rs, nrows = min(kRows, R - r0);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, hi = lane >> 5;
  const int W = kDc + dr;
  const int TW = W + 8;  // LDS row stride: 16 bytes of padding spread the rows over the banks
  typedef __attribute__((address_space(3))) uint16_t lds_u16;
  typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
  lds_u16* const tile = (lds_u16*)ab_smem;
  __attribute__((address_space(3))) double* const inv_freq =
      (__attribute__((address_space(3))) double*)(ab_smem + kRows * TW * 2);
  for (int i = threadIdx.x; i < dr / 2; i += blockDim.x) inv_freq[i] = pow(double(rope_base), -2.0 * i / dr);

  // B operands: both row blocks of q_c, loaded once
  bf16x8 bq[RB][kDk / 16];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = r0 + 32 * rb + (lane & 31);
    const uint16_t* qrow = q_c + (size_t(r < R ? r : 0) * H + h) * kDk + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < kDk / 16; ++ks) bq[rb][ks] = r < R ? load_bf16x8(qrow + 16 * ks) : bf16x8{};
  }
  // A operands of all four column blocks, loaded together with the B operands so that the wave
  // waits for memory once
  const uint16_t* wbase = w_uk + (size_t(h) * kDc + 128 * wave + (lane & 31)) * kDk + 8 * hi;
  bf16x8 a[4][kDk / 16];
#pragma unroll
  for (int jb = 0; jb < 4; ++jb)
#pragma unroll
    for (int ks = 0; ks < kDk / 16; ++ks) a[jb][ks] = load_bf16x8(wbase + size_t(32 * jb) * kDk + 16 * ks);
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) {
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
    // D layout: lane holds row 32rb + lane%32 and columns j = 128w + 32jb + 8g + 4hi + 0..3
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      lds_u16* trow = tile + (32 * rb + (lane & 31)) * TW + 128 * wave + 32 * jb + 4 * hi;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 v;
        v[0] = uint32_t(f32_to_bf16(acc[rb][4 * g] * qscale)) |
               (uint32_t(f32_to_bf16(acc[rb][4 * g + 1] * qscale)) << 16);
        v[1] = uint32_t(f32_to_bf16(acc[rb][4 * g + 2] * qscale)) |
               (uint32_t(f32_to_bf16(acc[rb][4 * g + 3] * qscale)) << 16);
        *(lds_u32x2*)(trow + 8 * g) = v;
      }
    }
  }
  __syncthreads();  // inv_freq ready
  // rotary columns: one thread per (row, 4 pairs) with 16-byte loads of q_r
  const int quads = dr / 8;  // dr is a multiple of 8 here
  for (int idx = threadIdx.x; idx < nrows * quads; idx += blockDim.x) {
    const int rr = idx / quads, qd = idx % quads, r = r0 + rr;
    const u32x4 in = *reinterpret_cast<const u32x4*>(q_r + (size_t(r) * H + h) * dr + 8 * qd);
    const double p = double(pos[r]);
    u32x4 outv;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = 4 * qd + k;
      // angle in double, reduced to [-pi, pi] before the float32 sine/cosine
      const double ang = p * inv_freq[i];
      const double red = ang - 6.283185307179586 * rint(ang * 0.15915494309189535);
      float sn, cs;
      sincosf(float(red), &sn, &cs);
      const float x1 = bf16_to_f32(uint16_t(in[k] & 0xffffu)), x2 = bf16_to_f32(uint16_t(in[k] >> 16));
      outv[k] = uint32_t(f32_to_bf16((x1 * cs - x2 * sn) * qscale)) |
                (uint32_t(f32_to_bf16((x1 * sn + x2 * cs) * qscale)) << 16);
    }
    *(lds_u32x4*)(tile + rr * TW + kDc + 8 * qd) = outv;
  }
  __syncthreads();
  // write the tile: row rr of the workgroup is q_hat[(r0 + rr) * H + h][0 .. W)
  const int chunks = W / 8;
  for (int idx = threadIdx.x; idx < nrows * chunks; idx += blockDim.x) {
    const int rr = idx / chunks, c = idx % chunks;
    const u32x4 v = *(const lds_u32x4*)(tile + rr * TW + 8 * c);
    *reinterpret_cast<u32x4*>(q_hat + (size_t(r0 + rr) * H + h) * W + 8 * c) = v;
  }
}

// ---------------------------------------------------------------------------------------- out_proj
constexpr int kOpCols = 64;                    // v columns per workgroup
constexpr int kOpRowB = kOpCols * 2;           // 128 bytes per W row slice in LDS
constexpr int kOpLds = kDc * kOpRowB;          // 64 KiB
constexpr int kOpRows = 128;                   // rows per workgroup: 4 blocks of 32, two per wave

// LDS place of 16-byte chunk c (0..7) of W row j: rows j and j+2 sit half a row apart, so that
// the 4-row x 64-byte transposing reads cover all 64 banks.
__device__ __forceinline__ int op_chunk(int j, int c) { return c ^ (((j >> 1) & 1) << 2); }

// z[r][16ks + 8hi .. +7] as a bf16 hi + lo pair (zero for rows past the end)
__device__ __forceinline__ void split_hilo(float4 z0, float4 z1, bool valid, bf16x8& zh, bf16x8& zl) {
  const float zv[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    const float v = valid ? zv[x] : 0.f;
    zh[x] = (__bf16)v;
    zl[x] = (__bf16)(v - float(zh[x]));
  }
}

// 4 waves: wave w owns v block (w & 1) and row blocks (w >> 1) and (w >> 1) + 2 of the
// workgroup's 128 rows; the two row blocks share every A read.
template <bool TWO>
__device__ __forceinline__ void out_proj_rows(const lds_u8* lw, int H, int R, int h, int v0, int vb, int rbA,
                                              const float* __restrict__ z, float* __restrict__ out) {
  const int lane = threadIdx.x & 63, hi = lane >> 5, g = lane >> 4, ii = lane & 15;
  const int rq = ii >> 2, ccol = vb * 32 + 16 * (g & 1) + 4 * (ii & 3);
  auto tr_addr = [&](int j) -> const lds_u8* {
    return lw + j * kOpRowB + 16 * op_chunk(j, ccol >> 3) + 2 * (ccol & 7);
  };
  const int ra = rbA + (lane & 31), rb = ra + 64;
  const bool va = ra < R, vbb = TWO && rb < R;
  const float* za = z + (size_t(va ? ra : 0) * H + h) * kDc + 8 * hi;
  const float* zb = z + (size_t(vbb ? rb : 0) * H + h) * kDc + 8 * hi;
  f32x16 acc0, acc1;
#pragma unroll
  for (int x = 0; x < 16; ++x) acc0[x] = acc1[x] = 0.f;
  constexpr int kPre = TWO ? 4 : 8;  // z steps loaded ahead: enough bytes in flight to cover HBM latency
  float4 ra0[kPre], ra1[kPre], rb0[kPre], rb1[kPre];
#pragma unroll
  for (int p = 0; p < kPre; ++p) {
    ra0[p] = *reinterpret_cast<const float4*>(za + 16 * p);
    ra1[p] = *reinterpret_cast<const float4*>(za + 16 * p + 4);
    if (TWO) {
      rb0[p] = *reinterpret_cast<const float4*>(zb + 16 * p);
      rb1[p] = *reinterpret_cast<const float4*>(zb + 16 * p + 4);
    }
  }
#pragma unroll
  for (int ks = 0; ks < kDc / 16; ++ks) {
    const int jr = 16 * ks + 8 * (g >> 1) + rq;
    const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)tr_addr(jr));
    const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)tr_addr(jr + 4));
    const bf16x8 aw = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
    bf16x8 zh, zl;
    const int sl = ks % kPre;
    split_hilo(ra0[sl], ra1[sl], va, zh, zl);
    if (ks + kPre < kDc / 16) {
      ra0[sl] = *reinterpret_cast<const float4*>(za + 16 * (ks + kPre));
      ra1[sl] = *reinterpret_cast<const float4*>(za + 16 * (ks + kPre) + 4);
    }
    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw, zh, acc0, 0, 0, 0);
    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw, zl, acc0, 0, 0, 0);
    if (TWO) {
      split_hilo(rb0[sl], rb1[sl], vbb, zh, zl);
      if (ks + kPre < kDc / 16) {
        rb0[sl] = *reinterpret_cast<const float4*>(zb + 16 * (ks + kPre));
        rb1[sl] = *reinterpret_cast<const float4*>(zb + 16 * (ks + kPre) + 4);
      }
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw, zh, acc1, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw, zl, acc1, 0, 0, 0);
    }
  }
  if (va) {
    float* o = out + (size_t(ra) * H + h) * kDv + v0 + vb * 32 + 4 * hi;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<float4*>(o + 8 * q) = make_float4(acc0[4 * q], acc0[4 * q + 1], acc0[4 * q + 2], acc0[4 * q + 3]);
  }
  if (vbb) {
    float* o = out + (size_t(rb) * H + h) * kDv + v0 + vb * 32 + 4 * hi;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<float4*>(o + 8 * q) = make_float4(acc1[4 * q], acc1[4 * q + 1], acc1[4 * q + 2], acc1[4 * q + 3]);
  }
}

// One workgroup per (head, 64 value columns, 128 rows), a head's workgroups on its XCD so that the
// two column halves of a row slice read the same z rows from that XCD's L2.
__global__ __launch_bounds__(256) void out_proj_mfma_kernel(int H, int R, const float* __restrict__ z,
                                                            const uint16_t* __restrict__ w_uv,
                                                            float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kOpLds];
  lds_u8* const lw = (lds_u8*)smem;
  constexpr int kHalves = kDv / kOpCols;
  const int slices = (R + kOpRows - 1) / kOpRows;
  int h, inner;
  if (!xcd_head_map(kHalves * slices, H, h, inner)) return;
  const int v0 = kOpCols * (inner % kHalves), rs = inner / kHalves;
  const int wave = threadIdx.x >> 6;
  // stage W_UV[h][:, v0 .. v0+63]: 512 rows x 8 chunks of 16 B, 16 per thread, all loads issued
  // before the first LDS write
  constexpr int kPer = kDc * 8 / 256;
  u32x4 wv[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int c = threadIdx.x + 256 * k, j = c >> 3, ch = c & 7;
    wv[k] = *reinterpret_cast<const u32x4*>(w_uv + (size_t(h) * kDc + j) * kDv + v0 + 8 * ch);
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int c = threadIdx.x + 256 * k, j = c >> 3, ch = c & 7;
    *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(lw + j * kOpRowB + 16 * op_chunk(j, ch)) = wv[k];
  }
  __syncthreads();
  const int rbA = kOpRows * rs + 32 * (wave >> 1);
  if (rbA >= R) return;  // no barrier follows
  if (rbA + 64 < R)
    out_proj_rows<true>(lw, H, R, h, v0, wave & 1, rbA, z, out);
  else
    out_proj_rows<false>(lw, H, R, h, v0, wave & 1, rbA, z, out);
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
  if (rows <= 4 * 32)  // small batch: 32-row workgroups
    absorb_mfma_kernel<1><<<dim3(xcd_grid((rows + 31) / 32, d.H)), 256, 0, s>>>(
        d.H, rows, d.dr, d.rope_base, qscale, qc, qr, wk, pos, static_cast<uint16_t*>(q_hat));
  else
    absorb_mfma_kernel<2><<<dim3(xcd_grid((rows + 63) / 64, d.H)), 256, 0, s>>>(
        d.H, rows, d.dr, d.rope_base, qscale, qc, qr, wk, pos, static_cast<uint16_t*>(q_hat));
  return hipGetLastError();
}

hipError_t launch_out_proj_mfma(const Dims& d, const float* z, const void* w_uv, int rows, float* out,
                                hipStream_t s) {
  out_proj_mfma_kernel<<<dim3(xcd_grid((kDv / kOpCols) * ((rows + kOpRows - 1) / kOpRows), d.H)), 256, 0, s>>>(
      d.H, rows, z, static_cast<const uint16_t*>(w_uv), out);
  return hipGetLastError();
}

}  // namespace mla
