// Per-head projections on bf16 MFMA (gfx950): the absorbed query and the value up-projection.
//
// mla_absorb_query ([ase] "Key 투영을 Query 쪽으로 옮기기", Fig. 3 equation):
//   q_hat[r,h,j] = (sum_k q_c[r,h,k] W_UK[h,j,k]) * qscale,  j < d_c
//   q_hat[r,h,d_c+2i, d_c+2i+1] = rotation of (q_r[r,h,2i], q_r[r,h,2i+1]) by pos[r]*base^(-2i/d_r), * qscale
// computed transposed, q_hat^T = W_UK[h] . q_c^T, so that W_UK rows (contiguous over k) are the
// A operand and query rows (contiguous over k) the B operand, both straight from global memory,
// and each lane stores four consecutive outputs.  One workgroup per (head, 128 latent columns):
// every weight is read once.
//
// mla_out_proj ([ase] "Value 투영을 가중합 뒤로 옮기기", Fig. 4 equation):
//   out[r,h,v] = sum_j z[r,h,j] W_UV[h,j,v]
// computed as out^T = W_UV[h]^T . z^T.  The contraction runs over j, the row index of W_UV, so
// the workgroup stages its 512 x 64 slice of W_UV in LDS and reads the A operand with the
// transposing ds_read_b64_tr_b16.  z is float32: it is split into bf16 hi + lo parts and both are
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
constexpr int kMaxDr = 512;

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

// ---------------------------------------------------------------------------------------- absorb
// grid (d_c / 128, H); 4 waves, wave w owns latent columns [128*blockIdx.x + 32w, +32).
__global__ __launch_bounds__(256) void absorb_mfma_kernel(int H, int R, int dr, float rope_base, float qscale,
                                                          const uint16_t* __restrict__ q_c,
                                                          const uint16_t* __restrict__ q_r,
                                                          const uint16_t* __restrict__ w_uk,
                                                          const int32_t* __restrict__ pos, uint16_t* __restrict__ q_hat) {
  const int h = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, hi = lane >> 5;
  const int W = kDc + dr;
  const int j0 = 128 * blockIdx.x + 32 * wave;
  // A operand: W_UK[h][j0 + lane%32][8*hi + 16*ks .. +7], kept for all row blocks
  bf16x8 a[kDk / 16];
  {
    const uint16_t* wrow = w_uk + (size_t(h) * kDc + j0 + (lane & 31)) * kDk + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < kDk / 16; ++ks) a[ks] = load_bf16x8(wrow + 16 * ks);
  }
  for (int rb = 0; rb < R; rb += 32) {
    const int r = rb + (lane & 31);
    const bool rv = r < R;
    f32x16 acc;
#pragma unroll
    for (int x = 0; x < 16; ++x) acc[x] = 0.f;
    const uint16_t* qrow = q_c + (size_t(rv ? r : 0) * H + h) * kDk + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < kDk / 16; ++ks) {
      bf16x8 bq = load_bf16x8(qrow + 16 * ks);
      if (!rv) bq = bf16x8{};
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], bq, acc, 0, 0, 0);
    }
    if (rv) {
      uint16_t* out = q_hat + (size_t(r) * H + h) * W + j0 + 4 * hi;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 v;
        v[0] = uint32_t(f32_to_bf16(acc[4 * g] * qscale)) | (uint32_t(f32_to_bf16(acc[4 * g + 1] * qscale)) << 16);
        v[1] = uint32_t(f32_to_bf16(acc[4 * g + 2] * qscale)) | (uint32_t(f32_to_bf16(acc[4 * g + 3] * qscale)) << 16);
        *reinterpret_cast<u32x2*>(out + 8 * g) = v;
      }
    }
  }
  // rotary part: the first column group of each head rotates q_r for every row
  if (blockIdx.x == 0) {
    __shared__ double inv_freq[kMaxDr / 2];
    const int pairs = dr / 2;
    for (int i = threadIdx.x; i < pairs; i += blockDim.x) inv_freq[i] = pow(double(rope_base), -2.0 * i / dr);
    __syncthreads();
    for (int idx = threadIdx.x; idx < R * pairs; idx += blockDim.x) {
      const int r = idx / pairs, i = idx % pairs;
      // angle in double, reduced to [-pi, pi] before the float32 sine/cosine
      const double ang = double(pos[r]) * inv_freq[i];
      const double red = ang - 6.283185307179586 * rint(ang / 6.283185307179586);
      float sn, cs;
      sincosf(float(red), &sn, &cs);
      const size_t qi = (size_t(r) * H + h) * dr + 2 * i;
      const float x1 = bf16_to_f32(q_r[qi]), x2 = bf16_to_f32(q_r[qi + 1]);
      uint16_t* out = q_hat + (size_t(r) * H + h) * W + kDc + 2 * i;
      out[0] = f32_to_bf16((x1 * cs - x2 * sn) * qscale);
      out[1] = f32_to_bf16((x1 * sn + x2 * cs) * qscale);
    }
  }
}

// ---------------------------------------------------------------------------------------- out_proj
constexpr int kOpCols = 64;                    // v columns per workgroup
constexpr int kOpRowB = kOpCols * 2;           // 128 bytes per W row slice in LDS
constexpr int kOpLds = kDc * kOpRowB;          // 64 KiB

// LDS place of 16-byte chunk c (0..7) of W row j: rows j and j+2 sit half a row apart, so that
// the 4-row x 64-byte transposing reads cover all 64 banks.
__device__ __forceinline__ int op_chunk(int j, int c) { return c ^ (((j >> 1) & 1) << 2); }

// grid (d_v / 64, H); 4 waves: wave w owns v block (w & 1) and row blocks (w >> 1) + 2i.
__global__ __launch_bounds__(256) void out_proj_mfma_kernel(int H, int R, const float* __restrict__ z,
                                                            const uint16_t* __restrict__ w_uv,
                                                            float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kOpLds];
  lds_u8* const lw = (lds_u8*)smem;
  const int h = blockIdx.y, v0 = kOpCols * blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, hi = lane >> 5;
  // stage W_UV[h][:, v0 .. v0+63]: 512 rows x 8 chunks of 16 B
  for (int c = threadIdx.x; c < kDc * 8; c += blockDim.x) {
    const int j = c >> 3, ch = c & 7;
    const u32x4 v = *reinterpret_cast<const u32x4*>(w_uv + (size_t(h) * kDc + j) * kDv + v0 + 8 * ch);
    *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(lw + j * kOpRowB + 16 * op_chunk(j, ch)) = v;
  }
  __syncthreads();
  const int vb = wave & 1;
  // transposing read of the A operand (M = v, K = j): lane group g reads rows j0 + 8*(g/2) + q,
  // q = 0..3 (first read) and +4 (second), columns vb*32 + 16*(g%2) + 4*(lane%4) .. +3
  const int g = lane >> 4, ii = lane & 15;
  const int rq = ii >> 2, ccol = vb * 32 + 16 * (g & 1) + 4 * (ii & 3);
  auto tr_addr = [&](int j) -> const lds_u8* {
    return lw + j * kOpRowB + 16 * op_chunk(j, ccol >> 3) + 2 * (ccol & 7);
  };
  for (int rb = 32 * (wave >> 1); rb < R; rb += 64) {
    const int r = rb + (lane & 31);
    const bool rv = r < R;
    const float* zrow = z + (size_t(rv ? r : 0) * H + h) * kDc + 8 * hi;
    f32x16 acc;
#pragma unroll
    for (int x = 0; x < 16; ++x) acc[x] = 0.f;
#pragma unroll 4
    for (int ks = 0; ks < kDc / 16; ++ks) {
      const int jr = 16 * ks + 8 * (g >> 1) + rq;
      const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)tr_addr(jr));
      const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)tr_addr(jr + 4));
      const bf16x8 aw = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
      // B operand: z[r][16ks + 8hi .. +7] as bf16 hi + lo
      float zv[8];
      const float4 z0 = *reinterpret_cast<const float4*>(zrow + 16 * ks);
      const float4 z1 = *reinterpret_cast<const float4*>(zrow + 16 * ks + 4);
      zv[0] = z0.x; zv[1] = z0.y; zv[2] = z0.z; zv[3] = z0.w;
      zv[4] = z1.x; zv[5] = z1.y; zv[6] = z1.z; zv[7] = z1.w;
      bf16x8 zh, zl;
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const float v = rv ? zv[x] : 0.f;
        zh[x] = (__bf16)v;
        zl[x] = (__bf16)(v - float(zh[x]));
      }
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw, zh, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw, zl, acc, 0, 0, 0);
    }
    if (rv) {
      float* o = out + (size_t(r) * H + h) * kDv + v0 + vb * 32 + 4 * hi;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(o + 8 * q) = make_float4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
    }
  }
}

}  // namespace

bool proj_mfma_supported(const Dims& d) {
  return d.dtype == MLA_BF16 && d.dc == kDc && d.dk == kDk && d.dv == kDv && d.dr % 2 == 0 && d.dr <= kMaxDr;
}

hipError_t launch_absorb_mfma(const Dims& d, const void* q_c, const void* q_r, const void* w_uk, const int32_t* pos,
                              int rows, void* q_hat, hipStream_t s) {
  absorb_mfma_kernel<<<dim3(kDc / 128, d.H), 256, 0, s>>>(
      d.H, rows, d.dr, d.rope_base, d.sm_scale * kLog2e, static_cast<const uint16_t*>(q_c),
      static_cast<const uint16_t*>(q_r), static_cast<const uint16_t*>(w_uk), pos, static_cast<uint16_t*>(q_hat));
  return hipGetLastError();
}

hipError_t launch_out_proj_mfma(const Dims& d, const float* z, const void* w_uv, int rows, float* out,
                                hipStream_t s) {
  out_proj_mfma_kernel<<<dim3(kDv / kOpCols, d.H), 256, 0, s>>>(d.H, rows, z, static_cast<const uint16_t*>(w_uv),
                                                                   out);
  return hipGetLastError();
}

}  // namespace mla
