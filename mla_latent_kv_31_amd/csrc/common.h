// Device helpers shared by the libmla kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla.h"

namespace mla {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- bfloat16 storage
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Round to nearest even; NaN stays NaN (quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// Element access for the two storage types.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void store(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
};

// ---------------------------------------------------------------- IEEE binary16 storage
// The absorbed query of the bf16 path is stored in binary16: 11 significant bits instead of bf16's
// 8 keep the score error of a 576-long dot product well inside the bf16 output tolerance.
struct f16_t {
  uint16_t bits;
};
__device__ __forceinline__ float f16_to_f32(uint16_t h) { return float(__builtin_bit_cast(_Float16, h)); }
// Round to nearest even; beyond +-65504 the result is +-inf.
__device__ __forceinline__ uint16_t f32_to_f16(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
template <> struct Elem<f16_t> {
  static __device__ __forceinline__ float load(const f16_t* p, size_t i) { return f16_to_f32(p[i].bits); }
  static __device__ __forceinline__ void store(f16_t* p, size_t i, float v) { p[i].bits = f32_to_f16(v); }
};
// Storage type of q_hat for a given storage type of the other tensors.
template <typename T> struct QHatOf { using type = T; };
template <> struct QHatOf<uint16_t> { using type = f16_t; };

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Block-wide reductions for blockDim.x a multiple of 64 (<= 1024). `red` holds >= 16 floats.
// Every thread receives the result.  Contains barriers: call from uniform control flow.
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < nw; ++i) r = fmaxf(r, red[i]);
  return r;
}
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < nw; ++i) r += red[i];
  return r;
}

// exp2 of x with exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Row address of token t of sequence b in a paged pool (row = d_c + d_r elements).
__device__ __forceinline__ size_t row_index(const int32_t* __restrict__ page_table, int max_pages,
                                            int page_size, int b, int t) {
  const int pg = page_table[size_t(b) * max_pages + t / page_size];
  return size_t(pg) * page_size + (t % page_size);
}

}  // namespace mla
