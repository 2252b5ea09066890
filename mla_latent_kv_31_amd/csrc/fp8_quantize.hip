// bf16 cache rows -> FP8 cache rows (fp8.h): one wave per row, lane l holds latent values
// 8l .. 8l+7; the row's largest magnitude (a wave maximum) fixes the power-of-two scale, every
// value becomes its nearest-even E4M3 code under it, the rotary values are copied unchanged.

#include "common.h"
#include "fp8.h"
#include "launch.h"

namespace mla {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kDc = 512, kW = 576;

__global__ __launch_bounds__(256) void quantize_rows_fp8_kernel(const uint16_t* __restrict__ src, int64_t rows,
                                                               unsigned char* __restrict__ dst) {
  const int64_t r = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;  // whole waves
  const int lane = threadIdx.x & 63;
  const uint16_t* s = src + r * kW;
  const u32x4 x = *reinterpret_cast<const u32x4*>(s + 8 * lane);
  float v[8], amax = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[2 * k] = __uint_as_float(x[k] << 16);
    v[2 * k + 1] = __uint_as_float(x[k] & 0xffff0000u);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(v[k]));
  const int e = fp8_scale_exp(wave_max(amax));
  uint32_t w0 = 0, w1 = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    w0 |= e4m3_code(ldexpf(v[k], -e)) << (8 * k);
    w1 |= e4m3_code(ldexpf(v[4 + k], -e)) << (8 * k);
  }
  unsigned char* d = dst + r * kFp8RowB;
  *reinterpret_cast<uint2*>(d + 8 * lane) = make_uint2(w0, w1);
  if (lane < 8) *reinterpret_cast<u32x4*>(d + kDc + 16 * lane) = *reinterpret_cast<const u32x4*>(s + kDc + 8 * lane);
  if (lane == 8) *reinterpret_cast<u32x4*>(d + kFp8ScaleOff) = u32x4{__float_as_uint(ldexpf(1.f, e)), 0u, 0u, 0u};
}

}  // namespace

hipError_t launch_quantize_rows_fp8(const void* src, int64_t rows, void* dst, hipStream_t stream) {
  const int64_t blocks = (rows + 3) / 4;
  quantize_rows_fp8_kernel<<<dim3(unsigned(blocks)), 256, 0, stream>>>(static_cast<const uint16_t*>(src), rows,
                                                                       static_cast<unsigned char*>(dst));
  return hipGetLastError();
}

}  // namespace mla
