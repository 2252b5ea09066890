// FP8 (E4M3) latent cache rows ([huny] section 5, FP8 mixed-precision item: E4M3 on the 512-wide
// latent with a per-token scale factor).
//
// Row of 656 bytes: 512 E4M3 codes of c / 2^e | the 64 bf16 rotary values unchanged | the scale
// 2^e as a float32 | 12 zero bytes (16-byte multiple, so rows stay aligned for 16-byte transfers).
// e is the smallest integer with max|c| <= 448 * 2^e: the scaled latent fills the E4M3 range, and
// a power of two keeps code value x scale exact in bf16 and fp32.  E4M3 is the OCP 8-bit format
// (bias 7, subnormals m * 2^-9, largest finite 448, S.1111.111 NaN); codes round to nearest even.
#pragma once

#include <math.h>
#include <stdint.h>

namespace mla {

constexpr int kFp8RowB = 656;
constexpr int kFp8ScaleOff = 640;

// Nearest-even E4M3 code of a finite x with |x| <= 448.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  uint32_t code;
  if (a < 0.015625f) {  // below 2^-6: multiples of 2^-9 (8 steps is the smallest normal, code 0x08)
    code = uint32_t(__builtin_rintf(a * 512.f));
  } else {
    const uint32_t u = __float_as_uint(a);
    const uint32_t m = u & 0x7FFFFFu;
    const uint32_t q = (m + 0x7FFFFu + ((m >> 20) & 1u)) >> 20;  // 3 mantissa bits, ties to even; 8 carries
    code = (((u >> 23) - 127u + 7u) << 3) + q;
  }
  return sign | code;
}

// Exponent of the per-token scale: the smallest e with amax <= 448 * 2^e; 0 for amax == 0.
// With amax = M * 2^E, 1 <= M < 2: 448 * 2^(E-8) = 1.75 * 2^E, so e = E - 8 when M <= 1.75, else E - 7.
__device__ __forceinline__ int fp8_scale_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  int ex;
  const float m = frexpf(amax, &ex);  // amax = m * 2^ex, 0.5 <= m < 1
  return 2.f * m <= 1.75f ? ex - 1 - 8 : ex - 1 - 7;
}

}  // namespace mla
