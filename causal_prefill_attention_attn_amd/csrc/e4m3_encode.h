// fp32 -> OCP E4M3FN encoder and a one-word clear kernel, shared by the
// quantization kernels (per-tensor FP8 quantization of Q, K and V, the
// largest source of FP8 error per "Precisao, estabilidade e efeito na
// pratica" on the miraibroadcast.com page).  The encoder works on the fp32
// bit pattern: exponent re-bias plus round-to-nearest-even on the dropped
// mantissa bits for normal results, an exact multiply by 2^9 and rint for
// the subnormal range, and saturation to the largest finite code (448);
// NaN maps to 0x7F.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpattn {
namespace {

__global__ void zero_u32(uint32_t* p) { *p = 0u; }

__device__ __forceinline__ uint8_t e4m3_from_f32(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7f;                 // NaN
  if (a >= 0x43e00000u) return (uint8_t)(sign | 0x7e);  // |x| >= 448 (incl. inf): saturate
  if (a < 0x3c800000u) {                            // |x| < 2^-6: multiples of 2^-9
    const float m = rintf(__uint_as_float(a) * 512.0f);  // exact scaling, RNE
    return (uint8_t)(sign | (uint32_t)m);           // m == 8 is the code of 2^-6
  }
  // normal: keep 3 of 23 mantissa bits, round half to even, re-bias 127 -> 7
  const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
  const uint32_t code = (r >> 20) - ((127u - 7u) << 3);
  return (uint8_t)(sign | (code > 0x7eu ? 0x7eu : code));
}

}  // namespace
}  // namespace cpattn
