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

// Magnitude of a float as a bit pattern: non-negative floats order like
// unsigned integers, so a max over these is exact, order-free and needs no
// float compare; NaN patterns (above the infinity pattern) count as zero.
__device__ __forceinline__ uint32_t mag_bits(float v) {
  const uint32_t a = __float_as_uint(v) & 0x7fffffffu;
  return a <= 0x7f800000u ? a : 0u;
}

// Amax passes run kAmaxThreads-thread blocks, at most kAmaxBlocks of them
// (one per compute unit): every block ends in one atomic max on the same
// word, and those atomics serialize across the chip, about 12 ns each
// (4096 blocks cost ~48 us whatever the tensor size).  512 or 1024 blocks,
// or eight loads in flight per thread instead of four, measured no faster.
constexpr int kAmaxThreads = 1024;
constexpr int kAmaxBlocks = 256;

// Block max of m (a bit pattern from mag_bits) folded into *out with one
// atomic; every thread of the kAmaxThreads-thread block calls it.
__device__ __forceinline__ void amax_commit(uint32_t m, uint32_t* out) {
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  __shared__ uint32_t wmax[kAmaxThreads / 64];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t b = 0u;
#pragma unroll
    for (int w = 0; w < kAmaxThreads / 64; ++w) b = max(b, wmax[w]);
    atomicMax(out, b);
  }
}

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
