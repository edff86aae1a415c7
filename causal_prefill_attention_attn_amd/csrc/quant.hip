// Per-tensor FP8 quantization helpers: amax and fp32 -> E4M3FN.
//
// Most of the FP8 error of the attention comes from rounding Q, K and V to
// FP8 ("Precisao, estabilidade e efeito na pratica" on the
// miraibroadcast.com page); these kernels produce the e4m3 codes and the
// per-tensor scale that attn_fwd consumes (the encoder is in
// e4m3_encode.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_kernels.h"
#include "e4m3_encode.h"

namespace cpattn {
namespace {

// Largest magnitude (as a bit pattern) of x, folded into *out.  vec: x is
// 16-byte aligned and each thread has four 16-byte loads in flight per step
// (coalesced across the block); the scalar loop takes the elements past the
// last whole group of four, or all of them when x is not aligned.
__global__ void __launch_bounds__(kAmaxThreads) amax_kernel(const float* __restrict__ x, int64_t n,
                                                            int vec, uint32_t* __restrict__ out) {
  uint32_t m = 0u;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t tail = 0;
  if (vec) {
    const int64_t n4 = n >> 2;
    const float4* x4 = reinterpret_cast<const float4*>(x);
    for (int64_t i = i0; i < n4; i += 4 * stride) {
      float4 v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        v[q] = i + q * stride < n4 ? x4[i + q * stride] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        m = max(max(m, max(mag_bits(v[q].x), mag_bits(v[q].y))),
                max(mag_bits(v[q].z), mag_bits(v[q].w)));
    }
    tail = n4 << 2;
  }
  for (int64_t i = tail + i0; i < n; i += stride) m = max(m, mag_bits(x[i]));
  amax_commit(m, out);
}

// descale from device memory when dptr is set (the whole quantization then
// runs without a host round trip), else the argument.
// vec: x and out are 16-byte aligned.  Whole runs of 1024 values go a wave
// at a time: lane t of the wave whose run starts at float4 4*base reads
// float4s 4*base + 64*q + t (q = 0..3), so each load covers 1 KB and each
// 4-byte store of codes 256 B contiguous (17-19% faster than 16 consecutive
// values per thread).  i - lane is a multiple of 64 and so is nw, so a wave
// with i < nw has its whole run below nw.  The groups of 16 values past the
// last whole run take 16 consecutive values per thread, and the values past
// the last whole group (or all of them when a buffer is not aligned) a
// scalar loop.
__global__ void __launch_bounds__(256) quantize_kernel(const float* __restrict__ x, int64_t n,
                                                       int vec, const float* __restrict__ dptr,
                                                       float dval, uint8_t* __restrict__ out) {
  const float descale = dptr != nullptr ? *dptr : dval;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  auto code4 = [&](const float4 v) {
    return (uint32_t)e4m3_from_f32(v.x / descale) |
           ((uint32_t)e4m3_from_f32(v.y / descale) << 8) |
           ((uint32_t)e4m3_from_f32(v.z / descale) << 16) |
           ((uint32_t)e4m3_from_f32(v.w / descale) << 24);
  };
  int64_t tail = 0;
  if (vec) {
    const int64_t n16 = n >> 4;
    const int64_t nw = (n >> 10) << 6;
    const float4* x4 = reinterpret_cast<const float4*>(x);
    uint32_t* o4 = reinterpret_cast<uint32_t*>(out);
    const int lane = threadIdx.x & 63;
    for (int64_t i = i0; i < nw; i += stride) {
      const int64_t f0 = (i - lane) * 4 + lane;
      float4 v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = x4[f0 + 64 * q];
#pragma unroll
      for (int q = 0; q < 4; ++q) o4[f0 + 64 * q] = code4(v[q]);
    }
    uint4* o16 = reinterpret_cast<uint4*>(out);
    for (int64_t i = nw + i0; i < n16; i += stride)
      o16[i] = make_uint4(code4(x4[4 * i]), code4(x4[4 * i + 1]), code4(x4[4 * i + 2]),
                          code4(x4[4 * i + 3]));
    tail = n16 << 4;
  }
  for (int64_t i = tail + i0; i < n; i += stride) out[i] = e4m3_from_f32(x[i] / descale);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// The per-tensor scale rule of the FP8 quantization, in place: *p holds
// amax (as written by the amax kernels) and becomes amax / 448 in fp32, or
// 1 for an all-zero tensor, so the largest magnitude lands on the largest
// finite E4M3FN value, 448.
__global__ void descale_from_amax(float* p) {
  if (threadIdx.x == 0) {
    const float a = *p;
    *p = a > 0.0f ? a / 448.0f : 1.0f;
  }
}

}  // namespace

int launch_clear_i32(int32_t* p, hipStream_t stream) {
  hipLaunchKernelGGL(zero_u32, dim3(1), dim3(1), 0, stream, reinterpret_cast<uint32_t*>(p));
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_amax_f32(const float* x, int64_t n, float* amax_out, hipStream_t stream) {
  hipLaunchKernelGGL(zero_u32, dim3(1), dim3(1), 0, stream, reinterpret_cast<uint32_t*>(amax_out));
  const int vec = aligned16(x) ? 1 : 0;
  int64_t blocks = (n / (vec ? 16 : 1) + kAmaxThreads - 1) / kAmaxThreads;
  if (blocks < 1) blocks = 1;
  if (blocks > kAmaxBlocks) blocks = kAmaxBlocks;
  hipLaunchKernelGGL(amax_kernel, dim3((unsigned)blocks), dim3(kAmaxThreads), 0, stream, x, n, vec,
                     reinterpret_cast<uint32_t*>(amax_out));
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

namespace {
void launch_quantize(const float* x, int64_t n, const float* dptr, float dval, uint8_t* out,
                     hipStream_t stream) {
  const int vec = aligned16(x) && aligned16(out) ? 1 : 0;
  int64_t blocks = (n / (vec ? 16 : 1) + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, n, vec,
                     dptr, dval, out);
}
}  // namespace

int launch_quantize_e4m3(const float* x, int64_t n, float descale, uint8_t* out,
                         hipStream_t stream) {
  launch_quantize(x, n, nullptr, descale, out, stream);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_quantize_fp8(const float* x, int64_t rows, int d, bool rotate, uint8_t* codes,
                        float* descale, hipStream_t stream) {
  const int64_t n = rows * d;
  int rc = rotate ? launch_hadamard_amax(x, rows, d, descale, stream)
                  : launch_amax_f32(x, n, descale, stream);
  if (rc != 0) return rc;
  hipLaunchKernelGGL(descale_from_amax, dim3(1), dim3(64), 0, stream, descale);
  if (hipGetLastError() != hipSuccess) return -1;
  if (rotate) return launch_hadamard_quantize_dev(x, rows, d, descale, codes, stream);
  launch_quantize(x, n, descale, 1.0f, codes, stream);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace cpattn
