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

__global__ void __launch_bounds__(256) amax_kernel(const float* __restrict__ x, int64_t n,
                                                   uint32_t* __restrict__ out) {
  // magnitudes as bit patterns: non-negative floats order like unsigned
  // integers, so the max is exact, order-free and needs no float compare;
  // NaN patterns (above the infinity pattern) are skipped
  uint32_t m = 0u;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t a = __float_as_uint(x[i]) & 0x7fffffffu;
    m = max(m, a <= 0x7f800000u ? a : 0u);
  }
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  __shared__ uint32_t wmax[4];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) atomicMax(out, max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3])));
}

// descale from device memory when dptr is set (the whole quantization then
// runs without a host round trip), else the argument
__global__ void __launch_bounds__(256) quantize_kernel(const float* __restrict__ x, int64_t n,
                                                       const float* __restrict__ dptr,
                                                       float dval, uint8_t* __restrict__ out) {
  const float descale = dptr != nullptr ? *dptr : dval;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    out[i] = e4m3_from_f32(x[i] / descale);
}

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

int launch_amax_f32(const float* x, int64_t n, float* amax_out, hipStream_t stream) {
  hipLaunchKernelGGL(zero_u32, dim3(1), dim3(1), 0, stream, reinterpret_cast<uint32_t*>(amax_out));
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(amax_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, n,
                     reinterpret_cast<uint32_t*>(amax_out));
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_quantize_e4m3(const float* x, int64_t n, float descale, uint8_t* out,
                         hipStream_t stream) {
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, n,
                     (const float*)nullptr, descale, out);
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
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, n,
                     (const float*)descale, 1.0f, codes);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace cpattn
