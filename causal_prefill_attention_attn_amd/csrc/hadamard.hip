// Walsh-Hadamard rotation of head-dimension rows (fp32 or bf16).
//
// Rotating Q, K and V by an orthogonal matrix before FP8 quantization
// spreads outlier channels over the whole row and so shrinks the rounding
// error of the per-tensor quantization, the largest part of the FP8 error
// ("Precisao, estabilidade e efeito na pratica" on the miraibroadcast.com
// page: about half of it, for about 0.1% of the attention time).  With the
// same orthogonal H on Q and K the scores are unchanged, (QH)(KH)^T = QK^T;
// V rotated by H gives O H, undone by applying H once more (H is symmetric
// and H H = I).
//
// H is the normalized Sylvester-Hadamard matrix in blocks along the row:
// one block of 128 for rows of 128 elements, three blocks of 64 for rows of
// 192.  Lane l of a wave holds elements l, l + 64, ... of one row; the
// butterflies of strides 1..32 cross lanes through shuffles, the stride-64
// butterfly of a 128-block is in-lane.  Rows are independent, so y may be x
// (in place).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_kernels.h"
#include "e4m3_encode.h"

namespace cpattn {
namespace {

// Rotated row r of x into v (lane l holds elements l, l + 64, ...)
template <int D, bool kBF16>
__device__ __forceinline__ void rotate_row(const void* x, int64_t r, int lane,
                                           float (&v)[D / 64]) {
  constexpr int J = D / 64;
  constexpr float kNorm = D == 128 ? 0.088388347648318440550f : 0.125f;  // 1/sqrt(block)
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int64_t i = r * D + j * 64 + lane;
    if constexpr (kBF16) v[j] = (float)reinterpret_cast<const __bf16*>(x)[i];
    else v[j] = reinterpret_cast<const float*>(x)[i];
  }
  // strides 1..32 inside each 64-block: the element whose stride bit is
  // clear takes a + b, the other a - b
#pragma unroll
  for (int h = 1; h < 64; h <<= 1)
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const float p = __shfl_xor(v[j], h);
      v[j] = (lane & h) ? p - v[j] : v[j] + p;
    }
  if constexpr (D == 128) {  // stride 64: in-lane
    const float a = v[0] + v[1], b = v[0] - v[1];
    v[0] = a;
    v[1] = b;
  }
#pragma unroll
  for (int j = 0; j < J; ++j) v[j] *= kNorm;
}

// x and y may be the same buffer (an in-place rotation): each wave reads its
// whole row into registers before it writes that row, and rows are disjoint
// between waves, so neither pointer is declared __restrict__.
template <int D, bool kBF16>
__global__ void __launch_bounds__(256) hadamard_kernel(const void* x, int64_t rows, void* y) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * (blockDim.x >> 6);
  for (int64_t r = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); r < rows;
       r += nw) {
    float v[D / 64];
    rotate_row<D, kBF16>(x, r, lane, v);
#pragma unroll
    for (int j = 0; j < D / 64; ++j) {
      const int64_t i = r * D + j * 64 + lane;
      if constexpr (kBF16) reinterpret_cast<__bf16*>(y)[i] = (__bf16)v[j];
      else reinterpret_cast<float*>(y)[i] = v[j];
    }
  }
}

// amax of the rotated rows (magnitudes as bit patterns, as in quant.hip);
// *out must be zero on entry
template <int D>
__global__ void __launch_bounds__(256) hadamard_amax_kernel(const float* __restrict__ x,
                                                            int64_t rows,
                                                            uint32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * (blockDim.x >> 6);
  uint32_t m = 0u;
  for (int64_t r = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); r < rows;
       r += nw) {
    float v[D / 64];
    rotate_row<D, false>(x, r, lane, v);
#pragma unroll
    for (int j = 0; j < D / 64; ++j) {
      const uint32_t a = __float_as_uint(v[j]) & 0x7fffffffu;
      m = max(m, a <= 0x7f800000u ? a : 0u);
    }
  }
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  __shared__ uint32_t wmax[4];
  if (lane == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) atomicMax(out, max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3])));
}

// e4m3 codes of the rotated rows divided by descale (read from device memory
// when dptr is set, else the argument)
template <int D>
__global__ void __launch_bounds__(256) hadamard_quantize_kernel(const float* __restrict__ x,
                                                                int64_t rows,
                                                                const float* __restrict__ dptr,
                                                                float dval,
                                                                uint8_t* __restrict__ out) {
  const float descale = dptr != nullptr ? *dptr : dval;
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * (blockDim.x >> 6);
  for (int64_t r = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); r < rows;
       r += nw) {
    float v[D / 64];
    rotate_row<D, false>(x, r, lane, v);
#pragma unroll
    for (int j = 0; j < D / 64; ++j) out[r * D + j * 64 + lane] = e4m3_from_f32(v[j] / descale);
  }
}

}  // namespace

namespace {
unsigned hadamard_grid(int64_t rows) {
  int64_t blocks = (rows + 3) / 4;  // four waves (rows) per block and pass
  return (unsigned)(blocks > 16384 ? 16384 : blocks);
}
}  // namespace

int launch_hadamard(const void* x, int64_t rows, int d, bool bf16, void* y, hipStream_t stream) {
  const dim3 grid(hadamard_grid(rows)), block(256);
  if (d == 128) {
    if (bf16) hipLaunchKernelGGL((hadamard_kernel<128, true>), grid, block, 0, stream, x, rows, y);
    else hipLaunchKernelGGL((hadamard_kernel<128, false>), grid, block, 0, stream, x, rows, y);
  } else {
    if (bf16) hipLaunchKernelGGL((hadamard_kernel<192, true>), grid, block, 0, stream, x, rows, y);
    else hipLaunchKernelGGL((hadamard_kernel<192, false>), grid, block, 0, stream, x, rows, y);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_hadamard_amax(const float* x, int64_t rows, int d, float* amax_out,
                         hipStream_t stream) {
  uint32_t* out = reinterpret_cast<uint32_t*>(amax_out);
  hipLaunchKernelGGL(zero_u32, dim3(1), dim3(1), 0, stream, out);
  const dim3 grid(hadamard_grid(rows)), block(256);
  if (d == 128) hipLaunchKernelGGL(hadamard_amax_kernel<128>, grid, block, 0, stream, x, rows, out);
  else hipLaunchKernelGGL(hadamard_amax_kernel<192>, grid, block, 0, stream, x, rows, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

namespace {
int hadamard_quantize(const float* x, int64_t rows, int d, const float* dptr, float dval,
                      uint8_t* out, hipStream_t stream) {
  const dim3 grid(hadamard_grid(rows)), block(256);
  if (d == 128)
    hipLaunchKernelGGL(hadamard_quantize_kernel<128>, grid, block, 0, stream, x, rows, dptr, dval,
                       out);
  else
    hipLaunchKernelGGL(hadamard_quantize_kernel<192>, grid, block, 0, stream, x, rows, dptr, dval,
                       out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
}  // namespace

int launch_hadamard_quantize(const float* x, int64_t rows, int d, float descale, uint8_t* out,
                             hipStream_t stream) {
  return hadamard_quantize(x, rows, d, nullptr, descale, out, stream);
}

int launch_hadamard_quantize_dev(const float* x, int64_t rows, int d, const float* descale,
                                 uint8_t* out, hipStream_t stream) {
  return hadamard_quantize(x, rows, d, descale, 1.0f, out, stream);
}

}  // namespace cpattn
