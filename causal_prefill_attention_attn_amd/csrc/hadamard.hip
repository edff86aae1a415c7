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
// 192.  Two layouts compute the same butterflies in the same order (so the
// same bits):
//  - 16-byte-aligned buffers: each thread holds 16 consecutive elements
//    (16-byte loads and stores).  Strides 1..8 are in-thread; strides 16, 32
//    and (for 128-blocks) 64 cross the 4 or 8 threads of a block through DPP
//    quad permutes and a swizzle.
//  - otherwise: lane l of a wave holds elements l, l + 64, ... of one row;
//    the butterflies of strides 1..32 cross lanes through shuffles, and the
//    stride-64 butterfly of a 128-block is in-lane.
// Rows are independent, so y may be x (in place).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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

// amax of the rotated rows (magnitudes as bit patterns); *out must be zero
// on entry
template <int D>
__global__ void __launch_bounds__(kAmaxThreads) hadamard_amax_kernel(const float* __restrict__ x,
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
    for (int j = 0; j < D / 64; ++j) m = max(m, mag_bits(v[j]));
  }
  amax_commit(m, out);
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

// ---- 16 elements per thread ---------------------------------------------
//
// The BK/16 threads of a block of BK elements each hold 16 of its elements,
// as 16/CH chunks of CH consecutive elements: thread j holds chunks
// j, j + BK/16, ... of the block.  Within a chunk the butterflies are
// in-thread; strides CH .. BK/16*CH - 1 cross the threads of the block; the
// larger strides pair chunks of one thread.  Each load or store instruction
// of a group of threads then covers BK/16 * CH * element-size contiguous
// bytes.  Chunks of one 16-byte piece (4 fp32, 8 bf16) give whole 128-byte
// lines per 8 threads for 128-blocks; chunks of 16 elements, one thread
// per 64 bytes, were 13% slower for the fp32 rotation, which stores 4 bytes
// per element.
constexpr int kChF32 = 4;
constexpr int kChBF16 = 8;

// value of lane (lane ^ S) for S = 1, 2, 4 (all inside one quad or 8-lane
// group, so every lane of a Hadamard block reads a lane of the same block)
template <int S>
__device__ __forceinline__ float lane_xor(float v) {
  const int i = __float_as_int(v);
  if constexpr (S == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(i, 0xB1, 0xF, 0xF, true));
  else if constexpr (S == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(i, 0x4E, 0xF, 0xF, true));
  else return __int_as_float(__builtin_amdgcn_ds_swizzle(i, 0x1F | (S << 10)));  // and 31, xor S
}

// Rotation of one thread's 16 elements of a block of BK (v[e] is element
// CH * (j + BK/16 * (e / CH)) + e % CH, j = lane % (BK/16)).  The strides run
// 1, 2, 4, ... as in the row-per-wave kernels.  Each butterfly is a + b for
// the element whose stride bit is clear and a - b for the other; across
// lanes the partner's p and the own v give v + p or p - v, one rounding
// each, written as fma(+-1, v, p).
template <int BK, int CH>
__device__ __forceinline__ void rotate16(float (&v)[16], int lane) {
  constexpr int T = BK / 16;
  constexpr float kNorm = BK == 128 ? 0.088388347648318440550f : 0.125f;  // 1/sqrt(block)
  auto in_thread = [&](auto hc) {
    constexpr int H = decltype(hc)::value;  // index distance inside v
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (!(e & H)) {
        const float x0 = v[e], x1 = v[e + H];
        v[e] = x0 + x1;
        v[e + H] = x0 - x1;
      }
  };
  auto across = [&](auto sc) {
    constexpr int S = decltype(sc)::value;  // lane distance
    const float sg = (lane & S) ? -1.0f : 1.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = __builtin_fmaf(sg, v[e], lane_xor<S>(v[e]));
  };
  auto stage = [&](auto stc) {
    constexpr int St = decltype(stc)::value;  // element stride
    if constexpr (St < CH) in_thread(std::integral_constant<int, St>{});
    else if constexpr (St < CH * T) across(std::integral_constant<int, St / CH>{});
    else in_thread(std::integral_constant<int, CH * (St / (CH * T))>{});
  };
  stage(std::integral_constant<int, 1>{});
  stage(std::integral_constant<int, 2>{});
  stage(std::integral_constant<int, 4>{});
  stage(std::integral_constant<int, 8>{});
  stage(std::integral_constant<int, 16>{});
  stage(std::integral_constant<int, 32>{});
  if constexpr (BK == 128) stage(std::integral_constant<int, 64>{});
#pragma unroll
  for (int e = 0; e < 16; ++e) v[e] *= kNorm;
}

// First element of chunk q of thread g: blocks start at multiples of BK and
// the thread count is a multiple of BK/16, so a block's threads are
// consecutive; the grid stride is a multiple of 256 threads, so they are
// always active together.
template <int BK, int CH>
__device__ __forceinline__ int64_t chunk_at(int64_t g, int q) {
  constexpr int T = BK / 16;
  const int j = (int)(g % T);
  return (g - j) * 16 + CH * (j + T * q);
}

template <int BK, int CH, bool kBF16>
__device__ __forceinline__ void load16(const void* x, int64_t g, float (&v)[16]) {
  static_assert(CH % (kBF16 ? 8 : 4) == 0, "chunks hold whole 16-byte pieces");
#pragma unroll
  for (int q = 0; q < 16 / CH; ++q) {
    const int64_t i0 = chunk_at<BK, CH>(g, q);
    if constexpr (kBF16) {
#pragma unroll
      for (int p = 0; p < CH / 8; ++p) {
        const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const __bf16*>(x) + i0 + 8 * p);
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          v[CH * q + 8 * p + 2 * k] = __uint_as_float(u[k] << 16);
          v[CH * q + 8 * p + 2 * k + 1] = __uint_as_float(u[k] & 0xffff0000u);
        }
      }
    } else {
#pragma unroll
      for (int p = 0; p < CH / 4; ++p) {
        const float4 w = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + i0 + 4 * p);
        v[CH * q + 4 * p] = w.x;
        v[CH * q + 4 * p + 1] = w.y;
        v[CH * q + 4 * p + 2] = w.z;
        v[CH * q + 4 * p + 3] = w.w;
      }
    }
  }
}

template <int BK, bool kBF16>
__global__ void __launch_bounds__(256) hadamard16_kernel(const void* x, int64_t groups, void* y) {
  constexpr int CH = kBF16 ? kChBF16 : kChF32;
  const int lane = threadIdx.x & 63;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < groups; g += stride) {
    float v[16];
    load16<BK, CH, kBF16>(x, g, v);
    rotate16<BK, CH>(v, lane);
#pragma unroll
    for (int q = 0; q < 16 / CH; ++q) {
      const int64_t i0 = chunk_at<BK, CH>(g, q);
      if constexpr (kBF16) {
#pragma unroll
        for (int p = 0; p < CH / 8; ++p) {
          uint32_t u[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const __bf16 lo = (__bf16)v[CH * q + 8 * p + 2 * k];
            const __bf16 hi = (__bf16)v[CH * q + 8 * p + 2 * k + 1];
            u[k] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                   ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
          }
          *reinterpret_cast<uint4*>(reinterpret_cast<__bf16*>(y) + i0 + 8 * p) =
              make_uint4(u[0], u[1], u[2], u[3]);
        }
      } else {
#pragma unroll
        for (int p = 0; p < CH / 4; ++p) {
          const float* w = &v[CH * q + 4 * p];
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + i0 + 4 * p) =
              make_float4(w[0], w[1], w[2], w[3]);
        }
      }
    }
  }
}

template <int BK>
__global__ void __launch_bounds__(kAmaxThreads) hadamard16_amax_kernel(const float* __restrict__ x,
                                                                       int64_t groups,
                                                                       uint32_t* __restrict__ out) {
  constexpr int CH = kChF32;
  const int lane = threadIdx.x & 63;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  uint32_t m = 0u;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < groups; g += stride) {
    float v[16];
    load16<BK, CH, false>(x, g, v);
    rotate16<BK, CH>(v, lane);
#pragma unroll
    for (int e = 0; e < 16; ++e) m = max(m, mag_bits(v[e]));
  }
  amax_commit(m, out);
}

template <int BK>
__global__ void __launch_bounds__(256) hadamard16_quantize_kernel(const float* __restrict__ x,
                                                                  int64_t groups,
                                                                  const float* __restrict__ dptr,
                                                                  float dval,
                                                                  uint8_t* __restrict__ out) {
  constexpr int CH = kChF32;
  const float descale = dptr != nullptr ? *dptr : dval;
  const int lane = threadIdx.x & 63;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < groups; g += stride) {
    float v[16];
    load16<BK, CH, false>(x, g, v);
    rotate16<BK, CH>(v, lane);
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = (uint32_t)e4m3_from_f32(v[4 * k] / descale) |
             ((uint32_t)e4m3_from_f32(v[4 * k + 1] / descale) << 8) |
             ((uint32_t)e4m3_from_f32(v[4 * k + 2] / descale) << 16) |
             ((uint32_t)e4m3_from_f32(v[4 * k + 3] / descale) << 24);
    // codes of chunk q at chunk_at(g, q): CH bytes, 4 per word
#pragma unroll
    for (int q = 0; q < 16 / CH; ++q) {
      uint8_t* o = out + chunk_at<BK, CH>(g, q);
      if constexpr (CH == 4) *reinterpret_cast<uint32_t*>(o) = w[q];
      else if constexpr (CH == 8) *reinterpret_cast<uint2*>(o) = make_uint2(w[2 * q], w[2 * q + 1]);
      else *reinterpret_cast<uint4*>(o) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// grid of the 16-element kernels: one group per thread per pass, at most
// 16384 blocks
unsigned grid16(int64_t groups) {
  int64_t blocks = (groups + 255) / 256;
  return (unsigned)(blocks > 16384 ? 16384 : blocks);
}

}  // namespace

namespace {
unsigned hadamard_grid(int64_t rows) {
  int64_t blocks = (rows + 3) / 4;  // four waves (rows) per block and pass
  return (unsigned)(blocks > 16384 ? 16384 : blocks);
}
}  // namespace

int launch_hadamard(const void* x, int64_t rows, int d, bool bf16, void* y, hipStream_t stream) {
  if (aligned16(x) && aligned16(y)) {
    const int64_t groups = rows * d / 16;
    const dim3 grid(grid16(groups)), block(256);
    if (d == 128) {
      if (bf16) hipLaunchKernelGGL((hadamard16_kernel<128, true>), grid, block, 0, stream, x, groups, y);
      else hipLaunchKernelGGL((hadamard16_kernel<128, false>), grid, block, 0, stream, x, groups, y);
    } else {
      if (bf16) hipLaunchKernelGGL((hadamard16_kernel<64, true>), grid, block, 0, stream, x, groups, y);
      else hipLaunchKernelGGL((hadamard16_kernel<64, false>), grid, block, 0, stream, x, groups, y);
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
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
  if (aligned16(x)) {
    const int64_t groups = rows * d / 16;
    int64_t blocks = (groups + kAmaxThreads - 1) / kAmaxThreads;
    const dim3 grid((unsigned)(blocks > kAmaxBlocks ? kAmaxBlocks : blocks)), block(kAmaxThreads);
    if (d == 128)
      hipLaunchKernelGGL(hadamard16_amax_kernel<128>, grid, block, 0, stream, x, groups, out);
    else
      hipLaunchKernelGGL(hadamard16_amax_kernel<64>, grid, block, 0, stream, x, groups, out);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  const int64_t blocks = (rows + kAmaxThreads / 64 - 1) / (kAmaxThreads / 64);  // a row per wave
  const dim3 grid((unsigned)(blocks > kAmaxBlocks ? kAmaxBlocks : blocks)), block(kAmaxThreads);
  if (d == 128) hipLaunchKernelGGL(hadamard_amax_kernel<128>, grid, block, 0, stream, x, rows, out);
  else hipLaunchKernelGGL(hadamard_amax_kernel<192>, grid, block, 0, stream, x, rows, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

namespace {
int hadamard_quantize(const float* x, int64_t rows, int d, const float* dptr, float dval,
                      uint8_t* out, hipStream_t stream) {
  if (aligned16(x) && aligned16(out)) {
    const int64_t groups = rows * d / 16;
    const dim3 grid(grid16(groups)), block(256);
    if (d == 128)
      hipLaunchKernelGGL(hadamard16_quantize_kernel<128>, grid, block, 0, stream, x, groups, dptr,
                         dval, out);
    else
      hipLaunchKernelGGL(hadamard16_quantize_kernel<64>, grid, block, 0, stream, x, groups, dptr,
                         dval, out);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
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
