// BF16 causal prefill attention forward for gfx950 (CDNA4).
//
// The two products Q.K^T and P.V run on the matrix cores with the softmax
// between them on the vector unit ("Por que a atencao FP8 tem desempenho
// inferior no MI355X?" on the acheiumaia.com.br page); work is done in
// blocks of 32 queries against the keys of a tile, the unit the pages cost
// their cycle budget in (same section).  The softmax is the online form
// (running row max and row sum), so the S x S score matrix never exists.
//
// Formulation (per wave of 64 lanes, 32 query rows):
//   S^T = K . Q^T   with v_mfma_f32_32x32x16_bf16: A = K rows (keys), B =
//                   Q^T (one query per lane column).  In the 32x32 result
//                   lane l holds query (l % 32) and the 16 keys
//                   (i/4)*8 + (l/32)*4 + i%4 of a 32-key block, so row
//                   reductions over keys are in-lane plus one exchange
//                   between the two lane halves (v_permlane32_swap).
//   O^T += V^T . P^T  A = V^T (one value column per lane), B = P^T taken
//                   straight from the S^T registers after exp2 and bf16
//                   rounding: no LDS round trip for P.  The O accumulator of
//                   lane l belongs to query (l % 32) only, so the online
//                   rescale and the final 1/l are per-lane scalars.
// V^T needs keys contiguous per value column; the tile is transposed in
// registers while it is staged into LDS, with the keys of each 16-key group
// stored in the order the P^T operand enumerates them (bits 2 and 3 of the
// key offset swapped), so each lane fetches its 8 keys with one 16-byte read.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_kernels.h"

namespace cpattn {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;            // waves per workgroup
constexpr int kBM = 32 * kWaves;     // query rows per workgroup
constexpr int kBN = 64;              // keys per tile
constexpr int kDV = 128;             // value head dimension
constexpr int kThreads = 64 * kWaves;

// v_permlane32_swap on two copies of x leaves {own value, value of lane l^32}
// in its two results (which one is which depends on the lane half), so
// combining both with a commutative operation gives the pair result in
// every lane.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// position of key offset r (0..63) inside a Vt row: bits 2 and 3 swapped
__device__ __forceinline__ int vt_pos(int r) {
  return (r & ~12) | ((r >> 2) & 1) << 3 | ((r >> 3) & 1) << 2;
}

template <int DQK>
struct Smem {
  static constexpr int kPitch = DQK + 8;   // bf16 elements per K row (+16 B breaks bank aliasing)
  static constexpr int vPitch = kBN + 8;   // bf16 elements per V^T row
  __bf16 k[kBN * kPitch];
  __bf16 vt[kDV * vPitch];
};

template <int DQK>
__global__ void __launch_bounds__(kThreads, 2)
attn_fwd_bf16_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                     const __bf16* __restrict__ v, __bf16* __restrict__ o,
                     float* __restrict__ lse, int S, int H, int BH, int nqb, float c_log2,
                     int causal) {
  constexpr int kSteps = DQK / 16;           // k-steps of the QK^T product
  constexpr int kChunksPerRow = DQK / 8;     // 16-byte chunks per K row
  constexpr int kKChunks = kBN * kChunksPerRow / kThreads;
  static_assert(kBN * kChunksPerRow % kThreads == 0, "K tile split");
  static_assert(kBN / 4 * kDV / 8 == kThreads, "V tile split: one 4x8 block per thread");
  using SM = Smem<DQK>;
  __shared__ SM sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;  // query column / key row / value column inside a 32-block
  const int half = lane >> 5;

  // longest-first order: the last query blocks (most keys) are issued first;
  // all blocks of one (b, h) are H*B apart in launch order
  const int id = blockIdx.x;
  const int qb = nqb - 1 - id / BH;
  const int bh = id % BH;
  const int b = bh / H;
  const int h = bh % H;
  const int q0 = qb * kBM;
  const int q0w = q0 + wave * 32;
  const int64_t rowStrideQK = (int64_t)H * DQK;
  const int64_t rowStrideV = (int64_t)H * kDV;
  const __bf16* qbh = q + ((int64_t)b * S * H + h) * DQK;
  const __bf16* kbh = k + ((int64_t)b * S * H + h) * DQK;
  const __bf16* vbh = v + ((int64_t)b * S * H + h) * kDV;

  // ---- Q^T operand, kept in registers for the whole key loop
  bf16x8 qreg[kSteps];
  {
    const int qi = q0w + col;
    #pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      if (qi < S)
        qreg[s] = *reinterpret_cast<const bf16x8*>(qbh + qi * rowStrideQK + s * 16 + half * 8);
      else
        qreg[s] = bf16x8{};
    }
  }

  const int nkt_all = (S + kBN - 1) / kBN;
  const int nkt = causal ? min(nkt_all, (q0 + kBM - 1) / kBN + 1) : nkt_all;

  // ---- register staging of one K/V tile (prefetched one tile ahead)
  uint4 kst[kKChunks];
  uint4 vst[4];
  const int va = tid >> 4;        // key group: keys 4*va .. 4*va+3
  const int vc = tid & 15;        // value chunk: columns 8*vc .. 8*vc+7
  auto load_tile = [&](int t) {
    const int key0 = t * kBN;
    #pragma unroll
    for (int j = 0; j < kKChunks; ++j) {
      const int c = tid + j * kThreads;
      const int r = c / kChunksPerRow, cc = c % kChunksPerRow;
      const int key = key0 + r;
      kst[j] = key < S ? *reinterpret_cast<const uint4*>(kbh + key * rowStrideQK + cc * 8)
                       : make_uint4(0, 0, 0, 0);
    }
    #pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = key0 + va * 4 + r;
      vst[r] = key < S ? *reinterpret_cast<const uint4*>(vbh + key * rowStrideV + vc * 8)
                       : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tile = [&]() {
    #pragma unroll
    for (int j = 0; j < kKChunks; ++j) {
      const int c = tid + j * kThreads;
      const int r = c / kChunksPerRow, cc = c % kChunksPerRow;
      *reinterpret_cast<uint4*>(&sm.k[r * SM::kPitch + cc * 8]) = kst[j];
    }
    // 4 keys x 8 columns -> 8 columns x 4 keys
    const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&vst[0]);
    const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&vst[1]);
    const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&vst[2]);
    const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&vst[3]);
    const int pos = vt_pos(va * 4);
    #pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int d = j >> 1;
      uint2 out;
      if (j & 1) {
        out.x = (w0[d] >> 16) | (w1[d] & 0xffff0000u);
        out.y = (w2[d] >> 16) | (w3[d] & 0xffff0000u);
      } else {
        out.x = (w0[d] & 0xffffu) | (w1[d] << 16);
        out.y = (w2[d] & 0xffffu) | (w3[d] << 16);
      }
      *reinterpret_cast<uint2*>(&sm.vt[(vc * 8 + j) * SM::vPitch + pos]) = out;
    }
  };

  f32x16 oacc[kDV / 32];
  #pragma unroll
  for (int i = 0; i < kDV / 32; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY;  // running row max of c*s (log2 domain)
  float l_run = 0.f;        // this lane's partial row sum (its half of the keys)

  if (nkt > 0) load_tile(0);
  for (int t = 0; t < nkt; ++t) {
    __syncthreads();  // everyone is done reading the previous tile
    store_tile();
    __syncthreads();
    if (t + 1 < nkt) load_tile(t + 1);

    const int key0 = t * kBN;
    if (causal && key0 > q0w + 31) continue;  // tile entirely above this wave's diagonal

    // ---- S^T = K . Q^T for two 32-key blocks
    f32x16 sacc[kBN / 32];
    #pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb) {
      sacc[kb] = f32x16{};
      const __bf16* krow = &sm.k[(kb * 32 + col) * SM::kPitch + half * 8];
      #pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + s * 16);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[s], sacc[kb], 0, 0, 0);
      }
    }

    // ---- mask (diagonal and ragged-tail tiles only), running max
    const int qi = q0w + col;
    const bool need_mask = (causal && key0 + kBN - 1 > q0w) || key0 + kBN > S;
    if (need_mask) {
      #pragma unroll
      for (int kb = 0; kb < kBN / 32; ++kb)
        #pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + kb * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
          if (key >= S || (causal && key > qi)) sacc[kb][i] = -INFINITY;
        }
    }
    float mx = -INFINITY;
    #pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb)
      #pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
    mx = pair_max(mx);
    const float m_new = fmaxf(m_run, mx * c_log2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;

    // ---- P = exp2(c*s - m), bf16, laid out as the B operand of P.V
    bf16x8 pb[kBN / 16];
    float psum = 0.f;
    #pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb)
      #pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][i], c_log2, -m_new));
        psum += p;
        pb[kb * 2 + (i >> 3)][i & 7] = (__bf16)p;
      }
    l_run = l_run * alpha + psum;
    #pragma unroll
    for (int d = 0; d < kDV / 32; ++d)
      #pragma unroll
      for (int i = 0; i < 16; ++i) oacc[d][i] *= alpha;

    // ---- O^T += V^T . P^T
    #pragma unroll
    for (int d = 0; d < kDV / 32; ++d) {
      const __bf16* vrow = &sm.vt[(d * 32 + col) * SM::vPitch + half * 8];
      #pragma unroll
      for (int u = 0; u < kBN / 16; ++u) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(vrow + u * 16);
        oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[u], oacc[d], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: O / l -> bf16, lse = ln2 * (m + log2 l)
  const float l_tot = pair_sum(l_run);
  const int qi = q0w + col;
  if (qi < S) {
    const float inv = 1.0f / l_tot;
    __bf16* orow = o + ((int64_t)b * S * H + (int64_t)qi * H + h) * kDV;
    #pragma unroll
    for (int d = 0; d < kDV / 32; ++d)
      #pragma unroll
      for (int g = 0; g < 4; ++g) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 w;
        #pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(oacc[d][g * 4 + e] * inv);
        *reinterpret_cast<bf16x4*>(orow + d * 32 + g * 8 + half * 4) = w;
      }
    if (lse != nullptr && half == 0)
      lse[(int64_t)bh * S + qi] = (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
  }
}

}  // namespace

int launch_attn_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int S, int H, int d_qk, float softmax_scale, int causal,
                     hipStream_t stream) {
  const int nqb = (S + kBM - 1) / kBM;
  const int BH = B * H;
  const dim3 grid((unsigned)nqb * (unsigned)BH);
  const float c_log2 = softmax_scale * 1.4426950408889634f;
  if (d_qk == 128)
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<128>, grid, dim3(kThreads), 0, stream,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (__bf16*)o, lse, S,
                       H, BH, nqb, c_log2, causal);
  else
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<192>, grid, dim3(kThreads), 0, stream,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (__bf16*)o, lse, S,
                       H, BH, nqb, c_log2, causal);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace cpattn
