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
// V^T comes from a row-major V tile in LDS through ds_read_b64_tr_b16: 16
// lanes supply four key rows of 16 values and each lane receives one value
// column of those four keys.  Rows are stored with a 32-byte chunk swizzle
// so that the eight 32-byte pieces one read instruction touches per 32
// lanes fall in distinct banks.  K/V tiles are double-buffered in LDS with
// global loads two tiles ahead, one workgroup barrier per tile.  The row
// sum adds the probabilities in fp32 before their bf16 rounding.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_device.h"
#include "attn_kernels.h"

namespace cpattn {

namespace {

constexpr int kWaves = 4;            // waves per workgroup
constexpr int kBM = 32 * kWaves;     // query rows per workgroup
constexpr int kDV = 128;             // value head dimension
constexpr int kThreads = 64 * kWaves;
constexpr int kVRow = kDV * 2;       // bytes per V row

// 32-byte chunk swizzle of a V row: the four consecutive keys one transposed
// read covers land on four distinct even chunk slots
__device__ __forceinline__ int v_swz(int key) { return (key & 3) << 1; }

template <int DQK, int BN>
struct Smem {
  static constexpr int kPitch = DQK * 2 + 16;  // bytes per K row (+16 B breaks bank aliasing)
  uint8_t k[2][BN * kPitch];
  uint8_t v[2][BN * kVRow];
};

template <int DQK, int BN>
__global__ void __launch_bounds__(kThreads, 2)
attn_fwd_bf16_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                     const __bf16* __restrict__ v, __bf16* __restrict__ o,
                     float* __restrict__ lse, int S, int H, int BH, int nqb, float c_log2,
                     int causal) {
  constexpr int kSteps = DQK / 16;                 // k-steps of the QK^T product
  constexpr int kNKB = BN / 32;                    // 32-key S blocks per tile
  constexpr int kKRowChunks = DQK * 2 / 16;        // 16-byte chunks per K row
  constexpr int kKChunks = BN * kKRowChunks / kThreads;
  constexpr int kVChunks = BN * (kVRow / 16) / kThreads;
  static_assert(BN * kKRowChunks % kThreads == 0 && BN * (kVRow / 16) % kThreads == 0, "split");
  using SM = Smem<DQK, BN>;
  __shared__ __attribute__((aligned(16))) SM sm;

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
  const uint32_t rsQK = (uint32_t)H * DQK * 2;  // bytes between rows
  const uint32_t rsV = (uint32_t)H * kVRow;
  const int64_t bstrQK = (int64_t)S * rsQK;
  const int64_t bstrV = (int64_t)S * rsV;
  const uint8_t* qb8 = reinterpret_cast<const uint8_t*>(q) + b * bstrQK;
  const uint8_t* kb8 = reinterpret_cast<const uint8_t*>(k) + b * bstrQK;
  const uint8_t* vb8 = reinterpret_cast<const uint8_t*>(v) + b * bstrV;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qb8, (uint32_t)bstrQK);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb8, (uint32_t)bstrQK);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb8, (uint32_t)bstrV);

  // ---- Q^T operand, kept in registers for the whole key loop
  bf16x8 qreg[kSteps];
  {
    const uint32_t off = (uint32_t)(q0w + col) * rsQK + h * DQK * 2 + half * 16;
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
      qreg[s] = __builtin_bit_cast(bf16x8, buffer_load16(rq, off + s * 32));
  }

  const int nkt_all = (S + BN - 1) / BN;
  const int nkt = causal ? min(nkt_all, (q0 + kBM - 1) / BN + 1) : nkt_all;

  // ---- register staging of one K/V tile
  uint32_t koff[kKChunks], vofs[kVChunks];
  int klds[kKChunks], vlds[kVChunks];
#pragma unroll
  for (int j = 0; j < kKChunks; ++j) {
    const int c = tid + j * kThreads;
    const int r = c / kKRowChunks, cc = c % kKRowChunks;
    koff[j] = (uint32_t)r * rsQK + h * DQK * 2 + cc * 16;
    klds[j] = r * SM::kPitch + cc * 16;
  }
#pragma unroll
  for (int j = 0; j < kVChunks; ++j) {
    const int c = tid + j * kThreads;
    const int r = c >> 4, cc = c & 15;  // 16-byte chunk cc of row r
    vofs[j] = (uint32_t)r * rsV + h * kVRow + cc * 16;
    vlds[j] = r * kVRow + (((cc >> 1) ^ v_swz(r)) << 5) + (cc & 1) * 16;
  }
  u32x4 kst[kKChunks], vst[kVChunks];
  auto load_tile = [&](int t) {
    const uint32_t kb0 = (uint32_t)(t * BN) * rsQK, vb0 = (uint32_t)(t * BN) * rsV;
#pragma unroll
    for (int j = 0; j < kKChunks; ++j) kst[j] = buffer_load16(rk, kb0 + koff[j]);
#pragma unroll
    for (int j = 0; j < kVChunks; ++j) vst[j] = buffer_load16(rv, vb0 + vofs[j]);
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int j = 0; j < kKChunks; ++j) lds_store16(&sm.k[buf][klds[j]], kst[j]);
#pragma unroll
    for (int j = 0; j < kVChunks; ++j) lds_store16(&sm.v[buf][vlds[j]], vst[j]);
  };

  // V^T operand reads: lane j of a 16-lane group supplies row j/4 (one key)
  // and bytes (j%4)*8 of the 32-byte chunk (d*2 + (lane/16)%2) of that row.
  // Operand element e of lane half h is key u*16 + (e/4)*8 + h*4 + e%4, so
  // read A covers keys u*16 + h*4 + 0..3 and read B the same plus 8.
  const int gj = lane & 15;
  const int vgrp = (lane >> 4) & 1;
  const int vrow = half * 4 + (gj >> 2);            // key offset of read A inside 16 keys
  const int vbyte = (gj & 3) * 8;

  f32x16 oacc[kDV / 32];
#pragma unroll
  for (int i = 0; i < kDV / 32; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY;  // running row max of c*s (log2 domain)
  float l_run = 0.f;        // this lane's partial row sum (its half of the keys)

  if (nkt > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  if (nkt > 1) load_tile(1);

  for (int t = 0; t < nkt; ++t) {
    const int buf = t & 1;
    const int key0 = t * BN;
    if (!(causal && key0 > q0w + 31)) {  // else: tile entirely above this wave's diagonal
      const uint8_t* kt = sm.k[buf];
      const uint8_t* vt = sm.v[buf];

      // ---- S^T = K . Q^T
      f32x16 sacc[kNKB];
#pragma unroll
      for (int kb = 0; kb < kNKB; ++kb) {
        sacc[kb] = f32x16{};
        const uint8_t* krow = kt + (kb * 32 + col) * SM::kPitch + half * 16;
#pragma unroll
        for (int s = 0; s < kSteps; ++s)
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, lds_load16(krow + s * 32)), qreg[s], sacc[kb], 0, 0, 0);
      }

      // ---- mask (diagonal and ragged-tail tiles only), running max
      if ((causal && key0 + BN - 1 > q0w) || key0 + BN > S) {
        const int lim = causal ? min(q0w + col, S - 1) : S - 1;  // last visible key
#pragma unroll
        for (int kb = 0; kb < kNKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = key0 + kb * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
            sacc[kb][i] = key > lim ? -INFINITY : sacc[kb][i];
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < kNKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
      const float tmax = pair_max(mx) * c_log2;
      if (__any(tmax > m_run)) {
        const float m_new = fmaxf(m_run, tmax);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int d = 0; d < kDV / 32; ++d)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[d][i] *= alpha;
      }

      // ---- P = exp2(c*s - m), bf16, laid out as the B operand of P.V
      bf16x8 pb[BN / 16];
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < kNKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][i], c_log2, -m_run));
          psum += p;
          pb[kb * 2 + (i >> 3)][i & 7] = (__bf16)p;
        }
      l_run += psum;

      // ---- O^T += V^T . P^T
#pragma unroll
      for (int u = 0; u < BN / 16; ++u) {
        const int keyA = u * 16 + vrow, keyB = keyA + 8;
#pragma unroll
        for (int d = 0; d < kDV / 32; ++d) {
          const int c32 = d * 2 + vgrp;
          const i16x4 ra = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(vt + keyA * kVRow +
                                                          ((c32 ^ v_swz(keyA)) << 5) + vbyte));
          const i16x4 rb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(vt + keyB * kVRow +
                                                          ((c32 ^ v_swz(keyB)) << 5) + vbyte));
          const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(ra, rb, 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[u], oacc[d], 0, 0, 0);
        }
      }
    }

    // ---- stage the next tile into the other buffer, then prefetch t+2
    if (t + 1 < nkt) store_tile(buf ^ 1);
    __syncthreads();
    if (t + 2 < nkt) load_tile(t + 2);
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
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<128, 64>), grid, dim3(kThreads), 0, stream,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (__bf16*)o, lse, S,
                       H, BH, nqb, c_log2, causal);
  else
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<192, 32>), grid, dim3(kThreads), 0, stream,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (__bf16*)o, lse, S,
                       H, BH, nqb, c_log2, causal);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace cpattn
