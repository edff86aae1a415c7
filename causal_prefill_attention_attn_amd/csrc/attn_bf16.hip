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
// lanes fall in distinct banks; K rows with a 16-byte chunk swizzle so that
// 16 consecutive keys read 16 distinct chunks.  The row sum adds the
// bf16-rounded probabilities that enter P.V on the matrix unit (16x16x32
// products of each P^T block with a lane-group selector, fp32 accumulation).
//
// Schedule: eight waves per workgroup (two per SIMD) share every K/V tile
// in LDS.  Tiles reach LDS through buffer-to-LDS loads issued by waves 0-3
// three tiles ahead into four stages (rows past the end read as zero), one
// workgroup barrier per tile.  Each wave is software-pipelined one tile deep
// and carries the scores of the next tile and their row maximum: P(t) is
// formed while the matrix unit computes S(t+1), and the maximum of S(t+1)
// is taken while it runs P(t).V(t), so its own matrix and vector work
// overlap.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_device.h"
#include "attn_kernels.h"

namespace cpattn {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Keep a value's computation above this point: the empty volatile statement
// reads and rewrites the registers, so the instructions that produce them
// cannot sink below a later barrier (they touch no memory, so the compiler
// would otherwise move them into the next iteration).
__device__ __forceinline__ void pin(f32x16& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }

constexpr int kWaves = 8;            // waves per workgroup, two per SIMD
constexpr int kBM = 32 * kWaves;     // query rows per workgroup
constexpr int kDV = 128;             // value head dimension
constexpr int kThreads = 64 * kWaves;
constexpr int kVRow = kDV * 2;       // bytes per V row
constexpr int kAhead = 3;            // tiles loaded ahead of the current one
constexpr int kStages = 4;
// The running maximum m is refreshed (and O, l rescaled) only when a row's
// tile maximum exceeds it by more than this many octaves, so probabilities
// can reach 2^kLazyLog2.  P is rounded to bf16, a floating-point format, so
// its relative rounding error does not depend on how far m lags the true
// maximum; O, l and lse = m + log2(l) are the same up to that rounding.
constexpr float kLazyLog2 = 8.0f;

// 32-byte chunk swizzle of a V row: the four consecutive keys one transposed
// read covers land on four distinct even chunk slots
__device__ __forceinline__ int v_swz(int key) { return (key & 3) << 1; }

// wait until at most N vector-memory operations of this wave are in flight
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[15:14]
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// LDS stage of BN keys: K rows of kKPitch bytes (16-byte chunk c of key r
// at slot c ^ (r & 15); for d_qk = 192 the row has 32 slots, 24 used), V
// rows of 256 bytes (32-byte chunk c of key r at c ^ v_swz(r)).
template <int DQK, int BN>
struct Layout {
  static constexpr int kKC = DQK == 128 ? 16 : 32;   // 16-byte slots per K row
  static constexpr int kKPitch = kKC * 16;
  static constexpr int kKBytes = BN * kKPitch;
  static constexpr int kVBytes = BN * kVRow;
};

// f(integral_constant<int, I>) for I = B .. E-1, in order
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

template <int DQK, int BN>
struct Smem {
  using L = Layout<DQK, BN>;
  uint8_t k[kStages][L::kKBytes];
  uint8_t v[kStages][L::kVBytes];
  uint8_t epi[kWaves][4096];  // per wave: its output rows on their way to memory
};

template <int DQK, int BN>
__global__ void __launch_bounds__(kThreads, 1)
attn_fwd_bf16_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                     const __bf16* __restrict__ v, __bf16* __restrict__ o,
                     float* __restrict__ lse, const int32_t* __restrict__ cu, int64_t total,
                    int S_max, int H, int BH, int nqb, float c_log2,
                     int causal, int n_static, int q_cut, int* __restrict__ tail_ctr) {
  using LY = Layout<DQK, BN>;
  constexpr int kSteps = DQK / 16;                 // k-steps of the QK^T product
  constexpr int kNKB = BN / 32;                    // 32-key S blocks per tile
  constexpr int kKRowsPerLoad = 1024 / LY::kKPitch;
  constexpr int kKL = BN / kKRowsPerLoad;          // 1 KB loads of K per tile
  constexpr int kVL = BN / 4;                      // 1 KB loads of V per tile
  constexpr int kLoads = kKL + kVL;
  // the loads of a tile are issued by waves 0-3, the older wave of each
  // SIMD, which the arbiter favours: they reach the barrier first, so the
  // issue work costs least there
  constexpr int kIssuers = 4;
  static_assert(kLoads % kIssuers == 0 && kKL % kIssuers == 0, "uniform load split");
  constexpr int kMine = kLoads / kIssuers;           // loads each issuing wave issues per tile
  using SM = Smem<DQK, BN>;
  __shared__ __attribute__((aligned(1024))) SM sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;  // query column / key row / value column inside a 32-block
  const int half = lane >> 5;

  int qb, bh;
  if (!block_claim(blockIdx.x, nqb, BH, n_static, q_cut, tail_ctr,
                   reinterpret_cast<int*>(&sm.epi[0][0]), qb, bh))
    return;
  const int b = bh / H;
  const int h = bh % H;
  // rows of this problem (a batch entry or a packed sequence); S is its length
  const SeqRows sr = seq_rows(cu, b, S_max, H, total);
  const int S = sr.len;
  const int q0 = qb * kBM;
  if (q0 >= S) return;  // past the end of a shorter sequence: nothing to do
  const int q0w = q0 + wave * 32;
  const uint32_t rsQK = (uint32_t)H * DQK * 2;  // bytes between rows
  const uint32_t rsV = (uint32_t)H * kVRow;
  const int64_t bstrQK = (int64_t)S * rsQK;
  const int64_t bstrV = (int64_t)S * rsV;
  const uint8_t* qb8 = reinterpret_cast<const uint8_t*>(q) + sr.row0 * rsQK;
  const uint8_t* kb8 = reinterpret_cast<const uint8_t*>(k) + sr.row0 * rsQK;
  const uint8_t* vb8 = reinterpret_cast<const uint8_t*>(v) + sr.row0 * rsV;
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

  // ---- tile t lives in LDS stage t % kStages: kLoads buffer-to-LDS loads of
  // 1 KB (K first, then V); wave w < 4 issues loads w, w + 4, ...
  uint32_t go[kMine];  // global offset inside the tile (0xfffffff0: padding, reads zeros)
  int lo_[kMine];      // LDS offset inside the stage (K region, then V region)
#pragma unroll
  for (int i = 0; i < kMine; ++i) {
    const int j = wave % kIssuers + i * kIssuers;
    if (i * kIssuers < kKL) {  // the same kind of load for every wave
      const int row = j * kKRowsPerLoad + lane / LY::kKC;
      const int lc = (lane % LY::kKC) ^ (row & 15);  // logical chunk held by this slot
      go[i] = lc * 16 < DQK * 2 ? (uint32_t)row * rsQK + h * DQK * 2 + lc * 16 : 0xfffffff0u;
      lo_[i] = j * 1024;
    } else {
      const int jv = j - kKL;
      const int row = jv * 4 + lane / 16;
      const int sl = lane % 16;                              // 16-byte slot of the row
      const int lc = (((sl >> 1) ^ v_swz(row)) << 1) | (sl & 1);  // logical 16-byte chunk
      go[i] = (uint32_t)row * rsV + h * kVRow + lc * 16;
      lo_[i] = jv * 1024;
    }
  }
  auto issue_tile = [&](int t) {
    const int st = t % kStages;
    const uint32_t kb0 = (uint32_t)(t * BN) * rsQK, vb0 = (uint32_t)(t * BN) * rsV;
    if (wave >= kIssuers) return;  // waves 4-7 have no loads (their vmcnt waits are no-ops)
#pragma unroll
    for (int i = 0; i < kMine; ++i) {
      if (i * kIssuers < kKL)
        buffer_load_lds16(rk, &sm.k[st][lo_[i]], go[i] == 0xfffffff0u ? go[i] : kb0 + go[i]);
      else
        buffer_load_lds16(rv, &sm.v[st][lo_[i]], vb0 + go[i]);
    }
  };

  // K operand of S block kb, step s: key kb*32 + col, logical chunk 2s + half
  // at slot (2s + half) ^ (col & 15) = (2s) ^ hs with hs = half ^ (col & 15)
  const int kbase = col * LY::kKPitch + ((half ^ (col & 15)) << 4);
  auto kread = [&](const uint8_t* kt, int kb, int s) {
    return __builtin_bit_cast(
        bf16x8, lds_load16(kt + kb * 32 * LY::kKPitch + (kbase ^ (s << 5))));
  };
  // V^T operand reads: lane j of a 16-lane group supplies row j/4 (one key)
  // and bytes (j%4)*8 of the 32-byte chunk (d*2 + (lane/16)%2) of that row.
  // Operand element e of lane half h is key u*16 + (e/4)*8 + h*4 + e%4, so
  // read A covers keys u*16 + h*4 + 0..3 and read B the same plus 8.  The row
  // swizzle depends on key & 3 = (j/4) & 3 only, so one per-lane base serves
  // every (u, d): chunk d*2 + vgrp sits at (vbase ^ (d << 6)) and the keys
  // of block u at +u*16 rows (+8 rows for read B).
  const int gj = lane & 15;
  const int vgrp = (lane >> 4) & 1;
  const int vrow = half * 4 + (gj >> 2);
  const int vbase = vrow * kVRow + (gj & 3) * 8 + ((vgrp ^ v_swz(vrow)) << 5);

  auto active = [&](int t) { return t < nkt && !(causal && t * BN > q0w + 31); };
  // tile t needs the mask (diagonal or ragged) for some row of this wave
  auto masked = [&](int t) {
    const int key0 = t * BN;
    return (causal && key0 + BN - 1 > q0w) || key0 + BN > S;
  };

  f32x16 oacc[kDV / 32];
#pragma unroll
  for (int i = 0; i < kDV / 32; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY;  // running row max of c*s (log2 domain)
  // row sums on v_mfma_f32_16x16x32_bf16: column n of its B operand (a P^T
  // block) is lanes n, n+16, n+32, n+48, i.e. queries n and n+16 with both
  // halves of their keys.  Row m of the A operand comes from lanes m, m+16,
  // m+32, m+48; rows 0 and 8 select the lane groups of query n, rows 4 and
  // 12 those of query n+16, so the first accumulator register of lane l
  // holds the row sum of its own query (the others stay zero).
  f32x4 lacc = f32x4{};
  bf16x8 lsel;
  {
    const int m = lane & 15, g = lane >> 4;
    const bool on = ((m == 0 || m == 8) && !(g & 1)) || ((m == 4 || m == 12) && (g & 1));
    const __bf16 v = on ? (__bf16)1.0f : (__bf16)0.0f;
    lsel = bf16x8{v, v, v, v, v, v, v, v};
  }
  f32x16 sa[kNKB], sb[kNKB];  // score buffers of consecutive tiles

  auto qk = [&](int t, f32x16* sc) {
    const uint8_t* kt = sm.k[t % kStages];
#pragma unroll
    for (int kb = 0; kb < kNKB; ++kb) {
      sc[kb] = f32x16{};
#pragma unroll
      for (int s = 0; s < kSteps; ++s)
        sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kread(kt, kb, s), qreg[s], sc[kb], 0, 0, 0);
    }
  };
  // mask of tile t (diagonal and ragged-tail tiles only)
  auto apply_mask = [&](int t, f32x16* sc) {
    // last visible key offset, less this lane half's 4-key shift, so the
    // comparisons below are against compile-time constants
    const int lim = (causal ? min(q0w + col, S - 1) : S - 1) - t * BN - half * 4;
#pragma unroll
    for (int kb = 0; kb < kNKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kofs = kb * 32 + (i >> 2) * 8 + (i & 3);
        sc[kb][i] = kofs > lim ? -INFINITY : sc[kb][i];
      }
  };
  // row max of a tile: two chains of three-input maxima (max(max(m, a), b)
  // is one v_max3; max(m, max(a, b)) was compiled as two instructions)
  auto tile_max = [&](const f32x16* sc) {
    float ma = -INFINITY, mb = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < kNKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; i += 4) {
        ma = fmaxf(fmaxf(ma, sc[kb][i]), sc[kb][i + 1]);
        mb = fmaxf(fmaxf(mb, sc[kb][i + 2]), sc[kb][i + 3]);
      }
    return pair_max(fmaxf(ma, mb)) * c_log2;
  };
  auto refresh = [&](float tmax) {
    if (__any(tmax > m_run + kLazyLog2)) {
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      lacc[0] *= alpha;
#pragma unroll
      for (int d = 0; d < kDV / 32; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[d][i] *= alpha;
    }
  };
  // P = exp2(c*s - m), bf16, laid out as the B operand of P.V; the row sum
  // adds the rounded probabilities (selector products above)
  auto probs = [&](const f32x16* scur, bf16x8* pb) {
#pragma unroll
    for (int kb = 0; kb < kNKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        pb[kb * 2 + (i >> 3)][i & 7] =
            (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(scur[kb][i], c_log2, -m_run));
#pragma unroll
    for (int u = 0; u < BN / 16; ++u) lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lsel, pb[u], lacc, 0, 0, 0);
  };
  // O^T += V^T . P^T, V^T reads two operands ahead of their use
  auto pv = [&](int t, const bf16x8* pb) {
    constexpr int kPV = (BN / 16) * (kDV / 32);
    const uint32_t vt = lds_addr(sm.v[t % kStages]);
    auto vread = [&](int m) {
      const int u = m / (kDV / 32), d = m % (kDV / 32);
      const uint32_t a = vt + u * 16 * kVRow + (vbase ^ (d << 6));
      const i16x4 ra = ds_read_tr16<0>(a);
      const i16x4 rb = ds_read_tr16<8 * kVRow>(a);
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(ra, rb, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8 vop[kPV];
    vop[0] = vread(0);
    vop[1] = vread(1);
#pragma unroll
    for (int m = 0; m < kPV; ++m) {
      if (m + 2 < kPV) {
        vop[m + 2] = vread(m + 2);
        lds_wait_n<4>(vop[m]);
      } else if (m + 1 < kPV) {
        lds_wait_n<2>(vop[m]);
      } else {
        lds_wait_n<0>(vop[m]);
      }
      const int u = m / (kDV / 32), d = m % (kDV / 32);
      oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[m], pb[u], oacc[d], 0, 0, 0);
    }
  };

  // ---- prologue: tiles 0..2 issued, 0 and 1 complete, S(0) and its max
  float tmax_a = 0.f, tmax_b = 0.f;  // row maxima of the two score buffers
#pragma unroll
  for (int t = 0; t < kAhead; ++t)
    if (t < nkt) issue_tile(t);
  if (nkt > 2) wait_vmcnt<kMine>();
  else wait_vmcnt<0>();
  barrier_nofence();
  if (active(0)) {
    qk(0, sa);
    if (masked(0)) apply_mask(0, sa);
    tmax_a = tile_max(sa);
  }

  // Iteration t: P(t) from S(t) and its max, S(t+1) = K(t+1).Q^T, O += P(t).V(t),
  // then the max of S(t+1).  While tile t+1 is fully visible to every row of
  // the wave the iteration is branch-free apart from the rescale, so the
  // compiler spreads the matrix instructions through the vector work of the
  // same wave: P(t) alongside S(t+1), the max of S(t+1) alongside
  // O += P(t).V(t).  Masked or inactive tiles take the general form.  Each
  // iteration ends in one workgroup barrier.
  static_assert(kAhead == 3, "wait counts assume three tiles ahead");
  auto fast_step = [&](int t, f32x16* scur, f32x16* snext, float tcur, float& tnext) {
    // tile t+3 goes to the stage of tile t-1, finished before the last barrier
    if (t + kAhead < nkt) issue_tile(t + kAhead);
    // d = 192 (32-key tiles): wave priority 1 for the P half and 0 for the
    // P.V half, so that the wave of a SIMD that gets ahead yields to the
    // other before the barrier (measured neutral to negative at d = 128)
    if constexpr (DQK == 192) __builtin_amdgcn_s_setprio(1);
    refresh(tcur);
    bf16x8 pb[BN / 16];
    probs(scur, pb);
    qk(t + 1, snext);
    if constexpr (DQK == 192) __builtin_amdgcn_s_setprio(0);
    pv(t, pb);
    tnext = tile_max(snext);
#pragma unroll
    for (int d = 0; d < kDV / 32; ++d) pin(oacc[d]);
    asm volatile("" : "+v"(lacc));
    pin(tnext);
    // tile t+2 complete for S(t+2) in the next step (tile t+3 may stay in flight)
    if (t + 3 < nkt) wait_vmcnt<kMine>();
    else wait_vmcnt<0>();
    barrier_nofence();
  };
  auto slow_step = [&](int t, f32x16* scur, f32x16* snext, float tcur, float& tnext) {
    if (t + kAhead < nkt) issue_tile(t + kAhead);
    if (active(t)) {
      refresh(tcur);
      bf16x8 pb[BN / 16];
      probs(scur, pb);
      if (active(t + 1)) qk(t + 1, snext);
      pv(t, pb);
      if (active(t + 1)) {
        if (masked(t + 1)) apply_mask(t + 1, snext);
        tnext = tile_max(snext);
      }
    }
    if (t + 3 < nkt) wait_vmcnt<kMine>();
    else wait_vmcnt<0>();
    barrier_nofence();
  };
  // iterations below t_fe have a fully visible next tile (t + 1 < nkt)
  const int lim_all = causal ? min(q0w + 1, S) : S;  // keys [0, lim_all) visible to every row
  const int t_fe = max(0, lim_all / BN - 1);
  // unrolled by two so that the score buffers swap roles without copies; an
  // odd exit copies the scores once
  int t = 0;
  {
    // Steady state: four iterations per pass, one per LDS stage, so that
    // every stage index and LDS address offset is a compile-time constant
    // (no per-tile address or stage arithmetic), and every tile issued ahead
    // exists (t + 6 < nkt), so no load is tested.
    const uint32_t kx0 = lds_addr(sm.k[0]);
    const uint32_t vx0 = lds_addr(sm.v[0]);
    auto issue_c = [&](auto J, int t0) {  // tile t0 + J + 3 into stage (J + 3) % 4
      constexpr int j = decltype(J)::value;
      constexpr int st = (j + kAhead) % kStages;
      const uint32_t kb0 = (uint32_t)((t0 + j + kAhead) * BN) * rsQK;
      const uint32_t vb0 = (uint32_t)((t0 + j + kAhead) * BN) * rsV;
      if (wave >= kIssuers) return;
#pragma unroll
      for (int i = 0; i < kMine; ++i) {
        // tiles of a pass lie inside the buffers: the tile's offset goes in
        // the scalar offset field, except for d = 192 K rows, whose padding
        // slots must read past the buffer (zeros)
        if (i * kIssuers < kKL) {
          if constexpr (LY::kKC * 16 == DQK * 2) {
            buffer_load_lds16_so(rk, &sm.k[st][lo_[i]], go[i], kb0);
          } else {
            buffer_load_lds16(rk, &sm.k[st][lo_[i]], go[i] == 0xfffffff0u ? go[i] : kb0 + go[i]);
          }
        } else {
          buffer_load_lds16_so(rv, &sm.v[st][lo_[i]], go[i], vb0);
        }
      }
    };
    auto qk_c = [&](auto ST, f32x16* sc) {
      constexpr int st = decltype(ST)::value;
#pragma unroll
      for (int kb = 0; kb < kNKB; ++kb) {
        sc[kb] = f32x16{};
#pragma unroll
        for (int s2 = 0; s2 < kSteps; ++s2) {
          const bf16x8 kop = __builtin_bit_cast(
              bf16x8, *(const __attribute__((address_space(3))) u32x4*)(uintptr_t)(
                          kx0 + st * LY::kKBytes + kb * 32 * LY::kKPitch + (kbase ^ (s2 << 5))));
          sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qreg[s2], sc[kb], 0, 0, 0);
        }
      }
    };
    auto pv_c = [&](auto ST, const bf16x8* pb) {
      constexpr int st = decltype(ST)::value;
      constexpr int kPV = (BN / 16) * (kDV / 32);
      auto vread = [&](auto M) {
        constexpr int m = decltype(M)::value;
        constexpr int u = m / (kDV / 32), d = m % (kDV / 32);
        constexpr int off = st * LY::kVBytes + u * 16 * kVRow;
        const uint32_t a = vx0 + (vbase ^ (d << 6));
        const i16x4 ra = ds_read_tr16<off>(a);
        const i16x4 rb = ds_read_tr16<off + 8 * kVRow>(a);
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(ra, rb, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      bf16x8 vop[kPV];
      vop[0] = vread(std::integral_constant<int, 0>{});
      vop[1] = vread(std::integral_constant<int, 1>{});
      auto body = [&](auto M) {
        constexpr int m = decltype(M)::value;
        if constexpr (m + 2 < kPV) {
          vop[m + 2] = vread(std::integral_constant<int, m + 2>{});
          lds_wait_n<4>(vop[m]);
        } else if constexpr (m + 1 < kPV) {
          lds_wait_n<2>(vop[m]);
        } else {
          lds_wait_n<0>(vop[m]);
        }
        constexpr int u = m / (kDV / 32), d = m % (kDV / 32);
        oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[m], pb[u], oacc[d], 0, 0, 0);
      };
      static_for<0, kPV>(body);
    };
    auto step_c = [&](auto J, int t0, f32x16* scur, f32x16* snext, float tcur, float& tnext) {
      constexpr int j = decltype(J)::value;
      issue_c(J, t0);
      if constexpr (DQK == 192) __builtin_amdgcn_s_setprio(1);
      refresh(tcur);
      bf16x8 pb[BN / 16];
      probs(scur, pb);
      qk_c(std::integral_constant<int, (j + 1) % kStages>{}, snext);
      if constexpr (DQK == 192) __builtin_amdgcn_s_setprio(0);
      pv_c(std::integral_constant<int, j>{}, pb);
      tnext = tile_max(snext);
#pragma unroll
      for (int d = 0; d < kDV / 32; ++d) pin(oacc[d]);
      asm volatile("" : "+v"(lacc));
      pin(tnext);
      wait_vmcnt<kMine>();
      barrier_nofence();
    };
    for (; t + kStages - 1 < t_fe && t + kStages - 1 + kAhead < nkt; t += kStages) {
      step_c(std::integral_constant<int, 0>{}, t, sa, sb, tmax_a, tmax_b);
      step_c(std::integral_constant<int, 1>{}, t, sb, sa, tmax_b, tmax_a);
      step_c(std::integral_constant<int, 2>{}, t, sa, sb, tmax_a, tmax_b);
      step_c(std::integral_constant<int, 3>{}, t, sb, sa, tmax_b, tmax_a);
    }
  }
  for (; t + 1 < t_fe; t += 2) {
    fast_step(t, sa, sb, tmax_a, tmax_b);
    fast_step(t + 1, sb, sa, tmax_b, tmax_a);
  }
  if (t < t_fe) {
    fast_step(t, sa, sb, tmax_a, tmax_b);
#pragma unroll
    for (int kb = 0; kb < kNKB; ++kb) sa[kb] = sb[kb];
    tmax_a = tmax_b;
    ++t;
  }
  for (; t < nkt; t += 2) {
    slow_step(t, sa, sb, tmax_a, tmax_b);
    if (t + 1 < nkt) slow_step(t + 1, sb, sa, tmax_b, tmax_a);
  }

  // ---- epilogue: O / l -> bf16, lse = ln2 * (m + log2 l)
  const float l_tot = lacc[0];
  const int qi = q0w + col;
  store_rows_bf16<kDV>(oacc, 1.0f / l_tot, sm.epi[wave], o, sr.row0 + q0w, (int64_t)H * kDV,
                       (int64_t)h * kDV, S - q0w, lane);
  if (qi < S && lse != nullptr && half == 0)
    lse[sr.lse0 + h * sr.lse_hs + qi] = (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
}

}  // namespace

int launch_attn_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                     const int32_t* cu, int64_t total, int B, int S, int H, int d_qk,
                     float softmax_scale, int causal, int32_t* tail_ctr, hipStream_t stream) {
  const int nqb = (S + kBM - 1) / kBM;
  const int BH = B * H;
  const BlockGrid bg = block_grid(nqb, BH, cu == nullptr, tail_ctr != nullptr);
  if (bg.q_cut && launch_clear_i32(tail_ctr, stream) != 0) return -1;
  const dim3 grid((unsigned)bg.grid);
  const float c_log2 = softmax_scale * 1.4426950408889634f;
  if (d_qk == 128)
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<128, 64>), grid, dim3(kThreads), 0, stream,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (__bf16*)o, lse, cu, total, S,
                       H, BH, nqb, c_log2, causal, bg.n_static, bg.q_cut, (int*)tail_ctr);
  else
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<192, 32>), grid, dim3(kThreads), 0, stream,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (__bf16*)o, lse, cu, total, S,
                       H, BH, nqb, c_log2, causal, bg.n_static, bg.q_cut, (int*)tail_ctr);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace cpattn
