// FP8 (OCP E4M3FN) causal prefill attention forward for gfx950 (CDNA4).
//
// Both products run on v_mfma_scale_f32_32x32x64_f8f6f4, the FP8 matrix
// path that runs at twice the BF16 rate; the softmax between them runs on
// the vector unit at the same speed in either precision ("Por que a atencao
// FP8 tem desempenho inferior no MI355X?" on the acheiumaia.com.br page).
// Work is organised per wave as 32 queries against the keys of a tile, the
// unit the pages cost (same section).
//
// Per wave (32 query rows), per tile of 64 keys:
//   S^T = K . Q^T   A = K rows (one key per lane column), B = Q^T (one query
//                   per lane column), 32 bytes of the head dimension per
//                   lane per step.  Lane l of the result holds query l%32 and
//                   16 keys of each 32-key block, so row maxima are in-lane
//                   plus one exchange between lane halves.
//   P               each 64-key block of a row is scaled by a power of two
//                   2^k before rounding to e4m3, with k chosen from the
//                   block's largest score so the block maximum lands in
//                   (128, 256]; the scale is removed inside the scaled
//                   matrix instruction through its E8M0 operand (the block
//                   scaling of "Como o motor de atencao FP8 da Zyphra
//                   funciona" on the miraibroadcast.com page).  In the
//                   32x32x64 instruction a lane's scale covers the 32-key
//                   block held by bytes 0-15 (or 16-31) of both lane halves,
//                   so both halves carry the same 64-key exponent.
//   l               the row sum is taken from the rounded P that enters
//                   P.V, with one extra matrix instruction per 64-key block
//                   that multiplies P^T by a selector matrix of ones and
//                   zeros (same section of that page): the half-size
//                   16x16x128 instruction sums each lane's own query, and the
//                   block's 2^-k is applied to that sum on the vector unit.
//   O^T += V^T.P^T  A = V^T read from a row-major V tile in LDS with
//                   ds_read_b64_tr_b8 (16 lanes cooperatively read 8 rows of
//                   16 bytes and each receives one column), B = P^T straight
//                   from registers.
// The running max m of a row is refreshed when it sees a larger tile
// maximum, and only the lanes of the rows whose maximum grew multiply their
// O and l (skipped when no row of the wave grew): the others would multiply
// by exactly 1, and lanes masked off draw less power, which under the
// board's power limit is returned as clock.  With m equal to the row max,
// the row's largest probability becomes exactly 2^8 before rounding, so the
// dominant weight of peaked rows is exact in e4m3.  (Refreshing only past a
// threshold saves rescales but makes the top weight inexact: measured a few
// per cent faster with several times the LSE error of peaked rows.)
//
// Two ways to form P (template flag kLean):
//   exact  p = exp2(c*s - m + k) on the transcendental unit, then
//          v_cvt_pk_fp8_f32 (round to nearest even), two bytes per op.
//   lean   no exponential: the e4m3 bit pattern of 2^y (y = c*s - m + k) is
//          written directly as the integer round(8*(y + 7) - d): the integer
//          part of y lands in the exponent field (bias 7) and 8*frac(y) in
//          the three mantissa bits, i.e. 2^f is replaced by 1 + f.  That is
//          one multiply-add per probability plus an integer conversion: the
//          multiply-add yields (256 z + 127.5) / 65535 for the code z, the
//          16-bit normalised conversion (round to nearest, clamp to [0, 1])
//          of a pair holds round(z) in each high byte, and one byte permute
//          gathers four codes, 1.75 instructions per probability (the lean-P
//          technique of "Como o motor de atencao FP8 da Zyphra funciona" on
//          the miraibroadcast.com page).  The shift d = 0.4567
//          makes the approximation unbiased on average (mean of decoded
//          value / 2^y over a uniform fractional part is 1), so the row sum
//          and the LSE carry no systematic bias; the block maximum y = 8
//          still maps exactly to 256 (byte 0x78).
//
// K/V tiles pass through LDS stages filled directly by buffer-to-LDS loads
// issued by waves 0-3 (rows past the end read as zero): eight stages with
// tile t+4 issued at t and a barrier after every second tile at d = 128,
// four stages with tile t+3 issued at t and a barrier per tile at d = 192.
// The bulk of the iterations run one per stage per pass (eight at d = 128,
// four at d = 192), with every LDS address offset a compile-time constant.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_device.h"
#include "attn_kernels.h"

namespace cpattn {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kDV = 128;
constexpr int kE8M0One = 127;      // E8M0 encoding of 2^0
constexpr float kLeanShift = 0.4567f;  // lean-P re-centring, in units of 1/8 octave
// the lean code's offset in the units of the 16-bit normalised conversion:
// (256 (8 x - kLeanShift) + 127.5) / 65535 = kOfsK x + kOfsC
constexpr float kOfsK = 2048.0f / 65535.0f;
constexpr float kOfsC = (127.5f - 256.0f * kLeanShift) / 65535.0f;

__device__ __forceinline__ f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c, int scale_a, int scale_b) {
  // operand formats 0/0 = E4M3 x E4M3; op_sel 0 = byte 0 of each scale VGPR
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, scale_a, 0, scale_b);
}
// The same product without block scales: zero scale operands select the
// unscaled instruction (v_mfma_f32_32x32x64_f8f6f4), whose result equals the
// scaled one with both scales 2^0 and which needs no scale registers.
__device__ __forceinline__ f32x16 mfma_f8_plain(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Keep a value's computation above this point: the empty volatile statement
// reads and rewrites the registers, so the instructions that produce them
// cannot sink below a later barrier (they touch no memory, so the compiler
// would otherwise move them into the next iteration).
__device__ __forceinline__ void pin(f32x16& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }

// 16-byte chunk swizzle of a V row (128 bytes = 8 chunks) so that the eight
// key rows one ds_read_b64_tr_b8 touches fall in distinct LDS banks
__device__ __forceinline__ int v_swz(int key) { return ((key >> 1) & 1) * 2 + ((key >> 3) & 1) * 4; }

// key (offset inside a 64-key block) whose probability sits in byte e of the
// P^T operand of lane half h: byte e < 16 comes from S block 0 register e,
// e >= 16 from S block 1 register e-16
__device__ __forceinline__ int p_key(int h, int e) {
  return (e >> 4) * 32 + ((e & 15) >> 2) * 8 + h * 4 + (e & 3);
}

// wait until at most n vector-memory operations of this wave are in flight
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[15:14]
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// LDS layout of one pipeline stage: K rows of kKPitch bytes whose 16-byte
// chunks are XOR-swizzled (conflict-free 16-byte reads by 16 consecutive
// keys), V rows of 128 bytes swizzled by v_swz.  Rows are filled by
// buffer-to-LDS loads: each load instruction writes 64 lanes x 16 bytes to
// consecutive LDS addresses, so a lane picks the global chunk that belongs
// at its slot (padding slots read past the end of the buffer: zeros).
template <int DQK, int BN>
struct Layout {
  static constexpr int kKC = DQK == 128 ? 8 : 16;          // chunk slots per K row
  static constexpr int kKPitch = kKC * 16;
  static constexpr int kKBytes = BN * kKPitch;
  static constexpr int kVBytes = BN * kDV;
  // d = 128: eight stages, tile t+4 issued at t and a workgroup barrier
  // after every second tile; d = 192 (24 KB per stage):
  // four stages and a barrier per tile (tile t+3 issued at t)
  static constexpr bool kPair = DQK == 128;
  static constexpr int kStages = kPair ? 8 : 4;
  __device__ static int k_swz(int row) { return DQK == 128 ? (row >> 1) & 7 : row & 15; }
};

// O rows times the Sylvester-Hadamard matrix of order 128 (unnormalised),
// in place.  Undoes a V rotated by the normalised matrix before quantization
// (the rotation of "Precisao, estabilidade e efeito na pratica" on the
// miraibroadcast.com page): (P.(V H)) H = P.V since H H = 128 I.  Lane
// (col, half) holds element j = d*32 + g*8 + half*4 + e of row col at
// oacc[d][g*4 + e]; the butterfly on bit b of j pairs (x_j, x_{j+2^b}) into
// (x_j + x_{j+2^b}, x_j - x_{j+2^b}).  Bits 0, 1, 3, 4, 5, 6 are inside the
// lane; bit 2 is the lane half, exchanged by a permlane32 swap.
__device__ __forceinline__ void hadamard_o_rows(f32x16* oacc, int half) {
#pragma unroll
  for (int m = 1; m < 16; m <<= 1)  // bits of g*4 + e
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (!(i & m)) {
          const float a = oacc[d][i], b = oacc[d][i | m];
          oacc[d][i] = a + b;
          oacc[d][i | m] = a - b;
        }
#pragma unroll
  for (int m = 1; m < 4; m <<= 1)  // bits of d
#pragma unroll
    for (int d = 0; d < 4; ++d)
      if (!(d & m)) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float a = oacc[d][i], b = oacc[d | m][i];
          oacc[d][i] = a + b;
          oacc[d | m][i] = a - b;
        }
      }
  // bit 2 of j: the swap leaves the lower-half lane's value in r[0] and the
  // upper-half lane's in r[1] in every lane
  const float sgn = half ? -1.0f : 1.0f;
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(oacc[d][i]),
                                                      __float_as_uint(oacc[d][i]), false, false);
      oacc[d][i] = __builtin_fmaf(sgn, __uint_as_float(r[1]), __uint_as_float(r[0]));
    }
}

template <int DQK, int BN>
struct Smem {
  using L = Layout<DQK, BN>;
  uint8_t k[L::kStages][L::kKBytes];
  uint8_t v[L::kStages][L::kVBytes];
  uint8_t epi[8][4096];  // per wave: its output rows on their way to memory
};

// One workgroup of 4*kOcc waves per compute unit (kOcc waves per SIMD),
// each wave owning 32 query rows; the 32*4*kOcc rows of the workgroup share
// every K/V tile in LDS, which keeps K/V re-reads from L2 low.  Each wave is
// software-pipelined one tile deep and carries the scores of the next tile
// and their row maximum from one iteration to the next.  Iteration t forms
// P(t) on the vector unit while the matrix unit computes S(t+1) = K(t+1).Q^T,
// then runs O += P(t).V(t) on the matrix unit while the vector unit takes the
// row maximum of S(t+1).  Both halves are branch-free in the iterations whose
// next tile needs no mask, so the compiler spreads the matrix instructions
// through the vector work of the same wave, and the other wave of the SIMD
// fills the remaining gaps (the overlap of matrix and vector work that "Como
// o motor de atencao FP8 da Zyphra funciona" on the miraibroadcast.com page
// describes, obtained here from instruction order inside each wave).  A
// wave runs the first half at priority 1 and the second at priority 0, so
// the wave of a SIMD that gets ahead yields to the other (the arbiter
// otherwise favours the older wave throughout and it idles at the barrier).
template <int DQK, int BN, bool kLean, int kOcc>
__global__ void __launch_bounds__(256 * kOcc, 1)
attn_fwd_fp8_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ k,
                    const uint8_t* __restrict__ v, __bf16* __restrict__ o,
                    float* __restrict__ lse, const int32_t* __restrict__ cu, int64_t total,
                    int S_max, int H, int BH, int nqb, float c_log2, float c8n,
                    float v_descale, int causal, int rot_o, int n_static, int q_cut,
                    int* __restrict__ tail_ctr) {
  using LY = Layout<DQK, BN>;
  constexpr int kWaves = 4 * kOcc;
  static_assert(kWaves <= 8, "one 4 KB output staging area per wave");
  constexpr int kBM = 32 * kWaves;                 // query rows per workgroup
  constexpr int kSteps = DQK / 64;                 // 32x32x64 steps of Q.K^T
  constexpr int kKRowsPerLoad = 1024 / LY::kKPitch;
  constexpr int kKL = BN / kKRowsPerLoad;          // 1 KB loads of K per tile
  constexpr int kVL = BN / 8;                      // 1 KB loads of V per tile
  constexpr int kLoads = kKL + kVL;
  static_assert(BN == 64, "one 64-key scale block per tile");
  using SM = Smem<DQK, BN>;
  __shared__ __attribute__((aligned(1024))) SM sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int col = lane & 31;
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
  const uint32_t rsQK = (uint32_t)H * DQK;  // bytes between consecutive rows
  const uint32_t rsV = (uint32_t)H * kDV;
  const int64_t bstrQK = (int64_t)S * rsQK;
  const int64_t bstrV = (int64_t)S * rsV;
  // one batch of q/k/v per buffer resource; rows >= S read as zero
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + sr.row0 * rsQK, (uint32_t)bstrQK);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + sr.row0 * rsQK, (uint32_t)bstrQK);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + sr.row0 * rsV, (uint32_t)bstrV);

  // ---- Q^T operand: lane (query col, half) holds d = s*64 + half*32 .. +31
  i32x8 qreg[kSteps];
  {
    const uint32_t off = (uint32_t)(q0w + col) * rsQK + h * DQK + half * 32;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const u32x4 lo = buffer_load16(rq, off + s * 64);
      const u32x4 hi = buffer_load16(rq, off + s * 64 + 16);
      qreg[s] = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  }

  const int nkt_all = (S + BN - 1) / BN;
  const int nkt = causal ? min(nkt_all, (q0 + kBM - 1) / BN + 1) : nkt_all;

  // ---- tile t (K and V) lives in LDS buffer t % kStages.  A tile is kLoads
  // buffer-to-LDS loads of 1 KB (K first, then V), all issued by waves
  // 0-3 (wave w issues loads w, w + 4, ..., the same number and kinds in
  // each).  Those waves are the older wave of each SIMD, which the
  // arbiter favours: they reach the end of an iteration first and wait at the
  // barrier, so the issue work costs least there.
  constexpr int kIssuers = 4;
  static_assert(kLoads % kIssuers == 0 && kKL % kIssuers == 0, "uniform load split");
  constexpr int kMine = kLoads / kIssuers;   // loads each issuing wave issues per tile
  uint32_t go[kMine];  // global offset inside the tile (0xfffffff0: padding, reads zeros)
  int lo_[kMine];      // LDS offset inside the stage (K region, then V region)
#pragma unroll
  for (int i = 0; i < kMine; ++i) {
    const int j = wave % kIssuers + i * kIssuers;
    if (i * kIssuers < kKL) {  // the same kind of load for every wave
      const int row = j * kKRowsPerLoad + lane / LY::kKC;
      const int lc = (lane % LY::kKC) ^ LY::k_swz(row);  // logical chunk held by this slot
      go[i] = lc * 16 < DQK ? (uint32_t)row * rsQK + h * DQK + lc * 16 : 0xfffffff0u;
      lo_[i] = j * 1024;
    } else {
      const int jv = j - kKL;
      const int row = jv * 8 + lane / 8;
      const int lc = (lane % 8) ^ v_swz(row);
      go[i] = (uint32_t)row * rsV + h * kDV + lc * 16;
      lo_[i] = jv * 1024;
    }
  }
  auto issue_tile = [&](int t) {
    const int buf = t % LY::kStages;
    const uint32_t kb = (uint32_t)(t * BN) * rsQK, vb = (uint32_t)(t * BN) * rsV;
    if (wave >= kIssuers) return;  // waves 4-7 have no loads (their vmcnt waits are no-ops)
#pragma unroll
    for (int i = 0; i < kMine; ++i) {
      if (i * kIssuers < kKL)
        buffer_load_lds16(rk, &sm.k[buf][lo_[i]], go[i] == 0xfffffff0u ? go[i] : kb + go[i]);
      else
        buffer_load_lds16(rv, &sm.v[buf][lo_[i]], vb + go[i]);
    }
  };

  // V^T operand reads: the key of operand byte group t4 is p_key(half, t4*8 +
  // gi/2) = that of group 0 plus 16*t4, and its row swizzle (key bits 1 and
  // 3) does not depend on t4, so one base address serves all four reads: the
  // chunk (d*2 + dvhalf) ^ swz sits at byte (vbase ^ (d << 5)) + 2048*t4,
  // with vbase = row*128 + (gi%2)*8 + dvhalf*16 + (swz/2)*32.
  const int gi = lane & 15;
  const int dvhalf = (lane >> 4) & 1;
  const int vkey0 = p_key(half, gi >> 1);
  const int vbase = vkey0 * kDV + (gi & 1) * 8 + dvhalf * 16 + (v_swz(vkey0) >> 1) * 32;
  // K operand reads: row kb*32 + col (its swizzle depends on col only) and
  // logical chunk s*4 + half*2 + part; the swizzled chunk offset is
  // kbase ^ ((s*4 + part) << 4) with kbase = row offset | ((half*2 ^ swz) << 4)
  const int kbase = col * LY::kKPitch + (((half * 2) ^ LY::k_swz(col)) << 4);

  // row sums on v_mfma_f32_16x16x128_f8f6f4: column n of its B operand is
  // lanes n, n+16, n+32, n+48 of the P^T registers, i.e. queries n and n+16,
  // each with both of its key halves.  Row m of the A operand comes from
  // lanes m, m+16, m+32, m+48; rows 0 and 8 select the lane groups of query
  // n, rows 4 and 12 those of query n+16, so output row 4*(l/16) of lane l
  // (its first accumulator register) is the sum over the tile of lane l's
  // own query.
  i32x8 lsel;
  {
    const int m = lane & 15, g = lane >> 4;
    const bool on = ((m == 0 || m == 8) && !(g & 1)) || ((m == 4 || m == 12) && (g & 1));
    const int v = on ? 0x38383838 : 0;  // e4m3 1.0 or 0
    lsel = i32x8{v, v, v, v, v, v, v, v};
  }

  auto qk = [&](int t, f32x16* sa) {  // S^T of tile t = K(t) . Q^T, two 32-key blocks
    const uint8_t* kt = sm.k[t % LY::kStages];
    sa[0] = f32x16{};
    sa[1] = f32x16{};
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint8_t* kblk = kt + kb * 32 * LY::kKPitch;
        const i32x4 lo = *reinterpret_cast<const i32x4*>(kblk + (kbase ^ ((s * 4) << 4)));
        const i32x4 hi = *reinterpret_cast<const i32x4*>(kblk + (kbase ^ ((s * 4 + 1) << 4)));
        sa[kb] = mfma_f8_plain(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), qreg[s], sa[kb]);
      }
  };
  auto active = [&](int t) { return t < nkt && !(causal && t * BN > q0w + 31); };
  // tile t needs the mask (diagonal or ragged) for some row of this wave
  auto masked = [&](int t) {
    const int key0 = t * BN;
    return (causal && key0 + BN - 1 > q0w) || key0 + BN > S;
  };

  f32x16 oacc[kDV / 32];
#pragma unroll
  for (int i = 0; i < kDV / 32; ++i) oacc[i] = f32x16{};
  float l_run = 0.f;        // row sum of this lane's query
  float m_run = -INFINITY;  // max of c*s in use (log2 domain)
  f32x16 sa[2], sb[2];      // score buffers of consecutive tiles

  // mask of tile t (diagonal or ragged) applied to its scores
  auto apply_mask = [&](int t, f32x16* s) {
    const int key0 = t * BN;
    const int lim = (causal ? min(q0w + col, S - 1) : S - 1) - key0;  // last visible offset
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kofs = kb * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
        s[kb][i] = kofs > lim ? -INFINITY : s[kb][i];
      }
  };
  // largest c*s of the row in a tile (block 0 chain, then block 1)
  auto tile_max = [&](const f32x16* s) {
    float mx0 = fmaxf(s[0][0], s[0][1]), mx1 = fmaxf(s[1][0], s[1][1]);
#pragma unroll
    for (int i = 2; i < 16; i += 2) mx0 = fmaxf(fmaxf(mx0, s[0][i]), s[0][i + 1]);
#pragma unroll
    for (int i = 2; i < 16; i += 2) mx1 = fmaxf(fmaxf(mx1, s[1][i]), s[1][i + 1]);
    return pair_max(fmaxf(mx0, mx1)) * c_log2;
  };
  // running max refresh: the lanes of the rows whose max grew (and only
  // those) take the new max and rescale O and l.  A per-lane branch: the
  // region runs with EXEC set to those lanes and is skipped when there are
  // none, with no vector instruction spent on the test beyond the compare.
  auto refresh = [&](float bmax) {
    if (bmax > m_run) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - bmax);
      m_run = bmax;
#pragma unroll
      for (int d = 0; d < kDV / 32; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[d][i] *= alpha;
      l_run *= alpha;
    }
  };
  // P = e4m3(2^(c*s - m + k)); k = 8 - ceil(block max - m) puts the block
  // maximum in (2^7, 2^8]; k >= 0 since block max <= m after the refresh
  auto probs = [&](const f32x16* scur, float bmax, int& pscale) {
    // k = 8 - ce with ce = ceil(block max - m) in [-118, 0]: the E8M0 code
    // of 2^-k is 127 - k = 119 + ce
    const float ce = fmaxf(__builtin_ceilf(bmax - m_run), -118.0f);
    pscale = (int)(ce + 119.0f);
    i32x8 pw = __builtin_nondeterministic_value(pw);  // every byte is written below
    if constexpr (kLean) {
      // z = 8 c s + 8 (7 + k - m) - shift is the code in units of 1/8
      // octave; the 16-bit normalised conversion of (256 z + 127.5) / 65535
      // (round to nearest, clamped to [0, 1]) holds round(z) in its high
      // byte, and one byte permute gathers the high bytes of two pairs.  The
      // offset is kOfsK (15 - ce - m) + kOfsC in those units.
      const float ofsn = __builtin_fmaf(-ce, kOfsK, __builtin_fmaf(-m_run, kOfsK, 15.0f * kOfsK + kOfsC));
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int kb = w >> 2;
        const int i0 = (w & 3) * 4;
        const auto lo = __builtin_amdgcn_cvt_pknorm_u16(__builtin_fmaf(scur[kb][i0 + 0], c8n, ofsn),
                                                        __builtin_fmaf(scur[kb][i0 + 1], c8n, ofsn));
        const auto hi = __builtin_amdgcn_cvt_pknorm_u16(__builtin_fmaf(scur[kb][i0 + 2], c8n, ofsn),
                                                        __builtin_fmaf(scur[kb][i0 + 3], c8n, ofsn));
        pw[w] = (int)__builtin_amdgcn_perm(__builtin_bit_cast(unsigned, hi),
                                           __builtin_bit_cast(unsigned, lo), 0x07050301u);
      }
    } else {
      const float ofs = (8.0f - ce) - m_run;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int kb = w >> 2;
        const int i0 = (w & 3) * 4;
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(scur[kb][i0 + 0], c_log2, ofs));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(scur[kb][i0 + 1], c_log2, ofs));
        const float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(scur[kb][i0 + 2], c_log2, ofs));
        const float p3 = __builtin_amdgcn_exp2f(__builtin_fmaf(scur[kb][i0 + 3], c_log2, ofs));
        int word = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, pw[w], false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, word, true);
        pw[w] = word;
      }
    }
    return pw;
  };
  // O^T += V^T . P^T and the row sum of P; V^T operands of the four 32-row
  // blocks of d read two blocks ahead (inline assembly: the reads wait for
  // no buffer-to-LDS load in flight)
  auto pv = [&](int t, const i32x8& pw, int pscale) {
    const uint32_t vt = lds_addr(sm.v[t % LY::kStages]);
    i32x2 r[2][4];
    auto vread = [&](int d, i32x2* x) {
      const uint32_t a = vt + (vbase ^ (d << 5));
      x[0] = ds_read_tr8<0 * 16 * kDV>(a);
      x[1] = ds_read_tr8<1 * 16 * kDV>(a);
      x[2] = ds_read_tr8<2 * 16 * kDV>(a);
      x[3] = ds_read_tr8<3 * 16 * kDV>(a);
    };
    vread(0, r[0]);
    vread(1, r[1]);
#pragma unroll
    for (int d = 0; d < kDV / 32; ++d) {
      i32x2* x = r[d & 1];
      if (d + 1 < kDV / 32) lds_wait4<4>(x[0], x[1], x[2], x[3]);  // block d+1 may be in flight
      else lds_wait4<0>(x[0], x[1], x[2], x[3]);
      const i32x8 a = __builtin_shufflevector(
          __builtin_shufflevector(x[0], x[1], 0, 1, 2, 3),
          __builtin_shufflevector(x[2], x[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
      oacc[d] = mfma_f8(a, pw, oacc[d], kE8M0One, pscale);
      if (d + 2 < kDV / 32) vread(d + 2, x);
    }
    {
      const f32x4 lt = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(lsel, pw, f32x4{}, 0, 0, 0, 0, 0, 0);
      l_run = __builtin_fmaf(lt[0], __uint_as_float((unsigned)pscale << 23), l_run);
    }
  };

  // ---- prologue: tiles 0..2 issued, 0 and 1 complete, S(0) and its max
  float bmax_a = 0.0f, bmax_b = 0.0f;  // tile maxima of the two score buffers
#pragma unroll
  for (int t = 0; t < (LY::kPair ? 4 : 3); ++t)
    if (t < nkt) issue_tile(t);
  // tiles 0..2 (pairs) or 0..1 complete; the last issued may stay in flight
  if (nkt > (LY::kPair ? 3 : 2)) wait_vmcnt<kMine>(); else wait_vmcnt<0>();
  barrier_nofence();
  if (active(0)) {
    qk(0, sa);
    if (masked(0)) apply_mask(0, sa);
    bmax_a = tile_max(sa);
  }

  // Loads ahead and barriers.  Per tile: tile t+3 goes to the stage of tile
  // t-1, finished before the last barrier; after the iteration each wave
  // waits for its own loads of tile t+2 (needed for S(t+2) next), then the
  // barrier (no fence: a release would wait for the loads of tile t+3 too).
  // Per pair (d = 128): at every t tile t+4 goes to the stage of tile t-4,
  // finished before the last barrier (after iteration t-1 or t-2); after
  // odd t each wave waits for its loads of tile t+3 (needed for S(t+3) in
  // iteration t+2, before the next barrier) and the barrier.
  auto issue_ahead = [&](int t) {
    if constexpr (LY::kPair) {
      if (t + 4 < nkt) issue_tile(t + 4);
    } else {
      if (t + 3 < nkt) issue_tile(t + 3);
    }
  };
  auto sync_after = [&](int t) {
    if constexpr (LY::kPair) {
      if (t & 1) {
        if (t + 4 < nkt) wait_vmcnt<kMine>(); else wait_vmcnt<0>();
        barrier_nofence();
      }
    } else {
      if (t + 3 < nkt) wait_vmcnt<kMine>(); else wait_vmcnt<0>();
      barrier_nofence();
    }
  };

  // Iteration t: P(t) from S(t) and its max, S(t+1) = K(t+1).Q^T, O += P(t).V(t),
  // then the max of S(t+1).  While tile t+1 is fully visible to every row of
  // the wave (all but the last iterations of a wave) the iteration is two
  // straight-line regions whose matrix instructions are interleaved with the
  // vector work: P(t) alongside S(t+1), and the max of S(t+1) alongside
  // O += P(t).V(t).  The remaining iterations (masked or inactive tiles) run
  // the general form.  Barriers come after fixed iterations (every one, or
  // every odd one with tile pairs), so all waves pass the same number.
  auto fast_step = [&](int t, f32x16* scur, f32x16* snext, float bcur, float& bnext) {
    issue_ahead(t);
    // Wave priority 1 for the first half, 0 for the second: the two waves of
    // a SIMD start the iteration together after the barrier, and the one
    // that gets ahead drops below the other once it reaches P.V, so the
    // arbiter (which otherwise favours the older wave throughout) lets the
    // lagging wave catch up before the next barrier.
    __builtin_amdgcn_s_setprio(1);
    refresh(bcur);
    int pscale;
    const i32x8 pw = probs(scur, bcur, pscale);
    qk(t + 1, snext);
    __builtin_amdgcn_s_setprio(0);
    pv(t, pw, pscale);
    bnext = tile_max(snext);
#pragma unroll
    for (int d = 0; d < kDV / 32; ++d) pin(oacc[d]);
    pin(l_run);
    pin(bnext);
    sync_after(t);
  };
  auto slow_step = [&](int t, f32x16* scur, f32x16* snext, float bcur, float& bnext) {
    issue_ahead(t);
    if (active(t)) {
      refresh(bcur);
      int pscale;
      const i32x8 pw = probs(scur, bcur, pscale);
      if (active(t + 1)) qk(t + 1, snext);
      pv(t, pw, pscale);
      if (active(t + 1)) {
        if (masked(t + 1)) apply_mask(t + 1, snext);
        bnext = tile_max(snext);
      }
    }
    sync_after(t);
  };
  // first iteration whose next tile is masked: iterations below it take the
  // straight-line form (tile t+1 < nkt is then fully visible)
  int t_fe = 0;
  {
    const int lim = causal ? min(q0w + 1, S) : S;   // keys [0, lim) visible to every row
    t_fe = max(0, lim / BN - 1);
  }
  // unrolled by two so that the two score buffers swap roles without copies;
  // an odd exit copies the scores once
  int t = 0;
  {
    // Steady state: one iteration per LDS stage per pass (eight at d = 128,
    // four at d = 192), so that every stage index and LDS address offset is
    // a compile-time constant (no per-tile address or stage arithmetic), and
    // every tile issued ahead exists, so no load is tested.
    constexpr int kS = LY::kStages;
    constexpr int kAhead = LY::kPair ? 4 : 3;     // tiles issued ahead
    // per-lane LDS addresses of the K and V^T operand reads in stage 0: K
    // logical chunk s*4 + part of this lane's row, V^T block d
    uint32_t kx[2 * kSteps], vx[kDV / 32];
#pragma unroll
    for (int c = 0; c < 2 * kSteps; ++c)
      kx[c] = lds_addr(sm.k[0]) + (kbase ^ ((((c >> 1) * 4) + (c & 1)) << 4));
#pragma unroll
    for (int d = 0; d < kDV / 32; ++d) vx[d] = lds_addr(sm.v[0]) + (vbase ^ (d << 5));
    auto issue_c = [&](auto J, int t0) {  // tile t0 + J + kAhead into its stage
      constexpr int j = decltype(J)::value;
      constexpr int buf = (j + kAhead) % kS;
      const uint32_t kb = (uint32_t)((t0 + j + kAhead) * BN) * rsQK;
      const uint32_t vb = (uint32_t)((t0 + j + kAhead) * BN) * rsV;
      if (wave >= kIssuers) return;
#pragma unroll
      for (int i = 0; i < kMine; ++i) {
        // every tile of a pass lies inside the buffers, so the tile's
        // offset goes in the scalar offset field; at d = 192 the 4 padding
        // slots of a 256-byte K row must read past the buffer (zeros), so
        // those rows keep the whole offset in the bounds-checked part
        if (i * kIssuers < kKL) {
          if constexpr (LY::kKC * 16 == DQK) {
            buffer_load_lds16_so(rk, &sm.k[buf][lo_[i]], go[i], kb);
          } else {
            const uint32_t g = go[i] == 0xfffffff0u ? go[i] : kb + go[i];
            buffer_load_lds16(rk, &sm.k[buf][lo_[i]], g);
          }
        } else {
          buffer_load_lds16_so(rv, &sm.v[buf][lo_[i]], go[i], vb);
        }
      }
    };
    auto qk_c = [&](auto ST, f32x16* sout) {  // S^T of the tile in stage ST
      constexpr int st = decltype(ST)::value;
      sout[0] = f32x16{};
      sout[1] = f32x16{};
#pragma unroll
      for (int s2 = 0; s2 < kSteps; ++s2)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const uint32_t off = st * LY::kKBytes + kb * 32 * LY::kKPitch;
          typedef const __attribute__((address_space(3))) i32x4* lds_i32x4;
          const i32x4 lo = *(lds_i32x4)(uintptr_t)(kx[s2 * 2 + 0] + off);
          const i32x4 hi = *(lds_i32x4)(uintptr_t)(kx[s2 * 2 + 1] + off);
          sout[kb] = mfma_f8_plain(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), qreg[s2], sout[kb]);
        }
    };
    auto pv_c = [&](auto ST, const i32x8& pw, int pscale) {
      constexpr int st = decltype(ST)::value;
      constexpr int so = st * LY::kVBytes;
      i32x2 r[2][4];
      auto vread = [&](int d, i32x2* x) {
        x[0] = ds_read_tr8<so + 0 * 16 * kDV>(vx[d]);
        x[1] = ds_read_tr8<so + 1 * 16 * kDV>(vx[d]);
        x[2] = ds_read_tr8<so + 2 * 16 * kDV>(vx[d]);
        x[3] = ds_read_tr8<so + 3 * 16 * kDV>(vx[d]);
      };
      vread(0, r[0]);
      vread(1, r[1]);
#pragma unroll
      for (int d = 0; d < kDV / 32; ++d) {
        i32x2* x = r[d & 1];
        if (d + 1 < kDV / 32) lds_wait4<4>(x[0], x[1], x[2], x[3]);
        else lds_wait4<0>(x[0], x[1], x[2], x[3]);
        const i32x8 a = __builtin_shufflevector(
            __builtin_shufflevector(x[0], x[1], 0, 1, 2, 3),
            __builtin_shufflevector(x[2], x[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[d] = mfma_f8(a, pw, oacc[d], kE8M0One, pscale);
        if (d + 2 < kDV / 32) vread(d + 2, x);
      }
      const f32x4 lt = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(lsel, pw, f32x4{}, 0, 0, 0, 0, 0, 0);
      l_run = __builtin_fmaf(lt[0], __uint_as_float((unsigned)pscale << 23), l_run);
    };
    auto step_c = [&](auto J, int t0, f32x16* scur, f32x16* snext, float bcur, float& bnext) {
      constexpr int j = decltype(J)::value;
      issue_c(J, t0);
      __builtin_amdgcn_s_setprio(1);
      refresh(bcur);
      int pscale;
      const i32x8 pw = probs(scur, bcur, pscale);
      qk_c(std::integral_constant<int, (j + 1) % kS>{}, snext);
      __builtin_amdgcn_s_setprio(0);
      pv_c(std::integral_constant<int, j>{}, pw, pscale);
      bnext = tile_max(snext);
#pragma unroll
      for (int d = 0; d < kDV / 32; ++d) pin(oacc[d]);
      pin(l_run);
      pin(bnext);
      if constexpr (!LY::kPair || (j & 1)) {
        wait_vmcnt<kMine>();
        barrier_nofence();
      }
    };
    for (; t + kS - 1 < t_fe && t + kS - 1 + kAhead < nkt; t += kS) {
      step_c(std::integral_constant<int, 0>{}, t, sa, sb, bmax_a, bmax_b);
      step_c(std::integral_constant<int, 1>{}, t, sb, sa, bmax_b, bmax_a);
      step_c(std::integral_constant<int, 2>{}, t, sa, sb, bmax_a, bmax_b);
      step_c(std::integral_constant<int, 3>{}, t, sb, sa, bmax_b, bmax_a);
      if constexpr (kS == 8) {
        step_c(std::integral_constant<int, 4>{}, t, sa, sb, bmax_a, bmax_b);
        step_c(std::integral_constant<int, 5>{}, t, sb, sa, bmax_b, bmax_a);
        step_c(std::integral_constant<int, 6>{}, t, sa, sb, bmax_a, bmax_b);
        step_c(std::integral_constant<int, 7>{}, t, sb, sa, bmax_b, bmax_a);
      }
    }
  }
  for (; t + 1 < t_fe; t += 2) {
    fast_step(t, sa, sb, bmax_a, bmax_b);
    fast_step(t + 1, sb, sa, bmax_b, bmax_a);
  }
  if (t < t_fe) {
    fast_step(t, sa, sb, bmax_a, bmax_b);
    sa[0] = sb[0];
    sa[1] = sb[1];
    bmax_a = bmax_b;
    ++t;
  }
  for (; t < nkt; t += 2) {
    slow_step(t, sa, sb, bmax_a, bmax_b);
    if (t + 1 < nkt) slow_step(t + 1, sb, sa, bmax_b, bmax_a);
  }

  // ---- epilogue
  if (rot_o) hadamard_o_rows(oacc, half);
  const float l_tot = l_run;
  const int qi = q0w + col;
  // 1/sqrt(128) normalises the rotation
  const float inv = v_descale / l_tot * (rot_o ? 0.08838834764831845f : 1.0f);
  store_rows_bf16<kDV>(oacc, inv, sm.epi[wave], o, sr.row0 + q0w, (int64_t)H * kDV,
                       (int64_t)h * kDV, S - q0w, lane);
  if (qi < S && lse != nullptr && half == 0)
    lse[sr.lse0 + h * sr.lse_hs + qi] = (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
}

}  // namespace

int launch_attn_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int32_t* cu, int64_t total, int B, int S, int H, int d_qk,
                    float softmax_scale, int causal, float q_descale, float k_descale,
                    float v_descale, bool rot_o, bool exact_p, int32_t* tail_ctr,
                    hipStream_t stream) {
  const int occ = 2;                      // waves per SIMD (register budget)
  const int bm = 128 * occ;               // query rows per workgroup
  const int nqb = (S + bm - 1) / bm;
  const int BH = B * H;
  const BlockGrid bg = block_grid(nqb, BH, cu == nullptr, tail_ctr != nullptr);
  if (bg.q_cut && launch_clear_i32(tail_ctr, stream) != 0) return -1;
  const dim3 grid((unsigned)bg.grid);
  const float c_log2 = softmax_scale * q_descale * k_descale * 1.4426950408889634f;
  // the lean code's scale 8 c in units of the 16-bit normalised conversion,
  // passed in so that its 32 FMAs per tile read it from a scalar register
  // (the scalar unit has no float multiply to form it in the kernel)
  const float c8n = 8.0f * c_log2 * (256.0f / 65535.0f);
  const bool lean = !exact_p;  // probabilities: lean (default) or exact exp2 + convert
#define CPATTN_LAUNCH_FP8(DQK, BN, LEAN, OCC)                                                     \
  hipLaunchKernelGGL((attn_fwd_fp8_kernel<DQK, BN, LEAN, OCC>), grid, dim3(256 * OCC), 0, stream, \
                     (const uint8_t*)q, (const uint8_t*)k, (const uint8_t*)v, (__bf16*)o, lse, cu, \
                     total, S, H, BH, nqb, c_log2, c8n, v_descale, causal, (int)rot_o,       \
                     bg.n_static, bg.q_cut, (int*)tail_ctr)
  if (d_qk == 128) {
    if (lean) CPATTN_LAUNCH_FP8(128, 64, true, 2);
    else CPATTN_LAUNCH_FP8(128, 64, false, 2);
  } else {
    if (lean) CPATTN_LAUNCH_FP8(192, 64, true, 2);
    else CPATTN_LAUNCH_FP8(192, 64, false, 2);
  }
#undef CPATTN_LAUNCH_FP8
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace cpattn
