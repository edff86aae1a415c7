// Decode step against a paged KV cache (gfx950): one new query token per
// sequence attends to every cached key of its sequence.  Decode and paged KV
// caches are the kernels' stated future work ("Ce que couvrent les noyaux",
// ai-daily-news.org page); the step is the last row of causal attention,
// o = softmax(tau q.K^T) V over keys 0 .. L-1.
//
// Paged cache: K [pages, page_size, H_kv, d_qk], V [pages, page_size, H_kv,
// 128]; key j of sequence b is slot j % page_size of page
// table[b][j / page_size].  Query head h reads key/value head h / G,
// G = H_q / H_kv.
//
// One query row per head makes this a matrix-vector product: 2 FLOPs per
// cached element (2G with G grouped query heads per key/value head), far
// below the matrix cores' ridge, so the kernel is bound by HBM: what matters
// is streaming the cache with wide, coalesced loads and enough workgroups in
// flight.  The scores of the G heads still go to the matrix cores: on the
// vector ALU, their dot products, lane sums and a softmax repeated in every
// lane of a key row cost more time than the memory at G = 4.
//
// Split over keys.  Workgroup (split s, key/value head hk, sequence b) takes
// keys [s*split, min((s+1)*split, L)) for the G query heads of hk, and leaves
// per head a partial output normalised by its own sum plus the partial's
// log-sum-exp.  decode_merge_kernel combines the partials of each head in
// split order, so results do not depend on timing.
//
// Inside a workgroup: 4 waves; a wave takes tiles of 16 consecutive keys
// (tiles w, w+4, ...), which lie in one page since pages hold a multiple of
// 16 keys and splits start at multiples of 64.  The scores of a tile for the
// G query heads of the key/value head are one 16x16 matrix-core product
// (keys x heads, heads past G are zero columns).  In its accumulator, lane
// group j (16 lanes) holds keys 4j .. 4j+3 of the tile and lane j*16 + g
// holds head g, so each (lane group, head) pair runs its own online softmax
// over its keys on the lane's four values.  The probabilities then go through
// a wave-private LDS slot to the P.V layout, where lane group j holds the same
// four keys' value rows and each lane 8 of the 128 output columns for every
// head; P.V stays in fp32 on the vector ALU.  The 16 streams of a workgroup
// are merged at the end.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "attn_device.h"
#include "attn_kernels.h"

namespace cpattn {
namespace {

constexpr int kWaves = 4;
constexpr int kDV = 128;
constexpr int kTile = 16;  // keys per wave tile: 4 lane groups x 4 steps
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNoKeys = -1e30f;  // running max of a stream that has seen no key

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// One lane's share of a row of `d` elements: elements 8*sub .. 8*sub+7 of the
// first 128, and for d = 192 elements 128 + 4*sub .. +3 as well, as raw words
// (bf16 pairs, or four e4m3 codes).
template <int DQK, bool kFP8>
struct RowPart {
  static constexpr int kA = kFP8 ? 2 : 4;              // words of the first 128 elements
  static constexpr int kB = DQK == 192 ? kA / 2 : 0;   // words of the last 64
  uint32_t a[kA];
  uint32_t b[kB > 0 ? kB : 1];
};

template <int DQK, bool kFP8>
__device__ __forceinline__ RowPart<DQK, kFP8> load_row(const uint8_t* row, int sub) {
  constexpr int esz = kFP8 ? 1 : 2;
  RowPart<DQK, kFP8> r;
  if constexpr (kFP8) {
    const u32x2 x = *reinterpret_cast<const u32x2*>(row + sub * 8);
    r.a[0] = x[0];
    r.a[1] = x[1];
    if constexpr (DQK == 192) r.b[0] = *reinterpret_cast<const uint32_t*>(row + 128 + sub * 4);
  } else {
    const u32x4 x = *reinterpret_cast<const u32x4*>(row + sub * 16);
    r.a[0] = x[0];
    r.a[1] = x[1];
    r.a[2] = x[2];
    r.a[3] = x[3];
    if constexpr (DQK == 192) {
      const u32x2 y = *reinterpret_cast<const u32x2*>(row + 128 * esz + sub * 8);
      r.b[0] = y[0];
      r.b[1] = y[1];
    }
  }
  return r;
}

// Words -> fp32 values, in element order.
__device__ __forceinline__ void bf16_words(const uint32_t* w, int n, float* out) {
  for (int i = 0; i < n; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void e4m3_words(const uint32_t* w, int n, float* out) {
  for (int i = 0; i < n; ++i) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
    out[4 * i] = lo[0];
    out[4 * i + 1] = lo[1];
    out[4 * i + 2] = hi[0];
    out[4 * i + 3] = hi[1];
  }
}

// A lane's quarter of a query or key row as a matrix-core operand: lane
// group j (lanes 16j .. 16j+15) holds bytes [j, j+1) * DQK*esz/4 of the row.
// The query (B operand) and the keys (A operand) use the same split, so every
// element of the row meets its partner in one product.
template <int DQK, bool kFP8>
struct Quarter {
  static constexpr int kWords = DQK * (kFP8 ? 1 : 2) / 16;  // 8 / 12 (e4m3), 16 / 24 (bf16)
  uint32_t w[kWords];
};

template <int DQK, bool kFP8>
__device__ __forceinline__ Quarter<DQK, kFP8> load_quarter(const uint8_t* row, int part) {
  using QT = Quarter<DQK, kFP8>;
  QT r;
  const u32x4* src = reinterpret_cast<const u32x4*>(row + part * QT::kWords * 4);
#pragma unroll
  for (int i = 0; i < QT::kWords / 4; ++i) {
    const u32x4 x = src[i];
#pragma unroll
    for (int c = 0; c < 4; ++c) r.w[4 * i + c] = x[c];
  }
  return r;
}

// S^T (16 keys x 16 heads) of one tile: the fp32 sum of the products of a
// lane's quarter of its key row with the same quarter of its head's query,
// over the four quarters.  Accumulator: lane l holds head l % 16 and keys
// 4 (l / 16) + i, i = 0..3.  e4m3 uses the 16x16x128 form (a d = 192 row
// leaves a 16-code remainder, padded with zero codes on both sides); bf16
// the 16x16x32 form.
template <int DQK, bool kFP8>
__device__ __forceinline__ f32x4 tile_scores(const Quarter<DQK, kFP8>& k,
                                             const Quarter<DQK, kFP8>& q) {
  using QT = Quarter<DQK, kFP8>;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (kFP8) {
#pragma unroll
    for (int c = 0; c < QT::kWords / 8; ++c) {
      i32x8 a, bq;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        a[i] = (int)k.w[8 * c + i];
        bq[i] = (int)q.w[8 * c + i];
      }
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bq, acc, 0, 0, 0, 0, 0, 0);
    }
    if constexpr (QT::kWords % 8 != 0) {
      constexpr int c0 = QT::kWords / 8 * 8;
      i32x8 a = {0, 0, 0, 0, 0, 0, 0, 0}, bq = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = (int)k.w[c0 + i];
        bq[i] = (int)q.w[c0 + i];
      }
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bq, acc, 0, 0, 0, 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int c = 0; c < QT::kWords / 4; ++c) {
      u32x4 a = {k.w[4 * c], k.w[4 * c + 1], k.w[4 * c + 2], k.w[4 * c + 3]};
      u32x4 bq = {q.w[4 * c], q.w[4 * c + 1], q.w[4 * c + 2], q.w[4 * c + 3]};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, bq), acc, 0, 0, 0);
    }
  }
  return acc;
}

template <int DQK, bool kFP8>
__device__ __forceinline__ void row_values(const RowPart<DQK, kFP8>& r, float* out) {
  using R = RowPart<DQK, kFP8>;
  if constexpr (kFP8) {
    e4m3_words(r.a, R::kA, out);
    if constexpr (R::kB > 0) e4m3_words(r.b, R::kB, out + 4 * R::kA);
  } else {
    bf16_words(r.a, R::kA, out);
    if constexpr (R::kB > 0) bf16_words(r.b, R::kB, out + 2 * R::kA);
  }
}

// Tiles each wave keeps in flight beyond the one it works on: chosen so that
// the ring of tile buffers (16 registers per e4m3 tile, 32 per bf16 tile)
// leaves the kernel's occupancy where it was with one tile ahead.
template <bool kFP8, int G>
constexpr int prefetch_tiles() {
  if (kFP8) return G <= 4 ? 3 : 1;
  return G <= 2 ? 2 : 1;
}

template <int DQK, int G, bool kFP8>
__global__ void __launch_bounds__(64 * kWaves)
decode_split_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ kc,
                    const uint8_t* __restrict__ vc, const int32_t* __restrict__ table,
                    const int32_t* __restrict__ lens, float* __restrict__ opart,
                    float* __restrict__ lpart, int Hkv, int maxp, int npages, int ps_log2,
                    int lcap, int split, int nsplit, float c_log2, float v_descale) {
  constexpr int esz = kFP8 ? 1 : 2;
  const int sp = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  int L = lens[b];
  L = L < 0 ? 0 : (L > lcap ? lcap : L);
  const int k0 = sp * split;
  if (k0 >= L) return;  // whole workgroup: this split is past the sequence's end
  const int k1 = min(L, k0 + split);
  const int ntile = (k1 - k0 + kTile - 1) / kTile;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = lane >> 4, sub = lane & 15;
  const int Hq = Hkv * G;
  const int ps = 1 << ps_log2;

  // B operand: column sub is query head hk*G + sub, a zero column for sub >= G
  using QT = Quarter<DQK, kFP8>;
  QT qq = load_quarter<DQK, kFP8>(q + ((int64_t)b * Hq + hk * G + (sub < G ? sub : 0)) * DQK * esz,
                                  grp);
  if (sub >= G) {
#pragma unroll
    for (int i = 0; i < QT::kWords; ++i) qq.w[i] = 0u;
  }

  const int64_t rsK = (int64_t)Hkv * DQK * esz;  // bytes between slots
  const int64_t rsV = (int64_t)Hkv * kDV * esz;
  const uint8_t* kbase = kc + (int64_t)hk * DQK * esz;
  const uint8_t* vbase = vc + (int64_t)hk * kDV * esz;
  const int32_t* trow = table + (int64_t)b * maxp;

  struct Tile {
    QT k;                      // key row sub of the tile, quarter grp
    RowPart<128, kFP8> v[4];   // value rows 4*grp + r, columns 8*sub .. 8*sub+7
  };
  // keys at or past k1 read the tile's first row (a valid key) and are
  // masked below
  auto load_tile = [&](int t) {
    Tile x;
    const int key0 = k0 + t * kTile;
    int page = trow[key0 >> ps_log2];
    page = page < 0 ? 0 : (page >= npages ? npages - 1 : page);
    const int64_t slot0 = (int64_t)page * ps + (key0 & (ps - 1));
    x.k = load_quarter<DQK, kFP8>(kbase + (slot0 + (key0 + sub < k1 ? sub : 0)) * rsK, grp);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int dk = 4 * grp + r;
      x.v[r] = load_row<128, kFP8>(vbase + (slot0 + (key0 + dk < k1 ? dk : 0)) * rsV, sub);
    }
    return x;
  };

  // softmax stream of (lane group grp, head sub): keys 4*grp .. 4*grp+3 of
  // every tile, in log2 units (meaningful for sub < G)
  float m_s = kNoKeys, l_s = 0.0f;
  float o[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[g][e] = 0.0f;

  // wave-private exchange slots: lane l's four probabilities and its rescale
  // factor.  Only this wave touches them, and a wave's LDS accesses complete
  // in order, so no workgroup barrier is needed.
  __shared__ f32x4 sP[kWaves][64];
  __shared__ float sA[kWaves][64];

  // one tile: scores, online softmax update, P.V
  auto process = [&](const Tile& x, int t) {
    const int key0 = k0 + t * kTile;
    const f32x4 acc = tile_scores<DQK, kFP8>(x.k, qq);
    f32x4 p;
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = key0 + 4 * grp + i < k1 ? acc[i] * c_log2 : -INFINITY;
    const float mx = fmaxf(fmaxf(p[0], p[1]), fmaxf(p[2], p[3]));
    const float mn = fmaxf(m_s, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_s - mn);
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(p[i] - mn);
    l_s = fmaf(l_s, alpha, (p[0] + p[1]) + (p[2] + p[3]));
    m_s = mn;
    sP[wave][lane] = p;
    sA[wave][lane] = alpha;
    __builtin_amdgcn_wave_barrier();
    f32x4 pg[G];
    float al[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      pg[g] = sP[wave][16 * grp + g];
      al[g] = sA[wave][16 * grp + g];
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[g][e] *= al[g];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float vv[8];
      row_values<128, kFP8>(x.v[r], vv);
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[g][e] = fmaf(pg[g][r], vv[e], o[g][e]);
    }
  };

  // Ring of kAhead + 1 tile buffers in registers, indexed at compile time
  // (the loop is unrolled by the ring size): while tile t is processed,
  // tiles t+4 .. t+4*kAhead are in flight.  The body has no condition, so the
  // compiler's count of outstanding loads stays exact: the wave's tile count
  // is rounded up to whole rings, loads past the last tile reload it (a cache
  // hit) and tiles past the last one are processed fully masked, which
  // leaves m, l and o unchanged (alpha = 1, p = 0).
  constexpr int kAhead = prefetch_tiles<kFP8, G>();
  constexpr int kRing = kAhead + 1;
  const int nmine = wave < ntile ? (ntile - wave + kWaves - 1) / kWaves : 0;
  Tile ring[kRing];
#pragma unroll
  for (int i = 0; i < kAhead; ++i) ring[i] = load_tile(min(wave + kWaves * i, ntile - 1));
  for (int it = 0; it < nmine; it += kRing) {
#pragma unroll
    for (int j = 0; j < kRing; ++j) {
      const int t = wave + kWaves * (it + j);
      ring[(j + kAhead) % kRing] = load_tile(min(t + kWaves * kAhead, ntile - 1));
      process(ring[j], t);
      // keep each step's loads in its own step: hoisting later loads only
      // lengthens register live ranges
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // each lane of group grp takes the stream state of its group's G heads
  float m[G], l[G];
  __builtin_amdgcn_wave_barrier();
  sP[wave][lane] = f32x4{m_s, l_s, 0.0f, 0.0f};
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const f32x4 st = sP[wave][16 * grp + g];
    m[g] = st[0];
    l[g] = st[1];
  }

  // merge the four lane groups of the wave (lanes sub, sub+16, sub+32, sub+48
  // hold the same output columns)
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float M = fmaxf(m[g], __shfl_xor(m[g], 16));
    M = fmaxf(M, __shfl_xor(M, 32));
    const float w = __builtin_amdgcn_exp2f(m[g] - M);
    float lw = l[g] * w;
    lw += __shfl_xor(lw, 16);
    lw += __shfl_xor(lw, 32);
    l[g] = lw;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = o[g][e] * w;
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      o[g][e] = x;
    }
    m[g] = M;
  }

  // merge the waves through LDS, in wave order
  __shared__ float sO[kWaves][G][kDV];
  __shared__ float sM[kWaves][G], sL[kWaves][G];
  if (grp == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sO[wave][g][sub * 8 + e] = o[g][e];
      if (sub == 0) {
        sM[wave][g] = m[g];
        sL[wave][g] = l[g];
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < G * kDV; i += 64 * kWaves) {
    const int g = i / kDV, d = i % kDV;
    float M = sM[0][g];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sM[w][g]);
    float lt = 0.0f, ot = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = __builtin_amdgcn_exp2f(sM[w][g] - M);
      lt = fmaf(sL[w][g], f, lt);
      ot = fmaf(sO[w][g][d], f, ot);
    }
    // key k0 is valid, so lt > 0
    const int64_t ph = ((int64_t)b * Hq + hk * G + g) * nsplit + sp;
    opart[ph * kDV + d] = ot / lt * v_descale;
    if (d == 0) lpart[ph] = (M + __builtin_amdgcn_logf(lt)) / kLog2e;
  }
}

// o[b, h] = sum_s e^{lse_s} o_s / sum_s e^{lse_s} over the splits that hold
// keys of sequence b, in split order; lse = log sum_s e^{lse_s}.  An empty
// sequence gives o = 0 and lse = -inf.
__global__ void __launch_bounds__(kDV)
decode_merge_kernel(const float* __restrict__ opart, const float* __restrict__ lpart,
                    const int32_t* __restrict__ lens, __bf16* __restrict__ o,
                    float* __restrict__ lse, int Hq, int lcap, int split, int nsplit) {
  const int bh = blockIdx.x;
  const int b = bh / Hq;
  const int d = threadIdx.x;
  int L = lens[b];
  L = L < 0 ? 0 : (L > lcap ? lcap : L);
  const int ns = (L + split - 1) / split;
  const float* lp = lpart + (int64_t)bh * nsplit;
  const float* op = opart + (int64_t)bh * nsplit * kDV;
  if (ns == 0) {
    o[(int64_t)bh * kDV + d] = (__bf16)0.0f;
    if (lse != nullptr && d == 0) lse[bh] = -INFINITY;
    return;
  }
  // unrolled so that the loads of several splits are in flight together;
  // the sums still run in split order
  float M = lp[0];
#pragma unroll 8
  for (int s = 1; s < ns; ++s) M = fmaxf(M, lp[s]);
  float wsum = 0.0f, acc = 0.0f;
#pragma unroll 8
  for (int s = 0; s < ns; ++s) {
    const float w = expf(lp[s] - M);
    wsum += w;
    acc = fmaf(w, op[(int64_t)s * kDV + d], acc);
  }
  o[(int64_t)bh * kDV + d] = (__bf16)(acc / wsum);
  if (lse != nullptr && d == 0) lse[bh] = M + logf(wsum);
}

template <int DQK, int G, bool kFP8>
void launch_split(const DecodeArgs& a, float* opart, float* lpart, float c_log2,
                  hipStream_t stream) {
  int ps_log2 = 0;
  while ((int64_t(1) << ps_log2) < a.page_size) ++ps_log2;
  hipLaunchKernelGGL((decode_split_kernel<DQK, G, kFP8>),
                     dim3(a.nsplit, (unsigned)a.Hkv, (unsigned)a.B), dim3(64 * kWaves), 0, stream,
                     (const uint8_t*)a.q, (const uint8_t*)a.k_cache, (const uint8_t*)a.v_cache,
                     a.block_table, a.seq_lens, opart, lpart, (int)a.Hkv,
                     (int)a.max_pages_per_seq, (int)a.num_pages, ps_log2, (int)a.max_seqlen,
                     a.split, a.nsplit, c_log2, a.dtype_fp8 ? a.v_descale : 1.0f);
}

template <int DQK, bool kFP8>
void launch_split_g(const DecodeArgs& a, int G, float* opart, float* lpart, float c_log2,
                    hipStream_t stream) {
  switch (G) {
    case 1: launch_split<DQK, 1, kFP8>(a, opart, lpart, c_log2, stream); break;
    case 2: launch_split<DQK, 2, kFP8>(a, opart, lpart, c_log2, stream); break;
    case 4: launch_split<DQK, 4, kFP8>(a, opart, lpart, c_log2, stream); break;
    default: launch_split<DQK, 8, kFP8>(a, opart, lpart, c_log2, stream); break;
  }
}

}  // namespace

void decode_split_policy(int64_t B, int64_t Hkv, int64_t max_seqlen, int* split, int* nsplit) {
  // about 4096 workgroups (16 per CU) if every sequence had max_seqlen keys;
  // splits of 256 .. 1024 keys, a multiple of 64.  The cap keeps shorter
  // sequences of a ragged batch spread over several workgroups (workgroups
  // past a sequence's end return at once).
  const int64_t per = B * Hkv;
  const int64_t want = (4096 + per - 1) / per;
  int64_t sp = (max_seqlen + want - 1) / want;
  sp = (sp + 63) / 64 * 64;
  if (sp < 256) sp = 256;
  if (sp > 1024) sp = 1024;
  *split = (int)sp;
  *nsplit = (int)((max_seqlen + sp - 1) / sp);
}

int64_t decode_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t max_seqlen) {
  int split, nsplit;
  decode_split_policy(B, Hkv, max_seqlen, &split, &nsplit);
  return B * Hq * nsplit * (kDV + 1) * 4;
}

int launch_decode(const DecodeArgs& a, hipStream_t stream) {
  float* opart = reinterpret_cast<float*>(a.workspace);
  float* lpart = opart + a.B * a.Hq * a.nsplit * kDV;
  const float c_log2 = a.softmax_scale * kLog2e * (a.dtype_fp8 ? a.q_descale * a.k_descale : 1.0f);
  const int G = (int)(a.Hq / a.Hkv);
  if (a.dtype_fp8) {
    if (a.d_qk == 128) launch_split_g<128, true>(a, G, opart, lpart, c_log2, stream);
    else launch_split_g<192, true>(a, G, opart, lpart, c_log2, stream);
  } else {
    if (a.d_qk == 128) launch_split_g<128, false>(a, G, opart, lpart, c_log2, stream);
    else launch_split_g<192, false>(a, G, opart, lpart, c_log2, stream);
  }
  if (hipGetLastError() != hipSuccess) return -1;
  hipLaunchKernelGGL(decode_merge_kernel, dim3((unsigned)(a.B * a.Hq)), dim3(kDV), 0, stream,
                     opart, lpart, a.seq_lens, (__bf16*)a.o, a.lse, (int)a.Hq,
                     (int)a.max_seqlen, a.split, a.nsplit);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Scratch held by the library for callers that cannot allocate device memory
// (attn_decode_paged_noalloc): the split partials of one decode step, up to
// kScratchBytes.  Each GPU the library runs on holds its own copy until the
// process ends.  In host code `scratch` is a stand-in, not a device address:
// only the address hipGetSymbolAddress returns for a device may reach a
// kernel.  Every call on a GPU shares that GPU's copy, so calls that overlap
// in time on one GPU race; the merge reads only partials the same step's
// split kernel wrote, so nothing needs clearing between calls.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // per device, filled on the first call there
}  // namespace

void* decode_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace cpattn
