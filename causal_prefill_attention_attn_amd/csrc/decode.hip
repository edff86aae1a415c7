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
// 16 keys and splits start at multiples of 64.  Tiles reach the wave through
// a ring of LDS slots filled by buffer-to-LDS loads (decode_split_kernel
// below says why).  The scores of a tile for the
// G query heads of the key/value head are one 16x16 matrix-core product
// (keys x heads, heads past G are zero columns).  In its accumulator, lane
// group j (16 lanes) holds keys 4j .. 4j+3 of the tile and lane j*16 + g
// holds head g, so each (lane group, head) pair runs its own online softmax
// over its keys on the lane's four values.  The probabilities then reach the
// P.V layout by DPP row broadcasts (lane g of each 16-lane row to the whole
// row), where lane group j holds the same four keys' value rows and each lane
// 8 of the 128 output columns for every head; P.V stays in fp32 on the
// vector ALU.  The 16 streams of a workgroup are merged at the end.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>
#include <utility>

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

// How the cache reaches the arithmetic.  Each wave streams its 16-key tiles
// into a private ring of slots in LDS with buffer-to-LDS loads (16 bytes per
// lane, 1 KB per instruction), waits for the oldest with an explicit vmcnt
// count and reads it back with LDS reads where it is used.  No loaded data is
// held in registers across the loop: with a ring of tiles in registers the
// compiler's wait count at the loop head falls back to waiting for every
// load in flight, once per ring, and the prefetch drains.  Here every wait is
// exact, and no registers are spent on tiles in flight.
template <int DQK, bool kFP8>
struct LdsTile {
  static constexpr int kEsz = kFP8 ? 1 : 2;
  static constexpr int kRowK = DQK * kEsz;  // bytes of a key row of one head
  static constexpr int kPitchK = (kRowK + 127) / 128 * 128;  // whole 128-byte swizzle groups
  static constexpr int kRowV = kDV * kEsz;
  static constexpr int kKBytes = kTile * kPitchK;
  static constexpr int kVBytes = kTile * kRowV;
  static constexpr int kBytes = kKBytes + kVBytes;
  static constexpr int kLoadsK = kKBytes / 1024;  // 1 KB loads per tile
  static constexpr int kLoadsV = kVBytes / 1024;
  static constexpr int kLoads = kLoadsK + kLoadsV;
  // slots: at most 72 KB of ring per workgroup, so that two workgroups fit
  // in a CU's LDS; between 2 and 4
  static constexpr int kFit = 73728 / (kWaves * kBytes);
  static constexpr int kDeep = kFit < 2 ? 2 : (kFit > 4 ? 4 : kFit);
};
// With grouped query heads (G > 1) a tile costs a wave several times the
// vector work of G = 1, and more resident workgroups (two slots: four per
// CU) hide it better than a deeper ring; with one head per key/value head
// the deeper ring streams best.
template <int DQK, int G, bool kFP8>
constexpr int decode_ring() {
  return G > 1 ? 2 : LdsTile<DQK, kFP8>::kDeep;
}

// 16-byte chunk c of key row `row` sits at chunk kswz(c, row) of its LDS
// row: the low three bits are XORed with the row, so the 16 rows that one
// quarter read touches spread over the banks.  The map is its own inverse.
__device__ __forceinline__ int kswz(int c, int row) { return (c & ~7) | ((c ^ row) & 7); }

template <int N>
__device__ __forceinline__ void decode_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

// value row part from LDS, as inline assembly so that the wait-count pass
// does not make it wait for the buffer-to-LDS loads in flight; the result is
// ordered with decode_lds_wait before use
template <bool kFP8>
struct VRead {
  typedef typename std::conditional<kFP8, i32x2, i32x4>::type T;
};
template <bool kFP8, int OFF>
__device__ __forceinline__ typename VRead<kFP8>::T v_read(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  typename VRead<kFP8>::T r;
  if constexpr (kFP8)
    asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
  else
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
  return r;
}
__device__ __forceinline__ u32x4 k_read(uint32_t addr) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(addr) : "memory");
  return r;
}
// s_waitcnt lgkmcnt(0) tied to the value reads, then to every key chunk:
// nothing that reads these registers can be placed above the wait
template <typename T, int N>
__device__ __forceinline__ void decode_lds_wait(T& a, T& b, T& c, T& d, u32x4 (&k)[N]) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(k[i]));
}

// x of lane g of the lane's 16-lane row (DPP row broadcast, no LDS)
template <int g>
__device__ __forceinline__ float row_bcast(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                               0x150 + g, 0xF, 0xF, false));
}
template <int... gs>
__device__ __forceinline__ void row_bcast_all(std::integer_sequence<int, gs...>, const f32x4& p,
                                              float a, f32x4* pg, float* al) {
  ((pg[gs] = f32x4{row_bcast<gs>(p[0]), row_bcast<gs>(p[1]), row_bcast<gs>(p[2]),
                   row_bcast<gs>(p[3])},
    al[gs] = row_bcast<gs>(a)),
   ...);
}

template <int DQK, int G, bool kFP8>
__global__ void __launch_bounds__(64 * kWaves)
decode_split_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ kc,
                        const uint8_t* __restrict__ vc, const int32_t* __restrict__ table,
                        const int32_t* __restrict__ lens, float* __restrict__ opart,
                        float* __restrict__ lpart, int Hkv, int maxp, int npages, int ps_log2,
                        int lcap, int split, int nsplit, float c_log2, float v_descale) {
  using LT = LdsTile<DQK, kFP8>;
  using QT = Quarter<DQK, kFP8>;
  constexpr int esz = LT::kEsz;
  constexpr int kRing = decode_ring<DQK, G, kFP8>();
  constexpr int kQC = QT::kWords / 4;  // 16-byte chunks in a quarter row
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kWaves][kRing][LT::kBytes];
  static_assert(sizeof(float) * kWaves * G * (kDV + 2) <= sizeof(ring),
                "merge buffers overlay the ring");

  const int sp = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = lane >> 4, sub = lane & 15;
  const int Hq = Hkv * G;
  const int ps = 1 << ps_log2;
  const int k0 = sp * split;

  // The sequence length, this split's pages and the query are loaded
  // together: neither the pages nor the query depend on the length, so the
  // first tile loads wait one memory round trip, not two.  Pages: one per
  // lane (a split of at most 1024 keys spans at most 64 pages of at least 16
  // keys); tile t takes its page by readlane.
  const int p0 = k0 >> ps_log2;
  const int npmax = ((k0 + split - 1) >> ps_log2) - p0 + 1;
  const int32_t* trow = table + (int64_t)b * maxp;
  int pg = 0;
  if (lane < npmax && p0 + lane < maxp) pg = trow[p0 + lane];
  // B operand: column sub is query head hk*G + sub, a zero column for sub >= G
  QT qq = load_quarter<DQK, kFP8>(q + ((int64_t)b * Hq + hk * G + (sub < G ? sub : 0)) * DQK * esz,
                                  grp);
  int L = lens[b];
  L = L < 0 ? 0 : (L > lcap ? lcap : L);
  if (k0 >= L) return;  // whole workgroup: this split is past the sequence's end
  const int k1 = min(L, k0 + split);
  const int ntile = (k1 - k0 + kTile - 1) / kTile;
  pg = pg < 0 ? 0 : (pg >= npages ? npages - 1 : pg);

  const int64_t rsK = (int64_t)Hkv * DQK * esz;  // bytes between slots
  const int64_t rsV = (int64_t)Hkv * kDV * esz;
  const uint8_t* kbase = kc + (int64_t)hk * DQK * esz;
  const uint8_t* vbase = vc + (int64_t)hk * kDV * esz;

  // Tile t of the split (keys k0 + 16t ..) into ring slot `slot`.  Lane l's
  // 16 bytes of load j land at byte 1024 j + 16 l of the slot: K rows of
  // kPitchK bytes (chunks swizzled; padding chunks of d = 192 rows read past
  // the buffer, i.e. zeros), then V rows.  Keys at or past k1 read the
  // tile's first row (a valid key); they are masked in the scores.  A tile
  // of 16 keys lies in one page (pages hold a power of two >= 16 keys, tiles
  // start at multiples of 16); its buffer resource starts at the tile's
  // first slot, so offsets stay small for any cache size.
  auto issue = [&](int t, int slot) {
    const int key0 = k0 + t * kTile;
    const int page = __builtin_amdgcn_readlane(pg, (key0 >> ps_log2) - p0);
    const int64_t slot0 = (int64_t)page * ps + (key0 & (ps - 1));
    const int nvalid = k1 - key0;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + slot0 * rsK, (uint32_t)(kTile * rsK));
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + slot0 * rsV, (uint32_t)(kTile * rsV));
    uint8_t* dst = ring[wave][slot];
#pragma unroll
    for (int j = 0; j < LT::kLoadsK; ++j) {
      const int pos = j * 1024 + 16 * lane;
      const int row = pos / LT::kPitchK;
      const int c = kswz((pos % LT::kPitchK) / 16, row);
      const uint32_t off = c * 16 >= LT::kRowK
                               ? 0xFFFFFFF0u
                               : (uint32_t)((row < nvalid ? row : 0) * rsK + c * 16);
      buffer_load_lds16(rk, dst + j * 1024, off);
    }
#pragma unroll
    for (int j = 0; j < LT::kLoadsV; ++j) {
      const int pos = j * 1024 + 16 * lane;
      const int row = pos / LT::kRowV;
      const uint32_t off = (uint32_t)((row < nvalid ? row : 0) * rsV + pos % LT::kRowV);
      buffer_load_lds16(rv, dst + LT::kKBytes + j * 1024, off);
    }
  };

  float m_s = kNoKeys, l_s = 0.0f;
  float o[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[g][e] = 0.0f;

  // one tile from ring slot `slot`: scores, online softmax update, P.V
  auto process = [&](int slot, int t) {
    const int key0 = k0 + t * kTile;
    const uint32_t base = lds_addr(ring[wave][slot]);
    // key row sub, quarter grp; value rows 4*grp + r, columns 8*sub .. +7
    u32x4 kx[kQC];
#pragma unroll
    for (int i = 0; i < kQC; ++i)
      kx[i] = k_read(base + sub * LT::kPitchK + kswz(grp * kQC + i, sub) * 16);
    const uint32_t va = base + LT::kKBytes + grp * 4 * LT::kRowV + sub * 8 * esz;
    auto v0 = v_read<kFP8, 0>(va);
    auto v1 = v_read<kFP8, LT::kRowV>(va);
    auto v2 = v_read<kFP8, 2 * LT::kRowV>(va);
    auto v3 = v_read<kFP8, 3 * LT::kRowV>(va);
    decode_lds_wait(v0, v1, v2, v3, kx);
    QT kq;
#pragma unroll
    for (int i = 0; i < kQC; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) kq.w[4 * i + c] = kx[i][c];
    const f32x4 acc = tile_scores<DQK, kFP8>(kq, qq);
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
    // probabilities and rescale factor of head g's stream (lane 16 grp + g)
    f32x4 pg4[G];
    float al[G];
    row_bcast_all(std::make_integer_sequence<int, G>{}, p, alpha, pg4, al);
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[g][e] *= al[g];
    RowPart<128, kFP8> vr[4];
    auto put = [&](RowPart<128, kFP8>& r, const typename VRead<kFP8>::T& x) {
#pragma unroll
      for (int i = 0; i < RowPart<128, kFP8>::kA; ++i) r.a[i] = (uint32_t)x[i];
    };
    put(vr[0], v0);
    put(vr[1], v1);
    put(vr[2], v2);
    put(vr[3], v3);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float vv[8];
      row_values<128, kFP8>(vr[r], vv);
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[g][e] = fmaf(pg4[g][r], vv[e], o[g][e]);
    }
  };

  // wave w takes tiles w, w+4, ...; its i-th tile goes to slot i % kRing.
  // Before tile i is read, the loads of tiles i+1 .. i+kRing-1 may still be
  // in flight: kLoads each.  The slot that tile i + kRing - 1 refills was
  // read (its reads waited on) in the previous step.
  const int nmine = wave < ntile ? (ntile - wave + kWaves - 1) / kWaves : 0;
#pragma unroll
  for (int i = 0; i < kRing - 1; ++i)
    if (i < nmine) issue(wave + kWaves * i, i);
  // zero columns past G, after the first tile loads are issued (using the
  // query earlier would make them wait for it)
  if (sub >= G) {
#pragma unroll
    for (int i = 0; i < QT::kWords; ++i) qq.w[i] = 0u;
  }
  for (int i0 = 0; i0 < nmine; i0 += kRing) {
#pragma unroll
    for (int j = 0; j < kRing; ++j) {
      const int i = i0 + j;
      if (i >= nmine) break;
      const int t = wave + kWaves * i;
      if (i + kRing - 1 < nmine) {
        issue(t + kWaves * (kRing - 1), (j + kRing - 1) % kRing);
        decode_wait_vmcnt<LT::kLoads * (kRing - 1)>();
      } else {
        const int younger = nmine - 1 - i;  // 0 .. kRing-2
        if (younger == 0) decode_wait_vmcnt<0>();
        else if (younger == 1) decode_wait_vmcnt<LT::kLoads>();
        else decode_wait_vmcnt<2 * LT::kLoads>();
      }
      process(j, t);
    }
  }

  // each lane of group grp takes the stream state of its group's G heads
  float m[G], l[G];
  {
    f32x4 st[G];
    row_bcast_all(std::make_integer_sequence<int, G>{}, f32x4{m_s, l_s, 0.0f, 0.0f}, 0.0f, st, l);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[g] = st[g][0];
      l[g] = st[g][1];
    }
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

  // merge the waves through LDS, in wave order; the partial outputs overlay
  // the ring, which every wave has finished reading at the barrier
  __syncthreads();
  float (*sO)[G][kDV] = reinterpret_cast<float (*)[G][kDV]>(&ring[0][0][0]);
  float (*sM)[G] = reinterpret_cast<float (*)[G]>(&ring[0][0][0] + sizeof(float) * kWaves * G * kDV);
  float (*sL)[G] = sM + kWaves;
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
  // up to 32 splits: every partial is loaded at once (one memory round
  // trip), then combined in split order as below
  if (ns <= 32) {
    float lv[32], ov[32];
#pragma unroll
    for (int s = 0; s < 32; ++s) {
      lv[s] = s < ns ? lp[s] : -INFINITY;
      ov[s] = s < ns ? op[(int64_t)s * kDV + d] : 0.0f;
    }
    float M = lv[0];
#pragma unroll
    for (int s = 1; s < 32; ++s) M = fmaxf(M, lv[s]);
    float wsum = 0.0f, acc = 0.0f;
#pragma unroll
    for (int s = 0; s < 32; ++s) {
      if (s < ns) {
        const float w = expf(lv[s] - M);
        wsum += w;
        acc = fmaf(w, ov[s], acc);
      }
    }
    o[(int64_t)bh * kDV + d] = (__bf16)(acc / wsum);
    if (lse != nullptr && d == 0) lse[bh] = M + logf(wsum);
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

namespace {
// Keys per split: about `target` workgroups if every sequence had max_seqlen
// keys, a multiple of 64 in [256, cap].  Sequences shorter than max_seqlen
// leave workgroups that return at once.
int split_keys(int64_t B, int64_t Hkv, int64_t max_seqlen, int64_t target, int64_t cap) {
  const int64_t per = B * Hkv;
  const int64_t want = (target + per - 1) / per;
  int64_t sp = (max_seqlen + want - 1) / want;
  sp = (sp + 63) / 64 * 64;
  if (sp < 256) sp = 256;
  if (sp > cap) sp = cap;
  return (int)sp;
}
}  // namespace

void decode_split_policy(int64_t B, int64_t Hkv, int64_t max_seqlen, int* split, int* nsplit) {
  // about 4096 workgroups (16 per CU), splits of at most 1024 keys: the e4m3
  // kernels' policy, and the most splits any call uses (sizes the workspace)
  const int sp = split_keys(B, Hkv, max_seqlen, 4096, 1024);
  *split = sp;
  *nsplit = (int)((max_seqlen + sp - 1) / sp);
}

void decode_launch_policy(const DecodeArgs& a, int* split, int* nsplit) {
  decode_split_policy(a.B, a.Hkv, a.max_seqlen, split, nsplit);
  if (a.dtype_fp8) return;
  // bf16 rows carry half the vector work per byte of e4m3 ones: fewer,
  // longer splits (about 512 workgroups, up to 4096 keys) stream better.  A
  // split spans at most 64 pages (one page index per lane).  Never more
  // splits than the workspace holds.
  const int sp = split_keys(a.B, a.Hkv, a.max_seqlen, 512,
                            a.page_size * 64 < 4096 ? a.page_size * 64 : 4096);
  const int ns = (int)((a.max_seqlen + sp - 1) / sp);
  if (ns <= *nsplit) {
    *split = sp;
    *nsplit = ns;
  }
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
