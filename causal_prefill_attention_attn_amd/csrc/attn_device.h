// Device helpers shared by the BF16 and FP8 attention kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpattn {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// v_permlane32_swap on two copies of x leaves {own value, value of lane
// l^32} in its two results (which one is which depends on the lane half),
// so combining both with a commutative operation gives the pair result in
// every lane.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroup id -> (query block qb, problem*head bh).  Workgroups go to the
// eight XCDs round-robin by id.  Default: the longest query blocks first
// across all (b, h).  When every (b, h) has at least 128 query blocks and B*H
// is a multiple of 8, each XCD runs its (b, h) one after another instead,
// longest blocks first, so that its resident workgroups stream the same K and
// V through its L2: at 32K tokens this fetches a third of the bytes.
__device__ __forceinline__ void block_order(int id, int nqb, int BH, int& qb, int& bh) {
  if (nqb >= 128 && (BH & 7) == 0) {
    const int x = id & 7, j = id >> 3;
    qb = nqb - 1 - j % nqb;
    bh = x + 8 * (j / nqb);
  } else {
    qb = nqb - 1 - id / BH;
    bh = id % BH;
  }
}

// The same order with the last part of the work shared among the XCDs.
// Which XCD runs slowest changes from launch to launch, and a static split
// leaves the others idle at the end (4-9% of the span at 32K tokens).  So the
// q_cut shortest query blocks of every (b, h) leave the static lists: in the
// head-major order XCD x = id & 7 runs blocks nqb-1 .. q_cut of its heads
// x, x+8, ...; in the query-block-major order the first n_static ids are
// those blocks already.  The workgroups after the static ids claim the
// remaining blocks, longest first, from a counter that starts at zero.  The
// fast XCDs reach their claiming workgroups first and take more of them;
// workgroups that find the pool empty end at once.  Outputs do not depend
// on which workgroup computes a block.  lds_slot is a word of the
// workgroup's LDS not yet in use.  Returns false when the workgroup has no
// block.
__device__ __forceinline__ bool block_claim(int id, int nqb, int BH, int n_static, int q_cut,
                                            int* ctr, int* lds_slot, int& qb, int& bh) {
  if (q_cut == 0) {
    block_order(id, nqb, BH, qb, bh);
    return true;
  }
  if (id < n_static) {
    if (nqb >= 128 && (BH & 7) == 0) {
      const int x = id & 7, j = id >> 3, nl = nqb - q_cut;
      qb = nqb - 1 - j % nl;
      bh = x + 8 * (j / nl);
    } else {
      block_order(id, nqb, BH, qb, bh);  // its first n_static ids: blocks nqb-1 .. q_cut
    }
    return true;
  }
  if (threadIdx.x == 0) *lds_slot = atomicAdd(ctr, 1);
  __syncthreads();
  const int t = __builtin_amdgcn_readfirstlane(*lds_slot);
  __syncthreads();
  if (t >= BH * q_cut) return false;
  qb = q_cut - 1 - t / BH;
  bh = t % BH;
  return true;
}

// Rows of one attention problem -- one batch entry of a dense [B,S,H,D]
// tensor, or one sequence of a packed [total,H,D] tensor -- and where its LSE
// goes (dense [B,H,S], packed [H,total]).
struct SeqRows {
  int64_t row0;    // first row of the problem in q/k/v/o
  int len;         // its rows
  int64_t lse0;    // LSE index of (head 0, row 0)
  int64_t lse_hs;  // LSE stride between heads
};
// Problem b: dense when cu is null (S rows each), else packed with bounds
// cu[b], cu[b+1] clamped to [0, total] and to S (the longest sequence), so
// that any contents of cu give in-bounds accesses.
__device__ __forceinline__ SeqRows seq_rows(const int32_t* cu, int b, int S, int H,
                                            int64_t total) {
  SeqRows r;
  if (cu == nullptr) {
    r.row0 = (int64_t)b * S;
    r.len = S;
    r.lse0 = (int64_t)b * H * S;
    r.lse_hs = S;
  } else {
    int64_t a = cu[b], e = cu[b + 1];
    a = a < 0 ? 0 : (a > total ? total : a);
    e = e < a ? a : (e > total ? total : e);
    if (e - a > S) e = a + S;
    r.row0 = a;
    r.len = (int)(e - a);
    r.lse0 = a;
    r.lse_hs = total;
  }
  return r;
}

// Buffer resource over `bytes` bytes from `base`: loads at byte offsets
// >= bytes return zero (the hardware range check), which pads ragged tiles.
// The whole offset goes in the VGPR operand so that it is range checked.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

// 16 bytes per lane from buffer offset `off` straight into LDS: lane l's
// data lands at lds_base + 16*l (lds_base must be the same in every lane);
// offsets past the buffer end write zeros.  Kept in a __device__ function:
// used directly inside a kernel template, the builtin stops the host pass
// from emitting the kernel's launch stub.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, void* lds_base,
                                                  uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base,
                                           16, (int)off, 0, 0, 0);
}
// The same with the wave-uniform part of the offset in the instruction's
// scalar offset field, so that no vector add forms the address.  Only for
// loads known to lie inside the buffer: the out-of-range zeros above are not
// relied on here.
__device__ __forceinline__ void buffer_load_lds16_so(__amdgpu_buffer_rsrc_t r, void* lds_base,
                                                     uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base,
                                           16, (int)voff, (int)soff, 0, 0);
}

// ds_read_b64_tr_b16 issued as inline assembly.  The compiler builtin for
// it carries no alias information, so the wait-count pass makes every such
// read wait until all buffer-to-LDS loads in flight have landed, which
// drains the K/V prefetch each tile.  As assembly the read waits for
// nothing; its result must be ordered with lds_wait_n() before use.  Lanes
// 4r..4r+3 of a 16-lane group supply the 16 values of row r (four rows) and
// lane i receives value i of every row.  `addr` is an LDS byte address; OFF
// a constant byte offset (< 65536).
template <int OFF>
__device__ __forceinline__ i16x4 ds_read_tr16(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  i16x4 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
  return r;
}
// ds_read_b64_tr_b8 as inline assembly, for the same reason: lanes 2r and
// 2r+1 of a 16-lane group supply row r (16 bytes) and lane i receives byte
// i of every row (eight rows).  Order its result with lds_wait4() before use.
template <int OFF>
__device__ __forceinline__ i32x2 ds_read_tr8(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  i32x2 r;
  asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
  return r;
}
// s_waitcnt lgkmcnt(N) tied to the four registers pairs of a transposed
// operand read, so that nothing that reads them (including the moves that
// assemble the operand) can be placed above the wait.
template <int N>
__device__ __forceinline__ void lds_wait4(i32x2& a, i32x2& b, i32x2& c, i32x2& d) {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d) : "i"(N));
}

// s_waitcnt lgkmcnt(N), tied to one operand register set so that its uses
// cannot be scheduled above it.  LDS operations complete in order, so with
// at most N of them (and any scalar loads) still in flight every older LDS
// read has landed.
template <int N>
__device__ __forceinline__ void lds_wait_n(bf16x8& a) {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a) : "i"(N));
}

// Workgroup barrier without a memory fence: s_barrier, guarded only
// against compiler reordering of memory accesses.  __syncthreads() adds a
// workgroup release, and the compiler counts every buffer-to-LDS load in
// flight as an LDS store that the release must wait for, so each barrier
// would drain the whole K/V prefetch.  Here a wave that issued such loads
// makes them visible by waiting for them itself (s_waitcnt vmcnt) before it
// arrives; every LDS read is consumed (its lgkmcnt wait passed) before the
// barrier after which its buffer is refilled.
__device__ __forceinline__ void barrier_nofence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS byte address of a pointer into a __shared__ object
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16-byte LDS read
__device__ __forceinline__ u32x4 lds_load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// One wave's 32 output rows to bf16 global memory through a 4 KB LDS area
// that only this wave uses.  Lane (col, half) = (lane % 32, lane / 32)
// holds, for row col, acc[d][4g + e] of column 32d + 8g + 4half + e
// (d < DV/32, g < 4, e < 4), the transposed layout of the P.V accumulators.
// Written straight from there, each 8-byte store instruction would touch 32
// rows, i.e. 32 partly written 128-byte lines.  Instead, per round of 64
// columns (128 bytes of a row) the wave writes its rows to LDS in 8-byte
// pieces and reads them back 16 bytes per lane, eight lanes per row, so
// that every store instruction writes 8 whole 128-byte row segments.  The
// 16-byte chunk c of LDS row r sits at chunk c ^ (r & 7), so that the 8
// lanes reading one row and the rows written together spread over the
// banks.  Row r of the wave is output row row0 + r, which starts at element
// (row0 + r) * rstride + col0 of o; rows r >= nvalid are not stored (nor
// their addresses formed).
template <int DV>
__device__ __forceinline__ void store_rows_bf16(const f32x16* acc, float scale, uint8_t* area,
                                                __bf16* o, int64_t row0, int64_t rstride,
                                                int64_t col0, int nvalid, int lane) {
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  lds_u8* a = (lds_u8*)(uintptr_t)lds_addr(area);
  const int col = lane & 31, half = lane >> 5;
#pragma unroll
  for (int rr = 0; rr < DV / 64; ++rr) {
#pragma unroll
    for (int dd = 0; dd < 2; ++dd)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(acc[2 * rr + dd][g * 4 + e] * scale);
        const int ch = dd * 4 + g;
        *(__attribute__((address_space(3))) bf16x4*)(a + col * 128 + ((ch ^ (col & 7)) << 4) +
                                                     half * 8) = w;
      }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (lane >> 3) + 8 * i, c = lane & 7;
      const bf16x8 x = *(const __attribute__((address_space(3))) bf16x8*)(a + r * 128 +
                                                                          ((c ^ (r & 7)) << 4));
      if (r < nvalid)
        *reinterpret_cast<bf16x8*>(o + (row0 + r) * rstride + col0 + rr * 64 + c * 8) = x;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
}
}  // namespace cpattn
