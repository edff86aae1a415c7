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
typedef short i16x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void lds_void;

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

// 16-byte LDS accesses
__device__ __forceinline__ u32x4 lds_load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void lds_store16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// 32-byte operand from two 16-byte LDS reads at p and p + second
__device__ __forceinline__ i32x8 lds_load32(const uint8_t* p, int second) {
  const i32x4 lo = *reinterpret_cast<const i32x4*>(p);
  const i32x4 hi = *reinterpret_cast<const i32x4*>(p + second);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

}  // namespace cpattn
