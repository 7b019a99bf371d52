// Device helpers shared by the gfx950 kernels of the native sparse
// attention library: vector types, LDS / constant address spaces, exp2,
// cross-lane reductions over the four 16-lane groups of an MFMA tile, the
// slot chunk swizzles, explicit vmcnt waits and range-checked buffer
// resources.  Internal, not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nsa {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#define NSA_LDS __attribute__((address_space(3)))
#define NSA_CONST __attribute__((address_space(4)))
// Third dword of a raw buffer resource (untyped loads, no swizzle).
constexpr int kBufferFlags = 0x00020000;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Maxima without the NaN quieting the compiler wraps around fmaxf for
// values it cannot prove canonical (MFMA results, lane exchanges): one
// v_max3_f32 / v_max_f32 each.  The operands are scores or -inf, never
// signalling NaNs.
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Lanes c, c+16, c+32, c+48 hold the same column.  v_permlane16_swap /
// v_permlane32_swap (gfx950) exchange 16-lane (resp. 32-lane) rows between
// their two registers in the VALU: with both operands = v, every lane gets
// back its own value and its partner's 16 (resp. 32) lanes away, in one
// order or the other, which a max or a sum does not mind.
__device__ __forceinline__ float max_over_groups(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = max_raw(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max_raw(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_over_groups(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 16-byte chunk swizzles of a slot.  K rows are read as ds_read_b128 by
// 16 consecutive rows, V rows by the transposing read in 4 x 16 tiles.
template <int D>
__device__ __forceinline__ int k_swizzle(int row) {
  constexpr int kRowsPer256 = (256 / (D * 2)) > 0 ? 256 / (D * 2) : 1;
  constexpr int kChunks = D / 8;
  return (row / kRowsPer256) & (kChunks - 1);
}
template <int D>
__device__ __forceinline__ int v_swizzle(int row) {
  constexpr int kRowsPer256 = (256 / (D * 2)) > 0 ? 256 / (D * 2) : 1;
  constexpr int kPairs = D / 16;
  return ((row / kRowsPer256) & (kPairs - 1)) << 1;
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// A pointer whose value is the same in every lane, held in scalar registers.
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return (const char*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Raw buffer resource for the rows from byte `at` of a K or V tensor of
// `total` bytes: the record count ends at the tensor's end (clamped to the
// 31-bit range), so loads past it read zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t group_rsrc(const char* base, int64_t at, int64_t total) {
  int64_t left = total - at;
  left = left < 0 ? 0 : (left > 0x7FFFFFFF ? 0x7FFFFFFF : left);
  return __builtin_amdgcn_make_buffer_rsrc((void*)uniform_ptr(base + at), 0, (int)left, kBufferFlags);
}

}  // namespace dev
}  // namespace nsa
