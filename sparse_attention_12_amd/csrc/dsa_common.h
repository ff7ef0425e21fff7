// Internal helpers shared by the libdsa kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

// float -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// 16x16x32 bf16 MFMA: A rows = lane%16, B cols = lane%16, both take k = (lane/16)*8 + [0,8);
// D[(lane/16)*4 + i][lane%16] = c[i].
__device__ __forceinline__ f32x4 mfma16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16x16x32 fp16 MFMA (same operand layout as mfma16).
__device__ __forceinline__ f32x4 mfma16h(const f16x8 &a, const f16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// two floats -> packed fp16 bits, round to nearest even (v_cvt_pk_f16_f32)
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const f16x2 v = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ f16x8 as_f16x8(const u32x4 &v) {
  return __builtin_bit_cast(f16x8, v);
}

// 32x32x16 bf16 MFMA: A rows = lane%32, B cols = lane%32, k = (lane/32)*8 + [0,8);
// D[(i/4)*8 + (lane/32)*4 + i%4][lane%32] = c[i].
__device__ __forceinline__ f32x16 mfma32(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4 &v) {
  return __builtin_bit_cast(bf16x8, v);
}

// Transposing LDS read: within each group of 16 lanes, lane i receives element i (in lane-then-
// element order) of each 4-lane block's four 8-byte reads.  With lanes 4r..4r+3 of a group
// pointing at columns [4c, 4c+4) of row r of a row-major bf16 tile, lane i gets rows r = 0..3
// of column i.
__device__ __forceinline__ u32x2 lds_read_tr16(const void *lds_ptr) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4 *)(lds_ptr));
  return __builtin_bit_cast(u32x2, v);
}

// Value of `x` held by lane (lane ^ 32).
__device__ __forceinline__ float swap_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(__lane_id() < 32 ? r[1] : r[0]);
}

// Value of `x` held by lane (lane ^ 16), without a trip through LDS (v_permlane16_swap: the
// first result holds the even 16-lane row's values, the second the odd row's).
__device__ __forceinline__ float xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((__lane_id() & 16) ? r[0] : r[1]);
}

__device__ __forceinline__ float xor_lane(float x, int mask) {
  return __shfl_xor(x, mask, 64);
}

// Orders LDS traffic of the calling wave (lanes exchanging data through LDS).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const unsigned l = __lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

}  // namespace dsa
