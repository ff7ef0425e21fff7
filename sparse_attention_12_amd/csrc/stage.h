// Staged key-gradient contributions: 16-bit block floating point rows, written by the kernels
// that form per-(query, slot) contributions and summed per key row after a counting sort.
#pragma once

#include "dsa_common.h"

namespace dsa {

// A staged row holds D channels in 16 blocks.  Block b = 4 qq + g holds the channels
// qq D/4 + 16 n + 4 g + i (n < D/64, i < 4): the channels that lane group g of the wave owning
// channel quarter qq holds for one slot.  With 2^e the smallest power of two above the block's
// largest magnitude (e = the float exponent field of that magnitude, minus 126), channel x is
// kept as the signed 16-bit m = round(32767 x / 2^e) and read back as m 2^e / 32767: an error of
// at most 2^-15 of the block's largest magnitude.  A staged row is D mantissas in channel
// order, then 16 exponent bytes (byte b: the field of block b's largest magnitude, at most
// 253).
template <int D>
constexpr int kStageWords = D / 2 + 4;  // 32-bit words per staged row
template <int D>
__device__ __forceinline__ int stage_exp_byte(int ch) {  // exponent byte of channel ch
  return ch / (D / 4) * 4 + ((ch >> 2) & 3);
}
__device__ __forceinline__ uint32_t pknorm16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pknorm_i16(a, b));
}
__device__ __forceinline__ float stage_factor(uint32_t eb) {  // 2^e / 32767
  return __uint_as_float((eb + 1u) << 23) * (1.0f / 32767.0f);
}
__device__ __forceinline__ f32x4 unpack_m16x4(const u32x2 &m, float f) {
  return f32x4{static_cast<float>(static_cast<int32_t>(m[0] << 16) >> 16) * f,
               static_cast<float>(static_cast<int32_t>(m[0]) >> 16) * f,
               static_cast<float>(static_cast<int32_t>(m[1] << 16) >> 16) * f,
               static_cast<float>(static_cast<int32_t>(m[1]) >> 16) * f};
}

}  // namespace dsa
