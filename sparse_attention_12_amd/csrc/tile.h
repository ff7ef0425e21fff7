// LDS tile of gathered latent rows shared by the sparse MLA kernels.
//
// A tile holds kSlots rows of DQK bf16 channels (row-major, no padding) and is filled with
// direct global->LDS loads (global_load_lds_dwordx4): lane i of a load instruction writes the
// 16 bytes it fetched to LDS offset base + 16 i.  The lane therefore fetches whichever 16-byte
// chunk belongs at that LDS position, which lets the tile use an XOR swizzle of the 16-byte
// chunks inside each row without any register traffic:
//     physical chunk = logical chunk ^ swz(row)
// swz keeps a chunk inside its aligned group of 8 (576-wide rows) or 16 (512-wide rows) and
// spreads the 16 rows read by one MFMA fragment over distinct LDS banks.
//
// Slots whose index is -1 (or beyond the valid prefix) are filled from latent row 0 so that no
// load is out of bounds; the kernels mask those slots (probability 0) so the values never
// contribute.
//
// The loads are issued through inline assembly so that the compiler does not treat them as
// pending LDS writes (it would otherwise wait for the next tile's loads before every read of
// the current tile).  The kernels wait for them explicitly with wait_tile() before the
// barrier that publishes a tile; the compiler's own waits for other vector-memory loads stay
// correct because extra older or younger loads only make an in-order vmcnt wait stricter.
#pragma once

#include "dsa_common.h"

namespace dsa {

// One wave-wide 16-byte-per-lane global -> LDS load: lane i's 16 bytes land at
// lds_dst + 16 i (lds_dst must be wave-uniform).  M0 is saved and restored.
__device__ __forceinline__ void dma16(const void *src, void *lds_dst) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) void *)lds_dst)));
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds)
      : "memory");
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void *)p));
}

// As dma16, with the global address split into a wave-uniform base (SGPR pair) and a 32-bit
// per-lane byte offset, and the destination given as a wave-uniform LDS byte address, so that
// moving to the next tile is scalar arithmetic only.
__device__ __forceinline__ void dma16_sv(const void *base, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(base), "s"(__builtin_amdgcn_readfirstlane(lds))
      : "memory");
}

// Make the compiler finish every load that produced `v` here (the value is pinned to VGPRs at
// this point).  Used before a kernel's main loop: the tile loads are invisible to the
// compiler, so a prologue load still pending at the loop header would make it wait for all
// vector-memory traffic (tile loads included) at the first use inside every iteration.
template <typename T>
__device__ __forceinline__ void settle(T &v) {
  asm volatile("" : "+v"(v));
}

// Wait until at most N vector-memory operations of this wave (including dma16) are still in
// flight (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_tile() { wait_vm<0>(); }

// Work-group barrier that orders LDS traffic only (it does not wait for outstanding global
// loads, unlike __syncthreads, so in-flight tile loads keep streaming across it).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int DQK>
struct Tile {
  static constexpr int kSlots = 32;
  static constexpr int kChunks = DQK / 8;            // 16-byte chunks per row
  static constexpr int kRowBytes = DQK * 2;
  static constexpr int kBytes = kSlots * kRowBytes;
  static constexpr int kLoads = kSlots * kChunks / 64;  // wave-wide DMA instructions per tile

  __device__ static __forceinline__ int swz(int row) {
    return DQK == 576 ? ((row >> 1) & 7) : (row & 15);
  }
  // byte offset of logical (row, chunk)
  __device__ static __forceinline__ int chunk_off(int row, int chunk) {
    return row * kRowBytes + ((chunk ^ swz(row)) << 4);
  }
  // byte offset of element `col` (a multiple of 4) of `row`: 8-byte aligned
  __device__ static __forceinline__ int elem_off(int row, int col) {
    return row * kRowBytes + (((col >> 3) ^ swz(row)) << 4) + ((col & 7) << 1);
  }

  // Issue this wave's share (loads k = wave, wave + NW, ...) of the DMA loads filling `tile`
  // with the latent rows of slots [c0, c0 + kSlots): `slot_rows` (LDS) holds the row of every
  // slot of the query (-1 = invalid), `lim` is the number of slots.
  template <int NW>
  __device__ static __forceinline__ void issue(unsigned char *tile, const uint16_t *kv,
                                               const int32_t *slot_rows, int c0, int lim,
                                               int wave) {
    const int lane = __lane_id();
#pragma unroll
    for (int k = wave; k < kLoads; k += NW) {
      const int pos = k * 64 + lane;          // physical chunk position in the tile
      const int row = pos / kChunks;
      const int chunk = (pos % kChunks) ^ swz(row);
      const int slot = c0 + row;
      int r = slot < lim ? slot_rows[slot] : -1;
      r = r < 0 ? 0 : r;
      const uint16_t *src = kv + static_cast<int64_t>(r) * DQK + chunk * 8;
      dma16(src, tile + k * 1024);
    }
  }
};

}  // namespace dsa
