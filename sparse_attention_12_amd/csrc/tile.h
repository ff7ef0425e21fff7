// LDS tile of gathered latent rows shared by the sparse MLA kernels.
//
// A tile holds kSlots rows of DQK bf16 channels (row-major, no padding) and is filled with
// direct global->LDS loads (global_load_lds_dwordx4): lane i of a load instruction writes the
// 16 bytes it fetched to LDS offset base + 16 i.  The lane therefore fetches whichever 16-byte
// chunk belongs at that LDS position, which lets the tile use an XOR swizzle of the 16-byte
// chunks inside each row without any register traffic:
//     physical chunk = logical chunk ^ swz(row)
// swz keeps a chunk inside its aligned group of 8 (576-wide rows) or 16 (512-wide rows) and
// spreads the rows read by one MFMA fragment, row-wise or transposed, over the LDS banks
// without conflicts.
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
  // the base is wave-uniform by contract; reading it from the first lane pins it to scalar
  // registers even where the compiler has lost track of that (folded away when it is scalar)
  // (readfirstlane yields a signed int: each half goes through uint32_t so that widening
  // zero-extends it; sign-extending the low half would corrupt the high half of the address)
  const uint64_t b = reinterpret_cast<uintptr_t>(base);
  const uint32_t blo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b)));
  const uint32_t bhi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32)));
  const uint64_t bs = static_cast<uint64_t>(blo) | (static_cast<uint64_t>(bhi) << 32);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(bs), "s"(__builtin_amdgcn_readfirstlane(lds))
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

// Slot-index ring of one query row: tiles of 32 slots (latent row per slot, -1 for an invalid
// slot or one beyond the row's valid prefix) in an LDS ring of 8 tiles.  One wave keeps it
// filled with ordinary loads issued in batches of four tiles, one batch interval (four tiles)
// before they are stored, so that no interval waits for a load it has just issued (such a wait
// would hold the whole work group at the next barrier).  start() stores tiles 0..3 and issues
// 4..7; step(c), at the top of interval c (every wave done with interval c - 1), stores tiles
// c + 4 .. c + 7 when c is a multiple of 4, into the ring slots of tiles c - 4 .. c - 1, and
// issues the next batch.
struct SlotRing {
  static constexpr int kSlots = 32, kTiles = 8, kBatch = 4;
  int32_t pend[kBatch];
  __device__ __forceinline__ static int32_t load(const int32_t *__restrict__ irow, int lim,
                                                 int j) {
    const int lane = __lane_id();
    const int slot = j * kSlots + lane;
    return lane < kSlots && slot < lim ? irow[slot] : -1;
  }
  __device__ __forceinline__ static void put(int32_t *ring, int j, int32_t v) {
    const int lane = __lane_id();
    if (lane < kSlots) ring[(j % kTiles) * kSlots + lane] = v;
  }
  __device__ __forceinline__ void start(const int32_t *__restrict__ irow, int lim, int nchunks,
                                        int32_t *ring) {
    int32_t first[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) first[j] = j < nchunks ? load(irow, lim, j) : -1;
#pragma unroll
    for (int b = 0; b < kBatch; ++b)
      pend[b] = kBatch + b < nchunks ? load(irow, lim, kBatch + b) : -1;
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (j < nchunks) put(ring, j, first[j]);
  }
  __device__ __forceinline__ void step(const int32_t *__restrict__ irow, int lim, int nchunks,
                                       int32_t *ring, int c) {
    if ((c & (kBatch - 1)) != 0 || c + kBatch >= nchunks) return;
#pragma unroll
    for (int b = 0; b < kBatch; ++b)
      if (c + kBatch + b < nchunks) put(ring, c + kBatch + b, pend[b]);
#pragma unroll
    for (int b = 0; b < kBatch; ++b)
      pend[b] = c + 2 * kBatch + b < nchunks ? load(irow, lim, c + 2 * kBatch + b) : -1;
  }
};

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

  // Chunk XOR of a row.  Two read patterns must be free of LDS bank conflicts: 16-byte reads
  // of one logical chunk from 16 consecutive rows, four adjacent chunks across the four lane
  // groups (MFMA fragments of rows), and the transposing 8-byte reads of two adjacent chunks
  // from 4 consecutive rows in each lane group (fragments of columns).  The XOR stays inside
  // the chunk's aligned group of 8 (576-wide rows) or 16 (512-wide rows).  Chosen by
  // measurement on gfx950 (SQ_LDS_BANK_CONFLICT over repeated reads of each pattern): row & 7
  // (576) and (row & 7) << 1 (512) leave both patterns without conflicts, while a swizzle built
  // for 64 four-byte banks served by 16 consecutive lanes stalled half of the row-fragment
  // reads' LDS cycles.
  __device__ static __forceinline__ int swz(int row) {
    return DQK == 576 ? (row & 7) : ((row & 7) << 1);
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

// Wait for the oldest tile when `ahead` later tiles (each L loads per wave) may stay in flight.
template <int L, int NBUF>
__device__ __forceinline__ void wait_tiles_ahead(int ahead) {
  if constexpr (NBUF >= 4) {
    if (ahead >= 2) { wait_vm<2 * L>(); return; }
  }
  if constexpr (NBUF >= 3) {
    if (ahead >= 1) { wait_vm<L>(); return; }
  }
  wait_vm<0>();
}

// Stream of a query's latent-row tiles through NBUF LDS buffers (tile c in buffer c % NBUF),
// filled by the NW waves of a work group with direct loads.  slot_rows (LDS) lists the latent
// row of every slot of the query, -1 for an invalid slot, up to a whole number of tiles; the
// latent tensor is below 4 GiB, so a 32-bit offset from its base addresses any row.
template <int DQK, int NW, int NBUF>
struct TileStream {
  using TL = Tile<DQK>;
  static constexpr int L = TL::kLoads / NW;  // loads per wave per tile
  static_assert(TL::kLoads % NW == 0, "loads must split evenly over the waves");
  int dma_row[L], dma_off[L];
  uint32_t tiles_lds;  // LDS address of buffer 0 plus this wave's first load slot

  __device__ __forceinline__ void init(const void *tiles, int wave) {
    const int lane = __lane_id();
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int pos = (i * NW + wave) * 64 + lane;
      dma_row[i] = pos / TL::kChunks;
      dma_off[i] = ((pos % TL::kChunks) ^ TL::swz(dma_row[i])) * 16;
    }
    tiles_lds = lds_addr(tiles) + wave * 1024;
  }
  __device__ __forceinline__ void issue(int c, const uint16_t *kv, const int32_t *slot_rows) const {
    const uint32_t dst = tiles_lds + (c % NBUF) * TL::kBytes;
    // every row index first: the loads are asm with a memory clobber, so an index read placed
    // between two of them would be waited for on its own
    uint32_t off[L];
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int r = slot_rows[c * TL::kSlots + dma_row[i]];
      off[i] = static_cast<uint32_t>(r < 0 ? 0 : r) * TL::kRowBytes + dma_off[i];  // -1: row 0
    }
#pragma unroll
    for (int i = 0; i < L; ++i) dma16_sv(kv, off[i], dst + i * NW * 1024);
  }
  // Before processing tile c of nchunks: wait for it and publish it to the work group.  The
  // barrier also means every wave is done with tile c - 1, whose buffer the caller may refill.
  __device__ static __forceinline__ void acquire(int c, int nchunks) {
    wait_tiles_ahead<L, NBUF>(min(NBUF - 2, nchunks - 1 - c));
    lds_barrier();
  }
};

// Per-lane LDS byte offsets into a Tile<DQK> for the 16x16x32 MFMA fragments of a 32-slot
// tile (lane = 16 g + hl, r4 = hl / 4, cq = lane % 4):
//   A operand of S^T = rows . q^T, rows mt*16 + hl, chunk 4 ks + g:
//       a_off(mt, ks) = sbase[mt][ks & 3] + (ks >> 2) * 256
//   transposing reads of columns 16 n + 4 cq .. + 3 of rows 4 g + r4 and 16 + 4 g + r4 (the
//   slot order that matches a P / dZ fragment held in registers):
//       v_off(half, n) = vbase[half][n & 7] + (n >> 3) * 256
// (the swizzle only permutes the low four bits of a chunk index, so chunk 16 a + b lands at
// (16 a + (b ^ swz)) * 16).
template <int DQK>
struct TileFrag {
  using TL = Tile<DQK>;
  int sbase[2][4], vbase[2][8];
  __device__ __forceinline__ void init() {
    const int lane = __lane_id();
    const int g = lane >> 4, hl = lane & 15, r4 = hl >> 2, cq = lane & 3;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) sbase[mt][j] = TL::chunk_off(mt * 16 + hl, j * 4 + g);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      vbase[0][j] = TL::elem_off(g * 4 + r4, j * 16 + cq * 4);
      vbase[1][j] = TL::elem_off(16 + g * 4 + r4, j * 16 + cq * 4);
    }
  }
  __device__ __forceinline__ bf16x8 a_frag(const unsigned char *tile, int mt, int ks) const {
    return as_bf16x8(*reinterpret_cast<const u32x4 *>(tile + sbase[mt][ks & 3] + (ks >> 2) * 256));
  }
  // rows^T fragment (16 columns x 32 slots in the register P/dZ slot order)
  __device__ __forceinline__ bf16x8 v_frag(const unsigned char *tile, int n) const {
    const u32x2 lo = lds_read_tr16(tile + vbase[0][n & 7] + (n >> 3) * 256);
    const u32x2 hi = lds_read_tr16(tile + vbase[1][n & 7] + (n >> 3) * 256);
    return as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
  }
};

// The transposing column reads of TileFrag::v_frag for NT consecutive 16-column tiles starting
// at tile n0 (n0 may differ between the waves of a work group: the offsets are computed, not
// indexed, so they stay in registers).
template <int DQK, int NT>
struct ColFrags {
  using TL = Tile<DQK>;
  int off[2][NT];
  __device__ __forceinline__ void init(int n0) {
    const int lane = __lane_id();
    const int g = lane >> 4, r4 = (lane & 15) >> 2, cq = lane & 3;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      off[0][n] = TL::elem_off(g * 4 + r4, (n0 + n) * 16 + cq * 4);
      off[1][n] = TL::elem_off(16 + g * 4 + r4, (n0 + n) * 16 + cq * 4);
    }
  }
  __device__ __forceinline__ bf16x8 frag(const unsigned char *tile, int n) const {
    const u32x2 lo = lds_read_tr16(tile + off[0][n]);
    const u32x2 hi = lds_read_tr16(tile + off[1][n]);
    return as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
  }
};

// Pack an S^T-layout fragment x[mt][i] (slot 16 mt + 4 g + i of this lane's head) into the
// bf16 MFMA operand whose contraction index 8 g + j is slot 4 g + j (j < 4) or 16 + 4 g + j - 4.
__device__ __forceinline__ bf16x8 pack_slots(const float x[2][4]) {
  u32x4 w;
  w[0] = pack_bf16x2(x[0][0], x[0][1]);
  w[1] = pack_bf16x2(x[0][2], x[0][3]);
  w[2] = pack_bf16x2(x[1][0], x[1][1]);
  w[3] = pack_bf16x2(x[1][2], x[1][3]);
  return as_bf16x8(w);
}

}  // namespace dsa
