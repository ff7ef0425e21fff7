// Absorbed sparse MLA backward (NeMo AutoModel cudnn_dsa API reference,
// _CudnnSparseAttention.backward: gradients for the query [T_q,H,576] and the gathered latent
// rows; SkyRL PR 2423 "Summary": query chunks are independent and key gradients sum).
//
// With P_j = exp(z_j - lse), dP_j = dO . v_j, Delta = dO . O and dZ_j = P_j (dP_j - Delta):
//   dq[t,h]   = scale * sum_j dZ_j kv_j
//   dkv[s_j] += scale * sum_h dZ_j q[t,h] + sum_h P_j dO[t,h]     (over every query t)
//
// Kernels, for query rows processed in passes of R rows (R as large as the caller's workspace
// allows):
//   rows   : one work group per query row, in two phases (layout of the waves below).  Both
//            recompute S^T and dP^T per 32-slot chunk of gathered latent rows; the dq phase
//            first forms Delta[t,h] = sum_c dO[t,h,c] O[t,h,c] from the forward output (kept
//            in the workspace for the second phase), then dq = scale dZ . rows; the
//            contribution phase forms C = scale dZ^T . q +
//            P^T . dO for every (query, slot) pair and stores C to a staging buffer (16-bit
//            block floating point, see below).
//   scan / fill : a counting sort of the pass's (query, slot) pairs by latent row (the rows
//            launch has counted them).
//   reduce : one work group per latent row adds up its staged contributions and adds the sum
//            to dkv (every row has a single owner, so no atomics touch dkv).
// Compared with fp32 atomics on dkv (bounded by the L2 atomic units at about one 4-byte add
// per channel per clock), staging moves about 4 bytes of HBM traffic per contribution element.
#include <algorithm>
#include <mutex>

#include "dsa_common.h"
#include "dsa_internal.h"
#include "stage.h"
#include "tile.h"

namespace dsa {
namespace {

constexpr int kSlots = 32;
constexpr int kDv = 512;

// ---------------------------------------------------------------------------------------
__global__ void fill_zero_kernel(float *__restrict__ p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t j = i; j < n; j += stride) p[j] = 0.0f;
}

// ---------------------------------------------------------------------------------------
// rows launch: one work group per query row of the pass computes the row's dq, then its
// key-gradient contributions (the second phase re-gathers the latent rows, mostly from L2).
// Keeping both phases in one work group gives every CU the same mix of work: with separate
// dq and contribution work groups the hardware's round-robin placement put each kind on its
// own half of the CUs, and the contribution half (about twice the work) set the time.  Both
// phases have 8 waves split by role, so that every SIMD runs one wave of each role and their
// work overlaps, and one barrier per 32-slot chunk:
//   SdP waves 0..3 (head group G = wave, 16 heads): S^T = rows . q^T and dP^T = V . dO^T
//     (16x16x32 MFMAs, A = LDS row fragments, B = q / dO blocks in registers), then
//     P = exp(S - lse) and dZ = P (dP - Delta).
//   dq phase, waves 4..7 (channel quarter qq): dq^T[channels x 64 heads] += rows^T . dZ^T
//     one chunk behind the SdP waves, dZ (bf16) of all head groups read from LDS; every
//     transposed row fragment feeds four MFMAs.  They also issue the latent-row tile loads.
//   contribution phase, waves 4..7 (channel quarter qq): C[32 slots x channels] =
//     scale dZ^T . q + P^T . dO one chunk behind, with q / dO held as head-contraction
//     fragments and scale dZ / P staged in LDS ([slot][head]), all as fp16 under per-row
//     power-of-two scales (C16Scales: 11 significant bits; with P or dZ rounded to bf16's 8
//     bits a latent row picked by many queries collects an error near the 2e-2 bar).  C is
//     stored as 16-bit block floating point (see kStageWords).
// Tile loads (direct to LDS, waited for with explicit load counts) come from waves that issue no
// other vector-memory operation, so that those counts stay exact and the compiler's own waits
// never wait for tiles.  The dq phase fetches slot indices into a small ring from SdP wave 0
// (ordinary loads, four tiles ahead); the contribution phase, whose channel waves store and
// whose SdP waves load tiles, reads the row's whole index list into LDS first.
constexpr int kRowWaves = 8;
constexpr int kDqBufs = 4;  // dq phase: a tile is read in two intervals
constexpr int kCBufs = 3;   // contribution phase: a tile is read in one interval
constexpr int kRing = 8;    // slot-index ring (tiles)
static_assert(kRing == SlotRing::kTiles && kSlots == SlotRing::kSlots, "slot-index ring layout");
constexpr int kSS = 72;     // staging row stride: 64 heads + 8 (bf16)
constexpr int kMaxK = 4096; // largest top-k of the contribution phase's index list

template <int DQK>
struct RowSmem {
  static constexpr int kTileB = Tile<DQK>::kBytes;
  // dq phase: tiles[4] | dZ[2][4 groups][64 lanes] bf16x8 | ring
  static constexpr int kDqZ = kDqBufs * kTileB;
  static constexpr int kDqRing = kDqZ + 2 * 4 * 64 * 16;
  static constexpr int kDqBytes = kDqRing + kRing * kSlots * 4;
  // contribution phase: tiles[3] | staging[2][z', P][32 slots][kSS] fp16 | slot rows (K
  // entries rounded up to a whole tile); the row's q ([64][DQK + 16]) and dO ([64][512 + 16])
  // pass through the tile area first, and the staging area starts with the prologue's exchange
  // of the row's largest |q| and |dO| (16 words)
  static constexpr int kCStageBytes = 2 * kSlots * kSS * 2;
  static constexpr int kCStage = kCBufs * kTileB;
  static constexpr int kCRows = kCStage + 2 * kCStageBytes;
  static constexpr int kCBytes = kCRows + kMaxK * 4;
  static size_t bytes(int K) {
    const size_t c = kCRows + static_cast<size_t>((K + kSlots - 1) / kSlots) * kSlots * 4;
    return c > kDqBytes ? c : static_cast<size_t>(kDqBytes);
  }
  static constexpr int kQStride = DQK + 16;
  static constexpr int kOStride = kDv + 16;
  static_assert(64 * kQStride * 2 <= kCStage, "q staging must fit the tile area");
  static_assert(kDqBytes <= 160 * 1024 && kCBytes <= 160 * 1024, "LDS per work group");
};

// This wave's share (loads k = 4 i + part) of the tile-c loads into buffer c % NBUF; rr lists
// the tile's 32 latent rows (-1: invalid slot).
template <int DQK, int NBUF>
__device__ __forceinline__ void issue_tile(uint32_t tiles_lds, const uint16_t *kv,
                                           const int32_t *rr, int c, int part) {
  using TL = Tile<DQK>;
  constexpr int kLoadsW = TL::kLoads / 4;
  const int lane = __lane_id();
  const uint32_t dst = tiles_lds + (c % NBUF) * TL::kBytes;
  // all row indices first: the loads are asm with a memory clobber, so an index read placed
  // between two of them would be waited for on its own
  uint32_t off[kLoadsW];
#pragma unroll
  for (int i = 0; i < kLoadsW; ++i) {
    const int pos = (4 * i + part) * 64 + lane;
    const int row = pos / TL::kChunks;
    const int chunk = (pos % TL::kChunks) ^ TL::swz(row);
    const int r = rr[row];
    off[i] = static_cast<uint32_t>(r < 0 ? 0 : r) * TL::kRowBytes + chunk * 16;  // -1: row 0
  }
#pragma unroll
  for (int i = 0; i < kLoadsW; ++i) dma16_sv(kv, off[i], dst + (4 * i + part) * 1024);
}

// Per-head operands of an SdP wave: q / dO blocks (B operands: lane -> head hl, dims ks*32 +
// g*8 + [0, 8)), and lse (base 2) / Delta of its head.
template <int DQK>
struct SdpHead {
  bf16x8 qf[DQK / 32], df[kDv / 32];
  float lse2, dlt;
  // q and dO blocks of head h from global memory, its lse, and Delta = dO . O computed from the
  // forward output (fp32 sums over the lane's eight channels of each block, then over the four
  // lane groups).
  __device__ __forceinline__ void load_delta_from_out(const uint16_t *__restrict__ q,
                                                      const uint16_t *__restrict__ dout,
                                                      const uint16_t *__restrict__ out,
                                                      const float *__restrict__ lse, int H,
                                                      int64_t t, int h) {
    const int g = __lane_id() >> 4;
    const bool hok = h < H;
#pragma unroll
    for (int ks = 0; ks < DQK / 32; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (hok) v = *reinterpret_cast<const u32x4 *>(q + ((t * H + h) * DQK + ks * 32 + g * 8));
      qf[ks] = as_bf16x8(v);
    }
    float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
    for (int ks = 0; ks < kDv / 32; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u}, o = {0u, 0u, 0u, 0u};
      if (hok) {
        v = *reinterpret_cast<const u32x4 *>(dout + ((t * H + h) * kDv + ks * 32 + g * 8));
        o = *reinterpret_cast<const u32x4 *>(out + ((t * H + h) * kDv + ks * 32 + g * 8));
      }
      df[ks] = as_bf16x8(v);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        d0 = fmaf(__uint_as_float(v[i] << 16), __uint_as_float(o[i] << 16), d0);
        d1 = fmaf(__uint_as_float(v[i] & 0xFFFF0000u), __uint_as_float(o[i] & 0xFFFF0000u), d1);
      }
    }
    float d = d0 + d1;
    d += __shfl_xor(d, 16, 64);
    d += __shfl_xor(d, 32, 64);
    dlt = d;
    const float l0 = hok ? lse[t * H + h] : -INFINITY;
    lse2 = l0 == -INFINITY ? INFINITY : l0 * kLog2e;  // empty row or padded head: P = 0
  }
  // q and dO blocks of head h from global memory
  __device__ __forceinline__ void load_q_dout(const uint16_t *__restrict__ q,
                                              const uint16_t *__restrict__ dout, int H, int64_t t,
                                              int h) {
    const int g = __lane_id() >> 4;
    const bool hok = h < H;
#pragma unroll
    for (int ks = 0; ks < DQK / 32; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (hok) v = *reinterpret_cast<const u32x4 *>(q + ((t * H + h) * DQK + ks * 32 + g * 8));
      qf[ks] = as_bf16x8(v);
    }
#pragma unroll
    for (int ks = 0; ks < kDv / 32; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (hok) v = *reinterpret_cast<const u32x4 *>(dout + ((t * H + h) * kDv + ks * 32 + g * 8));
      df[ks] = as_bf16x8(v);
    }
  }
  __device__ __forceinline__ void load_scalars(const float *__restrict__ lse,
                                               const float *__restrict__ delta, int H, int64_t t,
                                               int h) {
    const bool hok = h < H;
    const float l0 = hok ? lse[t * H + h] : -INFINITY;
    lse2 = l0 == -INFINITY ? INFINITY : l0 * kLog2e;  // empty row or padded head: P = 0
    dlt = hok ? delta[t * H + h] : 0.0f;
  }
  // q / dO blocks from a [head][stride] bf16 copy of the row in LDS
  __device__ __forceinline__ void q_from_lds(const uint16_t *rows, int stride, int h) {
    const int g = __lane_id() >> 4;
#pragma unroll
    for (int ks = 0; ks < DQK / 32; ++ks)
      qf[ks] = as_bf16x8(*reinterpret_cast<const u32x4 *>(rows + h * stride + ks * 32 + g * 8));
  }
  __device__ __forceinline__ void o_from_lds(const uint16_t *rows, int stride, int h) {
    const int g = __lane_id() >> 4;
#pragma unroll
    for (int ks = 0; ks < kDv / 32; ++ks)
      df[ks] = as_bf16x8(*reinterpret_cast<const u32x4 *>(rows + h * stride + ks * 32 + g * 8));
  }
  __device__ __forceinline__ void settle_all() {
#pragma unroll
    for (int ks = 0; ks < DQK / 32; ++ks) settle(qf[ks]);
#pragma unroll
    for (int ks = 0; ks < kDv / 32; ++ks) settle(df[ks]);
    settle(lse2);
    settle(dlt);
  }
  // P and dZ of the 32 slots of `tile` in the S^T fragment layout (slot 16 mt + 4 g + i);
  // pdp accumulates this lane's share of sum_j P_j dP_j
  __device__ __forceinline__ void grads(const unsigned char *tile, const TileFrag<DQK> &fr,
                                        const int32_t *rr, float scale_log2, float p[2][4],
                                        float dz[2][4], float &pdp) const {
    constexpr int kKS = DQK / 32;
    const int g = __lane_id() >> 4;
    f32x4 s[2][2] = {{f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}},
                     {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}}};
    f32x4 dp[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    // fragment reads run two k-steps ahead of the MFMAs
    bf16x8 a0[3], a1[3];
    a0[0] = fr.a_frag(tile, 0, 0);
    a1[0] = fr.a_frag(tile, 1, 0);
    a0[1] = fr.a_frag(tile, 0, 1);
    a1[1] = fr.a_frag(tile, 1, 1);
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      if (ks + 2 < kKS) {
        a0[(ks + 2) % 3] = fr.a_frag(tile, 0, ks + 2);
        a1[(ks + 2) % 3] = fr.a_frag(tile, 1, ks + 2);
      }
      s[0][ks & 1] = mfma16(a0[ks % 3], qf[ks], s[0][ks & 1]);
      s[1][ks & 1] = mfma16(a1[ks % 3], qf[ks], s[1][ks & 1]);
      if (ks < kDv / 32) {
        dp[0] = mfma16(a0[ks % 3], df[ks], dp[0]);
        dp[1] = mfma16(a1[ks % 3], df[ks], dp[1]);
      }
    }
    const u32x4 rv0 = *reinterpret_cast<const u32x4 *>(rr + g * 4);
    const u32x4 rv1 = *reinterpret_cast<const u32x4 *>(rr + 16 + g * 4);
    const f32x4 s0 = s[0][0] + s[0][1], s1 = s[1][0] + s[1][1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[0][i] = static_cast<int32_t>(rv0[i]) >= 0 ? __builtin_amdgcn_exp2f(s0[i] * scale_log2 - lse2) : 0.0f;
      p[1][i] = static_cast<int32_t>(rv1[i]) >= 0 ? __builtin_amdgcn_exp2f(s1[i] * scale_log2 - lse2) : 0.0f;
      dz[0][i] = p[0][i] * (dp[0][i] - dlt);
      dz[1][i] = p[1][i] * (dp[1][i] - dlt);
      pdp = fmaf(p[0][i], dp[0][i], pdp);
      pdp = fmaf(p[1][i], dp[1][i], pdp);
    }
  }
};

// ---------------------------------------------------------------------------------------
template <int DQK>
__device__ __forceinline__ void bwd_dq_row(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kv,
    const int32_t *__restrict__ idx, const int32_t *__restrict__ topk_length,
    const uint16_t *__restrict__ out, const float *__restrict__ lse, float *__restrict__ delta,
    const uint16_t *__restrict__ dout, int H, int K, float scale, float scale_log2,
    uint16_t *__restrict__ dq, int64_t t, unsigned char *smem) {
  using TL = Tile<DQK>;
  using SM = RowSmem<DQK>;
  constexpr int kNTq = DQK / 64;  // channel tiles per quarter (9 or 8)
  bf16x8 *zbuf = reinterpret_cast<bf16x8 *>(smem + SM::kDqZ);
  int32_t *ring = reinterpret_cast<int32_t *>(smem + SM::kDqRing);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, hl = lane & 15;
  const int lim = topk_length ? topk_length[t] : K;
  const int32_t *irow = idx + t * K;
  const int nchunks = (lim + kSlots - 1) / kSlots;

  if (wave < 4) {
    // ============================== SdP waves ==============================
    const int G = wave;
    SlotRing sr;  // wave 0 keeps the slot-index ring filled
    if (wave == 0) sr.start(irow, lim, nchunks, ring);
    SdpHead<DQK> hd;
    hd.load_delta_from_out(q, dout, out, lse, H, t, G * 16 + hl);
    __syncthreads();  // S0: indices of the first tiles are in the ring
    __syncthreads();  // S1: the first tiles are loaded
    hd.settle_all();  // see settle()
    TileFrag<DQK> fr;
    fr.init();
    float pdp = 0.0f;  // this lane's part of sum_j P_j dP_j for head G * 16 + hl
    for (int c = 0; c <= nchunks; ++c) {
      lds_barrier();  // B(c - 1)
      if (c == nchunks) break;
      if (wave == 0) sr.step(irow, lim, nchunks, ring, c);
      float p[2][4], dz[2][4];
      hd.grads(smem + (c % kDqBufs) * TL::kBytes, fr, ring + (c % kRing) * kSlots, scale_log2,
               p, dz, pdp);
      zbuf[((c & 1) * 4 + G) * 64 + lane] = pack_slots(dz);
    }
    // Delta of the key-gradient phase: sum_j P_j dP_j over the row's slots, equal to dO . O in
    // exact arithmetic but free of the rounding of the bf16 output (which dominates the key
    // gradient's error when many queries read one latent row)
    pdp += __shfl_xor(pdp, 16, 64);
    pdp += __shfl_xor(pdp, 32, 64);
    if (g == 0 && G * 16 + hl < H) delta[t * H + G * 16 + hl] = pdp;
    lds_barrier();  // Z
  } else {
    // ============================== dq waves ===============================
    const int qq = wave - 4;
    const uint32_t tiles_lds = lds_addr(smem);
    constexpr int kLoadsW = TL::kLoads / 4;
    __syncthreads();  // S0
    if (nchunks > 0) issue_tile<DQK, kDqBufs>(tiles_lds, kv, ring, 0, qq);
    if (nchunks > 1) issue_tile<DQK, kDqBufs>(tiles_lds, kv, ring + kSlots, 1, qq);
    if (nchunks > 0) {  // tile 0 before S1 (tile 1 may stay in flight)
      if (nchunks > 1) wait_vm<kLoadsW>();
      else wait_tile();
    }
    __syncthreads();  // S1
    ColFrags<DQK, kNTq> fr;
    fr.init(kNTq * qq);
    f32x4 acc[4][kNTq];  // acc[G][n][i] = dq[head 16 G + hl][channel 16 (kNTq qq + n) + 4 g + i]
#pragma unroll
    for (int G = 0; G < 4; ++G)
#pragma unroll
      for (int n = 0; n < kNTq; ++n) acc[G][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c <= nchunks; ++c) {
      lds_barrier();  // B(c - 1): dZ of chunk c - 1 is ready
      if (c + 2 < nchunks) issue_tile<DQK, kDqBufs>(tiles_lds, kv, ring + ((c + 2) % kRing) * kSlots, c + 2, qq);
      if (c > 0) {
        const unsigned char *tile = smem + ((c - 1) % kDqBufs) * TL::kBytes;
        bf16x8 zb[4];
#pragma unroll
        for (int G = 0; G < 4; ++G) zb[G] = zbuf[(((c - 1) & 1) * 4 + G) * 64 + lane];
#pragma unroll
        for (int n = 0; n < kNTq; ++n) {
          const bf16x8 va = fr.frag(tile, n);
#pragma unroll
          for (int G = 0; G < 4; ++G) acc[G][n] = mfma16(va, zb[G], acc[G][n]);
        }
      }
      if (c == nchunks) break;
      if (c + 2 < nchunks) wait_vm<kLoadsW>();  // tile c + 1 before the next barrier
      else wait_tile();
    }
    lds_barrier();  // Z
#pragma unroll
    for (int G = 0; G < 4; ++G) {
      const int hh = G * 16 + hl;
      if (hh < H) {
        uint16_t *row = dq + (t * H + hh) * DQK + 16 * kNTq * qq + g * 4;
#pragma unroll
        for (int n = 0; n < kNTq; ++n) {
          u32x2 v;
          v[0] = pack_bf16x2(acc[G][n][0] * scale, acc[G][n][1] * scale);
          v[1] = pack_bf16x2(acc[G][n][2] * scale, acc[G][n][3] * scale);
          *reinterpret_cast<u32x2 *>(row + n * 16) = v;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// Per-row power-of-two scales of the contribution phase's fp16 operands.  The products are
//   C = scale dZ^T . q + P^T . dO
// with P in [0, 1].  dO and q are converted to fp16 as dO' = dO 2^-gd, q' = q 2^-gq, and scale dZ
// as z' = scale dZ 2^(gq - gd), so that both products accumulate 2^-gd C in one fp32 accumulator.
// gq puts the row's largest |q| in [2^14, 2^15): bf16 -> fp16 is then exact except for elements
// more than 2^28 below it.  gd does the same for dO, raised when needed so that z' cannot leave the
// fp16 range: |dP_j| <= 512 max|dO| max|kv| and |Delta| <= max_j |dP_j|, so
// |scale dZ| <= scale 1024 max|dO| max|kv| =: bound, and 2^(gq - gd) bound <= 2^15.
struct C16Scales {
  int gq, gd;
  __device__ __forceinline__ static int expo(float x) {  // floor(log2 x) for normal x > 0
    return static_cast<int>((__float_as_uint(x) >> 23) & 0xFF) - 127;
  }
  __device__ __forceinline__ void init(uint32_t mq_bits, uint32_t md_bits, uint32_t mv_bits,
                                       float scale) {
    const float mq = bf16_to_f32(static_cast<uint16_t>(mq_bits));
    const float md = bf16_to_f32(static_cast<uint16_t>(md_bits));
    const float mv = bf16_to_f32(static_cast<uint16_t>(mv_bits));
    // bf16 subnormals have a zero exponent field: expo() then reads -127, which only makes the
    // scaled maximum smaller
    gq = mq > 0.0f ? expo(mq) - 14 : 0;
    gd = md > 0.0f ? expo(md) - 14 : 0;
    const float bound = scale * 1024.0f * md * mv;
    if (bound > 0.0f) gd = max(gd, gq + expo(fminf(bound, 3.0e38f)) + 1 - 15);
  }
};

// eight bf16 values (bit patterns) times 2^-g, as fp16 bit patterns, in place
__device__ __forceinline__ void bf16_to_f16_scaled_inplace(u32x4 &w, int g) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = pack_f16x2(ldexpf(__uint_as_float(w[i] << 16), -g),
                      ldexpf(__uint_as_float(w[i] & 0xFFFF0000u), -g));
}

// largest bf16 magnitude (bits) among the eight values of v
__device__ __forceinline__ uint32_t absmax_bits(const u32x4 &v, uint32_t m) {
#pragma unroll
  for (int i = 0; i < 4; ++i) m = max(m, max(v[i] & 0x7FFFu, (v[i] >> 16) & 0x7FFFu));
  return m;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t m) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), o, 64)));
  return m;
}

// Key-gradient contributions of query row t, stored to staged row `slot` of stage for every
// valid slot.
template <int DQK>
__device__ __forceinline__ void bwd_contrib_row(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kv,
    const int32_t *__restrict__ idx, const int32_t *__restrict__ topk_length,
    const float *__restrict__ lse, const float *__restrict__ delta,
    const uint16_t *__restrict__ dout, const uint32_t *__restrict__ vmax, int H, int K,
    float scale, float scale_log2, uint32_t *__restrict__ stage, int32_t *__restrict__ cnt,
    float *__restrict__ target, int64_t t, unsigned char *smem) {
  using TL = Tile<DQK>;
  using SM = RowSmem<DQK>;
  constexpr int kNTq = DQK / 64;  // channel tiles per quarter (9 or 8)
  uint16_t *qstage = reinterpret_cast<uint16_t *>(smem);  // prologue only
  _Float16 *stg = reinterpret_cast<_Float16 *>(smem + SM::kCStage);
  uint32_t *mx = reinterpret_cast<uint32_t *>(smem + SM::kCStage);  // prologue only
  int32_t *slot_rows = reinterpret_cast<int32_t *>(smem + SM::kCRows);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, hl = lane & 15;
  const int r = (lane & 15) >> 2, cq = lane & 3;
  const int lim = topk_length ? topk_length[t] : K;
  const int32_t *irow = idx + t * K;
  const int nchunks = (lim + kSlots - 1) / kSlots;

  // ---- prologue: the row's q, then dO, pass through LDS ([head][channel], padded heads zero)
  // as scaled fp16, from which the contribution waves read head-contraction fragments of their
  // channels; the SdP waves load their bf16 head blocks from global memory (the dq phase has
  // just read them).  The largest |q| and |dO| of the row are exchanged through LDS at P0.
  constexpr int kQV = 64 * (DQK / 8) / 512, kOV = 64 * (kDv / 8) / 512, kIV = kMaxK / 512;
  u32x4 qv[kQV], ov[kOV];
  int32_t iv[kIV];
#pragma unroll
  for (int j = 0; j < kQV; ++j) {
    const int e = threadIdx.x + j * 512, hh = e / (DQK / 8), col = (e % (DQK / 8)) * 8;
    qv[j] = u32x4{0u, 0u, 0u, 0u};
    if (hh < H) qv[j] = *reinterpret_cast<const u32x4 *>(q + (t * H + hh) * DQK + col);
  }
#pragma unroll
  for (int j = 0; j < kOV; ++j) {
    const int e = threadIdx.x + j * 512, hh = e / (kDv / 8), col = (e % (kDv / 8)) * 8;
    ov[j] = u32x4{0u, 0u, 0u, 0u};
    if (hh < H) ov[j] = *reinterpret_cast<const u32x4 *>(dout + (t * H + hh) * kDv + col);
  }
#pragma unroll
  for (int j = 0; j < kIV; ++j) {
    const int e = threadIdx.x + j * 512;
    iv[j] = e < lim ? irow[e] : -1;
  }
  const uint32_t mv_bits = *vmax;
  {
    uint32_t mq = 0u, md = 0u;
#pragma unroll
    for (int j = 0; j < kQV; ++j) mq = absmax_bits(qv[j], mq);
#pragma unroll
    for (int j = 0; j < kOV; ++j) md = absmax_bits(ov[j], md);
    mq = wave_max_u32(mq);
    md = wave_max_u32(md);
    if (lane == 0) {
      mx[wave] = mq;
      mx[8 + wave] = md;
    }
  }
  __syncthreads();  // P0: the maxima are exchanged
  C16Scales sc16;
  {
    uint32_t mq = 0u, md = 0u;
#pragma unroll
    for (int w = 0; w < kRowWaves; ++w) {
      mq = max(mq, mx[w]);
      md = max(md, mx[8 + w]);
    }
    sc16.init(mq, md, mv_bits, scale);
  }
#pragma unroll
  for (int j = 0; j < kQV; ++j) {
    const int e = threadIdx.x + j * 512, hh = e / (DQK / 8), col = (e % (DQK / 8)) * 8;
    bf16_to_f16_scaled_inplace(qv[j], sc16.gq);
    *reinterpret_cast<u32x4 *>(&qstage[hh * SM::kQStride + col]) = qv[j];
  }
  // dO and the slot rows (up to a whole number of tiles; the list lies outside the staging area);
  // each valid slot also counts one contribution for its latent row (the counting sort's first
  // step: the atomics need no result and complete while the phase runs)
  auto store_o_rows = [&]() {
#pragma unroll
    for (int j = 0; j < kOV; ++j) {
      const int e = threadIdx.x + j * 512, hh = e / (kDv / 8), col = (e % (kDv / 8)) * 8;
      bf16_to_f16_scaled_inplace(ov[j], sc16.gd);
      *reinterpret_cast<u32x4 *>(&qstage[hh * SM::kOStride + col]) = ov[j];
    }
#pragma unroll
    for (int j = 0; j < kIV; ++j) {
      const int e = threadIdx.x + j * 512;
      if (e < nchunks * kSlots) slot_rows[e] = iv[j];
      if (iv[j] >= 0) atomicAdd(&cnt[iv[j]], 1);  // iv is -1 beyond the valid prefix
    }
  };

  // The two roles are separate branches from here on (their register sets never overlap).
  if (wave < 4) {
    // ============================== SdP waves ==============================
    const int G = wave;
    const int h = G * 16 + hl;
    SdpHead<DQK> hd;
    hd.load_scalars(lse, delta, H, t, h);
    __syncthreads();  // P1: q (fp16) is staged
    hd.load_q_dout(q, dout, H, t, h);
    __syncthreads();  // P2: the contribution waves have read q
    store_o_rows();
    __syncthreads();  // P3: dO (fp16) is staged
    __syncthreads();  // P4: the staging is read (the tile area is free)
    const uint32_t tiles_lds = lds_addr(smem);
    constexpr int kLoadsW = TL::kLoads / 4;
    hd.settle_all();  // before the first tile load (see settle())
    if (nchunks > 0) issue_tile<DQK, kCBufs>(tiles_lds, kv, slot_rows, 0, G);
    if (nchunks > 1) issue_tile<DQK, kCBufs>(tiles_lds, kv, slot_rows + kSlots, 1, G);
    if (nchunks > 0) {
      if (nchunks > 1) wait_vm<kLoadsW>();
      else wait_tile();
    }
    __syncthreads();  // S1: tile 0 loaded
    TileFrag<DQK> fr;
    fr.init();
    const int zexp = sc16.gq - sc16.gd;  // z' = scale dZ 2^zexp
    for (int c = 0; c <= nchunks; ++c) {
      lds_barrier();  // B(c - 1): tile c complete; contribution waves are done with chunk c - 2
      if (c == nchunks) break;
      if (c + 2 < nchunks)  // into tile c - 1's buffer
        issue_tile<DQK, kCBufs>(tiles_lds, kv, slot_rows + (c + 2) * kSlots, c + 2, G);
      float p[2][4], dz[2][4], pdp = 0.0f;
      hd.grads(smem + (c % kCBufs) * TL::kBytes, fr, slot_rows + c * kSlots, scale_log2, p, dz,
               pdp);
      _Float16 *zs = stg + (c & 1) * (SM::kCStageBytes / 2);
      _Float16 *ps = zs + kSlots * kSS;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int o = (mt * 16 + g * 4 + i) * kSS + h;
          zs[o] = static_cast<_Float16>(ldexpf(dz[mt][i] * scale, zexp));
          ps[o] = static_cast<_Float16>(p[mt][i]);
        }
      if (c + 2 < nchunks) wait_vm<kLoadsW>();  // tile c + 1 before the next barrier
      else wait_tile();
    }
    lds_barrier();  // Z
  } else {
    // ========================== contribution waves =========================
    const int qq = wave - 4;
    float tgt_total = 0.0f;  // wave 0 of this role: the row's KL-target sum (lanes < 32)
    const int ch0 = qq * 16 * kNTq;
    // head-contraction fragments of the scaled fp16 q' and dO'
    u32x4 qh[2][kNTq], oh[2][kNTq];
    __syncthreads();  // P1
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int n = 0; n < kNTq; ++n) {
        const uint16_t *base = &qstage[(kh * 32 + g * 8 + r) * SM::kQStride + ch0 + n * 16 + cq * 4];
        const u32x2 lo = lds_read_tr16(base);
        const u32x2 hi = lds_read_tr16(base + 4 * SM::kQStride);
        qh[kh][n] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
    __syncthreads();  // P2: q is read (dO overwrites it)
    store_o_rows();
    __syncthreads();  // P3
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int n = 0; n < kNTq; ++n) {
        const int ch = ch0 + n * 16;
        oh[kh][n] = u32x4{0u, 0u, 0u, 0u};
        if (ch < kDv) {
          const uint16_t *base = &qstage[(kh * 32 + g * 8 + r) * SM::kOStride + ch + cq * 4];
          const u32x2 lo = lds_read_tr16(base);
          const u32x2 hi = lds_read_tr16(base + 4 * SM::kOStride);
          oh[kh][n] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
      }
    __syncthreads();  // P4
    __syncthreads();  // S1
    for (int c = 0; c <= nchunks; ++c) {
      lds_barrier();  // B(c - 1): P / dZ of chunk c - 1 are staged
      if (c > 0) {
        const int cc = c - 1;
        const _Float16 *zs = stg + (cc & 1) * (SM::kCStageBytes / 2);
        const _Float16 *ps = zs + kSlots * kSS;
        const int32_t *rr = slot_rows + cc * kSlots;
        if (target && qq == 0 && lane < kSlots) {
          // KL-loss target: head sum of the staged P of slot cc*32 + lane (unnormalised here,
          // renormalised over the row at the end; invalid slots hold P = 0)
          const int j = cc * kSlots + lane;
          float v = 0.0f;
#pragma unroll
          for (int b = 0; b < 8; ++b) {
            const f16x8 pv = as_f16x8(*reinterpret_cast<const u32x4 *>(&ps[lane * kSS + 8 * b]));
#pragma unroll
            for (int e = 0; e < 8; ++e) v += static_cast<float>(pv[e]);
          }
          if (j < K) target[t * K + j] = v;
          tgt_total += v;
        }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          f32x4 acc[kNTq];
#pragma unroll
          for (int n = 0; n < kNTq; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kh = 0; kh < 2; ++kh) {
            const int off = (mt * 16 + hl) * kSS + kh * 32 + g * 8;
            const f16x8 za = as_f16x8(*reinterpret_cast<const u32x4 *>(&zs[off]));
            const f16x8 pa = as_f16x8(*reinterpret_cast<const u32x4 *>(&ps[off]));
            // 2^-gd C^T = q'^T . z' + dO'^T . P: the head-contraction fragments serve as the A
            // operand (rows = channels) and the staged [slot][head] fragments as B (columns =
            // slots), so that each lane ends with four consecutive channels of one slot.  Two
            // passes over the channel tiles keep consecutive MFMAs independent (the dO fragments
            // of RoPE channels are zero; skipping them would need a branch per MFMA).
#pragma unroll
            for (int n = 0; n < kNTq; ++n) acc[n] = mfma16h(as_f16x8(qh[kh][n]), za, acc[n]);
#pragma unroll
            for (int n = 0; n < kNTq; ++n) acc[n] = mfma16h(as_f16x8(oh[kh][n]), pa, acc[n]);
          }
          // C = acc 2^gd, channels ch0 + 16n + 4g .. + 3 of staged row cc*32 + 16mt + hl: one
          // block per lane (valid slots only).  The mantissas are those of acc against its own
          // block exponent; the factor 2^gd only moves the stored exponent.
          if (rr[mt * 16 + hl] >= 0) {
            float mxa = 0.0f;
#pragma unroll
            for (int n = 0; n < kNTq; ++n)
#pragma unroll
              for (int i = 0; i < 4; ++i) mxa = fmaxf(mxa, fabsf(acc[n][i]));
            const int ea = static_cast<int>(min(__float_as_uint(mxa) >> 23, 253u));
            const int ec = ea + sc16.gd;  // exponent field of the block's largest |C|
            const uint32_t eb = static_cast<uint32_t>(min(max(ec, 0), 253));
            // 2^-e of acc; a block below the smallest normal fp32 is stored as zero
            const float sc = ec >= 0 ? __uint_as_float(static_cast<uint32_t>(253 - ea) << 23) : 0.0f;
            uint32_t *row =
                stage + static_cast<int64_t>(cc * kSlots + mt * 16 + hl) * kStageWords<DQK>;
            uint32_t *mrow = row + ((ch0 + 4 * g) >> 1);  // channel tile n at word 8 n
            // plain stores: the L2 merges the pieces of a row into whole lines (written with the
            // non-temporal hint the pieces reach HBM separately, at about half the rate)
#pragma unroll
            for (int n = 0; n < kNTq; ++n) {
              u32x2 v;
              v[0] = pknorm16(acc[n][0] * sc, acc[n][1] * sc);
              v[1] = pknorm16(acc[n][2] * sc, acc[n][3] * sc);
              *reinterpret_cast<u32x2 *>(mrow + 8 * n) = v;
            }
            reinterpret_cast<unsigned char *>(row + DQK / 2)[4 * qq + g] =
                static_cast<unsigned char>(eb);
          }
        }
      }
      if (c == nchunks) break;
    }
    lds_barrier();  // Z
    if (target && qq == 0) {
      // renormalise the row's target over its slots (each lane rereads what it wrote) and
      // zero the slots past the last chunk
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) tgt_total += __shfl_xor(tgt_total, o, 64);
      const float inv = tgt_total > 0.0f ? 1.0f / tgt_total : 0.0f;
      float *trow = target + t * K;
      if (lane < kSlots)
        for (int j = lane; j < nchunks * kSlots && j < K; j += kSlots) trow[j] *= inv;
      for (int j = nchunks * kSlots + lane; j < K; j += 64) trow[j] = 0.0f;
    }
  }
}

// Largest |kv| over n bf16 values (n a multiple of 8), as bf16 magnitude bits, into *out (which
// holds 0 before the launch).
__global__ __launch_bounds__(256) void kv_absmax_kernel(const uint16_t *__restrict__ kv, int64_t n8,
                                                        uint32_t *__restrict__ out) {
  uint32_t m = 0u;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n8;
       i += stride)
    m = absmax_bits(*reinterpret_cast<const u32x4 *>(kv + 8 * i), m);
  m = wave_max_u32(m);
  if ((threadIdx.x & 63) == 0 && m > 0u) atomicMax(out, m);
}

__global__ void check_indices_kernel(const int32_t *__restrict__ idx,
                                     const int32_t *__restrict__ topk_length, int64_t T_q, int K,
                                     int64_t T_kv, int32_t *__restrict__ bad) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= T_q * K) return;
  const int64_t t = i / K;
  const int j = static_cast<int>(i % K);
  const int lim = topk_length ? topk_length[t] : K;
  if (topk_length && (lim < 0 || lim > K)) {
    atomicOr(bad, 1);
    return;
  }
  const int32_t v = idx[i];
  if (j < lim && v != -1 && (v < 0 || v >= T_kv)) atomicOr(bad, 1);
}

// ---------------------------------------------------------------------------------------
template <int DQK>
__global__ __launch_bounds__(kRowWaves * 64) void bwd_rows_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kv,
    const int32_t *__restrict__ idx, const int32_t *__restrict__ topk_length,
    const uint16_t *__restrict__ out, const float *__restrict__ lse, float *__restrict__ delta,
    const uint16_t *__restrict__ dout, const uint32_t *__restrict__ vmax, int H, int K,
    float scale, float scale_log2, uint16_t *__restrict__ dq, uint32_t *__restrict__ stage,
    int32_t *__restrict__ cnt, float *__restrict__ target, int64_t row0) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int64_t i = blockIdx.x;
  const int64_t t = row0 + i;
  bwd_dq_row<DQK>(q, kv, idx, topk_length, out, lse, delta, dout, H, K, scale, scale_log2, dq,
                  t, smem);
  __syncthreads();  // every wave is done with the dq phase's LDS; the row's Delta is stored
  bwd_contrib_row<DQK>(q, kv, idx, topk_length, lse, delta, dout, vmax, H, K, scale, scale_log2,
                       stage + i * K * kStageWords<DQK>, cnt, target, t, smem);
}

// ---------------------------------------------------------------------------------------
// counting sort of the pass's (query, slot) pairs by latent row.  Pair p = (t - row0) * K + j.
__device__ __forceinline__ bool pair_row(const int32_t *__restrict__ idx,
                                         const int32_t *__restrict__ topk_length, int64_t row0,
                                         int64_t rows, int K, int64_t p, int32_t &s) {
  if (p >= rows * K) return false;
  const int64_t t = row0 + p / K;
  const int j = static_cast<int>(p % K);
  const int lim = topk_length ? topk_length[t] : K;
  s = idx[t * K + j];
  return j < lim && s >= 0;
}

__global__ void fill_zero_i32_kernel(int32_t *__restrict__ p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t j = i; j < n; j += stride) p[j] = 0;
}

// Exclusive scan of cnt[0, n) in place (cnt[n] receives the total) and cursor = the scan.
// One work group of 1024 threads; thread i scans a contiguous run of ceil(n / 1024) entries.
constexpr int kScanThreads = 1024;
__global__ __launch_bounds__(kScanThreads) void pair_scan_kernel(int32_t *__restrict__ cnt,
                                                                  int32_t *__restrict__ cursor,
                                                                  int64_t n) {
  __shared__ int32_t part[kScanThreads];
  const int tid = threadIdx.x;
  const int64_t per = (n + kScanThreads - 1) / kScanThreads;
  const int64_t b = tid * per, e = b + per < n ? b + per : n;
  int32_t sum = 0;
  for (int64_t i = b; i < e; ++i) sum += cnt[i];
  part[tid] = sum;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {  // Hillis-Steele inclusive scan
    const int32_t v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int32_t run = part[tid] - sum;
  for (int64_t i = b; i < e; ++i) {
    const int32_t c = cnt[i];
    cnt[i] = run;
    cursor[i] = run;
    run += c;
  }
  if (tid == kScanThreads - 1) cnt[n] = part[tid];
}

__global__ void pair_fill_kernel(const int32_t *__restrict__ idx,
                                 const int32_t *__restrict__ topk_length, int64_t row0,
                                 int64_t rows, int K, int32_t *__restrict__ cursor,
                                 int32_t *__restrict__ list) {
  const int64_t p = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  int32_t s;
  if (pair_row(idx, topk_length, row0, rows, K, p, s))
    list[atomicAdd(&cursor[s], 1)] = static_cast<int32_t>(p);
}

// dkv[s] += sum of the staged contributions of latent row s.  One wave per row; lane l owns
// the 16-byte pieces l + 64 c of a staged row (channels 8 (l + 64 c) .. + 7: two blocks, whose
// exponent bytes are adjacent), and four staged rows are in flight per step.
template <int DQK>
__global__ __launch_bounds__(256) void pair_reduce_kernel(const int32_t *__restrict__ off,
                                                          const int32_t *__restrict__ list,
                                                          const uint32_t *__restrict__ stage,
                                                          int64_t n_rows, float *__restrict__ dkv) {
  constexpr int kPieces = DQK / 8;           // 16-byte pieces per staged row (72 or 64)
  constexpr int kVec = (kPieces + 63) / 64;  // pieces per lane (2 or 1)
  constexpr int kW = kStageWords<DQK>;
  constexpr int kFly = 4;
  const int lane = threadIdx.x & 63;
  const int64_t s = static_cast<int64_t>(blockIdx.x) * 4 +
                    __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  if (s >= n_rows) return;
  const int b = off[s], e = off[s + 1];
  if (b == e) return;
  bool has[kVec];
  int eoff[kVec];  // byte offset of the piece's exponent pair (even)
#pragma unroll
  for (int c = 0; c < kVec; ++c) {
    has[c] = lane + 64 * c < kPieces;
    eoff[c] = DQK * 2 + stage_exp_byte<DQK>(8 * (lane + 64 * c));
  }
  f32x4 acc[kVec][2];
#pragma unroll
  for (int c = 0; c < kVec; ++c) acc[c][0] = acc[c][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto load = [&](int32_t pair, u32x4 (&m)[kVec], uint32_t (&ex)[kVec]) {
    const uint32_t *r = stage + static_cast<int64_t>(pair) * kW;
#pragma unroll
    for (int c = 0; c < kVec; ++c) {
      m[c] = u32x4{0u, 0u, 0u, 0u};
      ex[c] = 0u;
      if (has[c]) {
        m[c] = *reinterpret_cast<const u32x4 *>(r + 4 * (lane + 64 * c));
        ex[c] = *reinterpret_cast<const uint16_t *>(reinterpret_cast<const unsigned char *>(r) +
                                                     eoff[c]);
      }
    }
  };
  auto add = [&](const u32x4 (&m)[kVec], const uint32_t (&ex)[kVec]) {
#pragma unroll
    for (int c = 0; c < kVec; ++c) {
      acc[c][0] += unpack_m16x4(u32x2{m[c][0], m[c][1]}, stage_factor(ex[c] & 0xFFu));
      acc[c][1] += unpack_m16x4(u32x2{m[c][2], m[c][3]}, stage_factor(ex[c] >> 8));
    }
  };
  int k = b;
  for (; k + kFly <= e; k += kFly) {
    int32_t pr[kFly];  // one scalar load
#pragma unroll
    for (int i = 0; i < kFly; ++i) pr[i] = list[k + i];
    u32x4 m[kFly][kVec];
    uint32_t ex[kFly][kVec];
#pragma unroll
    for (int i = 0; i < kFly; ++i) load(pr[i], m[i], ex[i]);
#pragma unroll
    for (int i = 0; i < kFly; ++i) add(m[i], ex[i]);
  }
  for (; k < e; ++k) {
    u32x4 m[kVec];
    uint32_t ex[kVec];
    load(list[k], m, ex);
    add(m, ex);
  }
  float *d = dkv + s * DQK;
#pragma unroll
  for (int c = 0; c < kVec; ++c) {
    if (!has[c]) continue;
    f32x4 *dst = reinterpret_cast<f32x4 *>(d + 8 * (lane + 64 * c));
    dst[0] += acc[c][0];
    dst[1] += acc[c][1];
  }
}

template <int DQK>
hipError_t launch_rows(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                       const int32_t *topk_length, const uint16_t *out, const float *lse,
                       float *delta, const uint16_t *dout, const uint32_t *vmax, int64_t row0,
                       int64_t rows, int32_t H, int32_t K, float scale, uint16_t *dq,
                       float *target, const BwdPassBuffers &bb, hipStream_t s) {
  const size_t smem = RowSmem<DQK>::bytes(K);
  auto kern = bwd_rows_kernel<DQK>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(smem));
  if (e != hipSuccess) return e;
  DSA_LAUNCH("sparse_mla_bwd_rows", kern, dim3(static_cast<unsigned>(rows)),
             dim3(kRowWaves * 64), smem, s, q, kv, idx, topk_length, out, lse, delta, dout, vmax,
             H, K, scale, scale * kLog2e, dq, bb.stage, bb.off, target, row0);
  return hipGetLastError();
}

// Counting sort of pass [row0, row0 + rows) into buffer bb: the counts are cleared before the
// rows launch (launch_count_zero), which counts each latent row's contributions; the scan and
// the fill of the pair list follow it (launch_sort).
// Kernel names for the benchmark's event hooks: the attention backward's, or the indexer
// loss's (same kernels on its own pass buffers).
struct SortNames {
  const char *zero, *scan, *fill, *reduce;
};
constexpr SortNames kBwdNames = {"pair_zero", "pair_scan", "pair_fill", "sparse_mla_bwd_reduce"};
constexpr SortNames kKlNames = {"kl_pair_zero", "kl_pair_scan", "kl_pair_fill",
                                "indexer_kl_reduce"};

hipError_t launch_count_zero(int64_t T_kv, const BwdPassBuffers &bb, hipStream_t s,
                             const SortNames &nm = kBwdNames) {
  const unsigned zb = static_cast<unsigned>(std::min<int64_t>((T_kv + 256) / 256, 65536));
  DSA_LAUNCH(nm.zero, fill_zero_i32_kernel, dim3(zb), dim3(256), 0, s, bb.off, T_kv + 1);
  return hipGetLastError();
}

hipError_t launch_sort(const int32_t *idx, const int32_t *topk_length, int64_t row0,
                       int64_t rows, int64_t T_kv, int32_t K, const BwdPassBuffers &bb,
                       hipStream_t s, const SortNames &nm = kBwdNames) {
  const int64_t pairs = rows * K;
  const unsigned pb = static_cast<unsigned>((pairs + 255) / 256);
  DSA_LAUNCH(nm.scan, pair_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, bb.off, bb.cursor,
             T_kv);
  DSA_LAUNCH(nm.fill, pair_fill_kernel, dim3(pb), dim3(256), 0, s, idx, topk_length, row0, rows,
             K, bb.cursor, bb.list);
  return hipGetLastError();
}

template <int DQK>
hipError_t launch_reduce(int64_t T_kv, const BwdPassBuffers &bb, float *dkv, hipStream_t s,
                         const SortNames &nm = kBwdNames) {
  DSA_LAUNCH(nm.reduce, pair_reduce_kernel<DQK>, dim3(static_cast<unsigned>((T_kv + 3) / 4)),
             dim3(256), 0, s, bb.off, bb.list, bb.stage, T_kv, dkv);
  return hipGetLastError();
}

// Helper stream and events of the calling thread on the current device: created on first use
// and kept until the process ends (they hold none of the caller's memory).
struct BwdStreams {
  hipStream_t s2 = nullptr;
  hipEvent_t fork = nullptr, join = nullptr, rows_done[2] = {nullptr, nullptr},
             red_done[2] = {nullptr, nullptr};
};
hipError_t bwd_streams(BwdStreams *&out) {
  thread_local BwdStreams per_dev[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  BwdStreams &b = per_dev[dev];
  if (!b.s2) {
    hipEvent_t *evs[6] = {&b.fork, &b.join, &b.rows_done[0], &b.rows_done[1], &b.red_done[0],
                          &b.red_done[1]};
    for (hipEvent_t *ev : evs)
      if ((e = hipEventCreateWithFlags(ev, hipEventDisableTiming)) != hipSuccess) return e;
    if ((e = hipStreamCreateWithFlags(&b.s2, hipStreamNonBlocking)) != hipSuccess) return e;
  }
  out = &b;
  return hipSuccess;
}

template <int DQK>
hipError_t launch_passes(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                         const int32_t *topk_length, const uint16_t *out, const float *lse,
                         float *delta,
                         const uint16_t *dout, int64_t T_q, int64_t T_kv, int32_t H, int32_t K,
                         float scale, uint16_t *dq, float *dkv, float *target,
                         const BwdWorkspace &ws, hipStream_t s) {
  hipError_t e = hipSuccess;
  const int64_t R = ws.rows_per_pass;
  if (ws.nbuf == 1) {  // every pass in order on the caller's stream
    for (int64_t r0 = 0; e == hipSuccess && r0 < T_q; r0 += R) {
      const int64_t n = std::min<int64_t>(R, T_q - r0);
      e = launch_count_zero(T_kv, ws.buf[0], s);
      if (e == hipSuccess)
        e = launch_rows<DQK>(q, kv, idx, topk_length, out, lse, delta, dout, ws.vmax, r0, n, H,
                             K, scale, dq, target, ws.buf[0], s);
      if (e == hipSuccess) e = launch_sort(idx, topk_length, r0, n, T_kv, K, ws.buf[0], s);
      if (e == hipSuccess) e = launch_reduce<DQK>(T_kv, ws.buf[0], dkv, s);
    }
    return e;
  }
  // Two buffers: pass p clears its counts and computes (rows launch) on the caller's stream into
  // buffer p % 2; once the rows launch has finished, the scan, the list fill and the reduction
  // run on the helper stream while the caller's stream goes on with pass p + 1.  Pass p + 2 reuses the
  // buffer after pass p's reduction.  The helper stream forks from the caller's stream first
  // (so that it also joins a stream capture) and the caller's stream joins it at the end.
  BwdStreams *bs = nullptr;
  if ((e = bwd_streams(bs)) != hipSuccess) return e;
  if ((e = hipEventRecord(bs->fork, s)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(bs->s2, bs->fork, 0)) != hipSuccess) return e;
  int p = 0;
  for (int64_t r0 = 0; e == hipSuccess && r0 < T_q; r0 += R, ++p) {
    const int64_t n = std::min<int64_t>(R, T_q - r0);
    const int b = p & 1;
    if (p >= 2 && (e = hipStreamWaitEvent(s, bs->red_done[b], 0)) != hipSuccess) break;
    e = launch_count_zero(T_kv, ws.buf[b], s);
    if (e == hipSuccess)
      e = launch_rows<DQK>(q, kv, idx, topk_length, out, lse, delta, dout, ws.vmax, r0, n, H, K,
                           scale, dq, target, ws.buf[b], s);
    if (e == hipSuccess) e = hipEventRecord(bs->rows_done[b], s);
    if (e == hipSuccess) e = hipStreamWaitEvent(bs->s2, bs->rows_done[b], 0);
    if (e == hipSuccess) e = launch_sort(idx, topk_length, r0, n, T_kv, K, ws.buf[b], bs->s2);
    if (e == hipSuccess) e = launch_reduce<DQK>(T_kv, ws.buf[b], dkv, bs->s2);
    if (e == hipSuccess) e = hipEventRecord(bs->red_done[b], bs->s2);
  }
  // join (after an error too, so that no work is left unordered behind the caller's stream)
  hipError_t j = hipEventRecord(bs->join, bs->s2);
  if (j == hipSuccess) j = hipStreamWaitEvent(s, bs->join, 0);
  return e != hipSuccess ? e : j;
}

}  // namespace

hipError_t launch_sparse_mla_bwd(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                                 const int32_t *topk_length, const uint16_t *out,
                                 const float *lse, const uint16_t *dout, int64_t T_q,
                                 int64_t T_kv, int32_t H, int32_t D_qk, int32_t K, float scale,
                                 uint16_t *dq, float *dkv, bool accumulate,
                                 const BwdWorkspace &ws, hipStream_t s, float *target) {
  if (!accumulate && T_kv > 0) {
    const int64_t n = T_kv * D_qk;
    const int64_t blocks = (n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536;
    DSA_LAUNCH("dkv_zero", fill_zero_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                       dkv, n);
  }
  if (T_q == 0) return hipGetLastError();
  // largest |kv|, for the scales of the contribution phase's fp16 operands
  DSA_LAUNCH("kv_absmax_zero", fill_zero_i32_kernel, dim3(1), dim3(64), 0, s,
             reinterpret_cast<int32_t *>(ws.vmax), static_cast<int64_t>(1));
  {
    const int64_t n8 = T_kv * D_qk / 8;
    const int64_t blocks = std::min<int64_t>((n8 + 255) / 256, 2048);
    DSA_LAUNCH("kv_absmax", kv_absmax_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
               s, kv, n8, ws.vmax);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (D_qk == 576)
    return launch_passes<576>(q, kv, idx, topk_length, out, lse, ws.delta, dout, T_q, T_kv, H,
                              K, scale, dq, dkv, target, ws, s);
  if (D_qk == 512)
    return launch_passes<512>(q, kv, idx, topk_length, out, lse, ws.delta, dout, T_q, T_kv, H,
                              K, scale, dq, dkv, target, ws, s);
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------------------
// Scratch of the allocation-free backward (dsa_sparse_mla_bwd_noalloc): a fixed array in the
// code object, of which every GPU that loads the library holds its own copy until the process
// ends.  Host code never uses the array's name as an address: its device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void **ptr) {
  static std::mutex mu;
  static void *per_dev[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!per_dev[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    per_dev[dev] = p;
  }
  *ptr = per_dev[dev];
  return hipSuccess;
}

hipError_t launch_pair_count_zero(int64_t n_rows, const BwdPassBuffers &bb, hipStream_t s) {
  return launch_count_zero(n_rows, bb, s, kKlNames);
}

hipError_t launch_pair_sort(const int32_t *idx, const int32_t *topk_length, int64_t row0,
                            int64_t rows, int64_t n_rows, int32_t K, const BwdPassBuffers &bb,
                            hipStream_t s) {
  return launch_sort(idx, topk_length, row0, rows, n_rows, K, bb, s, kKlNames);
}

hipError_t launch_pair_reduce(int32_t D, int64_t n_rows, const BwdPassBuffers &bb, float *dst,
                              hipStream_t s) {
  if (D == 128) return launch_reduce<128>(n_rows, bb, dst, s, kKlNames);
  return hipErrorInvalidValue;
}

hipError_t launch_fill_zero(float *p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536;
  DSA_LAUNCH("kl_dk_zero", fill_zero_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
             p, n);
  return hipGetLastError();
}

hipError_t launch_check_indices(const int32_t *idx, const int32_t *topk_length, int64_t T_q,
                                int32_t K, int64_t T_kv, int32_t *bad_flag, hipStream_t s) {
  DSA_LAUNCH("flag_zero", fill_zero_kernel, dim3(1), dim3(64), 0, s, reinterpret_cast<float *>(bad_flag),
                     static_cast<int64_t>(1));
  const int64_t n = T_q * K;
  if (n == 0) return hipGetLastError();
  DSA_LAUNCH("check_indices", check_indices_kernel, dim3(static_cast<unsigned>((n + 255) / 256)),
                     dim3(256), 0, s, idx, topk_length, T_q, K, T_kv, bad_flag);
  return hipGetLastError();
}

}  // namespace dsa
