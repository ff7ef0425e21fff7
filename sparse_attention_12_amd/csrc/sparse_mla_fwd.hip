// Absorbed sparse MLA forward (NVIDIA GLM-5.2 cuDNN DSA page, "Why DSA needs fused kernels":
// all heads of a query attend one top-k set, so the MMA M axis is tiled from heads in an
// MQA-style layout; NeMo AutoModel cudnn_dsa API reference, cudnn_sparse_attention: q
// [T_q,H,576], latent rows [T_kv,576], values = first 512 channels, -1 slots masked, optional
// valid-prefix lengths, softmax_scale applied unchanged; SkyRL PR 2388 for the 512-wide NoPE
// layout and top-k widths that are not a multiple of 64).
//
// Up to 32 heads: work group = one query row, NW waves (1 for H <= 16, 2 for H <= 32), wave w
// owning HG = 1 group of 16 heads.  (33..64 heads use the role-split kernel further down.)
// The row's valid slots are processed in
// chunks of 32: the 32 latent rows are gathered into LDS with direct 16-byte loads (two
// buffers; two work groups share a CU so one computes while the other waits), then each wave
// computes, per head group,
//   S^T[32 slots x 16 heads] = rows . q^T          (16x16x32 bf16 MFMA, A = LDS rows,
//                                                   B = the wave's q block held in registers)
// runs the online softmax in fp32 (base 2), and accumulates
//   O^T[512 x 16 heads] += V^T . P^T                (A = V^T from transposing LDS reads of the
//                                                   same row tile, B = P straight from the S^T
//                                                   registers)
// The slot order inside the P.V contraction is permuted so that P needs no data movement: the
// lane holding S^T rows (lane/16)*4 + [0,4) of both 16-slot halves supplies exactly the eight
// contraction indices it owns in the MFMA B layout, and the transposing reads fetch V rows in
// the same order.  The output accumulators (HG x 128 per lane) stay in registers.
#include "dsa_common.h"
#include "dsa_internal.h"
#include "tile.h"

namespace dsa {
namespace {

constexpr int kSlots = 32;  // slots per chunk
constexpr int kDv = 512;
constexpr int kNBuf = 2;    // latent-row tile buffers per work group

template <int DQK, int SLOTCAP>
constexpr size_t fwd_smem_bytes() {
  return static_cast<size_t>(kNBuf) * Tile<DQK>::kBytes + SLOTCAP * sizeof(int32_t);
}

template <int DQK, int NW, int HG, int SLOTCAP>
__global__ __launch_bounds__(NW * 64) void sparse_mla_fwd_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kv,
    const int32_t *__restrict__ idx, const int32_t *__restrict__ topk_length, int H, int K,
    float scale_log2, uint16_t *__restrict__ out, float *__restrict__ lse) {
  using TL = Tile<DQK>;
  constexpr int kKSteps = DQK / 32;
  constexpr int kNT = kDv / 16;  // output tiles of 16 channels
  static_assert(TL::kLoads % NW == 0, "tile loads must split evenly over the waves");
  extern __shared__ __align__(16) unsigned char smem[];
  int32_t *slot_rows = reinterpret_cast<int32_t *>(smem + kNBuf * TL::kBytes);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t t = blockIdx.x;
  const int g = lane >> 4;   // lane group
  const int hl = lane & 15;  // head within a 16-head group
  const int lim = topk_length ? topk_length[t] : K;
  const int32_t *irow = idx + t * K;
  const int nchunks = (lim + kSlots - 1) / kSlots;

  // q blocks of this wave's head groups as MFMA B operands: lane -> head hl of group hg,
  // dims ks*32 + g*8 + [0,8)
  bf16x8 qf[HG][kKSteps];
#pragma unroll
  for (int hg = 0; hg < HG; ++hg) {
    const int h = (wave * HG + hg) * 16 + hl;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (h < H) v = *reinterpret_cast<const u32x4 *>(q + ((t * H + h) * DQK + ks * 32 + g * 8));
      qf[hg][ks] = as_bf16x8(v);
    }
  }
  // the query's slot -> latent row map (tail of the last chunk marked invalid)
  for (int j = threadIdx.x; j < nchunks * kSlots; j += NW * 64)
    slot_rows[j] = j < lim ? irow[j] : -1;
  // finish the q loads before the first tile load (see settle())
#pragma unroll
  for (int hg = 0; hg < HG; ++hg)
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) settle(qf[hg][ks]);
  __syncthreads();

  TileFrag<DQK> fr;
  fr.init();
  const uint32_t tiles_lds = lds_addr(smem);
  // this wave's DMA loads of tile c: load k (k = wave, wave + NW, ...) fills LDS bytes
  // [1024 k, 1024 k + 1024) of the tile, lane i the 16 bytes at 1024 k + 16 i
  auto issue = [&](int c) {
    const uint32_t dst = tiles_lds + (c % kNBuf) * TL::kBytes;
    uint32_t off[TL::kLoads / NW];  // row indices first (see the other kernel)
#pragma unroll
    for (int i = 0; i < TL::kLoads / NW; ++i) {
      const int pos = (i * NW + wave) * 64 + lane;
      const int row = pos / TL::kChunks;
      const int chunk = (pos % TL::kChunks) ^ TL::swz(row);
      const int r = slot_rows[c * kSlots + row];
      off[i] = static_cast<uint32_t>(r < 0 ? 0 : r) * TL::kRowBytes + chunk * 16;  // -1: row 0
    }
#pragma unroll
    for (int i = 0; i < TL::kLoads / NW; ++i) dma16_sv(kv, off[i], dst + (i * NW + wave) * 1024);
  };
  if (nchunks > 0) issue(0);

  f32x4 o[HG][kNT];  // O^T tiles: o[hg][n][i] = O[head hl of group hg][channel 16n + 4g + i]
#pragma unroll
  for (int hg = 0; hg < HG; ++hg)
#pragma unroll
    for (int n = 0; n < kNT; ++n) o[hg][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  // reference max (base-2 logits) per head; a finite floor keeps exp2(x - m_run) = 0 for
  // masked slots (x = -inf) even before the first valid slot
  float m_run[HG], l_run[HG];
#pragma unroll
  for (int hg = 0; hg < HG; ++hg) {
    m_run[hg] = -1e30f;
    l_run[hg] = 0.0f;  // this lane's partial softmax denominator of its head
  }

  for (int c = 0; c < nchunks; ++c) {
    wait_tile();    // this wave's loads of tile c (the only ones in flight)
    lds_barrier();  // tile c is complete in LDS; every wave is done with tile c - 1
    if (c + 1 < nchunks) issue(c + 1);
    const unsigned char *tile = smem + (c % kNBuf) * TL::kBytes;

    // ---- S^T = rows . q^T   (acc[hg][mt][i] = S^T[slot 16mt + 4g + i][head hl of group hg])
    f32x4 acc[HG][2];
#pragma unroll
    for (int hg = 0; hg < HG; ++hg) acc[hg][0] = acc[hg][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      const bf16x8 a0 = fr.a_frag(tile, 0, ks), a1 = fr.a_frag(tile, 1, ks);
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) {
        acc[hg][0] = mfma16(a0, qf[hg][ks], acc[hg][0]);
        acc[hg][1] = mfma16(a1, qf[hg][ks], acc[hg][1]);
      }
    }

    // ---- online softmax (base 2) with a lazily raised reference max: the reference only
    // moves when the running max exceeds it by more than 2^8, so P <= 256 and O is rescaled
    // only a handful of times per row.  Lanes hl, hl^16, hl^32, hl^48 share a head.
    const u32x4 rv0 = *reinterpret_cast<const u32x4 *>(&slot_rows[c * kSlots + g * 4]);
    const u32x4 rv1 = *reinterpret_cast<const u32x4 *>(&slot_rows[c * kSlots + 16 + g * 4]);
    bf16x8 pb[HG];
#pragma unroll
    for (int hg = 0; hg < HG; ++hg) {
      float x[2][4];
      float cmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[0][i] = static_cast<int32_t>(rv0[i]) >= 0 ? acc[hg][0][i] * scale_log2 : -INFINITY;
        x[1][i] = static_cast<int32_t>(rv1[i]) >= 0 ? acc[hg][1][i] * scale_log2 : -INFINITY;
        cmax = fmaxf(cmax, fmaxf(x[0][i], x[1][i]));
      }
      cmax = fmaxf(cmax, xor16(cmax));
      cmax = fmaxf(cmax, swap_halves(cmax));
      if (__ballot(cmax > m_run[hg] + 8.0f)) {
        const float m_new = cmax > m_run[hg] + 8.0f ? cmax : m_run[hg];
        const float alpha = __builtin_amdgcn_exp2f(m_run[hg] - m_new);  // 0 on the first raise
        l_run[hg] *= alpha;
#pragma unroll
        for (int n = 0; n < kNT; ++n) o[hg][n] *= alpha;
        m_run[hg] = m_new;
      }
      float p[2][4];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[mt][i] = __builtin_amdgcn_exp2f(x[mt][i] - m_run[hg]);  // 0 for masked slots
          l_run[hg] += p[mt][i];
        }
      pb[hg] = pack_slots(p);
    }

    // ---- O^T += V^T . P^T   (slot k-index 8g + j <-> tile row 4g + j (j < 4), 16 + 4g + j - 4)
#pragma unroll
    for (int n = 0; n < kNT; ++n) {
      const bf16x8 va = fr.v_frag(tile, n);
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) o[hg][n] = mfma16(va, pb[hg], o[hg][n]);
    }
  }

  // ---- finalize: denominator over the four lane groups, normalise, write
#pragma unroll
  for (int hg = 0; hg < HG; ++hg) {
    float l_tot = l_run[hg] + xor16(l_run[hg]);
    l_tot += swap_halves(l_tot);
    const int h = (wave * HG + hg) * 16 + hl;
    if (h < H) {
      const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
      if (g == 0)
        lse[t * H + h] =
            l_tot > 0.0f ? (m_run[hg] + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
      uint16_t *orow = out + (t * H + h) * kDv + g * 4;
#pragma unroll
      for (int n = 0; n < kNT; ++n) {
        u32x2 v;
        v[0] = pack_bf16x2(o[hg][n][0] * inv, o[hg][n][1] * inv);
        v[1] = pack_bf16x2(o[hg][n][2] * inv, o[hg][n][3] * inv);
        *reinterpret_cast<u32x2 *>(orow + n * 16) = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// 33..64 heads: one work group of 8 waves per query row, split by role so that every SIMD runs
// one wave of each kind and their work overlaps:
//   S waves 0..3 (head group G = wave): S^T = rows . q^T for 16 heads over all dims (four
//     independent MFMA chains), the online softmax, and P (bf16, already in the PV B-operand
//     layout) plus any rescale factor to LDS.  Wave 0 also fetches the slot indices of the
//     tile four chunks ahead into a small ring.
//   PV waves 4..7 (quarter qq): O^T[channels 128 qq .. + 127 x 64 heads] += V^T . P^T one chunk
//     behind the S waves; every V fragment read from LDS (transposing reads, the slow kind)
//     feeds four MFMAs, one per head group.  They also issue the latent-row tile loads, two
//     chunks ahead, which keeps the slow issue of the gathers off the S waves' path.
// One barrier per chunk: in interval c the S waves work on chunk c while the PV waves finish
// chunk c - 1, so P, the rescale factors and the flags are double buffered, and a latent-row
// tile stays in use for two intervals; four tile buffers keep two tiles in flight.  Only the
// PV waves issue the (compiler-invisible) tile loads and only the S waves issue ordinary
// global loads, so each wave's explicit load-count waits stay exact.
constexpr int kRoleNBuf = 4;
constexpr int kRedoGroups = 256;  // work groups of the second launch (one per CU)
constexpr int kRing = 8;  // slot-index ring (tiles)
static_assert(kRing == SlotRing::kTiles && kSlots == SlotRing::kSlots, "slot-index ring layout");

template <int DQK>
struct RoleSmem {
  static constexpr int kTiles = kRoleNBuf * Tile<DQK>::kBytes;
  static constexpr int kP = kTiles;                  // [2][4 groups][64 lanes] bf16x8
  static constexpr int kA = kP + 2 * 4 * 64 * 16;    // [2][4 groups][16 heads] fp32 rescale
  static constexpr int kI = kA + 2 * 4 * 16 * 4;     // [4 groups][16 heads] fp32 1/l
  static constexpr int kF = kI + 4 * 16 * 4;         // [2][4 groups] int32 rescale flags
  static constexpr int kRingOff = kF + 2 * 4 * 4;    // [kRing][32] int32 slot -> latent row
  static constexpr int kBytes = kRingOff + kRing * kSlots * 4;
};

// One query row t with a running maximum per head (the rows that the fast kernel flagged).
template <int DQK>
__device__ __forceinline__ void roles_row(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kv,
    const int32_t *__restrict__ idx, const int32_t *__restrict__ topk_length, int H, int K,
    float scale_log2, uint16_t *__restrict__ out, float *__restrict__ lse, int64_t t) {
  using TL = Tile<DQK>;
  using SM = RoleSmem<DQK>;
  constexpr int kKSteps = DQK / 32;
  constexpr int kLoadsW = TL::kLoads / 4;  // tile loads per PV wave
  extern __shared__ __align__(16) unsigned char smem[];
  bf16x8 *pbuf = reinterpret_cast<bf16x8 *>(smem + SM::kP);
  float *abuf = reinterpret_cast<float *>(smem + SM::kA);
  float *ibuf = reinterpret_cast<float *>(smem + SM::kI);
  int32_t *fbuf = reinterpret_cast<int32_t *>(smem + SM::kF);
  int32_t *ring = reinterpret_cast<int32_t *>(smem + SM::kRingOff);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int hl = lane & 15;
  const int lim = topk_length ? topk_length[t] : K;
  const int32_t *irow = idx + t * K;
  const int nchunks = (lim + kSlots - 1) / kSlots;

  if (wave < 4) {
    // ================================ S waves ================================
    const int G = wave;
    const int h = G * 16 + hl;
    // slot indices of tile j (lanes 0..31; -1 beyond the valid prefix)
    SlotRing sr;  // wave 0 keeps the slot-index ring filled
    if (wave == 0) sr.start(irow, lim, nchunks, ring);
    bf16x8 qf[kKSteps];  // head h, dims ks * 32 + g * 8 + [0, 8)
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (h < H) v = *reinterpret_cast<const u32x4 *>(q + ((t * H + h) * DQK + ks * 32 + g * 8));
      qf[ks] = as_bf16x8(v);
    }
    __syncthreads();  // S0: indices of the first tiles are in the ring
    __syncthreads();  // S1: PV waves have issued the first tiles and waited for tile 0
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) settle(qf[ks]);  // see settle()

    TileFrag<DQK> fr;
    fr.init();
    float m_run = -1e30f;  // reference max (base-2 logits) of head h
    float l_run = 0.0f;    // this lane's partial softmax denominator
    for (int c = 0; c <= nchunks; ++c) {
      lds_barrier();  // B(c - 1): tile c complete; PV waves are done with chunk c - 2
      if (c == nchunks) break;
      if (wave == 0) sr.step(irow, lim, nchunks, ring, c);
      const unsigned char *tile = smem + (c % kRoleNBuf) * TL::kBytes;
      // slot validity of this chunk, read before the MFMAs (the reads cannot move across the
      // scheduling fences below)
      const int32_t *rr = ring + (c % kRing) * kSlots;
      const u32x4 rv0 = *reinterpret_cast<const u32x4 *>(rr + g * 4);
      const u32x4 rv1 = *reinterpret_cast<const u32x4 *>(rr + 16 + g * 4);
      // ---- S^T = rows . q^T  (four chains: slot half mt, k-step parity); fragment reads run
      // kAhead k-steps ahead of the MFMAs (an LDS read under load takes longer than a few
      // MFMAs, so a shallow read-ahead leaves the MFMA pipe waiting)
      constexpr int kAhead = 2;
      f32x4 acc[2][2] = {{f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}},
                         {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}}};
      bf16x8 a0[kAhead + 1], a1[kAhead + 1];
#pragma unroll
      for (int j = 0; j < kAhead; ++j) {
        a0[j] = fr.a_frag(tile, 0, j);
        a1[j] = fr.a_frag(tile, 1, j);
      }
      // the scheduling fences keep this order (the compiler would otherwise pull each read
      // down next to its MFMA)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        if (ks + kAhead < kKSteps) {
          a0[(ks + kAhead) % (kAhead + 1)] = fr.a_frag(tile, 0, ks + kAhead);
          a1[(ks + kAhead) % (kAhead + 1)] = fr.a_frag(tile, 1, ks + kAhead);
        }
        acc[0][ks & 1] = mfma16(a0[ks % (kAhead + 1)], qf[ks], acc[0][ks & 1]);
        acc[1][ks & 1] = mfma16(a1[ks % (kAhead + 1)], qf[ks], acc[1][ks & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
      const f32x4 sv0 = acc[0][0] + acc[0][1], sv1 = acc[1][0] + acc[1][1];
      // ---- online softmax (base 2) with a lazily raised reference max: the reference only
      // moves when the running max exceeds it by more than 2^8, so P <= 256 and O is rescaled
      // only a handful of times per row.  Lanes hl, hl^16, hl^32, hl^48 share head h.
      float x[2][4];
      float cmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[0][i] = static_cast<int32_t>(rv0[i]) >= 0 ? sv0[i] * scale_log2 : -INFINITY;
        x[1][i] = static_cast<int32_t>(rv1[i]) >= 0 ? sv1[i] * scale_log2 : -INFINITY;
        cmax = fmaxf(cmax, fmaxf(x[0][i], x[1][i]));
      }
      cmax = fmaxf(cmax, xor16(cmax));
      cmax = fmaxf(cmax, swap_halves(cmax));
      int rescale = 0;
      if (__ballot(cmax > m_run + 8.0f)) {
        const float m_new = cmax > m_run + 8.0f ? cmax : m_run;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the first raise
        l_run *= alpha;
        m_run = m_new;
        if (g == 0) abuf[((c & 1) * 4 + G) * 16 + hl] = alpha;
        rescale = 1;
      }
      float p[2][4];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[mt][i] = __builtin_amdgcn_exp2f(x[mt][i] - m_run);  // 0 for masked slots
          l_run += p[mt][i];
        }
      pbuf[((c & 1) * 4 + G) * 64 + lane] = pack_slots(p);
      if (lane == 0) fbuf[(c & 1) * 4 + G] = rescale;
    }
    // ---- finalize: denominator over the four lane groups; 1/l for the PV waves
    float l_tot = l_run + xor16(l_run);
    l_tot += swap_halves(l_tot);
    if (h < H && g == 0)
      lse[t * H + h] = l_tot > 0.0f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
    if (g == 0) ibuf[G * 16 + hl] = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    lds_barrier();  // Z: 1/l ready
  } else {
    // ================================ PV waves ===============================
    const int qq = wave - 4;
    const uint32_t tiles_lds = lds_addr(smem);
    __syncthreads();  // S0: indices of the first tiles are in the ring
    // this wave's loads k = 4 i + qq of tile c: global byte offsets first (all row indices
    // are read before any load is issued: the loads are asm with a memory clobber, so an index
    // read placed between two of them would be waited for on its own)
    auto offsets = [&](int c, uint32_t (&off)[kLoadsW]) {
      const int32_t *rr = ring + (c % kRing) * kSlots;
#pragma unroll
      for (int i = 0; i < kLoadsW; ++i) {
        const int pos = (4 * i + qq) * 64 + lane;
        const int row = pos / TL::kChunks;
        const int chunk = (pos % TL::kChunks) ^ TL::swz(row);
        const int r = rr[row];
        off[i] = static_cast<uint32_t>(r < 0 ? 0 : r) * TL::kRowBytes + chunk * 16;  // -1: row 0
      }
    };
    auto load = [&](int c, int i, const uint32_t (&off)[kLoadsW]) {
      dma16_sv(kv, off[i], tiles_lds + (c % kRoleNBuf) * TL::kBytes + (4 * i + qq) * 1024);
    };
    auto issue = [&](int c) {
      uint32_t off[kLoadsW];
      offsets(c, off);
#pragma unroll
      for (int i = 0; i < kLoadsW; ++i) load(c, i, off);
    };
    if (nchunks > 0) issue(0);
    if (nchunks > 1) issue(1);
    if (nchunks > 0) {  // tile 0 before S1 (tile 1 may stay in flight)
      if (nchunks > 1) wait_vm<kLoadsW>();
      else wait_tile();
    }
    __syncthreads();  // S1

    TileFrag<DQK> fr;
    fr.init();
    f32x4 o[4][8];  // o[G][n][i] = O[head 16 G + hl][channel 128 qq + 16 n + 4 g + i]
#pragma unroll
    for (int G = 0; G < 4; ++G)
#pragma unroll
      for (int n = 0; n < 8; ++n) o[G][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c <= nchunks; ++c) {
      lds_barrier();  // B(c - 1): P and rescale factors of chunk c - 1 are ready
      // tile c + 2 goes into the buffer of tile c - 2 (PV done at B(c - 1)); its loads are
      // spread over the PV MFMAs below, so that the address unit drains them (1 KB each)
      // while the MFMAs run instead of stalling the wave up front
      const bool load_next = c + 2 < nchunks;
      uint32_t off[kLoadsW];
      if (load_next) offsets(c + 2, off);
      if (c == 0 && load_next) {
#pragma unroll
        for (int i = 0; i < kLoadsW; ++i) load(c + 2, i, off);
      }
      if (c > 0) {
        const int b = (c - 1) & 1;
        const unsigned char *tile = smem + ((c - 1) % kRoleNBuf) * TL::kBytes;
        const u32x4 fl = *reinterpret_cast<const u32x4 *>(fbuf + b * 4);
        bf16x8 pb[4];
#pragma unroll
        for (int G = 0; G < 4; ++G) {
          if (fl[G]) {  // wave-uniform
            const float alpha = abuf[(b * 4 + G) * 16 + hl];
#pragma unroll
            for (int n = 0; n < 8; ++n) o[G][n] *= alpha;
          }
          pb[G] = pbuf[(b * 4 + G) * 64 + lane];
        }
        static_assert(kLoadsW <= 16, "two loads per channel tile at most");
        // the fragment of channel tile n + 1 is read before tile n's loads are issued (a read
        // cannot move across those asm statements, so it would otherwise wait in full before
        // every group of MFMAs)
        bf16x8 va = fr.v_frag(tile, 8 * qq);
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          bf16x8 vn = va;
          if (n + 1 < 8) vn = fr.v_frag(tile, 8 * qq + n + 1);
          if (load_next) {
            if (n < kLoadsW) load(c + 2, n, off);
            if (n + 8 < kLoadsW) load(c + 2, n + 8, off);
          }
#pragma unroll
          for (int G = 0; G < 4; ++G) o[G][n] = mfma16(va, pb[G], o[G][n]);
          va = vn;
        }
      }
      if (c == nchunks) break;
      // tile c + 1 before the next barrier (tile c + 2 may stay in flight)
      if (c + 2 < nchunks) wait_vm<kLoadsW>();
      else wait_tile();
    }
    lds_barrier();  // Z: 1/l ready
#pragma unroll
    for (int G = 0; G < 4; ++G) {
      const int h = G * 16 + hl;
      const float inv = ibuf[G * 16 + hl];
      if (h < H) {
        uint16_t *orow = out + (t * H + h) * kDv + 128 * qq + g * 4;
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          u32x2 v;
          v[0] = pack_bf16x2(o[G][n][0] * inv, o[G][n][1] * inv);
          v[1] = pack_bf16x2(o[G][n][2] * inv, o[G][n][3] * inv);
          *reinterpret_cast<u32x2 *>(orow + n * 16) = v;
        }
      }
    }
  }
}

// Second launch: the rows whose first LSE entry the fast kernel left as NaN.  Each work group
// checks the rows blockIdx.x + i gridDim.x, 64 at a time (one per lane, the same in every wave,
// so the decisions are uniform), and computes the flagged ones.
template <int DQK>
__global__ __launch_bounds__(512) void sparse_mla_fwd_roles_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kv,
    const int32_t *__restrict__ idx, const int32_t *__restrict__ topk_length, int H, int K,
    float scale_log2, uint16_t *__restrict__ out, float *__restrict__ lse, int64_t T_q) {
  const int lane = threadIdx.x & 63;
  for (int64_t base = 0; blockIdx.x + base * gridDim.x < T_q; base += 64) {
    const int64_t tl = blockIdx.x + (base + lane) * gridDim.x;
    const bool flagged = tl < T_q && __builtin_isnan(lse[tl * H]);
    uint64_t m = __ballot(flagged);
    while (m != 0u) {
      const int i = __builtin_ctzll(m);
      m &= m - 1u;
      __syncthreads();  // the previous row is done with the LDS
      roles_row<DQK>(q, kv, idx, topk_length, H, K, scale_log2, out, lse,
                     blockIdx.x + (base + i) * gridDim.x);
    }
  }
}

// ---------------------------------------------------------------------------------------
// 33..64 heads, fast path.  As the role-split kernel above, except that S wave w takes the 32
// heads 32 (w >> 1) .. + 31 over the 16 slots 16 (w & 1) .. + 15 of every chunk: each
// latent-row fragment it reads feeds two MFMAs, which halves the S waves' LDS reads.  The two
// waves of a head pair see different slots of the same heads, so the softmax does not keep a
// running maximum: each head uses one reference, the larger of the pair's maxima over the
// first chunk (exchanged once in the prologue), and P = exp2(x - m_ref) needs neither
// rescaling nor per-chunk reductions.  A row in which a later logit exceeds its reference by
// more than kRefSlack (base 2), or whose first chunk has no valid slot for some head, is
// flagged by a NaN in its first LSE entry and computed again by the role-split kernel.
constexpr float kRefSlack = 24.0f;

template <int DQK>
struct PairSmem {
  static constexpr int kTiles = kRoleNBuf * Tile<DQK>::kBytes;
  static constexpr int kP = kTiles;                  // [2][4 groups][64 lanes] bf16x8
  static constexpr int kX = kP + 2 * 4 * 64 * 16;    // [4 waves][32 heads] fp32 exchange
  static constexpr int kI = kX + 4 * 32 * 4;         // [4 groups][16 heads] fp32 1/l
  static constexpr int kF = kI + 4 * 16 * 4;         // int32 redo flag (16 bytes)
  static constexpr int kRingOff = kF + 16;           // [kRing][32] int32 slot -> latent row
  static constexpr int kBytes = kRingOff + kRing * kSlots * 4;
};

template <int DQK>
__global__ __launch_bounds__(512) void sparse_mla_fwd_pair_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kv,
    const int32_t *__restrict__ idx, const int32_t *__restrict__ topk_length, int H, int K,
    float scale_log2, uint16_t *__restrict__ out, float *__restrict__ lse) {
  using TL = Tile<DQK>;
  using SM = PairSmem<DQK>;
  constexpr int kKSteps = DQK / 32;
  constexpr int kLoadsW = TL::kLoads / 4;  // tile loads per PV wave
  extern __shared__ __align__(16) unsigned char smem[];
  bf16x8 *pbuf = reinterpret_cast<bf16x8 *>(smem + SM::kP);
  float *xbuf = reinterpret_cast<float *>(smem + SM::kX);
  float *ibuf = reinterpret_cast<float *>(smem + SM::kI);
  int32_t *redo = reinterpret_cast<int32_t *>(smem + SM::kF);
  int32_t *ring = reinterpret_cast<int32_t *>(smem + SM::kRingOff);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t t = blockIdx.x;
  const int g = lane >> 4;
  const int hl = lane & 15;
  const int lim = topk_length ? topk_length[t] : K;
  const int32_t *irow = idx + t * K;
  const int nchunks = (lim + kSlots - 1) / kSlots;

  if (wave < 4) {
    // ================================ S waves ================================
    const int hp = wave >> 1;  // head pair: heads 32 hp .. + 31
    const int mh = wave & 1;   // slot half: slots 16 mh .. + 15 of each chunk
    SlotRing sr;                // wave 0 keeps the slot-index ring filled
    if (wave == 0) {
      sr.start(irow, lim, nchunks, ring);
      if (lane == 0) *redo = 0;
    }
    bf16x8 qf[2][kKSteps];  // head 32 hp + 16 hg + hl, dims ks * 32 + g * 8 + [0, 8)
#pragma unroll
    for (int hg = 0; hg < 2; ++hg) {
      const int h = 32 * hp + 16 * hg + hl;
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (h < H) v = *reinterpret_cast<const u32x4 *>(q + ((t * H + h) * DQK + ks * 32 + g * 8));
        qf[hg][ks] = as_bf16x8(v);
      }
    }
    // row fragments of this wave's slot half: rows 16 mh + hl, chunk 4 ks + g
    int sb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) sb[j] = TL::chunk_off(16 * mh + hl, j * 4 + g);
    __syncthreads();  // S0: indices of the first tiles are in the ring
    __syncthreads();  // S1: PV waves have issued the first tiles and waited for tile 0
#pragma unroll
    for (int hg = 0; hg < 2; ++hg)
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) settle(qf[hg][ks]);  // see settle()

    // logits (base 2) of chunk c for this wave's 16 slots (4 per lane: slot 16 mh + 4 g + i)
    // and 32 heads (hg); masked slots are -inf
    auto logits = [&](int c, float (&x)[2][4]) {
      const unsigned char *tile = smem + (c % kRoleNBuf) * TL::kBytes;
      const int32_t *rr = ring + (c % kRing) * kSlots;
      const u32x4 rv = *reinterpret_cast<const u32x4 *>(rr + 16 * mh + g * 4);
      f32x4 acc[2][2] = {{f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}},
                         {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}}};
      auto afrag = [&](int ks) {
        return as_bf16x8(*reinterpret_cast<const u32x4 *>(tile + sb[ks & 3] + (ks >> 2) * 256));
      };
      bf16x8 a[3];
      a[0] = afrag(0);
      a[1] = afrag(1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        if (ks + 2 < kKSteps) a[(ks + 2) % 3] = afrag(ks + 2);
        acc[0][ks & 1] = mfma16(a[ks % 3], qf[0][ks], acc[0][ks & 1]);
        acc[1][ks & 1] = mfma16(a[ks % 3], qf[1][ks], acc[1][ks & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int hg = 0; hg < 2; ++hg) {
        const f32x4 sv = acc[hg][0] + acc[hg][1];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          x[hg][i] = static_cast<int32_t>(rv[i]) >= 0 ? sv[i] * scale_log2 : -INFINITY;
      }
    };

    // ---- reference of each head: the larger of the two slot halves' maxima over chunk 0
    float m_ref[2] = {-INFINITY, -INFINITY};
    if (nchunks > 0) {
      float x[2][4];
      logits(0, x);
#pragma unroll
      for (int hg = 0; hg < 2; ++hg) {
        float m = fmaxf(fmaxf(x[hg][0], x[hg][1]), fmaxf(x[hg][2], x[hg][3]));
        m = fmaxf(m, xor16(m));
        m = fmaxf(m, swap_halves(m));
        m_ref[hg] = m;
      }
    }
    if (g == 0) {
      xbuf[wave * 32 + hl] = m_ref[0];
      xbuf[wave * 32 + 16 + hl] = m_ref[1];
    }
    lds_barrier();  // P1
#pragma unroll
    for (int hg = 0; hg < 2; ++hg) m_ref[hg] = fmaxf(m_ref[hg], xbuf[(wave ^ 1) * 32 + 16 * hg + hl]);
    float l_run[2] = {0.0f, 0.0f};  // this lane's partial denominators
    bool over = false;               // a logit exceeds its reference by more than kRefSlack
    for (int c = 0; c <= nchunks; ++c) {
      lds_barrier();  // B(c - 1): tile c complete; PV waves are done with chunk c - 2
      if (c == nchunks) break;
      if (wave == 0) sr.step(irow, lim, nchunks, ring, c);
      float x[2][4];
      logits(c, x);
#pragma unroll
      for (int hg = 0; hg < 2; ++hg) {
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool valid = x[hg][i] != -INFINITY;
          const float d = x[hg][i] - m_ref[hg];  // +inf if m_ref is -inf (chunk 0 had no slot)
          over = over || (valid && !(d <= kRefSlack));
          p[i] = valid ? __builtin_amdgcn_exp2f(d) : 0.0f;
          l_run[hg] += p[i];
        }
        // P of head group 2 hp + hg: this wave supplies slots 16 mh + 4 g + i, i.e. one half
        // of each lane's eight contraction entries (see pack_slots)
        u32x2 w;
        w[0] = pack_bf16x2(p[0], p[1]);
        w[1] = pack_bf16x2(p[2], p[3]);
        reinterpret_cast<u32x2 *>(&pbuf[((c & 1) * 4 + 2 * hp + hg) * 64 + lane])[mh] = w;
      }
    }
    if (__ballot(over)) {
      if (lane == 0) *redo = 1;  // every writer stores 1
    }
    // ---- finalize: denominators over the lane groups and the slot halves
#pragma unroll
    for (int hg = 0; hg < 2; ++hg) {
      float l = l_run[hg] + xor16(l_run[hg]);
      l += swap_halves(l);
      l_run[hg] = l;
    }
    if (g == 0) {
      xbuf[wave * 32 + hl] = l_run[0];
      xbuf[wave * 32 + 16 + hl] = l_run[1];
    }
    lds_barrier();  // Z1
    if (mh == 0) {
#pragma unroll
      for (int hg = 0; hg < 2; ++hg) {
        const float l = l_run[hg] + xbuf[(wave ^ 1) * 32 + 16 * hg + hl];
        const int h = 32 * hp + 16 * hg + hl;
        if (g == 0) {
          if (h < H)
            lse[t * H + h] = l > 0.0f ? (m_ref[hg] + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
          ibuf[(2 * hp + hg) * 16 + hl] = l > 0.0f ? 1.0f / l : 0.0f;
        }
      }
    }
    lds_barrier();  // Z2: 1/l ready
    if (wave == 0 && lane == 0 && *redo) lse[t * H] = __builtin_nanf("");
  } else {
    // ================================ PV waves ===============================
    const int qq = wave - 4;
    const uint32_t tiles_lds = lds_addr(smem);
    __syncthreads();  // S0: indices of the first tiles are in the ring
    auto offsets = [&](int c, uint32_t (&off)[kLoadsW]) {
      const int32_t *rr = ring + (c % kRing) * kSlots;
#pragma unroll
      for (int i = 0; i < kLoadsW; ++i) {
        const int pos = (4 * i + qq) * 64 + lane;
        const int row = pos / TL::kChunks;
        const int chunk = (pos % TL::kChunks) ^ TL::swz(row);
        const int r = rr[row];
        off[i] = static_cast<uint32_t>(r < 0 ? 0 : r) * TL::kRowBytes + chunk * 16;  // -1: row 0
      }
    };
    auto load = [&](int c, int i, const uint32_t (&off)[kLoadsW]) {
      dma16_sv(kv, off[i], tiles_lds + (c % kRoleNBuf) * TL::kBytes + (4 * i + qq) * 1024);
    };
    auto issue = [&](int c) {
      uint32_t off[kLoadsW];
      offsets(c, off);
#pragma unroll
      for (int i = 0; i < kLoadsW; ++i) load(c, i, off);
    };
    if (nchunks > 0) issue(0);
    if (nchunks > 1) issue(1);
    if (nchunks > 0) {  // tile 0 before S1 (tile 1 may stay in flight)
      if (nchunks > 1) wait_vm<kLoadsW>();
      else wait_tile();
    }
    __syncthreads();  // S1
    lds_barrier();    // P1
    TileFrag<DQK> fr;
    fr.init();
    f32x4 o[4][8];  // o[G][n][i] = O[head 16 G + hl][channel 128 qq + 16 n + 4 g + i]
#pragma unroll
    for (int G = 0; G < 4; ++G)
#pragma unroll
      for (int n = 0; n < 8; ++n) o[G][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c <= nchunks; ++c) {
      lds_barrier();  // B(c - 1): P of chunk c - 1 is ready
      // tile c + 2 first: its issue (ring reads, address arithmetic) runs while the S waves
      // start their MFMAs, and the MFMAs below overlap the S waves' softmax
      if (c + 2 < nchunks) issue(c + 2);
      if (c > 0) {
        const int b = (c - 1) & 1;
        const unsigned char *tile = smem + ((c - 1) % kRoleNBuf) * TL::kBytes;
        bf16x8 pb[4];
#pragma unroll
        for (int G = 0; G < 4; ++G) pb[G] = pbuf[(b * 4 + G) * 64 + lane];
        bf16x8 va = fr.v_frag(tile, 8 * qq);
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          bf16x8 vn = va;
          if (n + 1 < 8) vn = fr.v_frag(tile, 8 * qq + n + 1);
#pragma unroll
          for (int G = 0; G < 4; ++G) o[G][n] = mfma16(va, pb[G], o[G][n]);
          va = vn;
        }
      }
      if (c == nchunks) break;
      // tile c + 1 before the next barrier (tile c + 2 may stay in flight)
      if (c + 2 < nchunks) wait_vm<kLoadsW>();
      else wait_tile();
    }
    lds_barrier();  // Z1
    lds_barrier();  // Z2: 1/l ready
#pragma unroll
    for (int G = 0; G < 4; ++G) {
      const int h = G * 16 + hl;
      const float inv = ibuf[G * 16 + hl];
      if (h < H) {
        uint16_t *orow = out + (t * H + h) * kDv + 128 * qq + g * 4;
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          u32x2 v;
          v[0] = pack_bf16x2(o[G][n][0] * inv, o[G][n][1] * inv);
          v[1] = pack_bf16x2(o[G][n][2] * inv, o[G][n][3] * inv);
          *reinterpret_cast<u32x2 *>(orow + n * 16) = v;
        }
      }
    }
  }
}

template <int DQK>
hipError_t launch_roles(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                        const int32_t *topk_length, int64_t T_q, int32_t H, int32_t K,
                        float scale, uint16_t *out, float *lse, hipStream_t s) {
  constexpr size_t smem_p = PairSmem<DQK>::kBytes;
  auto fast = sparse_mla_fwd_pair_kernel<DQK>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(fast),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(smem_p));
  if (e != hipSuccess) return e;
  DSA_LAUNCH("sparse_mla_fwd", fast, dim3(static_cast<unsigned>(T_q)), dim3(512), smem_p, s, q,
             kv, idx, topk_length, H, K, scale * kLog2e, out, lse);
  // rows flagged by the fast kernel (a logit far above its reference) are computed again
  constexpr size_t smem = RoleSmem<DQK>::kBytes;
  auto kern = sparse_mla_fwd_roles_kernel<DQK>;
  e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
  if (e != hipSuccess) return e;
  const unsigned redo_groups = static_cast<unsigned>(T_q < kRedoGroups ? T_q : kRedoGroups);
  DSA_LAUNCH("sparse_mla_fwd_redo", kern, dim3(redo_groups), dim3(512), smem, s, q, kv, idx,
             topk_length, H, K, scale * kLog2e, out, lse, T_q);
  return hipGetLastError();
}

template <int DQK, int NW, int HG, int SLOTCAP>
hipError_t launch(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                  const int32_t *topk_length, int64_t T_q, int32_t H, int32_t K, float scale,
                  uint16_t *out, float *lse, hipStream_t s) {
  constexpr size_t smem = fwd_smem_bytes<DQK, SLOTCAP>();
  auto kern = sparse_mla_fwd_kernel<DQK, NW, HG, SLOTCAP>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(smem));
  if (e != hipSuccess) return e;
  DSA_LAUNCH("sparse_mla_fwd", kern, dim3(static_cast<unsigned>(T_q)), dim3(NW * 64), smem, s,
             q, kv, idx, topk_length, H, K, scale * kLog2e, out, lse);
  return hipGetLastError();
}

// Index rows of up to 2048 slots keep a work group within 80 KB of LDS (two per CU).
template <int DQK, int NW, int HG>
hipError_t launch_k(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                    const int32_t *topk_length, int64_t T_q, int32_t H, int32_t K, float scale,
                    uint16_t *out, float *lse, hipStream_t s) {
  if (K <= 2048)
    return launch<DQK, NW, HG, 2048>(q, kv, idx, topk_length, T_q, H, K, scale, out, lse, s);
  return launch<DQK, NW, HG, 4096>(q, kv, idx, topk_length, T_q, H, K, scale, out, lse, s);
}

template <int DQK>
hipError_t launch_w(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                    const int32_t *topk_length, int64_t T_q, int32_t H, int32_t K, float scale,
                    uint16_t *out, float *lse, hipStream_t s) {
  if (H <= 16) return launch_k<DQK, 1, 1>(q, kv, idx, topk_length, T_q, H, K, scale, out, lse, s);
  if (H <= 32) return launch_k<DQK, 2, 1>(q, kv, idx, topk_length, T_q, H, K, scale, out, lse, s);
  if (H <= 64) return launch_roles<DQK>(q, kv, idx, topk_length, T_q, H, K, scale, out, lse, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_sparse_mla_fwd(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                                 const int32_t *topk_length, int64_t T_q, int32_t H,
                                 int32_t D_qk, int32_t K, float scale, uint16_t *out, float *lse,
                                 hipStream_t s) {
  if (T_q == 0) return hipSuccess;
  if (D_qk == 576) return launch_w<576>(q, kv, idx, topk_length, T_q, H, K, scale, out, lse, s);
  if (D_qk == 512) return launch_w<512>(q, kv, idx, topk_length, T_q, H, K, scale, out, lse, s);
  return hipErrorInvalidValue;
}

}  // namespace dsa
