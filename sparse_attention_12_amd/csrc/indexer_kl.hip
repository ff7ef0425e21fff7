// Indexer training loss: the sparse KL loss that aligns the indexer's score distribution with
// the main attention's (NVIDIA GLM-5.2 cuDNN DSA page, "How DSA works": an auxiliary KL loss on
// a graph of its own; "GLM-5.2 training results": sparse formulation, coefficient 0.001, with
// a score-recompute step and an indexer backward; "cuDNN fused DSA kernels": the fused KL-score
// path).  The pages give no formula; the reading implemented here, for query row t with valid
// slots j and key rows s_j, is
//   target  p(j) = sum_h P[t,h,j] / sum_j' sum_h P[t,h,j']     (attention probabilities
//                  recomputed from q, kv and the forward's lse; no gradient)
//   indexer u(j) = softmax_j I(t, s_j),  I(t,s) = sum_h w[t,h] max(0, q_idx[t,h] . k_idx[s])
//   loss_t = sum_j p(j) (log p(j) - log u(j))
// and with upstream gradient g of sum_t loss_t, dI(t,j) = g (u(j) - p(j)), which flows to
//   dw[t,h] = sum_j dI max(0, d),  dq_idx[t,h] = sum_j dI w [d > 0] k_idx[s_j],
//   dk_idx[s] += sum_(t,j: s_j = s) sum_h dI w [d > 0] q_idx[t,h]      (d = q_idx[t,h] . k_idx[s_j]).
//
// Kernels (one work group per query row):
//   kl_target : S^T = rows . q^T per 32-slot tile of gathered latent rows (as the attention
//               backward recomputes it), P = exp(S - lse), the head sum per slot (lanes, then
//               waves through LDS), renormalised over the row -> target [T_q, K] fp32.
//   kl_bwd    : pass 1 recomputes the indexer scores of the row's slots (32x32x16 MFMAs on
//               gathered k_idx rows with the heads on the M axis, two waves of 32 heads; ReLU,
//               weights and head sum in fp32 registers) into LDS; the row's
//               softmax, loss and dI follow; pass 2 recomputes the dot products, forms
//               G = dI w [d > 0] and accumulates dq_idx^T += k_idx^T . G^T (transposing reads of
//               the tile), dw, and the key-gradient contribution C = q_idx^T . G of every slot
//               (G staged in LDS as a bf16 pair hi + lo, about 16 significant bits), which is
//               stored as a 16-bit block floating point row and summed per key row after a
//               counting sort, as for the attention's latent rows.  Four score waves (16 heads
//               each) load the tiles and do everything but C; four contribution waves form and
//               store C one chunk behind.
#include <algorithm>

#include "dsa_common.h"
#include "dsa_internal.h"
#include "stage.h"
#include "tile.h"

namespace dsa {
namespace {

constexpr int kSlots = 32;
constexpr int kWaves = 4;
constexpr int kDi = 128;   // indexer head dim of the training path
constexpr int kSS = 72;    // G staging row stride (64 heads + 8, bf16)


__device__ __forceinline__ int rows_rounded(int K) { return (K + kSlots - 1) / kSlots * kSlots; }

// ---------------------------------------------------------------------------------------
// kl_target: chunks of 64 slots, wave w taking slots 16 w .. + 15 of every chunk for all 64
// heads.  With the heads on the MFMA M axis, S[heads x slots] = q . rows^T takes the query
// blocks (held in registers) as the A operand and the gathered rows as B, so every row fragment
// read from LDS feeds four MFMAs (one per 16-head group), and a lane ends with 16 heads of one
// slot: the head sum is 15 register adds and two lane swaps.  A chunk is two 32-slot tiles;
// two chunks are double buffered (147 KB of LDS).  Wave 0 keeps the slot indices in a ring of
// four chunks, loaded two chunks ahead.
constexpr int kTChunk = 64;
constexpr int kTRing = 4;

template <int DQK>
struct TargetSmem {
  static constexpr int kTiles = 4 * Tile<DQK>::kBytes;        // 2 chunks x 2 tiles
  static constexpr int kRing = kTiles;                          // [kTRing][64] int32
  static constexpr int kTot = kRing + kTRing * kTChunk * 4;     // [4 waves] fp32
  static constexpr int kBytes = kTot + kWaves * 4;
  static_assert(kBytes <= 160 * 1024, "LDS per work group");
};

template <int DQK>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void kl_target_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ kv,
                      const int32_t *__restrict__ idx, const int32_t *__restrict__ topk_length,
                      const float *__restrict__ lse, int H, int K, float scale_log2,
                      float *__restrict__ target) {
  using TL = Tile<DQK>;
  using SM = TargetSmem<DQK>;
  constexpr int kKS = DQK / 32;
  constexpr int L = TL::kLoads / kWaves;  // DMA loads per wave per 32-slot tile
  extern __shared__ __align__(16) unsigned char smem[];
  int32_t *ring = reinterpret_cast<int32_t *>(smem + SM::kRing);
  float *tot = reinterpret_cast<float *>(smem + SM::kTot);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, hl = lane & 15;
  const int64_t t = blockIdx.x;
  const int lim = topk_length ? topk_length[t] : K;
  const int32_t *irow = idx + t * K;
  const int nch = (lim + kTChunk - 1) / kTChunk;
  auto slot_index = [&](int c) {  // slot c * 64 + lane of the row (-1: invalid)
    const int j = c * kTChunk + lane;
    return c < nch && j < lim ? irow[j] : -1;
  };
  int32_t pend = -1;
  if (wave == 0) {
    ring[lane] = slot_index(0);
    ring[kTChunk + lane] = slot_index(1);
    pend = slot_index(2);
  }
  // query blocks as A operands: head 16 G + hl, dims 32 ks + 8 g + [0, 8); lse (base 2) of the
  // heads 16 G + 4 g + i whose logits this lane receives
  bf16x8 qf[4][kKS];
  float lse2[4][4];
#pragma unroll
  for (int G = 0; G < 4; ++G) {
    const int h = 16 * G + hl;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (h < H) v = *reinterpret_cast<const u32x4 *>(q + ((t * H + h) * DQK + ks * 32 + g * 8));
      qf[G][ks] = as_bf16x8(v);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = 16 * G + 4 * g + i;
      const float l0 = hh < H ? lse[t * H + hh] : -INFINITY;
      lse2[G][i] = l0 == -INFINITY ? INFINITY : l0 * kLog2e;  // padded head / empty row: P = 0
    }
  }
#pragma unroll
  for (int G = 0; G < 4; ++G)
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) settle(qf[G][ks]);
  __syncthreads();  // ring holds chunks 0 and 1

  // DMA loads of chunk c (tiles 2c, 2c + 1) into buffer c % 2: this wave's loads k = wave,
  // wave + 4, ... of each tile; slot indices from the ring
  int dma_row[L], dma_off[L];
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const int pos = (i * kWaves + wave) * 64 + lane;
    dma_row[i] = pos / TL::kChunks;
    dma_off[i] = ((pos % TL::kChunks) ^ TL::swz(dma_row[i])) * 16;
  }
  const uint32_t tiles_lds = lds_addr(smem) + wave * 1024;
  auto issue = [&](int c) {
    const int32_t *rr = ring + (c % kTRing) * kTChunk;
    uint32_t off[2][L];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int i = 0; i < L; ++i) {
        const int r = rr[h2 * 32 + dma_row[i]];
        off[h2][i] = static_cast<uint32_t>(r < 0 ? 0 : r) * TL::kRowBytes + dma_off[i];
      }
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int i = 0; i < L; ++i)
        dma16_sv(kv, off[h2][i], tiles_lds + ((c & 1) * 2 + h2) * TL::kBytes + i * kWaves * 1024);
  };
  if (nch > 0) issue(0);
  // row fragments of this wave's 16 slots as B operands: slot 16 (wave & 1) + hl of tile
  // half (wave >> 1), dims 32 ks + 8 g + [0, 8)
  int sb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) sb[j] = TL::chunk_off(16 * (wave & 1) + hl, j * 4 + g);
  float total = 0.0f;
  float *trow = target + t * K;
  for (int c = 0; c < nch; ++c) {
    wait_vm<0>();    // chunk c's loads (the only ones in flight)
    lds_barrier();   // chunk c is in LDS; every wave is done with chunk c - 1
    if (wave == 0) {  // the ring slot of chunk c + 2 held chunk c - 2
      ring[((c + 2) % kTRing) * kTChunk + lane] = pend;
      pend = slot_index(c + 3);
    }
    if (c + 1 < nch) issue(c + 1);
    const unsigned char *tile = smem + ((c & 1) * 2 + (wave >> 1)) * TL::kBytes;
    f32x4 acc[4] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f},
                    f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    bf16x8 b[3];
    auto bfrag = [&](int ks) {
      return as_bf16x8(*reinterpret_cast<const u32x4 *>(tile + sb[ks & 3] + (ks >> 2) * 256));
    };
    b[0] = bfrag(0);
    b[1] = bfrag(1);
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      if (ks + 2 < kKS) b[(ks + 2) % 3] = bfrag(ks + 2);
#pragma unroll
      for (int G = 0; G < 4; ++G) acc[G] = mfma16(qf[G][ks], b[ks % 3], acc[G]);
    }
    // P of heads 16 G + 4 g + i for slot 16 wave + hl, summed over the heads
    const int32_t sidx = ring[(c % kTRing) * kTChunk + 16 * wave + hl];
    float v = 0.0f;
#pragma unroll
    for (int G = 0; G < 4; ++G)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        v += __builtin_amdgcn_exp2f(acc[G][i] * scale_log2 - lse2[G][i]);
    v += xor16(v);
    v += swap_halves(v);
    v = sidx >= 0 ? v : 0.0f;
    const int j = c * kTChunk + 16 * wave + hl;
    if (g == 0 && j < K) trow[j] = v;  // unnormalised (the last chunk may pass K)
    total += g == 0 ? v : 0.0f;
  }
  // row total over the waves, then the row is renormalised in place
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) total += __shfl_xor(total, o, 64);
  if (lane == 0) tot[wave] = total;
  __syncthreads();  // also orders this work group's writes of the row before the rereads
  const float sum = tot[0] + tot[1] + tot[2] + tot[3];
  const float inv = sum > 0.0f ? 1.0f / sum : 0.0f;
  for (int j = threadIdx.x; j < K; j += kWaves * 64)
    trow[j] = j < nch * kTChunk ? trow[j] * inv : 0.0f;
}

// ---------------------------------------------------------------------------------------
// kl_bwd: one work group of 8 waves per query row.  Score waves 0..3 (head group G = wave)
// stream the row's k_idx tiles with direct loads (kBwdNBuf buffers, three tiles in flight) and
// compute the dot products, the scores (pass 1), and in pass 2 G and dq_idx; contribution waves
// 4..7 (dims 32 qd .. + 31, qd = wave - 4) form C = q_idx^T . G one chunk behind from the staged
// G and store it.  The stores stay out of the score waves, whose explicit waits for tile loads
// would otherwise also wait for them (the vector-memory counter does not tell loads from stores).
constexpr int kBwdScoreWaves = 4;
constexpr int kBwdWaves = 8;
constexpr int kBwdNBuf = 5;

struct KlSmem {
  static constexpr int kTiles = kBwdNBuf * Tile<kDi>::kBytes;      // k_idx tiles
  static constexpr int kStage = kTiles;                            // [2][hi, lo][32][kSS] bf16
  static constexpr int kStageBytes = 2 * kSlots * kSS * 2;         // one buffer (hi + lo)
  static constexpr int kPart = kStage + 2 * kStageBytes;           // [2][4][32] fp32
  static constexpr int kRows = kPart + 2 * kBwdScoreWaves * kSlots * 4;  // slot rows [Kr] int32
  static size_t bytes(int K) {
    const size_t kr = static_cast<size_t>(K + kSlots - 1) / kSlots * kSlots;
    return kRows + kr * 4 /* slot rows */ + kr * 4 /* scores, then dI */;
  }
};

__global__ __launch_bounds__(kBwdWaves * 64, 4) void kl_bwd_kernel(
    const uint16_t *__restrict__ q_idx, const uint16_t *__restrict__ k_idx,
    const float *__restrict__ w, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ topk_length, const float *__restrict__ target, int Hi, int K,
    float grad, float *__restrict__ loss, uint16_t *__restrict__ dq_idx, float *__restrict__ dw,
    uint32_t *__restrict__ stage, int32_t *__restrict__ cnt, int64_t row0) {
  using TL = Tile<kDi>;
  using TS = TileStream<kDi, kBwdScoreWaves, kBwdNBuf>;
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t *stg = reinterpret_cast<uint16_t *>(smem + KlSmem::kStage);
  float *part = reinterpret_cast<float *>(smem + KlSmem::kPart);
  int32_t *slot_rows = reinterpret_cast<int32_t *>(smem + KlSmem::kRows);
  const int Kr = rows_rounded(K);
  float *ibuf = reinterpret_cast<float *>(smem + KlSmem::kRows + Kr * 4);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool scorer = wave < kBwdScoreWaves;
  const int g = lane >> 4, hl = lane & 15;
  const int64_t i_row = blockIdx.x;
  const int64_t t = row0 + i_row;
  const int lim = topk_length ? topk_length[t] : K;
  const int32_t *irow = idx + t * K;
  const int nch = (lim + kSlots - 1) / kSlots;
  // slot rows and one count per valid slot for the key rows' counting sort
  for (int j = threadIdx.x; j < nch * kSlots; j += kBwdWaves * 64) {
    const int32_t sj = j < lim ? irow[j] : -1;
    slot_rows[j] = sj;
    if (sj >= 0) atomicAdd(&cnt[sj], 1);
  }
  // score waves: B operands of the dot products, head h, dims 32 ks + 8 g + [0, 8)
  const int h = (wave & 3) * 16 + hl;
  const bool hok = scorer && h < Hi;
  bf16x8 qf[kDi / 32];
  float wv = 0.0f;
  // pass 1 (score waves 0 and 1): heads 32 wave .. + 31 on the M axis of 32x32x16 MFMAs, so
  // that a lane ends with 16 heads of one slot and the head sum is register arithmetic and one
  // swap with the lane 32 apart.  A: head 32 wave + lane % 32, dims 16 kk + 8 (lane / 32) +
  // [0, 8); wm: the weights of the heads (i / 4) 8 + (lane / 32) 4 + i % 4 of the output.
  const bool p1 = wave < 2;
  bf16x8 qm[kDi / 16];
  float wm[16];
  // contribution waves: A operands of C^T = q_idx^T . G, dims 32 qd + 16 m + hl, heads
  // 32 kh + 8 g + [0, 8)
  bf16x8 qa[2][2];
  if (scorer) {
#pragma unroll
    for (int ks = 0; ks < kDi / 32; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (hok) v = *reinterpret_cast<const u32x4 *>(q_idx + ((t * Hi + h) * kDi + ks * 32 + g * 8));
      qf[ks] = as_bf16x8(v);
    }
    wv = hok ? w[t * Hi + h] : 0.0f;
    const int hm = 32 * wave + (lane & 31);
#pragma unroll
    for (int kk = 0; kk < kDi / 16; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (p1 && hm < Hi)
        v = *reinterpret_cast<const u32x4 *>(q_idx + ((t * Hi + hm) * kDi + kk * 16 + (lane >> 5) * 8));
      qm[kk] = as_bf16x8(v);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int hh = 32 * wave + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
      wm[i] = p1 && hh < Hi ? w[t * Hi + hh] : 0.0f;
    }
#pragma unroll
    for (int ks = 0; ks < kDi / 32; ++ks) settle(qf[ks]);
#pragma unroll
    for (int kk = 0; kk < kDi / 16; ++kk) settle(qm[kk]);
#pragma unroll
    for (int i = 0; i < 16; ++i) settle(wm[i]);
  } else {
    const int qd = wave - kBwdScoreWaves;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const int dim = 32 * qd + 16 * m + hl;
        uint16_t e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int hh = 32 * kh + 8 * g + j;
          e[j] = hh < Hi ? q_idx[(t * Hi + hh) * kDi + dim] : static_cast<uint16_t>(0);
        }
        qa[m][kh] = as_bf16x8(u32x4{e[0] | (static_cast<uint32_t>(e[1]) << 16),
                                    e[2] | (static_cast<uint32_t>(e[3]) << 16),
                                    e[4] | (static_cast<uint32_t>(e[5]) << 16),
                                    e[6] | (static_cast<uint32_t>(e[7]) << 16)});
      }
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) settle(qa[m][kh]);
  }
  __syncthreads();  // slot rows

  TS ts;
  if (scorer) ts.init(smem, wave);
  TileFrag<kDi> fr;
  fr.init();
  // D^T = k rows . q_idx^T for the 32 slots of a tile (d[mt][i]: slot 16 mt + 4 g + i, head h)
  auto dots = [&](const unsigned char *tile, f32x4 (&d)[2]) {
    d[0] = d[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kDi / 32; ++ks) {
      d[0] = mfma16(fr.a_frag(tile, 0, ks), qf[ks], d[0]);
      d[1] = mfma16(fr.a_frag(tile, 1, ks), qf[ks], d[1]);
    }
  };
  auto gather_part = [&](int c) {  // wave 0: the scores of chunk c from the two head halves
    if (wave == 0 && lane < kSlots) {
      const float v = part[((c & 1) * kBwdScoreWaves + 0) * kSlots + lane] +
                      part[((c & 1) * kBwdScoreWaves + 1) * kSlots + lane];
      ibuf[c * kSlots + lane] = slot_rows[c * kSlots + lane] >= 0 ? v : -INFINITY;
    }
  };
  // tile c complete (up to three later tiles stay in flight) and published to the work group;
  // every wave is then done with tile c - 1, whose buffer the caller refills
  auto acquire = [&](int c) {
    const int ahead = min(kBwdNBuf - 2, nch - 1 - c);
    if (ahead >= 3) wait_vm<3 * TS::L>();
    else if (ahead == 2) wait_vm<2 * TS::L>();
    else if (ahead == 1) wait_vm<TS::L>();
    else wait_vm<0>();
    lds_barrier();
  };
  auto issue_first = [&]() {  // tiles 0 .. kBwdNBuf - 2 of a pass
#pragma unroll
    for (int c = 0; c < kBwdNBuf - 1; ++c)
      if (c < nch) ts.issue(c, k_idx, slot_rows);
  };

  // ---- pass 1: indexer scores of the row's slots (the contribution waves only keep step with
  // the barriers)
  if (scorer) issue_first();
  for (int c = 0; c < nch; ++c) {
    if (!scorer) {
      lds_barrier();
      continue;
    }
    acquire(c);
    if (c > 0) gather_part(c - 1);
    if (c + kBwdNBuf - 1 < nch) ts.issue(c + kBwdNBuf - 1, k_idx, slot_rows);
    if (p1) {
      // D[head][slot] = q_idx . rows^T, B = the tile's row fragments (slot lane % 32, chunk
      // 2 kk + lane / 32)
      const unsigned char *tile = smem + (c % kBwdNBuf) * TL::kBytes;
      f32x16 acc = {};
#pragma unroll
      for (int kk = 0; kk < kDi / 16; ++kk) {
        const bf16x8 b = as_bf16x8(*reinterpret_cast<const u32x4 *>(
            tile + TL::chunk_off(lane & 31, 2 * kk + (lane >> 5))));
        acc = mfma32(qm[kk], b, acc);
      }
      float sc = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) sc = fmaf(wm[i], fmaxf(acc[i], 0.0f), sc);
      sc += swap_halves(sc);  // the other 16 heads of this half
      if (lane < kSlots) part[((c & 1) * kBwdScoreWaves + wave) * kSlots + lane] = sc;
    }
  }
  lds_barrier();  // every wave is done with the tiles and with the last chunk's partial scores
  if (nch > 0) gather_part(nch - 1);
  // pass 2's first tiles load while the softmax runs
  if (scorer) issue_first();
  lds_barrier();  // scores complete
  // ---- the row's softmax over its slots, the loss and dI (the first contribution wave, which
  // has no tile loads in flight to wait for with its target loads)
  if (wave == kBwdScoreWaves) {
    const int n = nch * kSlots;
    float m = -INFINITY;
    for (int j = lane; j < n; j += 64) m = fmaxf(m, ibuf[j]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    float zs = 0.0f;
    for (int j = lane; j < n; j += 64) zs += ibuf[j] == -INFINITY ? 0.0f : __expf(ibuf[j] - m);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) zs += __shfl_xor(zs, o, 64);
    const float logz = m + __logf(zs);
    float ls = 0.0f;
    for (int j = lane; j < n; j += 64) {
      const float I = ibuf[j];
      float di = 0.0f;
      if (I != -INFINITY) {  // a valid slot (j < lim)
        const float logu = I - logz;
        const float p = target[t * K + j];
        if (p > 0.0f) ls += p * (__logf(p) - logu);
        di = grad * (__expf(logu) - p);
      }
      ibuf[j] = di;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ls += __shfl_xor(ls, o, 64);
    if (lane == 0) loss[t] = nch > 0 ? ls : 0.0f;
  }
  // ---- pass 2: gradients
  if (scorer) {
    f32x4 dq[kDi / 16];  // dq_idx^T[dim 16 n + 4 g + i][head h]
#pragma unroll
    for (int n = 0; n < kDi / 16; ++n) dq[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    float dwa = 0.0f;
    for (int c = 0; c <= nch; ++c) {
      // also: dI is published (c = 0); every wave is done with chunk c - 1's tile, and the
      // contribution waves with the G staged two chunks back
      if (c < nch) acquire(c);
      else lds_barrier();
      if (c == nch) break;
      if (c + kBwdNBuf - 1 < nch) ts.issue(c + kBwdNBuf - 1, k_idx, slot_rows);
      const unsigned char *tile = smem + (c % kBwdNBuf) * TL::kBytes;
      f32x4 d[2];
      dots(tile, d);
      float gv[2][4];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const f32x4 di = *reinterpret_cast<const f32x4 *>(ibuf + c * kSlots + mt * 16 + g * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          gv[mt][i] = d[mt][i] > 0.0f ? di[i] * wv : 0.0f;
          dwa = fmaf(di[i], fmaxf(d[mt][i], 0.0f), dwa);
        }
      }
      // G as a bf16 pair hi + lo: B operands of dq^T and the staged [slot][head] copy for C
      float gl[2][4];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) gl[mt][i] = gv[mt][i] - bf16_to_f32(f32_to_bf16(gv[mt][i]));
      const bf16x8 gh8 = pack_slots(gv), gl8 = pack_slots(gl);
#pragma unroll
      for (int n = 0; n < kDi / 16; ++n) {
        const bf16x8 va = fr.v_frag(tile, n);
        dq[n] = mfma16(va, gh8, dq[n]);
        dq[n] = mfma16(va, gl8, dq[n]);
      }
      uint16_t *zh = stg + (c & 1) * (KlSmem::kStageBytes / 2);
      uint16_t *zl = zh + kSlots * kSS;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int o = (mt * 16 + g * 4 + i) * kSS + h;
          const uint16_t hi = f32_to_bf16(gv[mt][i]);
          zh[o] = hi;
          zl[o] = f32_to_bf16(gv[mt][i] - bf16_to_f32(hi));
        }
    }
    // ---- dq_idx (bf16) and dw of this wave's heads
    if (hok) {
      uint16_t *row = dq_idx + (t * Hi + h) * kDi + g * 4;
#pragma unroll
      for (int n = 0; n < kDi / 16; ++n) {
        u32x2 v;
        v[0] = pack_bf16x2(dq[n][0], dq[n][1]);
        v[1] = pack_bf16x2(dq[n][2], dq[n][3]);
        *reinterpret_cast<u32x2 *>(row + n * 16) = v;
      }
    }
    dwa += __shfl_xor(dwa, 16, 64);
    dwa += __shfl_xor(dwa, 32, 64);
    if (hok && g == 0) dw[t * Hi + h] = dwa;
  } else {
    const int qd = wave - kBwdScoreWaves;
    for (int c = 0; c <= nch; ++c) {
      lds_barrier();  // G of chunk c - 1 is staged
      if (c == 0) continue;
      // C^T[dims 32 qd .. + 31 x 32 slots] of chunk c - 1 from the staged G (hi + lo)
      const int cc = c - 1;
      const uint16_t *zh = stg + (cc & 1) * (KlSmem::kStageBytes / 2);
      const uint16_t *zl = zh + kSlots * kSS;
      const int32_t *rr = slot_rows + cc * kSlots;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          const int off = (mt * 16 + hl) * kSS + kh * 32 + g * 8;
          const bf16x8 bh = as_bf16x8(*reinterpret_cast<const u32x4 *>(zh + off));
          const bf16x8 bl = as_bf16x8(*reinterpret_cast<const u32x4 *>(zl + off));
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            acc[m] = mfma16(qa[m][kh], bh, acc[m]);
            acc[m] = mfma16(qa[m][kh], bl, acc[m]);
          }
        }
        // staged row of slot cc*32 + 16 mt + hl: this lane's block is dims
        // 32 qd + 16 m + 4 g + i (block 4 qd + g)
        if (rr[mt * 16 + hl] >= 0) {
          float mx = 0.0f;
#pragma unroll
          for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(acc[m][i]));
          const uint32_t eb = min(__float_as_uint(mx) >> 23, 253u);
          const float sc = __uint_as_float((253u - eb) << 23);  // 2^-e
          uint32_t *row = stage + (i_row * K + cc * kSlots + mt * 16 + hl) * kStageWords<kDi>;
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            u32x2 v;
            v[0] = pknorm16(acc[m][0] * sc, acc[m][1] * sc);
            v[1] = pknorm16(acc[m][2] * sc, acc[m][3] * sc);
            *reinterpret_cast<u32x2 *>(row + ((32 * qd + 16 * m + 4 * g) >> 1)) = v;
          }
          reinterpret_cast<unsigned char *>(row + kDi / 2)[4 * qd + g] =
              static_cast<unsigned char>(eb);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_indexer_kl_target(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                                    const int32_t *topk_length, const float *lse, int64_t T_q,
                                    int32_t H, int32_t D_qk, int32_t K, float scale,
                                    float *target, hipStream_t s) {
  if (T_q == 0) return hipSuccess;
  auto go = [&](auto kern, size_t smem) -> hipError_t {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(smem));
    if (e != hipSuccess) return e;
    DSA_LAUNCH("indexer_kl_target", kern, dim3(static_cast<unsigned>(T_q)), dim3(kWaves * 64),
               smem, s, q, kv, idx, topk_length, lse, H, K, scale * kLog2e, target);
    return hipGetLastError();
  };
  if (D_qk == 576) return go(kl_target_kernel<576>, static_cast<size_t>(TargetSmem<576>::kBytes));
  if (D_qk == 512) return go(kl_target_kernel<512>, static_cast<size_t>(TargetSmem<512>::kBytes));
  return hipErrorInvalidValue;
}

hipError_t launch_indexer_kl_bwd(const uint16_t *q_idx, const uint16_t *k_idx, const float *w,
                                 const int32_t *idx, const int32_t *topk_length,
                                 const float *target, int64_t T_q, int64_t T_kv, int32_t H_i,
                                 int32_t K, float grad, float *loss, uint16_t *dq_idx, float *dw,
                                 float *dk_idx, bool accumulate, const BwdPassBuffers &bb,
                                 int64_t rows_per_pass, hipStream_t s) {
  hipError_t e = hipSuccess;
  if (!accumulate && (e = launch_fill_zero(dk_idx, T_kv * kDi, s)) != hipSuccess) return e;
  if (T_q == 0) return hipSuccess;
  const size_t smem = KlSmem::bytes(K);
  if ((e = hipFuncSetAttribute(reinterpret_cast<const void *>(kl_bwd_kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize,
                               static_cast<int>(smem))) != hipSuccess)
    return e;
  for (int64_t r0 = 0; e == hipSuccess && r0 < T_q; r0 += rows_per_pass) {
    const int64_t n = std::min<int64_t>(rows_per_pass, T_q - r0);
    e = launch_pair_count_zero(T_kv, bb, s);
    if (e != hipSuccess) break;
    DSA_LAUNCH("indexer_kl_bwd", kl_bwd_kernel, dim3(static_cast<unsigned>(n)), dim3(kBwdWaves * 64),
               smem, s, q_idx, k_idx, w, idx, topk_length, target, H_i, K, grad, loss, dq_idx, dw,
               bb.stage, bb.off, r0);
    if ((e = hipGetLastError()) != hipSuccess) break;
    e = launch_pair_sort(idx, topk_length, r0, n, T_kv, K, bb, s);
    if (e == hipSuccess) e = launch_pair_reduce(kDi, T_kv, bb, dk_idx, s);
  }
  return e;
}

}  // namespace dsa
