// Absorbed sparse MLA forward (NVIDIA GLM-5.2 cuDNN DSA page, "Why DSA needs fused kernels":
// all heads of a query attend one top-k set, so the MMA M axis is tiled from heads in an
// MQA-style layout; NeMo AutoModel cudnn_dsa API reference, cudnn_sparse_attention: q
// [T_q,H,576], latent rows [T_kv,576], values = first 512 channels, -1 slots masked, optional
// valid-prefix lengths, softmax_scale applied unchanged; SkyRL PR 2388 for the 512-wide NoPE
// layout and top-k widths that are not a multiple of 64).
//
// Work group = one query row, ceil(H/16) waves, wave w owning heads [16w, 16w+16).  The row's
// valid slots are processed in chunks of 32: the 32 latent rows are gathered into LDS with
// 16-byte loads, then each wave computes
//   S^T[32 slots x 16 heads] = rows . q^T          (16x16x32 bf16 MFMA, A = LDS rows,
//                                                   B = the wave's q block held in registers)
// runs the online softmax in fp32 (base 2), and accumulates
//   O[16 heads x 512] += P . V                       (A = P straight from the S^T registers,
//                                                   B = V read from the same row-major LDS
//                                                   tile with transposing LDS reads)
// The slot order inside the P.V contraction is permuted so that P needs no data movement:
// the lane holding S^T rows (lane/16)*4 + [0,4) of both 16-slot halves supplies exactly the
// eight contraction indices it owns in the MFMA A layout, and the transposing reads fetch V
// rows in the same order.
#include "dsa_common.h"
#include "dsa_internal.h"
#include "tile.h"

namespace dsa {
namespace {

constexpr int kSlots = 32;  // slots per chunk
constexpr int kDv = 512;
constexpr int kMaxK = 4096;  // largest top-k width whose index row fits the LDS copy

// Tile buffers in flight: a wave with few loads per tile keeps NBUF - 1 tiles in flight.
template <int NW>
constexpr int fwd_buffers() { return NW == 1 ? 2 : 4; }

template <int DQK, int NW>
constexpr size_t fwd_smem_bytes() {
  return static_cast<size_t>(fwd_buffers<NW>()) * Tile<DQK>::kBytes + kMaxK * sizeof(int32_t);
}

template <int DQK, int NW>
__global__ __launch_bounds__(NW * 64) void sparse_mla_fwd_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kv,
    const int32_t *__restrict__ idx, const int32_t *__restrict__ topk_length, int H, int K,
    float scale_log2, uint16_t *__restrict__ out, float *__restrict__ lse) {
  using TL = Tile<DQK>;
  constexpr int kKSteps = DQK / 32;
  constexpr int NBUF = fwd_buffers<NW>();
  constexpr int L = TL::kLoads / NW;  // DMA loads per wave per tile
  static_assert(TL::kLoads % NW == 0, "loads must split evenly over the waves");
  extern __shared__ __align__(16) unsigned char smem[];
  int32_t *slot_rows = reinterpret_cast<int32_t *>(smem + NBUF * TL::kBytes);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t t = blockIdx.x;
  const int h0 = wave * 16;
  const int g = lane >> 4;     // lane group
  const int hl = lane & 15;    // head within the wave's tile
  const int lim = topk_length ? topk_length[t] : K;
  const int32_t *irow = idx + t * K;
  const int nchunks = (lim + kSlots - 1) / kSlots;

  // q block of this wave as the MFMA B operand: lane -> head hl, dims ks*32 + g*8 + [0,8)
  bf16x8 qf[kKSteps];
  {
    const int h = h0 + hl;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (h < H) v = *reinterpret_cast<const u32x4 *>(q + ((t * H + h) * DQK + ks * 32 + g * 8));
      qf[ks] = as_bf16x8(v);
    }
  }
  // the query's slot -> latent row map (tail of the last chunk marked invalid)
  for (int j = threadIdx.x; j < nchunks * kSlots; j += NW * 64)
    slot_rows[j] = j < lim ? irow[j] : -1;
  // finish the q loads before the first tile load (see settle())
#pragma unroll
  for (int ks = 0; ks < kKSteps; ++ks) settle(qf[ks]);
  __syncthreads();

  // Per-lane LDS offsets, fixed for the whole kernel (the swizzle only permutes the low four
  // bits of a chunk index, so a chunk 16*a + b lands at (16*a + (b ^ swz)) * 16).
  //   S^T A operand, tile row mt*16 + hl, chunk ks*4 + g:  sbase[mt][ks & 3] + (ks >> 2) * 256
  //   V (transposing reads), rows 4g + r4 and 16 + 4g + r4, element col n*16 + cq*4:
  //                                                        vbase[j][n & 7] + (n >> 3) * 256
  const int r4 = (lane & 15) >> 2;
  const int cq = lane & 3;
  int sbase[2][4], vbase[2][8];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j) sbase[mt][j] = TL::chunk_off(mt * 16 + hl, j * 4 + g);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    vbase[0][j] = TL::elem_off(g * 4 + r4, j * 16 + cq * 4);
    vbase[1][j] = TL::elem_off(16 + g * 4 + r4, j * 16 + cq * 4);
  }
  // this lane's DMA targets: (tile row, byte offset inside the row) for each of its L loads;
  // the latent tensor is below 4 GiB (checked by the host), so a 32-bit offset from its base
  // addresses any row
  int dma_row[L], dma_off[L];
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const int pos = (i * NW + wave) * 64 + lane;
    dma_row[i] = pos / TL::kChunks;
    dma_off[i] = ((pos % TL::kChunks) ^ TL::swz(dma_row[i])) * 16;
  }
  const uint32_t smem_lds = lds_addr(smem);
  auto issue = [&](int c) {
    const uint32_t tile = smem_lds + (c % NBUF) * TL::kBytes + wave * 1024;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      int r = slot_rows[c * kSlots + dma_row[i]];
      r = r < 0 ? 0 : r;
      dma16_sv(kv, static_cast<uint32_t>(r) * TL::kRowBytes + dma_off[i],
               tile + i * NW * 1024);
    }
  };
#pragma unroll
  for (int c = 0; c < NBUF - 1; ++c)
    if (c < nchunks) issue(c);

  f32x4 o[kDv / 16];  // O^T tiles: o[n][i] = O[head hl][channel 16n + 4g + i]
#pragma unroll
  for (int n = 0; n < kDv / 16; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  // reference max (base-2 logits) of head hl; a finite floor keeps exp2(x - m_run) = 0 for
  // masked slots (x = -inf) even before the first valid slot
  float m_run = -1e30f;
  float l_run = 0.0f;       // this lane's partial softmax denominator of head hl

  for (int c = 0; c < nchunks; ++c) {
    const int ahead = min(NBUF - 2, nchunks - 1 - c);  // later tiles already issued
    wait_tiles_ahead<L, NBUF>(ahead);
    lds_barrier();  // tile c is complete in LDS; buffer (c - 1) % NBUF is free
    if (c + NBUF - 1 < nchunks) issue(c + NBUF - 1);
    const unsigned char *tile = smem + (c % NBUF) * TL::kBytes;

    // ---- S^T = rows . q^T   (acc[mt][i] = S^T[slot 16mt + 4g + i][head hl])
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4 *>(
            tile + sbase[mt][ks & 3] + (ks >> 2) * 256));
        acc[mt] = mfma16(a, qf[ks], acc[mt]);
      }
    }

    // ---- online softmax (base 2) with a lazily raised reference max: the reference only
    // moves when the running max exceeds it by more than 2^8, so P <= 256 and O is rescaled
    // only a handful of times per row.  Lanes hl, hl^16, hl^32, hl^48 share head hl.
    const u32x4 rv0 = *reinterpret_cast<const u32x4 *>(&slot_rows[c * kSlots + g * 4]);
    const u32x4 rv1 = *reinterpret_cast<const u32x4 *>(&slot_rows[c * kSlots + 16 + g * 4]);
    float x[2][4];
    float cmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[0][i] = static_cast<int32_t>(rv0[i]) >= 0 ? acc[0][i] * scale_log2 : -INFINITY;
      x[1][i] = static_cast<int32_t>(rv1[i]) >= 0 ? acc[1][i] * scale_log2 : -INFINITY;
      cmax = fmaxf(cmax, fmaxf(x[0][i], x[1][i]));
    }
    cmax = fmaxf(cmax, xor_lane(cmax, 16));
    cmax = fmaxf(cmax, swap_halves(cmax));
    if (__ballot(cmax > m_run + 8.0f)) {
      const float m_new = cmax > m_run + 8.0f ? cmax : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the first raise
      l_run *= alpha;
#pragma unroll
      for (int n = 0; n < kDv / 16; ++n) o[n] *= alpha;
      m_run = m_new;
    }
    float p[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[mt][i] = __builtin_amdgcn_exp2f(x[mt][i] - m_run);  // 0 for masked slots
        l_run += p[mt][i];
      }

    // ---- O^T += V^T . P^T   (slot k-index 8g + j <-> tile row 4g + j (j < 4), 16 + 4g + j - 4)
    u32x4 pw;
    pw[0] = pack_bf16x2(p[0][0], p[0][1]);
    pw[1] = pack_bf16x2(p[0][2], p[0][3]);
    pw[2] = pack_bf16x2(p[1][0], p[1][1]);
    pw[3] = pack_bf16x2(p[1][2], p[1][3]);
    const bf16x8 pb = as_bf16x8(pw);
#pragma unroll
    for (int n = 0; n < kDv / 16; ++n) {
      const u32x2 lo = lds_read_tr16(tile + vbase[0][n & 7] + (n >> 3) * 256);
      const u32x2 hi = lds_read_tr16(tile + vbase[1][n & 7] + (n >> 3) * 256);
      const u32x4 va = {lo[0], lo[1], hi[0], hi[1]};
      o[n] = mfma16(as_bf16x8(va), pb, o[n]);
    }
  }

  // ---- finalize: denominator over the four lane groups, normalise, write
  float l_tot = l_run + xor_lane(l_run, 16);
  l_tot += swap_halves(l_tot);
  const int h = h0 + hl;
  if (h < H) {
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    if (g == 0)
      lse[t * H + h] = l_tot > 0.0f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
    uint16_t *orow = out + (t * H + h) * kDv + g * 4;
#pragma unroll
    for (int n = 0; n < kDv / 16; ++n) {
      u32x2 v;
      v[0] = pack_bf16x2(o[n][0] * inv, o[n][1] * inv);
      v[1] = pack_bf16x2(o[n][2] * inv, o[n][3] * inv);
      *reinterpret_cast<u32x2 *>(orow + n * 16) = v;
    }
  }
}

template <int DQK, int NW>
hipError_t launch(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                  const int32_t *topk_length, int64_t T_q, int32_t H, int32_t K, float scale,
                  uint16_t *out, float *lse, hipStream_t s) {
  constexpr size_t smem = fwd_smem_bytes<DQK, NW>();
  auto kern = sparse_mla_fwd_kernel<DQK, NW>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(smem));
  if (e != hipSuccess) return e;
  DSA_LAUNCH("sparse_mla_fwd", kern, dim3(static_cast<unsigned>(T_q)), dim3(NW * 64), smem, s,
             q, kv, idx, topk_length, H, K, scale * kLog2e, out, lse);
  return hipGetLastError();
}

template <int DQK>
hipError_t launch_w(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                    const int32_t *topk_length, int64_t T_q, int32_t H, int32_t K, float scale,
                    uint16_t *out, float *lse, hipStream_t s) {
  if (H <= 16) return launch<DQK, 1>(q, kv, idx, topk_length, T_q, H, K, scale, out, lse, s);
  if (H <= 32) return launch<DQK, 2>(q, kv, idx, topk_length, T_q, H, K, scale, out, lse, s);
  if (H <= 64) return launch<DQK, 4>(q, kv, idx, topk_length, T_q, H, K, scale, out, lse, s);
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
