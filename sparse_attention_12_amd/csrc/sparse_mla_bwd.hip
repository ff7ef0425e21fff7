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
//   delta  : Delta[t,h] = sum_c dO[t,h,c] O[t,h,c]          (streaming, one wave per (t,h))
//   rows   : one launch whose even work groups compute dq and odd work groups the key-gradient
//            contributions of the same query rows, so the LDS/MFMA-bound dq work and the
//            HBM-bound contribution stores overlap on every CU.
//     dq   : waves own 16 heads each.  Per 32-slot chunk the latent rows are gathered into
//            LDS; S^T and dP^T come from 16x16x32 bf16 MFMAs with the row tile as A and the
//            wave's q / dO blocks (registers) as B; dZ is formed in registers and dq += dZ . rows
//            uses dZ as the A operand directly (same slot permutation as the forward's P . V)
//            and transposing LDS reads for the rows.
//     contributions : 4 waves.  The row's q and dO blocks are first staged through LDS and read
//            back transposed into registers so that the head axis is the MFMA contraction
//            axis; wave w owns a quarter of the latent channels.  Per chunk the waves recompute
//            S^T / dP^T for their head tile, publish scale * dZ^T and P^T in LDS, each as a bf16
//            pair hi + lo (hi = bf16(x), lo = bf16(x - hi), about 16 significant bits), and
//            every wave then forms C[32 slots x its channels] = (scale dZ)^T . q + P^T . dO from
//            the four bf16 products (plain bf16 rounding of P and dZ, 8 bits, would leave a
//            visible error in latent rows picked by thousands of queries).  C is stored in fp32
//            to a staging buffer, one row per (query, slot).
//   count / scan / fill : a counting sort of the pass's (query, slot) pairs by latent row.
//   reduce : one work group per latent row adds up its staged contributions and adds the sum
//            to dkv (every row has a single owner, so no atomics touch dkv).
// Compared with fp32 atomics on dkv (bounded by the L2 atomic units at about one 4-byte add
// per channel per clock), staging moves 8 bytes of HBM traffic per contribution element.
#include <algorithm>

#include "dsa_common.h"
#include "dsa_internal.h"
#include "tile.h"

namespace dsa {
namespace {

constexpr int kSlots = 32;
constexpr int kDv = 512;

// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_delta_kernel(const uint16_t *__restrict__ out,
                                                        const uint16_t *__restrict__ dout,
                                                        int64_t rows, float *__restrict__ delta) {
  const int lane = threadIdx.x & 63;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const u32x4 a = *reinterpret_cast<const u32x4 *>(out + r * kDv + lane * 8);
  const u32x4 b = *reinterpret_cast<const u32x4 *>(dout + r * kDv + lane * 8);
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s = fmaf(__uint_as_float(a[i] << 16), __uint_as_float(b[i] << 16), s);
    s = fmaf(__uint_as_float(a[i] & 0xFFFF0000u), __uint_as_float(b[i] & 0xFFFF0000u), s);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  if (lane == 0) delta[r] = s;
}

__global__ void fill_zero_kernel(float *__restrict__ p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t j = i; j < n; j += stride) p[j] = 0.0f;
}

constexpr int kRowWaves = 4;  // waves of a work group of the rows launch
constexpr int kRowBufs = 3;   // latent-row tile buffers
constexpr int kMaxK = 4096;   // largest top-k width whose index row fits the LDS copy

template <int DQK>
using RowStream = TileStream<DQK, kRowWaves, kRowBufs>;

// LDS of a rows work group: tile buffers | slot rows [kMaxK] | (contributions) dZ / P staging
template <int DQK, int HP>
struct RowSmem {
  static constexpr int kTiles = kRowBufs * Tile<DQK>::kBytes;
  static constexpr int kSlotRows = kTiles;
  static constexpr int kStage = kSlotRows + kMaxK * 4;
  static constexpr int kStageStride = HP + 8;  // [slot][head] bf16 rows (+16 B)
  static constexpr int kStageBytes = 4 * kSlots * kStageStride * 2;
  static constexpr int kBytes = kStage + kStageBytes;
  // prologue staging of the row's q ([HP][DQK+16]) and dO ([HP][512+16]) in the tile area
  static constexpr int kQStride = DQK + 16;
  static constexpr int kOStride = kDv + 16;
  static_assert(HP * kQStride * 2 <= kTiles, "q staging must fit the tile area");
};

// The query row's slot -> latent row map in LDS (-1 for invalid slots, padded to whole tiles),
// then the per-head operands shared by both row paths.
struct RowHead {
  int lim, nchunks;
  float lse2, dlt;
};

template <int DQK>
__device__ __forceinline__ RowHead row_setup(const int32_t *__restrict__ idx,
                                             const int32_t *__restrict__ topk_length,
                                             const float *__restrict__ lse,
                                             const float *__restrict__ delta, int H, int K,
                                             int64_t t, int h, int32_t *slot_rows) {
  RowHead r;
  r.lim = topk_length ? topk_length[t] : K;
  r.nchunks = (r.lim + kSlots - 1) / kSlots;
  const int32_t *irow = idx + t * K;
  for (int j = threadIdx.x; j < r.nchunks * kSlots; j += kRowWaves * 64)
    slot_rows[j] = j < r.lim ? irow[j] : -1;
  const bool hok = h < H;
  const float l0 = hok ? lse[t * H + h] : 0.0f;
  r.lse2 = l0 == -INFINITY ? INFINITY : l0 * kLog2e;  // empty row: P = 0
  r.dlt = hok ? delta[t * H + h] : 0.0f;
  return r;
}

// S^T and dP^T of the wave's 16-head tile over the 32 slots of `tile`, then P and dZ in the
// S^T fragment layout (slot 16 mt + 4 g + i, head hl).
template <int DQK>
__device__ __forceinline__ void slot_grads(const unsigned char *tile, const TileFrag<DQK> &fr,
                                           const int32_t *slot_rows_c, const bf16x8 *qf,
                                           const bf16x8 *df, float lse2, float dlt,
                                           float scale_log2, float p[2][4], float dz[2][4]) {
  const int g = __lane_id() >> 4;
  f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  f32x4 dp[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int ks = 0; ks < DQK / 32; ++ks) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const bf16x8 a = fr.a_frag(tile, mt, ks);
      s[mt] = mfma16(a, qf[ks], s[mt]);
      if (ks < kDv / 32) dp[mt] = mfma16(a, df[ks], dp[mt]);
    }
  }
  const u32x4 rv0 = *reinterpret_cast<const u32x4 *>(slot_rows_c + g * 4);
  const u32x4 rv1 = *reinterpret_cast<const u32x4 *>(slot_rows_c + 16 + g * 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool v0 = static_cast<int32_t>(rv0[i]) >= 0, v1 = static_cast<int32_t>(rv1[i]) >= 0;
    p[0][i] = v0 ? __builtin_amdgcn_exp2f(s[0][i] * scale_log2 - lse2) : 0.0f;
    p[1][i] = v1 ? __builtin_amdgcn_exp2f(s[1][i] * scale_log2 - lse2) : 0.0f;
    dz[0][i] = p[0][i] * (dp[0][i] - dlt);
    dz[1][i] = p[1][i] * (dp[1][i] - dlt);
  }
}

// q / dO block of the wave's head tile as MFMA B operands (lane -> head hl, dims ks*32 + g*8).
template <int DQK>
__device__ __forceinline__ void load_head_frags(const uint16_t *__restrict__ q,
                                                const uint16_t *__restrict__ dout, int H,
                                                int64_t t, int h, bf16x8 *qf, bf16x8 *df) {
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

// ---------------------------------------------------------------------------------------
// dq of query row t: dq^T[channels x 16 heads] += rows^T . dZ^T per tile (A = transposing
// reads of the row tile, B = dZ packed from registers), so a lane ends with channels
// 16 n + 4 g .. + 3 of head hl.
template <int DQK, int HP>
__device__ __forceinline__ void bwd_dq_row(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kv,
    const int32_t *__restrict__ idx, const int32_t *__restrict__ topk_length,
    const float *__restrict__ lse, const float *__restrict__ delta,
    const uint16_t *__restrict__ dout, int H, int K, float scale, float scale_log2,
    uint16_t *__restrict__ dq, int64_t t, unsigned char *smem) {
  using SM = RowSmem<DQK, HP>;
  constexpr int kNT = DQK / 16;
  int32_t *slot_rows = reinterpret_cast<int32_t *>(smem + SM::kSlotRows);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, hl = lane & 15;
  const int h = wave * 16 + hl;
  const bool active = wave * 16 < H;  // waves without heads only help with the loads

  bf16x8 qf[DQK / 32], df[kDv / 32];
  load_head_frags<DQK>(q, dout, H, t, h, qf, df);
  const RowHead rh = row_setup<DQK>(idx, topk_length, lse, delta, H, K, t, h, slot_rows);
#pragma unroll
  for (int ks = 0; ks < DQK / 32; ++ks) settle(qf[ks]);
#pragma unroll
  for (int ks = 0; ks < kDv / 32; ++ks) settle(df[ks]);
  __syncthreads();

  RowStream<DQK> ts;
  ts.init(smem, wave);
  TileFrag<DQK> fr;
  fr.init();
#pragma unroll
  for (int c = 0; c < kRowBufs - 1; ++c)
    if (c < rh.nchunks) ts.issue(c, kv, slot_rows);

  f32x4 acc[kNT];
#pragma unroll
  for (int n = 0; n < kNT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < rh.nchunks; ++c) {
    RowStream<DQK>::acquire(c, rh.nchunks);
    if (c + kRowBufs - 1 < rh.nchunks) ts.issue(c + kRowBufs - 1, kv, slot_rows);
    if (!active) continue;
    const unsigned char *tile = smem + (c % kRowBufs) * Tile<DQK>::kBytes;
    float p[2][4], dz[2][4];
    slot_grads<DQK>(tile, fr, slot_rows + c * kSlots, qf, df, rh.lse2, rh.dlt, scale_log2, p,
                    dz);
    const bf16x8 zb = pack_slots(dz);
#pragma unroll
    for (int n = 0; n < kNT; ++n) acc[n] = mfma16(fr.v_frag(tile, n), zb, acc[n]);
  }
  if (active && h < H) {
    uint16_t *row = dq + (t * H + h) * DQK + g * 4;
#pragma unroll
    for (int n = 0; n < kNT; ++n) {
      u32x2 v;
      v[0] = pack_bf16x2(acc[n][0] * scale, acc[n][1] * scale);
      v[1] = pack_bf16x2(acc[n][2] * scale, acc[n][3] * scale);
      *reinterpret_cast<u32x2 *>(row + n * 16) = v;
    }
  }
}

// ---------------------------------------------------------------------------------------
// Key-gradient contributions of query row t, stored to stage[slot][DQK] (fp32) for every
// valid slot.  Wave w owns latent channels [w DQK / 4, (w + 1) DQK / 4).
template <int DQK, int HP>  // HP: head count padded to the contraction width (32 or 64)
__device__ __forceinline__ void bwd_contrib_row(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kv,
    const int32_t *__restrict__ idx, const int32_t *__restrict__ topk_length,
    const float *__restrict__ lse, const float *__restrict__ delta,
    const uint16_t *__restrict__ dout, int H, int K, float scale, float scale_log2,
    float *__restrict__ stage, int64_t t, unsigned char *smem_raw) {
  using SM = RowSmem<DQK, HP>;
  constexpr int kChanPerWave = DQK / kRowWaves;  // 144 or 128
  constexpr int kNTw = kChanPerWave / 16;        // output tiles per wave (9 or 8)
  constexpr int kKH = HP / 32;                   // head contraction steps
  constexpr int kSS = SM::kStageStride;
  uint16_t *qstage = reinterpret_cast<uint16_t *>(smem_raw);  // prologue only
  int32_t *slot_rows = reinterpret_cast<int32_t *>(smem_raw + SM::kSlotRows);
  uint16_t *zst = reinterpret_cast<uint16_t *>(smem_raw + SM::kStage);  // scale*dZ^T hi
  uint16_t *zsl = zst + kSlots * kSS;                                    //            lo
  uint16_t *pst = zsl + kSlots * kSS;                                    // P^T        hi
  uint16_t *psl = pst + kSlots * kSS;                                    //            lo

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, hl = lane & 15;
  const int r = (lane & 15) >> 2;
  const int cq = lane & 3;
  const int ch0 = wave * kChanPerWave;  // first latent channel owned by this wave
  constexpr int kThreads = kRowWaves * 64;

  // ---- prologue: heads-as-contraction fragments of q and dO for this wave's channels
  bf16x8 qh[kKH][kNTw], oh[kKH][kNTw];
  for (int c = threadIdx.x; c < HP * (DQK / 8); c += kThreads) {
    const int hh = c / (DQK / 8), col = (c % (DQK / 8)) * 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (hh < H) v = *reinterpret_cast<const u32x4 *>(q + (t * H + hh) * DQK + col);
    *reinterpret_cast<u32x4 *>(&qstage[hh * SM::kQStride + col]) = v;
  }
  __syncthreads();
#pragma unroll
  for (int kh = 0; kh < kKH; ++kh)
#pragma unroll
    for (int n = 0; n < kNTw; ++n) {
      const uint16_t *base = &qstage[(kh * 32 + g * 8 + r) * SM::kQStride + ch0 + n * 16 + cq * 4];
      const u32x2 lo = lds_read_tr16(base);
      const u32x2 hi = lds_read_tr16(base + 4 * SM::kQStride);
      qh[kh][n] = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
    }
  __syncthreads();
  for (int c = threadIdx.x; c < HP * (kDv / 8); c += kThreads) {
    const int hh = c / (kDv / 8), col = (c % (kDv / 8)) * 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (hh < H) v = *reinterpret_cast<const u32x4 *>(dout + (t * H + hh) * kDv + col);
    *reinterpret_cast<u32x4 *>(&qstage[hh * SM::kOStride + col]) = v;
  }
  __syncthreads();
#pragma unroll
  for (int kh = 0; kh < kKH; ++kh)
#pragma unroll
    for (int n = 0; n < kNTw; ++n) {
      const int ch = ch0 + n * 16;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (ch < kDv) {
        const uint16_t *base = &qstage[(kh * 32 + g * 8 + r) * SM::kOStride + ch + cq * 4];
        const u32x2 lo = lds_read_tr16(base);
        const u32x2 hi = lds_read_tr16(base + 4 * SM::kOStride);
        v = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
      oh[kh][n] = as_bf16x8(v);
    }
  // padded heads of the staging arrays stay zero for the whole kernel
  for (int c = threadIdx.x; c < 4 * kSlots * kSS; c += kThreads) zst[c] = 0;

  // ---- this wave's head tile for the S^T / dP^T recompute (waves beyond the tiles idle)
  const int h = wave * 16 + hl;
  const bool tile_active = wave * 16 < H;
  const bool hok = h < H;
  bf16x8 qf[DQK / 32], df[kDv / 32];
  load_head_frags<DQK>(q, dout, H, t, h, qf, df);
  __syncthreads();  // the q / dO staging is read; the tile area may be refilled
  const RowHead rh = row_setup<DQK>(idx, topk_length, lse, delta, H, K, t, h, slot_rows);
#pragma unroll
  for (int ks = 0; ks < DQK / 32; ++ks) settle(qf[ks]);
#pragma unroll
  for (int ks = 0; ks < kDv / 32; ++ks) settle(df[ks]);
  __syncthreads();

  RowStream<DQK> ts;
  ts.init(smem_raw, wave);
  TileFrag<DQK> fr;
  fr.init();
#pragma unroll
  for (int c = 0; c < kRowBufs - 1; ++c)
    if (c < rh.nchunks) ts.issue(c, kv, slot_rows);

  for (int c = 0; c < rh.nchunks; ++c) {
    RowStream<DQK>::acquire(c, rh.nchunks);  // also: every wave is done with the staging
    if (c + kRowBufs - 1 < rh.nchunks) ts.issue(c + kRowBufs - 1, kv, slot_rows);
    const unsigned char *tile = smem_raw + (c % kRowBufs) * Tile<DQK>::kBytes;
    if (tile_active) {
      float p[2][4], dz[2][4];
      slot_grads<DQK>(tile, fr, slot_rows + c * kSlots, qf, df, rh.lse2, rh.dlt, scale_log2,
                      p, dz);
      if (hok) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int o = (mt * 16 + g * 4 + i) * kSS + h;
            const float zv = dz[mt][i] * scale;
            const uint16_t zh = f32_to_bf16(zv), ph = f32_to_bf16(p[mt][i]);
            zst[o] = zh;
            zsl[o] = f32_to_bf16(zv - bf16_to_f32(zh));
            pst[o] = ph;
            psl[o] = f32_to_bf16(p[mt][i] - bf16_to_f32(ph));
          }
      }
    }
    lds_barrier();
    // contributions[slot][channel] for this wave's channels
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x4 acc[kNTw];
#pragma unroll
      for (int n = 0; n < kNTw; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kh = 0; kh < kKH; ++kh) {
        const int off = (mt * 16 + hl) * kSS + kh * 32 + g * 8;
        const bf16x8 za = as_bf16x8(*reinterpret_cast<const u32x4 *>(&zst[off]));
        const bf16x8 zl = as_bf16x8(*reinterpret_cast<const u32x4 *>(&zsl[off]));
        const bf16x8 pa = as_bf16x8(*reinterpret_cast<const u32x4 *>(&pst[off]));
        const bf16x8 pl = as_bf16x8(*reinterpret_cast<const u32x4 *>(&psl[off]));
#pragma unroll
        for (int n = 0; n < kNTw; ++n) {
          acc[n] = mfma16(za, qh[kh][n], acc[n]);
          acc[n] = mfma16(zl, qh[kh][n], acc[n]);
          if (ch0 + n * 16 < kDv) {
            acc[n] = mfma16(pa, oh[kh][n], acc[n]);
            acc[n] = mfma16(pl, oh[kh][n], acc[n]);
          }
        }
      }
      // acc[n][i] -> stage[slot c*32 + 16mt + 4g + i][ch0 + 16n + hl] (valid slots only)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int sl = mt * 16 + g * 4 + i;
        if (slot_rows[c * kSlots + sl] >= 0) {
          float *dst = stage + static_cast<int64_t>(c * kSlots + sl) * DQK + ch0 + hl;
#pragma unroll
          for (int n = 0; n < kNTw; ++n) dst[n * 16] = acc[n][i];
        }
      }
    }
  }
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
// rows launch: work group 2i computes dq of query row row0 + i, 2i + 1 its contributions
template <int DQK, int HP>
constexpr size_t rows_smem_bytes() {
  return RowSmem<DQK, HP>::kBytes;
}

template <int DQK, int HP>
__global__ __launch_bounds__(kRowWaves * 64) void bwd_rows_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kv,
    const int32_t *__restrict__ idx, const int32_t *__restrict__ topk_length,
    const float *__restrict__ lse, const float *__restrict__ delta,
    const uint16_t *__restrict__ dout, int H, int K, float scale, float scale_log2,
    uint16_t *__restrict__ dq, float *__restrict__ stage, int64_t row0) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int64_t i = blockIdx.x >> 1;
  const int64_t t = row0 + i;
  if (blockIdx.x & 1)
    bwd_contrib_row<DQK, HP>(q, kv, idx, topk_length, lse, delta, dout, H, K, scale, scale_log2,
                             stage + i * K * DQK, t, smem);
  else
    bwd_dq_row<DQK, HP>(q, kv, idx, topk_length, lse, delta, dout, H, K, scale, scale_log2, dq,
                        t, smem);
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

__global__ void pair_count_kernel(const int32_t *__restrict__ idx,
                                  const int32_t *__restrict__ topk_length, int64_t row0,
                                  int64_t rows, int K, int32_t *__restrict__ cnt) {
  const int64_t p = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  int32_t s;
  if (pair_row(idx, topk_length, row0, rows, K, p, s)) atomicAdd(&cnt[s], 1);
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
// channels 4 l + 256 c (c < DQK / 256 rounded up).
template <int DQK>
__global__ __launch_bounds__(256) void pair_reduce_kernel(const int32_t *__restrict__ off,
                                                          const int32_t *__restrict__ list,
                                                          const float *__restrict__ stage,
                                                          int64_t n_rows, float *__restrict__ dkv) {
  constexpr int kVec = (DQK / 4 + 63) / 64;  // float4 per lane (3 for 576, 2 for 512)
  const int lane = threadIdx.x & 63;
  const int64_t s = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (s >= n_rows) return;
  const int b = off[s], e = off[s + 1];
  if (b == e) return;
  f32x4 acc[kVec];
#pragma unroll
  for (int c = 0; c < kVec; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  int k = b;
  for (; k + 1 < e; k += 2) {  // two contributions in flight per iteration
    const float *r0 = stage + static_cast<int64_t>(list[k]) * DQK;
    const float *r1 = stage + static_cast<int64_t>(list[k + 1]) * DQK;
    f32x4 v0[kVec], v1[kVec];
#pragma unroll
    for (int c = 0; c < kVec; ++c) {
      const int ch = 4 * lane + 256 * c;
      v0[c] = ch < DQK ? *reinterpret_cast<const f32x4 *>(r0 + ch) : f32x4{0.f, 0.f, 0.f, 0.f};
      v1[c] = ch < DQK ? *reinterpret_cast<const f32x4 *>(r1 + ch) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int c = 0; c < kVec; ++c) acc[c] += v0[c] + v1[c];
  }
  if (k < e) {
    const float *r0 = stage + static_cast<int64_t>(list[k]) * DQK;
#pragma unroll
    for (int c = 0; c < kVec; ++c) {
      const int ch = 4 * lane + 256 * c;
      if (ch < DQK) acc[c] += *reinterpret_cast<const f32x4 *>(r0 + ch);
    }
  }
  float *d = dkv + s * DQK;
#pragma unroll
  for (int c = 0; c < kVec; ++c) {
    const int ch = 4 * lane + 256 * c;
    if (ch < DQK) *reinterpret_cast<f32x4 *>(d + ch) += acc[c];
  }
}

template <int DQK, int HP>
hipError_t launch_rows(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                       const int32_t *topk_length, const float *lse, const float *delta,
                       const uint16_t *dout, int64_t row0, int64_t rows, int32_t H, int32_t K,
                       float scale, uint16_t *dq, float *stage, hipStream_t s) {
  constexpr size_t smem = rows_smem_bytes<DQK, HP>();
  auto kern = bwd_rows_kernel<DQK, HP>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(smem));
  if (e != hipSuccess) return e;
  DSA_LAUNCH("sparse_mla_bwd_rows", kern, dim3(static_cast<unsigned>(2 * rows)),
             dim3(kRowWaves * 64), smem, s, q, kv, idx, topk_length, lse, delta, dout, H, K,
             scale, scale * kLog2e, dq, stage, row0);
  return hipGetLastError();
}

template <int DQK>
hipError_t launch_pass(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                       const int32_t *topk_length, const float *lse, const float *delta,
                       const uint16_t *dout, int64_t row0, int64_t rows, int64_t T_kv,
                       int32_t H, int32_t K, float scale, uint16_t *dq, float *dkv,
                       const BwdWorkspace &ws, hipStream_t s) {
  hipError_t e = H <= 32 ? launch_rows<DQK, 32>(q, kv, idx, topk_length, lse, delta, dout, row0,
                                                rows, H, K, scale, dq, ws.stage, s)
                         : launch_rows<DQK, 64>(q, kv, idx, topk_length, lse, delta, dout, row0,
                                                rows, H, K, scale, dq, ws.stage, s);
  if (e != hipSuccess) return e;
  const int64_t pairs = rows * K;
  const unsigned pb = static_cast<unsigned>((pairs + 255) / 256);
  const unsigned zb = static_cast<unsigned>(std::min<int64_t>((T_kv + 256) / 256, 65536));
  DSA_LAUNCH("pair_zero", fill_zero_i32_kernel, dim3(zb), dim3(256), 0, s, ws.off, T_kv + 1);
  DSA_LAUNCH("pair_count", pair_count_kernel, dim3(pb), dim3(256), 0, s, idx, topk_length, row0,
             rows, K, ws.off);
  DSA_LAUNCH("pair_scan", pair_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, ws.off,
             ws.cursor, T_kv);
  DSA_LAUNCH("pair_fill", pair_fill_kernel, dim3(pb), dim3(256), 0, s, idx, topk_length, row0,
             rows, K, ws.cursor, ws.list);
  DSA_LAUNCH("sparse_mla_bwd_reduce", pair_reduce_kernel<DQK>,
             dim3(static_cast<unsigned>((T_kv + 3) / 4)), dim3(256), 0, s, ws.off, ws.list,
             ws.stage, T_kv, dkv);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_mla_bwd(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                                 const int32_t *topk_length, const uint16_t *out,
                                 const float *lse, const uint16_t *dout, int64_t T_q,
                                 int64_t T_kv, int32_t H, int32_t D_qk, int32_t K, float scale,
                                 uint16_t *dq, float *dkv, bool accumulate,
                                 const BwdWorkspace &ws, hipStream_t s) {
  if (!accumulate && T_kv > 0) {
    const int64_t n = T_kv * D_qk;
    const int64_t blocks = (n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536;
    DSA_LAUNCH("dkv_zero", fill_zero_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                       dkv, n);
  }
  if (T_q == 0) return hipGetLastError();
  const int64_t rows = T_q * H;
  DSA_LAUNCH("sparse_mla_bwd_delta", bwd_delta_kernel, dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0,
                     s, out, dout, rows, ws.delta);
  hipError_t e = hipGetLastError();
  for (int64_t r0 = 0; e == hipSuccess && r0 < T_q; r0 += ws.rows_per_pass) {
    const int64_t n = std::min<int64_t>(ws.rows_per_pass, T_q - r0);
    if (D_qk == 576)
      e = launch_pass<576>(q, kv, idx, topk_length, lse, ws.delta, dout, r0, n, T_kv, H, K,
                           scale, dq, dkv, ws, s);
    else if (D_qk == 512)
      e = launch_pass<512>(q, kv, idx, topk_length, lse, ws.delta, dout, r0, n, T_kv, H, K,
                           scale, dq, dkv, ws, s);
    else
      e = hipErrorInvalidValue;
  }
  return e;
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
