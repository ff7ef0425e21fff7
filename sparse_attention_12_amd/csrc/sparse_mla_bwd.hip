// Absorbed sparse MLA backward (NeMo AutoModel cudnn_dsa API reference,
// _CudnnSparseAttention.backward: gradients for the query [T_q,H,576] and the gathered latent
// rows; SkyRL PR 2423 "Summary": query chunks are independent and key gradients sum).
//
// With P_j = exp(z_j - lse), dP_j = dO . v_j, Delta = dO . O and dZ_j = P_j (dP_j - Delta):
//   dq[t,h]   = scale * sum_j dZ_j kv_j
//   dkv[s_j] += scale * sum_h dZ_j q[t,h] + sum_h P_j dO[t,h]     (over every query t)
//
// Three kernels:
//   delta  : Delta[t,h] = sum_c dO[t,h,c] O[t,h,c]          (streaming, one wave per (t,h))
//   dq     : one work group per query row, waves own 16 heads each.  Per 32-slot chunk the
//            latent rows are gathered into LDS; S^T and dP^T come from 16x16x32 bf16 MFMAs
//            with the row tile as A and the wave's q / dO blocks (registers) as B; dZ is
//            formed in registers and dq += dZ . rows uses dZ as the A operand directly (same
//            slot permutation as the forward's P . V) and transposing LDS reads for the rows.
//   dkv    : one work group of 4 waves per query row.  The row's q and dO blocks are first
//            staged through LDS and read back transposed into registers so that the head axis
//            is the MFMA contraction axis; wave w owns a quarter of the 576 latent channels.
//            Per chunk the waves recompute S^T / dP^T for their head tile, publish
//            scale * dZ^T and P^T in LDS, each as a bf16 pair hi + lo (hi = bf16(x),
//            lo = bf16(x - hi), about 16 significant bits), and every wave then forms
//            dkv_chunk[32 slots x its channels] = (scale dZ)^T . q + P^T . dO from the four
//            bf16 products and adds it to the fp32 dkv rows with atomics.  The split matters:
//            a latent row picked by many queries sums thousands of such products, and plain
//            bf16 rounding of P and dZ (8 bits) would leave a visible error in large rows.
// dq is recomputed-from-scratch per row and written once (deterministic); dkv is the only
// atomically accumulated output.
#include "dsa_common.h"
#include "dsa_internal.h"

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

template <int DQK>
struct BwdCfg {
  static constexpr int kStride = DQK + 16;
  static constexpr int kKSteps = DQK / 32;
  static constexpr int kChunksPerRow = DQK / 8;
  static constexpr int kNT = DQK / 16;  // 16-wide output tiles over the latent channels
};

// Gather the chunk's latent rows into the LDS tile (invalid slots -> zeros) and record the
// row index of each slot (-1 if invalid).
template <int DQK>
__device__ __forceinline__ void gather_rows(const uint16_t *__restrict__ kv,
                                            const int32_t *__restrict__ irow, int c0, int lim,
                                            uint16_t *tile, int32_t *srow, int nthreads) {
  using C = BwdCfg<DQK>;
  for (int c = threadIdx.x; c < kSlots * C::kChunksPerRow; c += nthreads) {
    const int j = c / C::kChunksPerRow;
    const int col = (c % C::kChunksPerRow) * 8;
    const int slot = c0 + j;
    const int32_t r = slot < lim ? irow[slot] : -1;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r >= 0) v = *reinterpret_cast<const u32x4 *>(kv + static_cast<int64_t>(r) * DQK + col);
    *reinterpret_cast<u32x4 *>(&tile[j * C::kStride + col]) = v;
    if (col == 0) srow[j] = r;
  }
}

// S^T and dP^T of one 16-head tile for the 32 slots in the LDS tile, then P and dZ.
// Returns p[mt][i], dz[mt][i] for slot 16mt + 4g + i, head hl (lane layout of 16x16 MFMA D).
template <int DQK>
__device__ __forceinline__ void slot_grads(const uint16_t *tile, const int32_t *srow,
                                           const bf16x8 *qf, const bf16x8 *df, float lse2,
                                           float dlt, float scale_log2, float p[2][4],
                                           float dz[2][4]) {
  using C = BwdCfg<DQK>;
  const int lane = __lane_id();
  const int g = lane >> 4, hl = lane & 15;
  f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  f32x4 dp[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int ks = 0; ks < C::kKSteps; ++ks) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const bf16x8 a = as_bf16x8(
          *reinterpret_cast<const u32x4 *>(&tile[(mt * 16 + hl) * C::kStride + ks * 32 + g * 8]));
      s[mt] = mfma16(a, qf[ks], s[mt]);
      if (ks < kDv / 32) dp[mt] = mfma16(a, df[ks], dp[mt]);
    }
  }
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool valid = srow[mt * 16 + g * 4 + i] >= 0;
      const float pp = valid ? __builtin_amdgcn_exp2f(s[mt][i] * scale_log2 - lse2) : 0.0f;
      p[mt][i] = pp;
      dz[mt][i] = pp * (dp[mt][i] - dlt);
    }
}

// ---------------------------------------------------------------------------------------
template <int DQK, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_dq_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kv,
    const int32_t *__restrict__ idx, const int32_t *__restrict__ topk_length,
    const float *__restrict__ lse, const float *__restrict__ delta,
    const uint16_t *__restrict__ dout, int H, int K, float scale, float scale_log2,
    uint16_t *__restrict__ dq) {
  using C = BwdCfg<DQK>;
  __shared__ __align__(16) uint16_t tile[kSlots * C::kStride];
  __shared__ int32_t srow[kSlots];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4, hl = lane & 15;
  const int64_t t = blockIdx.x;
  const int h = wave * 16 + hl;
  const bool hok = h < H;
  const int lim = topk_length ? topk_length[t] : K;
  const int32_t *irow = idx + t * K;

  bf16x8 qf[C::kKSteps], df[kDv / 32];
#pragma unroll
  for (int ks = 0; ks < C::kKSteps; ++ks) {
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
  const float l0 = hok ? lse[t * H + h] : 0.0f;
  const float lse2 = l0 == -INFINITY ? INFINITY : l0 * kLog2e;  // empty row: P = 0
  const float dlt = hok ? delta[t * H + h] : 0.0f;

  f32x4 acc[C::kNT];
#pragma unroll
  for (int n = 0; n < C::kNT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int r = (lane & 15) >> 2;
  const int cq = lane & 3;
  for (int c0 = 0; c0 < lim; c0 += kSlots) {
    gather_rows<DQK>(kv, irow, c0, lim, tile, srow, NW * 64);
    __syncthreads();
    float p[2][4], dz[2][4];
    slot_grads<DQK>(tile, srow, qf, df, lse2, dlt, scale_log2, p, dz);
    u32x4 zw;
    zw[0] = pack_bf16x2(dz[0][0], dz[0][1]);
    zw[1] = pack_bf16x2(dz[0][2], dz[0][3]);
    zw[2] = pack_bf16x2(dz[1][0], dz[1][1]);
    zw[3] = pack_bf16x2(dz[1][2], dz[1][3]);
    const bf16x8 za = as_bf16x8(zw);
    const uint16_t *v0 = &tile[(g * 4 + r) * C::kStride + cq * 4];
    const uint16_t *v1 = &tile[(16 + g * 4 + r) * C::kStride + cq * 4];
#pragma unroll
    for (int n = 0; n < C::kNT; ++n) {
      const u32x2 lo = lds_read_tr16(v0 + n * 16);
      const u32x2 hi = lds_read_tr16(v1 + n * 16);
      const u32x4 b = {lo[0], lo[1], hi[0], hi[1]};
      acc[n] = mfma16(za, as_bf16x8(b), acc[n]);
    }
    __syncthreads();
  }
  // acc[n][i] = dq[head 4g+i][channel 16n + hl] / scale
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hh = wave * 16 + g * 4 + i;
    if (hh < H) {
      uint16_t *row = dq + (t * H + hh) * DQK + hl;
#pragma unroll
      for (int n = 0; n < C::kNT; ++n) row[n * 16] = f32_to_bf16(acc[n][i] * scale);
    }
  }
}

// ---------------------------------------------------------------------------------------
constexpr int kDkvWaves = 4;

template <int DQK, int HP>  // HP: head count padded to the contraction width (32 or 64)
struct DkvCfg {
  static constexpr int kStride = DQK + 16;
  static constexpr int kTileElems = kSlots * kStride;
  static constexpr int kChanPerWave = DQK / kDkvWaves;  // 144 or 128
  static constexpr int kNTw = kChanPerWave / 16;        // output tiles per wave (9 or 8)
  static constexpr int kKH = HP / 32;                   // head contraction steps
  static constexpr int kStageStride = HP + 8;           // [slot][head] bf16 rows (+16 B)
  // staging of the row's q ([HP][DQK+16]) and dO ([HP][512+16]) at kernel start
  static constexpr int kQStride = DQK + 16;
  static constexpr int kOStride = kDv + 16;
  static constexpr int kMainElems = kTileElems + 4 * kSlots * kStageStride;
  static constexpr int kPrologElems = HP * kQStride;
  static constexpr int kSmemElems = kMainElems > kPrologElems ? kMainElems : kPrologElems;
};

template <int DQK, int HP>
__global__ __launch_bounds__(kDkvWaves * 64) void bwd_dkv_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kv,
    const int32_t *__restrict__ idx, const int32_t *__restrict__ topk_length,
    const float *__restrict__ lse, const float *__restrict__ delta,
    const uint16_t *__restrict__ dout, int H, int K, float scale, float scale_log2,
    float *__restrict__ dkv) {
  using C = DkvCfg<DQK, HP>;
  using B = BwdCfg<DQK>;
  __shared__ __align__(16) uint16_t smem[C::kSmemElems];
  __shared__ int32_t srow[kSlots];
  uint16_t *tile = smem;
  uint16_t *zst = smem + C::kTileElems;                     // scale*dZ^T [slot][head], hi
  uint16_t *zsl = zst + kSlots * C::kStageStride;           //                          lo
  uint16_t *pst = zsl + kSlots * C::kStageStride;           // P^T        [slot][head], hi
  uint16_t *psl = pst + kSlots * C::kStageStride;           //                          lo

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4, hl = lane & 15;
  const int r = (lane & 15) >> 2;
  const int cq = lane & 3;
  const int64_t t = blockIdx.x;
  const int lim = topk_length ? topk_length[t] : K;
  const int32_t *irow = idx + t * K;
  const int ch0 = wave * C::kChanPerWave;  // first latent channel owned by this wave
  constexpr int kThreads = kDkvWaves * 64;

  // ---- prologue: heads-as-contraction fragments of q and dO for this wave's channels
  bf16x8 qh[C::kKH][C::kNTw], oh[C::kKH][C::kNTw];
  for (int c = threadIdx.x; c < HP * (DQK / 8); c += kThreads) {
    const int hh = c / (DQK / 8), col = (c % (DQK / 8)) * 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (hh < H) v = *reinterpret_cast<const u32x4 *>(q + (t * H + hh) * DQK + col);
    *reinterpret_cast<u32x4 *>(&smem[hh * C::kQStride + col]) = v;
  }
  __syncthreads();
#pragma unroll
  for (int kh = 0; kh < C::kKH; ++kh)
#pragma unroll
    for (int n = 0; n < C::kNTw; ++n) {
      const uint16_t *base = &smem[(kh * 32 + g * 8 + r) * C::kQStride + ch0 + n * 16 + cq * 4];
      const u32x2 lo = lds_read_tr16(base);
      const u32x2 hi = lds_read_tr16(base + 4 * C::kQStride);
      qh[kh][n] = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
    }
  __syncthreads();
  for (int c = threadIdx.x; c < HP * (kDv / 8); c += kThreads) {
    const int hh = c / (kDv / 8), col = (c % (kDv / 8)) * 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (hh < H) v = *reinterpret_cast<const u32x4 *>(dout + (t * H + hh) * kDv + col);
    *reinterpret_cast<u32x4 *>(&smem[hh * C::kOStride + col]) = v;
  }
  __syncthreads();
#pragma unroll
  for (int kh = 0; kh < C::kKH; ++kh)
#pragma unroll
    for (int n = 0; n < C::kNTw; ++n) {
      const int ch = ch0 + n * 16;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (ch < kDv) {
        const uint16_t *base = &smem[(kh * 32 + g * 8 + r) * C::kOStride + ch + cq * 4];
        const u32x2 lo = lds_read_tr16(base);
        const u32x2 hi = lds_read_tr16(base + 4 * C::kOStride);
        v = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
      oh[kh][n] = as_bf16x8(v);
    }
  __syncthreads();
  // padded heads of the staging arrays stay zero for the whole kernel
  for (int c = threadIdx.x; c < 4 * kSlots * C::kStageStride; c += kThreads) zst[c] = 0;

  // ---- this wave's head tile for the S^T / dP^T recompute (waves beyond the tiles idle)
  const int h = wave * 16 + hl;
  const bool tile_active = wave * 16 < H;
  const bool hok = h < H;
  bf16x8 qf[B::kKSteps], df[kDv / 32];
#pragma unroll
  for (int ks = 0; ks < B::kKSteps; ++ks) {
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
  const float l0 = hok ? lse[t * H + h] : 0.0f;
  const float lse2 = l0 == -INFINITY ? INFINITY : l0 * kLog2e;
  const float dlt = hok ? delta[t * H + h] : 0.0f;
  __syncthreads();

  for (int c0 = 0; c0 < lim; c0 += kSlots) {
    gather_rows<DQK>(kv, irow, c0, lim, tile, srow, kThreads);
    __syncthreads();
    if (tile_active) {
      float p[2][4], dz[2][4];
      slot_grads<DQK>(tile, srow, qf, df, lse2, dlt, scale_log2, p, dz);
      if (hok) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int o = (mt * 16 + g * 4 + i) * C::kStageStride + h;
            const float zv = dz[mt][i] * scale;
            const uint16_t zh = f32_to_bf16(zv), ph = f32_to_bf16(p[mt][i]);
            zst[o] = zh;
            zsl[o] = f32_to_bf16(zv - bf16_to_f32(zh));
            pst[o] = ph;
            psl[o] = f32_to_bf16(p[mt][i] - bf16_to_f32(ph));
          }
      }
    }
    __syncthreads();
    // dkv_chunk[slot][channel] for this wave's channels
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x4 acc[C::kNTw];
#pragma unroll
      for (int n = 0; n < C::kNTw; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kh = 0; kh < C::kKH; ++kh) {
        const int off = (mt * 16 + hl) * C::kStageStride + kh * 32 + g * 8;
        const bf16x8 za = as_bf16x8(*reinterpret_cast<const u32x4 *>(&zst[off]));
        const bf16x8 zl = as_bf16x8(*reinterpret_cast<const u32x4 *>(&zsl[off]));
        const bf16x8 pa = as_bf16x8(*reinterpret_cast<const u32x4 *>(&pst[off]));
        const bf16x8 pl = as_bf16x8(*reinterpret_cast<const u32x4 *>(&psl[off]));
#pragma unroll
        for (int n = 0; n < C::kNTw; ++n) {
          acc[n] = mfma16(za, qh[kh][n], acc[n]);
          acc[n] = mfma16(zl, qh[kh][n], acc[n]);
          if (ch0 + n * 16 < kDv) {
            acc[n] = mfma16(pa, oh[kh][n], acc[n]);
            acc[n] = mfma16(pl, oh[kh][n], acc[n]);
          }
        }
      }
      // acc[n][i] -> dkv[row of slot 16mt + 4g + i][ch0 + 16n + hl]
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int32_t row = srow[mt * 16 + g * 4 + i];
        if (row >= 0) {
          float *dst = dkv + static_cast<int64_t>(row) * DQK + ch0 + hl;
#pragma unroll
          for (int n = 0; n < C::kNTw; ++n) atomicAdd(dst + n * 16, acc[n][i]);
        }
      }
    }
    __syncthreads();
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

template <int DQK, int NW>
hipError_t launch_dq(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                     const int32_t *topk_length, const float *lse, const float *delta,
                     const uint16_t *dout, int64_t T_q, int32_t H, int32_t K, float scale,
                     uint16_t *dq, hipStream_t s) {
  DSA_LAUNCH("sparse_mla_bwd_dq", (bwd_dq_kernel<DQK, NW>), dim3(static_cast<unsigned>(T_q)), dim3(NW * 64), 0,
                     s, q, kv, idx, topk_length, lse, delta, dout, H, K, scale, scale * kLog2e,
                     dq);
  return hipGetLastError();
}

template <int DQK>
hipError_t launch_all(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                      const int32_t *topk_length, const float *lse, const float *delta,
                      const uint16_t *dout, int64_t T_q, int32_t H, int32_t K, float scale,
                      uint16_t *dq, float *dkv, hipStream_t s) {
  const int nw = (H + 15) / 16;
  hipError_t e;
  switch (nw) {
    case 1: e = launch_dq<DQK, 1>(q, kv, idx, topk_length, lse, delta, dout, T_q, H, K, scale, dq, s); break;
    case 2: e = launch_dq<DQK, 2>(q, kv, idx, topk_length, lse, delta, dout, T_q, H, K, scale, dq, s); break;
    case 3: e = launch_dq<DQK, 3>(q, kv, idx, topk_length, lse, delta, dout, T_q, H, K, scale, dq, s); break;
    case 4: e = launch_dq<DQK, 4>(q, kv, idx, topk_length, lse, delta, dout, T_q, H, K, scale, dq, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  if (H <= 32)
    DSA_LAUNCH("sparse_mla_bwd_dkv", (bwd_dkv_kernel<DQK, 32>), dim3(static_cast<unsigned>(T_q)),
                       dim3(kDkvWaves * 64), 0, s, q, kv, idx, topk_length, lse, delta, dout, H,
                       K, scale, scale * kLog2e, dkv);
  else
    DSA_LAUNCH("sparse_mla_bwd_dkv", (bwd_dkv_kernel<DQK, 64>), dim3(static_cast<unsigned>(T_q)),
                       dim3(kDkvWaves * 64), 0, s, q, kv, idx, topk_length, lse, delta, dout, H,
                       K, scale, scale * kLog2e, dkv);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_mla_bwd(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                                 const int32_t *topk_length, const uint16_t *out,
                                 const float *lse, const uint16_t *dout, int64_t T_q,
                                 int64_t T_kv, int32_t H, int32_t D_qk, int32_t K, float scale,
                                 uint16_t *dq, float *dkv, bool accumulate, float *delta_ws,
                                 hipStream_t s) {
  if (!accumulate && T_kv > 0) {
    const int64_t n = T_kv * D_qk;
    const int64_t blocks = (n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536;
    DSA_LAUNCH("dkv_zero", fill_zero_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                       dkv, n);
  }
  if (T_q == 0) return hipGetLastError();
  const int64_t rows = T_q * H;
  DSA_LAUNCH("sparse_mla_bwd_delta", bwd_delta_kernel, dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0,
                     s, out, dout, rows, delta_ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (D_qk == 576)
    return launch_all<576>(q, kv, idx, topk_length, lse, delta_ws, dout, T_q, H, K, scale, dq,
                           dkv, s);
  if (D_qk == 512)
    return launch_all<512>(q, kv, idx, topk_length, lse, delta_ws, dout, T_q, H, K, scale, dq,
                           dkv, s);
  return hipErrorInvalidValue;
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
