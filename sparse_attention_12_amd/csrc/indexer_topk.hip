// Lightning indexer + streaming per-row top-k (NVIDIA GLM-5.2 cuDNN DSA page, "How DSA works"
// and "Why DSA needs fused kernels": the indexer scores every causal key of a query and keeps
// the top-k, and its S x S score matrix must stay on chip; NeMo AutoModel cudnn_dsa API
// reference, cudnn_indexer_topk and _compact_and_sort_indices for the output contract).
//
//   I(t,s) = sum_h w[t,h] * max(0, q[t,h,:] . k[s,:])      for seq_start(t) <= s <= t
//
// Work group = 4 waves = 4 consecutive query rows of one sequence (one wave per row).  The
// group streams the rows' common causal key range in tiles of 64 keys through LDS; each wave
// multiplies its row's [H x D] query block by the tile with 32x32x16 bf16 MFMAs (heads on the
// M axis, keys on N), so the ReLU, the head weights and the head sum are applied to fp32
// accumulators in registers: a lane ends up holding the partial sum over 32 heads of one key,
// and one cross-half exchange finishes it.
//
// Streaming top-k: each row owns a candidate buffer of (orderable score, key position) in LDS.
// Keys arrive in ascending position order and are appended in that order when their score
// exceeds the row's threshold tau (initially none).  When the buffer nears capacity the wave
// runs an exact radix select (4 passes of 8 bits over the orderable uint32 scores) for the
// K-th largest score, and a stable partition keeps the K best, ties resolved to the lower
// position because the buffer is in position order.  tau becomes the K-th score; later keys
// have higher positions, so a later key with score == tau can never enter the top K and the
// strict test score > tau is exact.  The buffer therefore always holds the exact running top
// K in ascending position order, which is also the required output order.
//
// Rows with L_t <= K select their whole causal prefix, which is written without scoring.
#include "dsa_common.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kWaves = kIdxRowsPerGroup;  // one wave per query row
constexpr int kThreads = 64 * kWaves;
constexpr int kTileKeys = 64;
constexpr int kCap = 4096;  // candidate entries per row
constexpr int kBins = 256;

template <int D>
struct IndexerSmem {
  uint32_t cand_key[kWaves][kCap];
  int32_t cand_pos[kWaves][kCap];
  uint32_t hist[kWaves][kBins];
  uint16_t tile[kTileKeys][D + 8];  // 16-byte pad keeps 16-lane b128 reads conflict free
};

// Monotone map float -> uint32 (larger float -> larger key); +0 and -0 map alike.
__device__ __forceinline__ uint32_t orderable(float f) {
  uint32_t u = __float_as_uint(f);
  if (f == 0.0f) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Keep the K best of the wave's `cnt` candidates (in place, order preserving) and return the
// K-th largest key.  Requires cnt >= K.
__device__ uint32_t select_top_k(uint32_t *ck, int32_t *cp, uint32_t *hist, int cnt, int K) {
  const int lane = __lane_id();
  wave_sync();
  int need = K;
  uint32_t prefix = 0, pmask = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = lane; b < kBins; b += 64) hist[b] = 0u;
    wave_sync();
    for (int e = lane; e < cnt; e += 64) {
      const uint32_t u = ck[e];
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 0xFFu], 1u);
    }
    wave_sync();
    // lane l owns bins 255-4l .. 252-4l, scanned from the top
    const uint32_t h0 = hist[255 - 4 * lane], h1 = hist[254 - 4 * lane];
    const uint32_t h2 = hist[253 - 4 * lane], h3 = hist[252 - 4 * lane];
    const uint32_t c = h0 + h1 + h2 + h3;
    uint32_t incl = c;
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t v = __shfl_up(incl, off, 64);
      if (lane >= off) incl += v;
    }
    const uint32_t excl = incl - c;
    const bool mine = excl < static_cast<uint32_t>(need) && static_cast<uint32_t>(need) <= incl;
    const uint64_t owner = __ballot(mine);
    const int src = __ffsll(static_cast<unsigned long long>(owner)) - 1;
    uint32_t digit = 0, above = 0;
    if (mine) {
      uint32_t a = excl;
      const uint32_t n = static_cast<uint32_t>(need);
      if (a + h0 >= n) {
        digit = 255 - 4 * lane;
      } else if ((a += h0) + h1 >= n) {
        digit = 254 - 4 * lane;
      } else if ((a += h1) + h2 >= n) {
        digit = 253 - 4 * lane;
      } else {
        a += h2;
        digit = 252 - 4 * lane;
      }
      above = a;
    }
    digit = __shfl(digit, src, 64);
    above = __shfl(above, src, 64);
    need -= static_cast<int>(above);
    prefix |= digit << shift;
    pmask |= 0xFFu << shift;
    wave_sync();
  }
  const uint32_t tau = prefix;  // exact K-th largest key; `need` copies of it are kept
  int written = 0, eq_seen = 0;
  const uint64_t lt = lanemask_lt();
  for (int base = 0; base < cnt; base += 64) {
    const int e = base + lane;
    const bool in = e < cnt;
    const uint32_t u = in ? ck[e] : 0u;
    const int32_t p = in ? cp[e] : 0;
    const bool gt = in && u > tau;
    const bool eq = in && u == tau;
    const uint64_t eqm = __ballot(eq);
    const bool keep = gt || (eq && eq_seen + __popcll(eqm & lt) < need);
    const uint64_t km = __ballot(keep);
    if (keep) {
      const int o = written + __popcll(km & lt);
      ck[o] = u;
      cp[o] = p;
    }
    written += __popcll(km);
    eq_seen += __popcll(eqm);
  }
  wave_sync();
  return tau;
}

template <int NMT, int D>
__global__ __launch_bounds__(kThreads) void indexer_topk_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const float *__restrict__ w,
    const int32_t *__restrict__ seq_start, const int32_t *__restrict__ groups, int64_t T, int H,
    int K, int32_t *__restrict__ idx_out, int32_t *__restrict__ len_out) {
  constexpr int NKK = D / 16;                        // k-steps of the 32x32x16 MFMA
  constexpr int kChunks = kTileKeys * D / 8 / kThreads;  // 16-byte chunks per thread per tile
  constexpr int kChunksPerKey = D / 8;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  IndexerSmem<D> &sm = *reinterpret_cast<IndexerSmem<D> *>(smem_raw);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t last = groups[blockIdx.x];
  const int64_t start = seq_start[last];
  const int64_t first = last - (kWaves - 1) > start ? last - (kWaves - 1) : start;
  const int64_t t = first + wave;
  const bool row_ok = t <= last;
  const int64_t L = row_ok ? t - start + 1 : 0;
  const bool compute = row_ok && L > K;

  if (row_ok && !compute) {
    int32_t *row = idx_out + t * K;
    for (int j = lane; j < K; j += 64) row[j] = j < L ? static_cast<int32_t>(start + j) : -1;
    if (lane == 0) len_out[t] = static_cast<int32_t>(L);
  }
  if (last - start + 1 <= K) return;  // every row of the group is a whole prefix (uniform)

  // ---- this row's query block (A operand) and head weights
  bf16x8 qa[NMT][NKK];
  float wv[NMT][16];
#pragma unroll
  for (int m = 0; m < NMT; ++m) {
    const int h = m * 32 + (lane & 31);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (compute && h < H)
        v = *reinterpret_cast<const u32x4 *>(q + ((t * H + h) * D + kk * 16 + (lane >> 5) * 8));
      qa[m][kk] = as_bf16x8(v);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int hh = m * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
      wv[m][i] = (compute && hh < H) ? w[t * H + hh] : 0.0f;
    }
  }

  uint32_t *ck = sm.cand_key[wave];
  int32_t *cp = sm.cand_pos[wave];
  uint32_t *hist = sm.hist[wave];
  int cnt = 0;
  uint32_t tau = 0u;
  bool has_tau = false;
  const uint64_t lt = lanemask_lt();

  u32x4 pf[kChunks];
  auto load_tile = [&](int64_t kb) {
#pragma unroll
    for (int r = 0; r < kChunks; ++r) {
      const int c = threadIdx.x + r * kThreads;
      const int64_t key = kb + c / kChunksPerKey;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (key <= last) v = *reinterpret_cast<const u32x4 *>(k + key * D + (c % kChunksPerKey) * 8);
      pf[r] = v;
    }
  };
  load_tile(start);

  for (int64_t kb = start; kb <= last; kb += kTileKeys) {
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kChunks; ++r) {
      const int c = threadIdx.x + r * kThreads;
      *reinterpret_cast<u32x4 *>(&sm.tile[c / kChunksPerKey][(c % kChunksPerKey) * 8]) = pf[r];
    }
    __syncthreads();
    if (kb + kTileKeys <= last) load_tile(kb + kTileKeys);
    if (!compute) continue;

#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int64_t kbase = kb + sub * 32;
      if (kbase > t) break;
      f32x16 acc[NMT];
#pragma unroll
      for (int m = 0; m < NMT; ++m) acc[m] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const bf16x8 b = as_bf16x8(
            *reinterpret_cast<const u32x4 *>(&sm.tile[sub * 32 + (lane & 31)][kk * 16 + (lane >> 5) * 8]));
#pragma unroll
        for (int m = 0; m < NMT; ++m) acc[m] = mfma32(qa[m][kk], b, acc[m]);
      }
      float s = 0.0f;
#pragma unroll
      for (int m = 0; m < NMT; ++m)
#pragma unroll
        for (int i = 0; i < 16; ++i) s = fmaf(wv[m][i], fmaxf(acc[m][i], 0.0f), s);
      s += swap_halves(s);
      const int64_t key = kbase + (lane & 31);
      const uint32_t u = orderable(s);
      const bool pass = lane < 32 && key <= t && (!has_tau || u > tau);
      const uint64_t pm = __ballot(pass);
      if (pass) {
        const int p = cnt + __popcll(pm & lt);
        ck[p] = u;
        cp[p] = static_cast<int32_t>(key);
      }
      cnt += __popcll(pm);
    }
    if (cnt > kCap - kTileKeys) {
      tau = select_top_k(ck, cp, hist, cnt, K);
      cnt = K;
      has_tau = true;
    }
  }

  if (compute) {
    if (cnt > K) {
      select_top_k(ck, cp, hist, cnt, K);
      cnt = K;
    }
    wave_sync();
    int32_t *row = idx_out + t * K;
    for (int j = lane; j < K; j += 64) row[j] = cp[j];
    if (lane == 0) len_out[t] = K;
  }
}

template <int NMT, int D>
hipError_t launch(const uint16_t *q, const uint16_t *k, const float *w, const int32_t *seq_start,
                  const int32_t *groups, int32_t n_groups, int64_t T, int32_t H, int32_t K,
                  int32_t *idx, int32_t *len, hipStream_t s) {
  const size_t smem = sizeof(IndexerSmem<D>);
  auto kern = indexer_topk_kernel<NMT, D>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(smem));
  if (e != hipSuccess) return e;
  DSA_LAUNCH("indexer_topk", kern, dim3(n_groups), dim3(kThreads), smem, s, q, k, w, seq_start, groups,
                     T, H, K, idx, len);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer_topk(const uint16_t *q, const uint16_t *k, const float *w,
                               const int32_t *seq_start, const int32_t *groups, int32_t n_groups,
                               int64_t T, int32_t H, int32_t D, int32_t K, int32_t *idx,
                               int32_t *len, hipStream_t s) {
  if (n_groups == 0) return hipSuccess;
  const bool two = H > 32;
  if (D == 128) return two ? launch<2, 128>(q, k, w, seq_start, groups, n_groups, T, H, K, idx, len, s)
                           : launch<1, 128>(q, k, w, seq_start, groups, n_groups, T, H, K, idx, len, s);
  if (D == 64) return two ? launch<2, 64>(q, k, w, seq_start, groups, n_groups, T, H, K, idx, len, s)
                          : launch<1, 64>(q, k, w, seq_start, groups, n_groups, T, H, K, idx, len, s);
  return hipErrorInvalidValue;
}

}  // namespace dsa
