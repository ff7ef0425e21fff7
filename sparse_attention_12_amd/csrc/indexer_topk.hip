// Lightning indexer + streaming per-row top-k (NVIDIA GLM-5.2 cuDNN DSA page, "How DSA works"
// and "Why DSA needs fused kernels": the indexer scores every causal key of a query and keeps
// the top-k, and its S x S score matrix must stay on chip; NeMo AutoModel cudnn_dsa API
// reference, cudnn_indexer_topk and _compact_and_sort_indices for the output contract).
//
//   I(t,s) = sum_h w[t,h] * max(0, q[t,h,:] . k[s,:])      for seq_start(t) <= s <= t
//
// Work group = 8 waves = 4 consecutive query rows of one sequence, two waves per row.  The
// group streams the rows' common causal key range in tiles of 64 keys, loaded straight into
// LDS (double buffered); the two waves of a row take the lower and upper 32 keys of each tile.
// A wave multiplies its row's [H x D] query block by its 32 keys with 32x32x16 bf16 MFMAs
// (heads on the M axis, keys on N), so the ReLU, the head weights and the head sum are applied
// to fp32 accumulators in registers: a lane ends up holding the partial sum over 32 heads of
// one key, and one cross-half exchange finishes it.  The two waves of a row sit on the same
// SIMD, so one's VALU epilogue overlaps the other's MFMAs.
//
// Streaming top-k: each row owns a candidate buffer of (orderable score, key position) in LDS.
// Keys arrive in ascending position order (tile by tile, lower half before upper half, lane
// order inside a half) and are appended in that order when their score exceeds the row's
// threshold tau (initially none).  When the buffer nears capacity one wave of the row runs an
// exact radix select (4 passes of 8 bits over the orderable uint32 scores) for the K-th
// largest score, and a stable partition keeps the K best, ties resolved to the lower position
// because the buffer is in position order.  tau becomes the K-th score; later keys have higher
// positions, so a later key with score == tau can never enter the top K and the strict test
// score > tau is exact.  The buffer therefore always holds the exact running top K in
// ascending position order, which is also the required output order.
//
// Rows with L_t <= K select their whole causal prefix, which is written without scoring.
#include "dsa_common.h"
#include "dsa_internal.h"
#include "tile.h"

namespace dsa {
namespace {

constexpr int kRows = kIdxRowsPerGroup;  // query rows per work group
constexpr int kWaves = 2 * kRows;        // two waves per row
constexpr int kThreads = 64 * kWaves;
constexpr int kTileKeys = 64;
constexpr int kBins = 256;

template <int D>
struct IndexerCfg {
  // candidate entries per row: as many as fit next to two key tiles
  static constexpr int kCap = D == 128 ? 3840 : 4096;
  static constexpr int kChunks = D / 8;                      // 16-byte chunks per key
  static constexpr int kTileBytes = kTileKeys * D * 2;
  static constexpr int kLoads = kTileKeys * kChunks / 64;    // wave-wide DMAs per tile
  static constexpr int kLoadsPerWave = kLoads / kWaves;
  static_assert(kLoads % kWaves == 0, "tile loads must split evenly");
  __device__ static __forceinline__ int swz(int key) { return key & (kChunks - 1); }
};

template <int D>
struct IndexerSmem {
  uint32_t cand_key[kRows][IndexerCfg<D>::kCap];
  int32_t cand_pos[kRows][IndexerCfg<D>::kCap];
  uint32_t hist[kRows][kBins];
  int32_t exch[2][kRows][2];  // per-tile candidate counts of the two halves (double buffered)
  uint32_t tau[kRows];
  int32_t has_tau[kRows];
  __align__(16) unsigned char tile[2][IndexerCfg<D>::kTileBytes];
};

// Monotone map float -> uint32 (larger float -> larger key); +0 and -0 map alike.
__device__ __forceinline__ uint32_t orderable(float f) {
  uint32_t u = __float_as_uint(f);
  if (f == 0.0f) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Keep the K best of the wave's `cnt` candidates (in place, order preserving) and return the
// K-th largest key.  Requires cnt >= K.  Executed by one wave.
__device__ uint32_t select_top_k(uint32_t *ck, int32_t *cp, uint32_t *hist, int cnt, int K) {
  const int lane = __lane_id();
  wave_sync();
  int need = K;
  uint32_t prefix = 0, pmask = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = lane; b < kBins; b += 64) hist[b] = 0u;
    wave_sync();
    for (int e0 = 0; e0 < cnt; e0 += 64) {
      const int e = e0 + lane;
      const uint32_t u = e < cnt ? ck[e] : 0u;
      const bool in = e < cnt && (u & pmask) == prefix;
      const uint32_t d = (u >> shift) & 0xFFu;
      // all matching lanes on one digit (common for the leading digit): one add
      const uint64_t inm = __ballot(in);
      const uint32_t d0 = __shfl(d, __ffsll(static_cast<unsigned long long>(inm | 1ull)) - 1, 64);
      const uint64_t same = __ballot(in && d == d0);
      if (same == inm) {
        if (inm != 0 && lane == 0) atomicAdd(&hist[d0], static_cast<uint32_t>(__popcll(inm)));
      } else if (in) {
        atomicAdd(&hist[d], 1u);
      }
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

// Streaming compaction: drop candidates that can no longer reach the top K, keeping at least
// K of them, in one counting pass.  With lo = the current threshold (or the smallest key) and
// hi = the largest key, the keys are binned by (u - lo) >> shift into at most 256 bins; the
// bin holding the K-th largest key gives a new threshold tau' = lo + (bin << shift) - 1 with
// at least K keys above it (so tau' never exceeds the true K-th largest key, and a later key
// at or below tau' can never enter the top K).  Keys <= tau' are removed with an order
// preserving partition.  Returns tau'; `cnt` becomes the number kept (>= K).
__device__ uint32_t prune_candidates(uint32_t *ck, int32_t *cp, uint32_t *hist, int &cnt, int K,
                                     bool has_tau, uint32_t tau) {
  const int lane = __lane_id();
  wave_sync();
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  for (int e = lane; e < cnt; e += 64) {
    const uint32_t u = ck[e];
    lo = min(lo, u);
    hi = max(hi, u);
  }
  for (int off = 32; off >= 1; off >>= 1) {
    lo = min(lo, static_cast<uint32_t>(__shfl_xor(static_cast<int>(lo), off, 64)));
    hi = max(hi, static_cast<uint32_t>(__shfl_xor(static_cast<int>(hi), off, 64)));
  }
  if (has_tau) lo = tau + 1u;  // every candidate is above the current threshold
  const uint32_t span = hi - lo;
  const int shift = span < 256u ? 0 : 32 - __clz(span) - 8;
  for (int b = lane; b < kBins; b += 64) hist[b] = 0u;
  wave_sync();
  for (int e = lane; e < cnt; e += 64) atomicAdd(&hist[(ck[e] - lo) >> shift], 1u);
  wave_sync();
  // bins scanned from the top: lane l owns bins 255-4l .. 252-4l
  const uint32_t h0 = hist[255 - 4 * lane], h1 = hist[254 - 4 * lane];
  const uint32_t h2 = hist[253 - 4 * lane], h3 = hist[252 - 4 * lane];
  const uint32_t c = h0 + h1 + h2 + h3;
  uint32_t incl = c;
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  const uint32_t excl = incl - c;
  const uint32_t n = static_cast<uint32_t>(K);
  const bool mine = excl < n && n <= incl;
  const uint64_t owner = __ballot(mine);
  const int src = __ffsll(static_cast<unsigned long long>(owner)) - 1;
  uint32_t bin = 0;
  if (mine) {
    uint32_t a = excl;
    if (a + h0 >= n) bin = 255 - 4 * lane;
    else if ((a += h0) + h1 >= n) bin = 254 - 4 * lane;
    else if ((a += h1) + h2 >= n) bin = 253 - 4 * lane;
    else bin = 252 - 4 * lane;
  }
  bin = __shfl(bin, src, 64);
  const uint32_t floor_key = lo + (bin << shift);  // keys >= floor_key: at least K of them
  int written = 0;
  const uint64_t lt = lanemask_lt();
  for (int base = 0; base < cnt; base += 64) {
    const int e = base + lane;
    const bool in = e < cnt;
    const uint32_t u = in ? ck[e] : 0u;
    const int32_t p = in ? cp[e] : 0;
    const bool keep = in && u >= floor_key;
    const uint64_t km = __ballot(keep);
    if (keep) {
      const int o = written + __popcll(km & lt);
      ck[o] = u;
      cp[o] = p;
    }
    written += __popcll(km);
  }
  wave_sync();
  cnt = written;
  return floor_key - 1u;  // floor_key > lo >= 1 whenever keys were dropped
}

// DMA targets of this wave's loads of a key tile: key index inside the tile and byte offset
// inside the key row (keys beyond `last` repeat key `last`; they lie beyond every row of the
// group and are never selected).
template <int D>
struct KeyTileLoads {
  int key[IndexerCfg<D>::kLoadsPerWave];
  int off[IndexerCfg<D>::kLoadsPerWave];
  __device__ __forceinline__ void init(int wave) {
    using C = IndexerCfg<D>;
    const int lane = __lane_id();
#pragma unroll
    for (int i = 0; i < C::kLoadsPerWave; ++i) {
      const int pos = (wave * C::kLoadsPerWave + i) * 64 + lane;
      key[i] = pos / C::kChunks;
      off[i] = ((pos % C::kChunks) ^ C::swz(key[i])) * 16;
    }
  }
  __device__ __forceinline__ void issue(unsigned char *tile, const uint16_t *k, int64_t kb,
                                        int64_t last, int wave) const {
    using C = IndexerCfg<D>;
#pragma unroll
    for (int i = 0; i < C::kLoadsPerWave; ++i) {
      int64_t s = kb + key[i];
      s = s <= last ? s : last;
      dma16(reinterpret_cast<const unsigned char *>(k) + s * (D * 2) + off[i],
            tile + (wave * C::kLoadsPerWave + i) * 1024);
    }
  }
};

template <int NMT, int D>
__global__ __launch_bounds__(kThreads) void indexer_topk_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const float *__restrict__ w,
    const int32_t *__restrict__ seq_start, const int32_t *__restrict__ groups, int64_t T, int H,
    int K, int32_t *__restrict__ idx_out, int32_t *__restrict__ len_out) {
  using C = IndexerCfg<D>;
  constexpr int NKK = D / 16;  // k-steps of the 32x32x16 MFMA
  extern __shared__ __align__(16) unsigned char smem_raw[];
  IndexerSmem<D> &sm = *reinterpret_cast<IndexerSmem<D> *>(smem_raw);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row = wave & (kRows - 1);  // waves w and w + 4 share a row (and a SIMD)
  const int half = wave >> 2;
  const int64_t last = groups[blockIdx.x];
  const int64_t start = seq_start[last];
  const int64_t first = last - (kRows - 1) > start ? last - (kRows - 1) : start;
  const int64_t t = first + row;
  const bool row_ok = t <= last;
  const int64_t L = row_ok ? t - start + 1 : 0;
  const bool compute = row_ok && L > K;

  if (row_ok && !compute && half == 0) {
    int32_t *out = idx_out + t * K;
    for (int j = lane; j < K; j += 64) out[j] = j < L ? static_cast<int32_t>(start + j) : -1;
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
  if (threadIdx.x < kRows) {
    sm.has_tau[threadIdx.x] = 0;
    sm.tau[threadIdx.x] = 0u;
  }
  uint32_t *ck = sm.cand_key[row];
  int32_t *cp = sm.cand_pos[row];
  // candidate counts of all four rows, tracked identically by every wave
  int cnt[kRows] = {0, 0, 0, 0};
  const uint64_t lt = lanemask_lt();
  // B-operand LDS offsets of this lane (key row half*32 + lane%32, dims kk*16 + (lane/32)*8)
  const int krow = half * 32 + (lane & 31);
  int boff[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk)
    boff[kk] = krow * (D * 2) + (((2 * kk + (lane >> 5)) ^ C::swz(krow)) << 4);
  KeyTileLoads<D> loads;
  loads.init(wave);

  loads.issue(sm.tile[0], k, start, last, wave);
  wait_tile();      // the tile loads are invisible to the compiler: wait for them explicitly
  __syncthreads();  // q, w, tau init and the first tile have landed

  int it = 0;
  for (int64_t kb = start; kb <= last; kb += kTileKeys, ++it) {
    const int buf = it & 1;
    if (it > 0) {
      wait_tile();
      lds_barrier();  // tile `it` complete; compactions of the previous tile finished
    }
    if (kb + kTileKeys <= last) loads.issue(sm.tile[buf ^ 1], k, kb + kTileKeys, last, wave);

    int n_pass = 0;
    uint64_t pm = 0;
    uint32_t u = 0;
    const int64_t kbase = kb + half * 32;
    const int64_t key = kbase + (lane & 31);
    if (compute && kbase <= t) {
      const unsigned char *tile = sm.tile[buf];
      f32x16 acc[NMT];
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const bf16x8 b = as_bf16x8(*reinterpret_cast<const u32x4 *>(tile + boff[kk]));
#pragma unroll
        for (int m = 0; m < NMT; ++m) acc[m] = mfma32(qa[m][kk], b, kk == 0 ? f32x16{} : acc[m]);
      }
      float s = 0.0f;
#pragma unroll
      for (int m = 0; m < NMT; ++m)
#pragma unroll
        for (int i = 0; i < 16; ++i) s = fmaf(wv[m][i], fmaxf(acc[m][i], 0.0f), s);
      s += swap_halves(s);
      u = orderable(s);
      const bool has_tau = sm.has_tau[row] != 0;
      const uint32_t tau = sm.tau[row];
      const bool pass = lane < 32 && key <= t && (!has_tau || u > tau);
      pm = __ballot(pass);
      n_pass = __popcll(pm);
    }
    if (lane == 0) sm.exch[buf][row][half] = n_pass;
    lds_barrier();
    int need_compact = 0;
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int n0 = sm.exch[buf][r][0], n1 = sm.exch[buf][r][1];
      if (r == row && (pm >> lane) & 1ull) {
        const int p = cnt[r] + (half ? n0 : 0) + __popcll(pm & lt);
        ck[p] = u;
        cp[p] = static_cast<int32_t>(key);
      }
      cnt[r] += n0 + n1;
      need_compact |= cnt[r] > C::kCap - kTileKeys;
    }
    if (need_compact) {
      lds_barrier();  // both halves' appends are visible
      if (half == 0 && cnt[row] > C::kCap - kTileKeys) {
        int c2 = cnt[row];
        uint32_t tau = prune_candidates(ck, cp, sm.hist[row], c2, K, sm.has_tau[row] != 0,
                                        sm.tau[row]);
        if (c2 > C::kCap - 2 * kTileKeys) {  // too many ties to make room: exact selection
          tau = select_top_k(ck, cp, sm.hist[row], c2, K);
          c2 = K;
        }
        if (lane == 0) {
          sm.tau[row] = tau;
          sm.has_tau[row] = 1;
          sm.exch[buf][row][0] = c2;
        }
      }
      lds_barrier();  // new thresholds and counts are visible
#pragma unroll
      for (int r = 0; r < kRows; ++r)
        if (cnt[r] > C::kCap - kTileKeys) cnt[r] = sm.exch[buf][r][0];
    }
  }

  lds_barrier();
  if (compute && half == 0) {
    if (cnt[row] > K) select_top_k(ck, cp, sm.hist[row], cnt[row], K);
    wave_sync();
    int32_t *out = idx_out + t * K;
    for (int j = lane; j < K; j += 64) out[j] = cp[j];
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
  DSA_LAUNCH("indexer_topk", kern, dim3(n_groups), dim3(kThreads), smem, s, q, k, w, seq_start,
             groups, T, H, K, idx, len);
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
