// Lightning indexer + streaming per-row top-k (NVIDIA GLM-5.2 cuDNN DSA page, "How DSA works"
// and "Why DSA needs fused kernels": the indexer scores every causal key of a query and keeps
// the top-k, and its S x S score matrix must stay on chip; NeMo AutoModel cudnn_dsa API
// reference, cudnn_indexer_topk and _compact_and_sort_indices for the output contract).
//
//   I(t,s) = sum_h w[t,h] * max(0, q[t,h,:] . k[s,:])      for seq_start(t) <= s <= t
//
// Work group = 8 waves = 4 consecutive query rows of one sequence, two waves per row.  The
// group streams the rows' common causal key range in tiles of 64 keys, loaded straight into
// LDS (three buffers, so a tile's loads have two tiles of compute to land); the two waves of a
// row take the lower and upper 32 keys of each tile.
// A wave multiplies its row's [H x D] query block by its 32 keys with 32x32x16 bf16 MFMAs
// (heads on the M axis, keys on N), so the ReLU, the head weights and the head sum are applied
// to fp32 accumulators in registers: a lane ends up holding the partial sum over 32 heads of
// one key, and one cross-half exchange finishes it.  The two waves of a row sit on the same
// SIMD, so one's VALU epilogue overlaps the other's MFMAs.
//
// Streaming top-k: each row owns a candidate buffer of (orderable score, key position) pairs in
// LDS, filled as two stacks (one per wave of the row, counts kept in registers, so no atomics;
// entries in no particular order).  A key is appended when its score exceeds the row's
// threshold tau (initially none).  When a row nears capacity it is
// pruned with one 512-bin counting pass: the bin holding the K-th largest score gives a new
// tau that never exceeds the true K-th largest score, and every candidate at or below it is
// dropped.  Keys arrive in ascending position order, so a later key equal to the K-th score
// would lose the tie to the candidates already kept: the strict test score > tau is exact.  On
// long rows a pruning may instead keep fewer than K (compaction_rank): the threshold that a
// uniform sample of the row would still pass K times over.  At the end an exact selection
// (histograms narrowing the K-th score, ties resolved to the lower positions) keeps exactly K
// candidates, and a bitmap over the row's key range writes their positions in ascending order;
// a row left with fewer than K candidates (a speculative pruning went too far) is marked and
// recomputed without speculation by a second launch.
//
// Rows with L_t <= K select their whole causal prefix, which is written without scoring.
#include <type_traits>

#include "dsa_common.h"
#include "dsa_internal.h"
#include "tile.h"

namespace dsa {
namespace {

constexpr int kRows = kIdxRowsPerGroup;  // query rows per work group
constexpr int kWaves = 2 * kRows;        // two waves per row
constexpr int kThreads = 64 * kWaves;
constexpr int kTileKeys = 64;
constexpr int kRedoGroups = 256;  // work groups of the second launch (one per CU)
// value bins of a compaction: narrower bins collide less in the LDS atomics
constexpr int kPruneBins = 512;

template <int D>
struct IndexerCfg {
  static constexpr int kNBuf = 3;  // key tile buffers
  // candidate entries per row: as many as fit next to the key tiles in 160 KB of LDS
  static constexpr int kCap = D == 128 ? 3320 : 4088;
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
  __align__(16) uint32_t hist[kRows][kPruneBins];
  __align__(16) int32_t cnt[kRows];   // entries of the lower stack of each row
  __align__(16) int32_t cntb[kRows];  // entries of the upper stack of each row
  uint32_t tau[kRows];                // per-row threshold: later keys enter only if above it
  int32_t has_tau[kRows];
  int32_t compact[2];  // compaction due in step i: compact[i & 1] (written by wave 0 in step i - 1)
  uint32_t xlo[kRows][2], xhi[kRows][2], xdrop[kRows][2];  // a compaction's per-stack results
  __align__(16) unsigned char tile[IndexerCfg<D>::kNBuf][IndexerCfg<D>::kTileBytes];
};
static_assert(sizeof(IndexerSmem<128>) <= 160 * 1024 && sizeof(IndexerSmem<64>) <= 160 * 1024,
              "indexer LDS");
// after the key stream the tile buffers hold 4 rows x (4 KB bitmap + 2 KB scratch list), and
// with 128-dim keys also 4 rows x a 4 KB (1024-bin) value histogram
template <int D>
constexpr int kFinalBins = D == 128 ? 1024 : 256;
static_assert(IndexerCfg<64>::kNBuf * IndexerCfg<64>::kTileBytes >= 4 * (4096 + 2048), "tile area");
static_assert(IndexerCfg<128>::kNBuf * IndexerCfg<128>::kTileBytes >= 4 * (4096 + 2048 + 4096),
              "tile area");

// Monotone map float -> uint32 (larger float -> larger key).  -0 would map just below +0; no
// score is -0: each half-sum starts at +0 and adds fmaf(w, max(x, 0), s) terms, whose exact
// value is 0 only as w * (+-0) + s with s = +0 (giving +0 in round-to-nearest), and a sum of
// two such values is -0 only if both are.
__device__ __forceinline__ uint32_t orderable(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---- per-row candidate selection, executed by one wave ------------------------------------
// A row's candidates are (key, position) pairs in two LDS arrays, in no particular order.
// Loops read four consecutive entries per lane (ds_read_b128); entries at or beyond `cnt`
// are masked.  Capacities are multiples of 4, so such reads stay inside the arrays.

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = __lane_id();
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t x = __shfl_up(v, off, 64);
    if (lane >= off) v += x;
  }
  return v;
}

// Smallest and largest of ck[0, cnt) (cnt >= 1).
__device__ __forceinline__ void key_range(const uint32_t *ck, int cnt, uint32_t &lo,
                                          uint32_t &hi) {
  const int lane = __lane_id();
  lo = 0xFFFFFFFFu;
  hi = 0u;
  for (int e = 4 * lane; e < cnt; e += 256) {
    const u32x4 v = *reinterpret_cast<const u32x4 *>(ck + e);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (e + j < cnt) {
        lo = min(lo, v[j]);
        hi = max(hi, v[j]);
      }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    lo = min(lo, static_cast<uint32_t>(__shfl_xor(static_cast<int>(lo), off, 64)));
    hi = max(hi, static_cast<uint32_t>(__shfl_xor(static_cast<int>(hi), off, 64)));
  }
}

// Bin width exponent for the key range [lo, hi]: (hi - lo) >> shift < 256.
__device__ __forceinline__ int range_shift(uint32_t lo, uint32_t hi) {
  const uint32_t span = hi - lo;
  return span < 256u ? 0 : 32 - __clz(static_cast<int>(span)) - 8;
}

// 256-bin histogram of the keys in [lo, hi], bin = (u - lo) >> shift.
__device__ void key_histogram(const uint32_t *ck, int cnt, uint32_t lo, uint32_t hi, int shift,
                              uint32_t *hist) {
  const int lane = __lane_id();
  *reinterpret_cast<u32x4 *>(hist + 4 * lane) = u32x4{0u, 0u, 0u, 0u};
  wave_sync();
  for (int e = 4 * lane; e < cnt; e += 256) {
    const u32x4 v = *reinterpret_cast<const u32x4 *>(ck + e);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (e + j < cnt && v[j] >= lo && v[j] <= hi) atomicAdd(&hist[(v[j] - lo) >> shift], 1u);
  }
  wave_sync();
}

// The bin holding the need-th largest key of a 256-bin histogram (1 <= need <= total); `above`
// receives the number of keys in higher bins.
__device__ __forceinline__ uint32_t bin_from_top(const uint32_t *hist, uint32_t need,
                                                 uint32_t &above) {
  const int lane = __lane_id();
  // lane l owns bins 255-4l .. 252-4l, i.e. hist[252-4l .. 255-4l] read as one vector
  const u32x4 hv = *reinterpret_cast<const u32x4 *>(hist + 252 - 4 * lane);
  const uint32_t c = hv[0] + hv[1] + hv[2] + hv[3];
  const uint32_t incl = wave_incl_scan(c);
  const uint32_t excl = incl - c;
  const bool mine = excl < need && need <= incl;
  const int src = __ffsll(static_cast<unsigned long long>(__ballot(mine))) - 1;
  uint32_t bin = 0, a = excl;
  if (mine) {
    if (a + hv[3] >= need) {
      bin = 255 - 4 * lane;
    } else if ((a += hv[3]) + hv[2] >= need) {
      bin = 254 - 4 * lane;
    } else if ((a += hv[2]) + hv[1] >= need) {
      bin = 253 - 4 * lane;
    } else {
      a += hv[1];
      bin = 252 - 4 * lane;
    }
  }
  above = __shfl(a, src, 64);
  return __shfl(bin, src, 64);
}

// As bin_from_top for a histogram of NB bins (NB a multiple of 256): lane l owns the NB/64
// bins NB-1-(NB/64) l downward.
template <int NB>
__device__ __forceinline__ uint32_t bin_from_top_n(const uint32_t *hist, uint32_t need,
                                                   uint32_t &above) {
  constexpr int P = NB / 64;  // bins per lane
  const int lane = __lane_id();
  const int lo = NB - P * (lane + 1);
  uint32_t hv[P];
#pragma unroll
  for (int i = 0; i < P; i += 4) {
    const u32x4 v = *reinterpret_cast<const u32x4 *>(hist + lo + i);
    hv[i] = v[0];
    hv[i + 1] = v[1];
    hv[i + 2] = v[2];
    hv[i + 3] = v[3];
  }
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < P; ++i) c += hv[i];
  const uint32_t incl = wave_incl_scan(c);
  const uint32_t excl = incl - c;
  const bool mine = excl < need && need <= incl;
  const int src = __ffsll(static_cast<unsigned long long>(__ballot(mine))) - 1;
  uint32_t bin = 0, a = excl;
  if (mine) {
    bool found = false;
#pragma unroll
    for (int i = P - 1; i >= 0; --i) {  // from this lane's highest bin down
      if (!found) {
        if (a + hv[i] >= need) {
          bin = static_cast<uint32_t>(lo + i);
          found = true;
        } else {
          a += hv[i];
        }
      }
    }
  }
  above = __shfl(a, src, 64);
  return __shfl(bin, src, 64);
}

// Keeps the entries for which keep(key, position) holds, packed at the front (order not
// preserved); returns their number and sets `dropped_max` to the largest key removed (0 if
// none).  In place: an iteration writes below the end of the block it has just read, and a
// wave's LDS operations complete in order.
template <typename Keep>
__device__ int compact_candidates(uint32_t *ck, int32_t *cp, int cnt, Keep keep,
                                  uint32_t &dropped_max) {
  const int lane = __lane_id();
  const uint64_t lt = lanemask_lt();
  int written = 0;
  uint32_t dmax = 0u;
  for (int base = 0; base < cnt; base += 256) {
    const int e = base + 4 * lane;
    u32x4 v = {0u, 0u, 0u, 0u}, p = {0u, 0u, 0u, 0u};
    if (e < cnt) {
      v = *reinterpret_cast<const u32x4 *>(ck + e);
      p = *reinterpret_cast<const u32x4 *>(cp + e);
    }
    bool kp[4];
    uint64_t m[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool in = e + j < cnt;
      kp[j] = in && keep(v[j], static_cast<int32_t>(p[j]));
      if (in && !kp[j]) dmax = max(dmax, v[j]);
      m[j] = __ballot(kp[j]);
    }
    int off = written;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (kp[j]) {
        const int o = off + __popcll(m[j] & lt);
        ck[o] = v[j];
        cp[o] = static_cast<int32_t>(p[j]);
      }
      off += __popcll(m[j]);
    }
    written = off;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1)
    dmax = max(dmax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(dmax), off, 64)));
  dropped_max = dmax;
  wave_sync();
  return written;
}

// Number of entries with key == tau and position <= pcut.
__device__ int count_ties_upto(const uint32_t *ck, const int32_t *cp, int cnt, uint32_t tau,
                               int64_t pcut) {
  const int lane = __lane_id();
  int c = 0;
  for (int e = 4 * lane; e < cnt; e += 256) {
    const u32x4 v = *reinterpret_cast<const u32x4 *>(ck + e);
    const u32x4 p = *reinterpret_cast<const u32x4 *>(cp + e);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      c += (e + j < cnt && v[j] == tau && static_cast<int32_t>(p[j]) <= pcut) ? 1 : 0;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off, 64);
  return c;
}

// Exact selection: keeps the K largest keys of ck[0, cnt) (cnt >= K), ties at the K-th key
// resolved to the lower positions, and returns the K-th largest key.  The key is narrowed one
// 256-bin histogram at a time (at most four levels); a tie straddling the cut is resolved by a
// bisection on position.  `pos_lo`/`pos_hi` bound the positions.
__device__ uint32_t select_exact(uint32_t *ck, int32_t *cp, uint32_t *hist, int &cnt, int K,
                                 int64_t pos_lo, int64_t pos_hi) {
  uint32_t lo, hi;
  key_range(ck, cnt, lo, hi);
  uint32_t need = static_cast<uint32_t>(K);
  uint32_t tau = lo;
  for (int level = 0; level < 4; ++level) {
    if (hi == lo) {
      tau = lo;
      break;
    }
    const int shift = range_shift(lo, hi);
    key_histogram(ck, cnt, lo, hi, shift, hist);
    uint32_t above;
    const uint32_t bin = bin_from_top(hist, need, above);
    need -= above;
    const uint32_t nlo = lo + (bin << shift);
    const uint64_t nhi = static_cast<uint64_t>(nlo) + ((1ull << shift) - 1ull);
    lo = nlo;
    hi = nhi < hi ? static_cast<uint32_t>(nhi) : hi;
    tau = lo;
    if (shift == 0) break;
  }
  // `need` keys equal to tau belong to the top K
  const int eq = count_ties_upto(ck, cp, cnt, tau, pos_hi);
  uint32_t dmax;
  if (eq == static_cast<int>(need)) {
    cnt = compact_candidates(ck, cp, cnt, [tau](uint32_t u, int32_t) { return u >= tau; }, dmax);
    return tau;
  }
  // smallest position cut with `need` tied keys at or below it
  int64_t a = pos_lo, b = pos_hi;
  while (a < b) {
    const int64_t mid = a + ((b - a) >> 1);
    if (count_ties_upto(ck, cp, cnt, tau, mid) >= static_cast<int>(need)) b = mid;
    else a = mid + 1;
  }
  const int64_t pcut = a;
  cnt = compact_candidates(ck, cp, cnt, [tau, pcut](uint32_t u, int32_t p) {
    return u > tau || (u == tau && p <= pcut);
  }, dmax);
  return tau;
}

// Inverse of orderable() (the +0 key maps back to +0).
__device__ __forceinline__ float key_to_float(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// NB bins of equal width in score value over [lo, hi] (keys).  bin(u) is non-decreasing in
// u (a rounded subtraction and a product with a positive constant are monotone), so
// {u : bin(u) >= b} is a set of keys at or above some key.
template <int NB>
struct ValueBinsN {
  float flo, scale;
  __device__ __forceinline__ bool init(uint32_t lo, uint32_t hi) {
    flo = key_to_float(lo);
    const float fhi = key_to_float(hi);
    scale = static_cast<float>(NB) / (fhi - flo);
    return fhi > flo && scale < INFINITY;
  }
  __device__ __forceinline__ int operator()(uint32_t u) const {
    return max(min(static_cast<int>((key_to_float(u) - flo) * scale), NB - 1), 0);
  }
};
using ValueBins = ValueBinsN<256>;

// NB-bin histogram of ck[0, cnt) (all keys within the bins' range).
template <int NB = 256>
__device__ void value_histogram(const uint32_t *ck, int cnt, const ValueBinsN<NB> &vb,
                                uint32_t *hist) {
  const int lane = __lane_id();
#pragma unroll
  for (int i = 0; i < NB / 256; ++i)
    *reinterpret_cast<u32x4 *>(hist + 256 * i + 4 * lane) = u32x4{0u, 0u, 0u, 0u};
  wave_sync();
  for (int e = 4 * lane; e < cnt; e += 256) {
    const u32x4 v = *reinterpret_cast<const u32x4 *>(ck + e);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (e + j < cnt) atomicAdd(&hist[vb(v[j])], 1u);
  }
  wave_sync();
}

// ---- the two stacks of a row's candidate buffer, seen from the wave that fills each ----------
// The lower-half wave's stack holds entries 0 .. n-1 of the buffer; the upper-half wave's stack
// holds its i-th entry at cap - 1 - i.  A Stack presents either as entries 0 .. n-1, read four
// at a time (four consecutive entries of the upper stack are one reversed 16-byte vector, since
// cap is a multiple of 4).
struct Stack {
  uint32_t *ck;
  int32_t *cp;
  int cap;
  bool up;
  __device__ __forceinline__ int at(int i) const { return up ? cap - 1 - i : i; }
  __device__ __forceinline__ u32x4 keys4(int e) const {
    if (!up) return *reinterpret_cast<const u32x4 *>(ck + e);
    const u32x4 v = *reinterpret_cast<const u32x4 *>(ck + cap - 4 - e);
    return u32x4{v[3], v[2], v[1], v[0]};
  }
  __device__ __forceinline__ u32x4 pos4(int e) const {
    if (!up) return *reinterpret_cast<const u32x4 *>(cp + e);
    const u32x4 v = *reinterpret_cast<const u32x4 *>(cp + cap - 4 - e);
    return u32x4{v[3], v[2], v[1], v[0]};
  }
};

// Smallest and largest key of a stack (lo = 0xFFFFFFFF, hi = 0 for an empty one).
__device__ __forceinline__ void stack_range(const Stack &st, int cnt, uint32_t &lo, uint32_t &hi) {
  const int lane = __lane_id();
  lo = 0xFFFFFFFFu;
  hi = 0u;
  for (int e = 4 * lane; e < cnt; e += 256) {
    const u32x4 v = st.keys4(e);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (e + j < cnt) {
        lo = min(lo, v[j]);
        hi = max(hi, v[j]);
      }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    lo = min(lo, static_cast<uint32_t>(__shfl_xor(static_cast<int>(lo), off, 64)));
    hi = max(hi, static_cast<uint32_t>(__shfl_xor(static_cast<int>(hi), off, 64)));
  }
}

// Adds a stack's keys to an NB-bin value histogram that the caller has cleared.
template <int NB>
__device__ void stack_histogram(const Stack &st, int cnt, const ValueBinsN<NB> &vb,
                                uint32_t *hist) {
  const int lane = __lane_id();
  for (int e = 4 * lane; e < cnt; e += 256) {
    const u32x4 v = st.keys4(e);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (e + j < cnt) atomicAdd(&hist[vb(v[j])], 1u);
  }
}

// As compact_candidates, on a stack: the kept entries become the stack's first entries.
template <typename Keep>
__device__ int compact_stack(const Stack &st, int cnt, Keep keep, uint32_t &dropped_max) {
  const int lane = __lane_id();
  const uint64_t lt = lanemask_lt();
  int written = 0;
  uint32_t dmax = 0u;
  for (int base = 0; base < cnt; base += 256) {
    const int e = base + 4 * lane;
    u32x4 v = {0u, 0u, 0u, 0u}, p = {0u, 0u, 0u, 0u};
    if (e < cnt) {
      v = st.keys4(e);
      p = st.pos4(e);
    }
    bool kp[4];
    uint64_t m[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool in = e + j < cnt;
      kp[j] = in && keep(v[j], static_cast<int32_t>(p[j]));
      if (in && !kp[j]) dmax = max(dmax, v[j]);
      m[j] = __ballot(kp[j]);
    }
    int off = written;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (kp[j]) {
        const int o = st.at(off + __popcll(m[j] & lt));
        st.ck[o] = v[j];
        st.cp[o] = static_cast<int32_t>(p[j]);
      }
      off += __popcll(m[j]);
    }
    written = off;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1)
    dmax = max(dmax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(dmax), off, 64)));
  dropped_max = dmax;
  wave_sync();
  return written;
}

// Final selection of exactly K of the row's cnt >= K candidates and their output in ascending
// position order.  One value histogram finds the bin b of the K-th largest key: every
// candidate in a higher bin is selected, and the `need` best of the bin-b candidates (copied
// to a scratch list of at most kScratch entries, ranked by key and then lower position) are
// added.  If bin b is too populous (massive ties), select_exact() runs on the whole buffer.
// The selected positions (all inside [start, t]) are marked in a bitmap one window of kWin
// positions at a time; lane l owns four bitmap words (128 positions), counts their bits, and
// writes its positions from its exclusive prefix onward, so no LDS read sits inside the
// emission loop.
constexpr int kScratch = 256;

template <int NB>
__device__ void select_and_write(uint32_t *ck, int32_t *cp, uint32_t *hist, uint32_t *hist256,
                                 int cnt, int K, bool has_tau, uint32_t tau, int64_t start,
                                 int64_t t, uint32_t *bm, uint32_t *sk, int32_t *sp,
                                 int32_t *out) {
  const int lane = __lane_id();
  ValueBinsN<NB> vb;
  int b = -1;        // bin of the K-th key; -1: every candidate in ck[0, cnt) is selected
  int nb = 0;        // scratch entries
  uint32_t keep4 = 0u;  // bit r: scratch entry lane + 64 r is selected
  if (cnt > K) {
    uint32_t lo, hi;
    key_range(ck, cnt, lo, hi);
    if (has_tau) lo = tau + 1u;
    bool fast = vb.init(lo, hi);
    uint32_t need = 0u;
    if (fast) {
      value_histogram<NB>(ck, cnt, vb, hist);
      uint32_t above;
      b = static_cast<int>(bin_from_top_n<NB>(hist, static_cast<uint32_t>(K), above));
      need = static_cast<uint32_t>(K) - above;
      nb = static_cast<int>(hist[b]);
      fast = nb <= kScratch;
    }
    if (fast) {
      // copy bin b to the scratch list; two blocks of 256 entries are read per trip
      const uint64_t lt = lanemask_lt();
      int w = 0;
      for (int e0 = 0; e0 < cnt; e0 += 512) {
        u32x4 v[2], p[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int e = e0 + 256 * h + 4 * lane;
          v[h] = u32x4{0u, 0u, 0u, 0u};
          p[h] = u32x4{0u, 0u, 0u, 0u};
          if (e < cnt) {
            v[h] = *reinterpret_cast<const u32x4 *>(ck + e);
            p[h] = *reinterpret_cast<const u32x4 *>(cp + e);
          }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bool in = e0 + 256 * h + 4 * lane + j < cnt && vb(v[h][j]) == b;
            const uint64_t m = __ballot(in);
            if (in) {
              const int o = w + __popcll(m & lt);
              sk[o] = v[h][j];
              sp[o] = static_cast<int32_t>(p[h][j]);
            }
            w += __popcll(m);
          }
      }
      wave_sync();
      // rank of each scratch entry among the bin: larger key first, then lower position (the
      // list is read four entries at a time, the same addresses for every lane)
      uint32_t ki[kScratch / 64], rank[kScratch / 64];
      int32_t pi[kScratch / 64];
#pragma unroll
      for (int r = 0; r < kScratch / 64; ++r) {
        const int i = lane + 64 * r;
        ki[r] = i < nb ? sk[i] : 0u;
        pi[r] = i < nb ? sp[i] : 0;
        rank[r] = 0u;
      }
      for (int j0 = 0; j0 < nb; j0 += 4) {
        const u32x4 kj = *reinterpret_cast<const u32x4 *>(sk + j0);
        const u32x4 pj = *reinterpret_cast<const u32x4 *>(sp + j0);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          if (j0 + jj < nb) {
#pragma unroll
            for (int r = 0; r < kScratch / 64; ++r)
              rank[r] += (kj[jj] > ki[r] || (kj[jj] == ki[r] && static_cast<int32_t>(pj[jj]) < pi[r])) ? 1u : 0u;
          }
        }
      }
#pragma unroll
      for (int r = 0; r < kScratch / 64; ++r)
        if (lane + 64 * r < nb && rank[r] < need) keep4 |= 1u << r;
    } else {
      int n = cnt;
      select_exact(ck, cp, hist256, n, K, start, t);
      cnt = K;
      b = -1;
      nb = 0;
    }
  }
  // ---- ascending output, one window of kWin positions at a time.  A single-window row stages
  // its output in cp (free by then: every candidate has been marked) and copies it out with
  // wide stores.
  constexpr int kWords = 256;
  constexpr int64_t kWin = 32 * kWords;
  const bool single = t - start < kWin;
  int done = 0;
  for (int64_t w0 = start; w0 <= t; w0 += kWin) {
    *reinterpret_cast<u32x4 *>(bm + 4 * lane) = u32x4{0u, 0u, 0u, 0u};
    wave_sync();
    for (int e0 = 0; e0 < cnt; e0 += 512) {
      u32x4 v[2], p[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int e = e0 + 256 * h + 4 * lane;
        v[h] = u32x4{0u, 0u, 0u, 0u};
        p[h] = u32x4{0u, 0u, 0u, 0u};
        if (e < cnt) {
          v[h] = *reinterpret_cast<const u32x4 *>(ck + e);
          p[h] = *reinterpret_cast<const u32x4 *>(cp + e);
        }
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t rel = static_cast<int32_t>(p[h][j]) - w0;
          if (e0 + 256 * h + 4 * lane + j < cnt && rel >= 0 && rel < kWin &&
              (b < 0 || vb(v[h][j]) > b))
            atomicOr(&bm[rel >> 5], 1u << (rel & 31));
        }
    }
#pragma unroll
    for (int r = 0; r < kScratch / 64; ++r) {
      const int i = lane + 64 * r;
      if (i < nb && ((keep4 >> r) & 1u)) {
        const int64_t rel = sp[i] - w0;
        if (rel >= 0 && rel < kWin) atomicOr(&bm[rel >> 5], 1u << (rel & 31));
      }
    }
    wave_sync();
    const u32x4 words = *reinterpret_cast<const u32x4 *>(bm + 4 * lane);
    const int c = __popc(words[0]) + __popc(words[1]) + __popc(words[2]) + __popc(words[3]);
    const int incl = static_cast<int>(wave_incl_scan(static_cast<uint32_t>(c)));
    const int tw = __shfl(incl, 63, 64);  // selected positions in this window
    int o = done + incl - c;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t bits = words[i];
      const int32_t base = static_cast<int32_t>(w0 + 128 * lane + 32 * i);
      while (bits != 0u) {
        const int32_t pos = base + __ffs(static_cast<int>(bits)) - 1;
        bits &= bits - 1u;
        if (single) cp[o] = pos;
        else out[o] = pos;
        ++o;
      }
    }
    done += tw;
    wave_sync();
  }
  if (single) {
    if ((K & 3) == 0) {
      for (int j = 4 * lane; j < K; j += 256)
        *reinterpret_cast<u32x4 *>(out + j) = *reinterpret_cast<const u32x4 *>(cp + j);
    } else {
      for (int j = lane; j < K; j += 64) out[j] = cp[j];
    }
  }
}

// This wave's share of the loads of one key tile: lane byte offsets relative to the tile's
// first key, for the i-th load (key index inside the tile and swizzled 16-byte chunk).  Keys
// beyond `last` (only in a group's final tile) are clamped to key `last`; they lie beyond every
// row of the group and are never selected.
template <int D>
struct KeyTileLoads {
  uint32_t voff[IndexerCfg<D>::kLoadsPerWave];
  int key[IndexerCfg<D>::kLoadsPerWave];
  __device__ __forceinline__ void init(int wave) {
    using C = IndexerCfg<D>;
    const int lane = __lane_id();
#pragma unroll
    for (int i = 0; i < C::kLoadsPerWave; ++i) {
      const int pos = (wave * C::kLoadsPerWave + i) * 64 + lane;
      key[i] = pos / C::kChunks;
      voff[i] = key[i] * (D * 2) + ((pos % C::kChunks) ^ C::swz(key[i])) * 16;
    }
  }
  // tile_lds: LDS byte address of the destination tile buffer
  // kb, last: key positions (32-bit: the host limits T to INT32_MAX - 4096)
  __device__ __forceinline__ void issue(uint32_t tile_lds, const uint16_t *k, int kb, int last,
                                        int wave) const {
    using C = IndexerCfg<D>;
    const unsigned char *base =
        reinterpret_cast<const unsigned char *>(k) + static_cast<int64_t>(kb) * (D * 2);
    const uint32_t dst = tile_lds + wave * C::kLoadsPerWave * 1024;
    if (kb + (kTileKeys - 1) <= last) {
#pragma unroll
      for (int i = 0; i < C::kLoadsPerWave; ++i) dma16_sv(base, voff[i], dst + i * 1024);
    } else {
      const int lim = last - kb;  // in [0, 63)
#pragma unroll
      for (int i = 0; i < C::kLoadsPerWave; ++i) {
        const int over = key[i] - lim;
        dma16_sv(base, voff[i] - (over > 0 ? over * (D * 2) : 0), dst + i * 1024);
      }
    }
  }
};

// Target rank of a compaction of a row of L keys after about ns of them (an upper bound) have
// been seen.  Without speculation it is K: every entry at or above the K-th largest key so far is
// kept, which can never drop a key of the final top-K.  With speculation it is the rank x, among
// the keys seen, of a threshold that the rest of the row is still expected to pass often enough:
// if the keys seen were a uniform sample of the row's scores, a fraction x / ns of all L keys
// would lie above the x-th largest, up to a relative sampling error of about 1 / sqrt(x).  x is
// the smallest rank for which L x / ns, lowered by five such errors, still exceeds K by five
// standard deviations of a count of K (solving y^2 - 5 y - a = 0 for y = sqrt(x)).  Only the
// check at the end of the row makes this exact: a row that ends with fewer than K entries above
// its threshold lost some of its top-K keys and is recomputed without speculation.
__device__ __forceinline__ int compaction_rank(bool spec, int K, int L, int ns) {
  if (!spec || ns >= L) return K;
  const float kf = static_cast<float>(K);
  const float a = (kf + 5.0f * sqrtf(kf)) * static_cast<float>(ns) / static_cast<float>(L);
  const float y = 0.5f * (5.0f + sqrtf(25.0f + 4.0f * a));
  const float x = ceilf(y * y);
  return x >= kf ? K : max(1, static_cast<int>(x));
}

// The rows of group g.  spec: compactions may use a speculative target rank (see
// compaction_rank); a row whose speculation failed gets the length -1 instead of its output.
template <int NMT, int D>
__device__ __forceinline__ void indexer_group(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const float *__restrict__ w,
    const int32_t *__restrict__ seq_start, const int32_t *__restrict__ causal_len,
    const int32_t *__restrict__ gpos, const int32_t *__restrict__ groups,
    const int32_t *__restrict__ group_first, int H, int K, int32_t *__restrict__ idx_out,
    int32_t *__restrict__ len_out, int g, bool spec) {
  using C = IndexerCfg<D>;
  constexpr int NKK = D / 16;  // k-steps of the 32x32x16 MFMA
  extern __shared__ __align__(16) unsigned char smem_raw[];
  IndexerSmem<D> &sm = *reinterpret_cast<IndexerSmem<D> *>(smem_raw);

  // Positions are 32-bit: the host limits T to INT32_MAX - 4096, so no key position computed
  // below (at most last + 4 tiles) overflows.
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = wave & (kRows - 1);  // waves w and w + 4 share a row (and a SIMD)
  const int half = wave >> 2;
  // Rows are local query rows (q, w and the output); key positions are global coordinates of
  // the key tensor.  Without local coordinates (gpos NULL) the two coincide and a group is the
  // run of up to kRows rows that ends at `last`, clipped at the sequence start.
  const int last = groups[g];
  const int start = seq_start[last];
  const int first = group_first ? group_first[g]
                                : (last - (kRows - 1) > start ? last - (kRows - 1) : start);
  const int lastg = gpos ? gpos[last] : last;  // key position of the group's last row
  const int t = first + row;                   // this wave's local row
  const bool row_ok = t <= last;
  // its key position: a row's own coordinate (the rows of a group may share one, as k-pool
  // rows that see the same pools do; the group's last row has the largest)
  const int tg = gpos ? (row_ok ? gpos[t] : lastg) : t;
  const int L = row_ok ? causal_len[t] : 0;    // 0 for a padding row
  const bool compute = row_ok && L > K;

  if (row_ok && !compute && half == 0) {
    int32_t *out = idx_out + static_cast<int64_t>(t) * K;
    for (int j = lane; j < K; j += 64) out[j] = j < L ? start + j : -1;
    if (lane == 0) len_out[t] = L;
  }
  // every row of the group is a whole prefix or padding (uniform): the last row is the longest
  if (causal_len[last] <= K) return;

  // tiles 0 and 1 in flight while the query block loads; tile it+2 is issued at the top of
  // iteration it
  const uint32_t tile_lds = lds_addr(&sm.tile[0][0]);
  KeyTileLoads<D> loads;
  loads.init(wave);
  loads.issue(tile_lds, k, start, lastg, wave);
  if (lastg - start >= kTileKeys) loads.issue(tile_lds + C::kTileBytes, k, start + kTileKeys, lastg, wave);

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
        v = *reinterpret_cast<const u32x4 *>(
            q + ((static_cast<int64_t>(t) * H + h) * D + kk * 16 + (lane >> 5) * 8));
      qa[m][kk] = as_bf16x8(v);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int hh = m * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
      wv[m][i] = (compute && hh < H) ? w[static_cast<int64_t>(t) * H + hh] : 0.0f;
    }
  }
  if (threadIdx.x < kRows) {
    sm.has_tau[threadIdx.x] = 0;
    sm.tau[threadIdx.x] = 0u;
    sm.cnt[threadIdx.x] = 0;
    sm.cntb[threadIdx.x] = 0;
  }
  if (threadIdx.x < 2) sm.compact[threadIdx.x] = 0;
  uint32_t *ck = sm.cand_key[row];
  int32_t *cp = sm.cand_pos[row];
  // The candidate buffer of a row is two stacks: the lower-half wave appends upward from entry
  // 0, the upper-half wave downward from entry kCap - 1.  Each wave keeps its own count in a
  // register (no atomics) and publishes it in sm.cnt / sm.cntb for the capacity decision; a
  // compaction or the final selection first moves the upper stack down behind the lower one.
  int my_n = 0;
  uint32_t my_tau = 0u;  // this row's threshold (wave-uniform copy)
  bool my_has_tau = false;
  // threshold for the append test: keys of finite scores are > 0, so 0 admits every key
  uint32_t tau_eff = 0u;
  // B-operand LDS offsets of this lane (key row half*32 + lane%32, dims kk*16 + (lane/32)*8)
  const int krow = half * 32 + (lane & 31);
  int boff[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk)
    boff[kk] = krow * (D * 2) + (((2 * kk + (lane >> 5)) ^ C::swz(krow)) << 4);

  // finish the query block loads here (and, with them, the first two tiles) so that no
  // compiler-visible load is pending inside the loop
#pragma unroll
  for (int m = 0; m < NMT; ++m) {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) settle(qa[m][kk]);
#pragma unroll
    for (int i = 0; i < 16; ++i) settle(wv[m][i]);
  }
  wait_tile();
  __syncthreads();  // q, w, counters and the first tiles have landed

  // The scores of a tile are finished one tile late: the VALU work that turns a tile's
  // accumulators into scores (ReLU, head weights, head sum) is interleaved with the MFMAs of the
  // next tile, so the matrix cores do not idle while it runs.  A tile's keys are therefore
  // appended during the next tile, and the capacity check leaves room for two tiles.
  constexpr int kElems = NMT * 16;       // accumulator elements per lane
  constexpr int kSlice = kElems / NKK;   // of them finished per MFMA k-step
  static_assert(kElems % NKK == 0, "score slices");
  // The two waves of a row share a SIMD.  The lower-half wave appends a tile's keys right
  // after the MFMAs that finish their scores; the upper-half wave appends them one step later,
  // before its MFMAs, so that one wave's appends overlap the other's MFMAs.
  float ap_sc = 0.0f;  // pending tile: this lane's partial score (half of the heads) ...
  int ap_key = 0;      // ... and key position
  bool ap_on = false;  // a tile is pending
  auto append = [&]() __attribute__((always_inline)) {
    // lanes l and l + 32 hold the two head halves of key l; lanes 0..31 finish the sum
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ap_sc),
                                                     __float_as_uint(ap_sc), false, false);
    const uint32_t u = orderable(ap_sc + __uint_as_float(sw[1]));
    const bool pass = ap_on && lane < 32 && ap_key <= tg && u > tau_eff;
    const uint64_t m = __ballot(pass);
    if (m) {
      const int o = my_n + static_cast<int>(__builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
      if (pass) {
        const int e = half == 0 ? o : C::kCap - 1 - o;
        ck[e] = u;
        cp[e] = ap_key;
      }
      my_n += __popcll(m);
      if (lane == 0) (half == 0 ? sm.cnt : sm.cntb)[row] = my_n;
    }
    ap_on = false;
  };

  // issue_kb >= 0: the tile at key issue_kb is loaded into buffer issue_buf behind the first
  // k-step's MFMAs
  auto mfma_tile = [&](const unsigned char *tile, f32x16 (&cur)[NMT], const f32x16 (&prev)[NMT],
                       auto with_prev, int issue_kb, int issue_buf) -> float {
    bf16x8 bf[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      bf[kk] = as_bf16x8(*reinterpret_cast<const u32x4 *>(tile + boff[kk]));
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
      for (int m = 0; m < NMT; ++m) cur[m] = mfma32(qa[m][kk], bf[kk], kk == 0 ? f32x16{} : cur[m]);
      if (kk == 0 && issue_kb >= 0)
        loads.issue(tile_lds + issue_buf * C::kTileBytes, k, issue_kb, lastg, wave);
      if constexpr (decltype(with_prev)::value) {
#pragma unroll
        for (int j = 0; j < kSlice; j += 2) {
          const int e = kk * kSlice + j;
          s0 = fmaf(wv[e >> 4][e & 15], fmaxf(prev[e >> 4][e & 15], 0.0f), s0);
          s1 = fmaf(wv[(e + 1) >> 4][(e + 1) & 15], fmaxf(prev[(e + 1) >> 4][(e + 1) & 15], 0.0f), s1);
        }
      }
    }
    return s0 + s1;
  };
  auto score_only = [&](const f32x16 (&prev)[NMT]) -> float {
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int e = 0; e < kElems; e += 2) {
      s0 = fmaf(wv[e >> 4][e & 15], fmaxf(prev[e >> 4][e & 15], 0.0f), s0);
      s1 = fmaf(wv[(e + 1) >> 4][(e + 1) & 15], fmaxf(prev[(e + 1) >> 4][(e + 1) & 15], 0.0f), s1);
    }
    return s0 + s1;
  };

  // The lower-half wave moves the upper stack of its row down behind its own entries (the
  // ranges cannot be overlapped destructively: the copy runs upward and its destination
  // always lies below its source); returns the row's entry count.  Called between barriers.
  auto merge_stacks = [&](int n_lo, int n_hi) -> int {
    for (int j = lane; j < n_hi; j += 64) {
      const uint32_t kv = ck[C::kCap - n_hi + j];
      const int32_t pv = cp[C::kCap - n_hi + j];
      wave_sync();
      ck[n_lo + j] = kv;
      cp[n_lo + j] = pv;
    }
    wave_sync();
    return n_lo + n_hi;
  };

  // Compaction of every row far enough above K, by both waves of the row, each on its own
  // stack.  Every wave calls it in the same step (the flag it follows was written by wave 0 in
  // the previous step), after its MFMAs and before its appends, and passes the same five
  // barriers: appends visible | key ranges and cleared histogram | histogram | kept entries and
  // the largest dropped key of each stack | the new threshold and counts.
  //   The keys above the current threshold (all of them before the first one) are binned by
  // value over [threshold, largest key]; the bin b holding the R-th largest key leaves at least
  // R keys in bins >= b, so every key in a lower bin lies below the R-th largest and is dropped,
  // and so is any later key that is not above the largest key dropped, which becomes the new
  // threshold.  R is the row's compaction rank after the keys before kb: K without
  // speculation, so that no key of the final top-K is dropped.
  auto compact_rows = [&](int kb) __attribute__((always_inline)) {
    lds_barrier();
    const int n_lo = __builtin_amdgcn_readfirstlane(sm.cnt[row]);
    const int n_hi = __builtin_amdgcn_readfirstlane(sm.cntb[row]);
    const bool go = n_lo + n_hi > (C::kCap + K) / 2;
    const Stack st{ck, cp, C::kCap, half == 1};
    uint32_t *hist = sm.hist[row];
    if (go) {
      uint32_t lo, hi;
      stack_range(st, my_n, lo, hi);
      *reinterpret_cast<u32x4 *>(hist + (kPruneBins / 2) * half + 4 * lane) = u32x4{0u, 0u, 0u, 0u};
      if (lane == 0) {
        sm.xlo[row][half] = lo;
        sm.xhi[row][half] = hi;
      }
    }
    lds_barrier();
    ValueBinsN<kPruneBins> vb;
    bool binned = false;
    if (go) {
      uint32_t lo = min(sm.xlo[row][0], sm.xlo[row][1]);
      const uint32_t hi = max(sm.xhi[row][0], sm.xhi[row][1]);
      if (my_has_tau) lo = my_tau + 1u;  // every candidate is above the current threshold
      binned = vb.init(lo, hi);
      if (binned) stack_histogram<kPruneBins>(st, my_n, vb, hist);
    }
    lds_barrier();
    bool pruned = false;
    if (binned) {
      uint32_t above;
      const int R = __builtin_amdgcn_readfirstlane(compaction_rank(spec, K, L, kb - start));
      const int b = static_cast<int>(bin_from_top_n<kPruneBins>(hist, static_cast<uint32_t>(R), above));
      if (b > 0) {
        uint32_t dmax;
        my_n = compact_stack(st, my_n, [vb, b](uint32_t u, int32_t) { return vb(u) >= b; }, dmax);
        pruned = true;
        if (lane == 0) {
          sm.xdrop[row][half] = dmax;
          (half == 0 ? sm.cnt : sm.cntb)[row] = my_n;
        }
      }
    }
    lds_barrier();
    if (go && half == 0) {
      uint32_t tau = my_tau;
      bool has = my_has_tau;
      if (pruned) {
        const uint32_t dmax = max(sm.xdrop[row][0], sm.xdrop[row][1]);
        tau = has ? max(tau, dmax) : dmax;
        has = true;
      }
      int n_hi2 = __builtin_amdgcn_readfirstlane(sm.cntb[row]);
      if (my_n + n_hi2 > C::kCap - 3 * kTileKeys) {  // too many ties to make room: exact selection
        // exactly K kept, all at or above the K-th key kth (> the old threshold); a later key
        // equal to kth loses the tie, but the threshold kth - 1 keeps every kept key above it
        int n = merge_stacks(my_n, n_hi2);
        const uint32_t kth = select_exact(ck, cp, hist, n, K, start, tg);
        if (kth > 0u) {
          tau = kth - 1u;
          has = true;
        }
        my_n = n;
        n_hi2 = 0;
      }
      if (lane == 0) {
        sm.tau[row] = tau;
        sm.has_tau[row] = has ? 1 : 0;
        sm.cnt[row] = my_n;
        sm.cntb[row] = n_hi2;
      }
    }
    lds_barrier();  // new thresholds and counts are visible
    my_has_tau = __builtin_amdgcn_readfirstlane(sm.has_tau[row]) != 0;
    my_tau = __builtin_amdgcn_readfirstlane(sm.tau[row]);
    tau_eff = my_has_tau ? my_tau : 0u;
    my_n = __builtin_amdgcn_readfirstlane(half == 0 ? sm.cnt[row] : sm.cntb[row]);
  };
  // Wave 0 decides whether the next step compacts.  The counts it reads hold every append up to
  // the previous step and perhaps some of this step's; until that compaction this step and the
  // next one append at most two tiles per row, hence the margin of three tiles.  Every row far
  // enough above K is compacted in the same round, so the rows of a group (whose counts grow
  // alike) rarely stop the group more than once per round.
  auto decide = [&](int slot) __attribute__((always_inline)) {
    if (wave == 0) {
      const int4 ca = *reinterpret_cast<const int4 *>(sm.cnt);
      const int4 cb = *reinterpret_cast<const int4 *>(sm.cntb);
      const int mx = max(max(ca.x + cb.x, ca.y + cb.y), max(ca.z + cb.z, ca.w + cb.w));
      if (lane == 0) sm.compact[slot] = mx > C::kCap - 3 * kTileKeys ? 1 : 0;
    }
  };

  // one tile: accumulate into `cur`, finish the pending tile held in `prev`
  int buf = 0;
  int sidx = 0;            // step number
  bool have_prev = false;  // `prev` holds the accumulators of an unfinished tile
  int key_prev = 0;
  auto step = [&](int kb, f32x16 (&cur)[NMT], f32x16 (&prev)[NMT]) __attribute__((always_inline)) {
    if (kb > start) {
      if (lastg - kb >= kTileKeys) wait_vm<C::kLoadsPerWave>();  // the next tile may stay in flight
      else wait_tile();
      lds_barrier();  // this tile is complete everywhere; the previous one is free; every
                      // append made so far is visible
    }
    // this step's compaction flag; read now, used after the MFMAs
    const int cflag = sm.compact[sidx & 1];
    // the tile two ahead goes into the previous tile's buffer, issued behind the first MFMAs
    const int issue_kb = lastg - kb >= 2 * kTileKeys ? kb + 2 * kTileKeys : -1;
    const int issue_buf = buf >= C::kNBuf - 2 ? buf + 2 - C::kNBuf : buf + 2;

    if (half == 1) append();  // the tile pending since the previous step
    // ---- this wave's 32 keys of the tile
    const int kbase = kb + half * 32;
    const bool do_cur = compute && kbase <= tg;
    float sc = 0.0f;
    if (do_cur && have_prev) {
      sc = mfma_tile(sm.tile[buf], cur, prev, std::true_type{}, issue_kb, issue_buf);
    } else if (do_cur) {
      mfma_tile(sm.tile[buf], cur, prev, std::false_type{}, issue_kb, issue_buf);
    } else {
      if (issue_kb >= 0) loads.issue(tile_lds + issue_buf * C::kTileBytes, k, issue_kb, lastg, wave);
      if (have_prev) sc = score_only(prev);
    }
    if (__builtin_amdgcn_readfirstlane(cflag)) compact_rows(kb);
    decide((sidx + 1) & 1);
    ap_sc = sc;  // prev's scores: appended now (lower half) or in the next step (upper half)
    ap_key = key_prev;
    ap_on = have_prev;
    if (half == 0) append();
    have_prev = do_cur;
    key_prev = kbase + (lane & 31);
    buf = buf == C::kNBuf - 1 ? 0 : buf + 1;
    ++sidx;
  };
  // the last tile: its append after the compaction (if any) decided in the last step
  auto drain = [&](const f32x16 (&last_acc)[NMT]) __attribute__((always_inline)) {
    float sc = 0.0f;
    if (have_prev) sc = score_only(last_acc);
    lds_barrier();  // every append of the key stream is visible; the flag is written
    if (__builtin_amdgcn_readfirstlane(sm.compact[sidx & 1])) compact_rows(start + L);
    append();  // the upper half's pending tile
    ap_sc = sc;
    ap_key = key_prev;
    ap_on = have_prev;
    append();
  };
  f32x16 acc_a[NMT], acc_b[NMT];
  int kb = start;
  while (true) {  // two tiles per trip so that the accumulator sets alternate without copies
    step(kb, acc_a, acc_b);
    kb += kTileKeys;
    if (kb > lastg) {
      drain(acc_a);
      break;
    }
    step(kb, acc_b, acc_a);
    kb += kTileKeys;
    if (kb > lastg) {
      drain(acc_b);
      break;
    }
  }

  lds_barrier();  // every append is visible; no tile load is in flight
  if (compute && half == 0) {
    // the key tiles are free now: per row a 4 KB bitmap and a kScratch-entry scratch list, and
    // with 128-dim keys (48 KB of tiles) a 1024-bin value histogram, whose narrower bins
    // collide less in the LDS atomics than the 256 of the compactions
    uint32_t *tiles = reinterpret_cast<uint32_t *>(&sm.tile[0][0]);
    uint32_t *bm = tiles + row * 1024;
    uint32_t *sk = tiles + 4 * 1024 + row * 2 * kScratch;
    int32_t *sp = reinterpret_cast<int32_t *>(sk + kScratch);
    const int n = merge_stacks(my_n, __builtin_amdgcn_readfirstlane(sm.cntb[row]));
    // Every key above the final threshold is an entry; fewer than K of them means that a
    // speculative compaction dropped keys of the top-K: the row is left to the second launch.
    if (n < K) {
      if (lane == 0) len_out[t] = -1;
      return;
    }
    if constexpr (kFinalBins<D> == 1024) {
      select_and_write<1024>(ck, cp, tiles + 6 * 1024 + row * 1024, sm.hist[row], n, K,
                             my_has_tau, my_tau, start, tg, bm, sk, sp,
                             idx_out + static_cast<int64_t>(t) * K);
    } else {
      select_and_write<256>(ck, cp, sm.hist[row], sm.hist[row], n, K, my_has_tau, my_tau, start,
                            tg, bm, sk, sp, idx_out + static_cast<int64_t>(t) * K);
    }
    if (lane == 0) len_out[t] = K;
  }
}

template <int NMT, int D>
__global__ __launch_bounds__(kThreads) void indexer_topk_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const float *__restrict__ w,
    const int32_t *__restrict__ seq_start, const int32_t *__restrict__ causal_len,
    const int32_t *__restrict__ gpos, const int32_t *__restrict__ groups,
    const int32_t *__restrict__ group_first, int H, int K, int32_t *__restrict__ idx_out,
    int32_t *__restrict__ len_out) {
  indexer_group<NMT, D>(q, k, w, seq_start, causal_len, gpos, groups, group_first, H, K, idx_out,
                        len_out, blockIdx.x, true);
}

// Second launch: recomputes, without speculation, every group that has a row of length -1.
// Each work group checks the groups blockIdx.x + i gridDim.x, 64 at a time (one per lane, the
// same in every wave, so the decisions are uniform), and then runs the flagged ones.
template <int NMT, int D>
__global__ __launch_bounds__(kThreads) void indexer_topk_redo_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const float *__restrict__ w,
    const int32_t *__restrict__ seq_start, const int32_t *__restrict__ causal_len,
    const int32_t *__restrict__ gpos, const int32_t *__restrict__ groups,
    const int32_t *__restrict__ group_first, int H, int K, int32_t *__restrict__ idx_out,
    int32_t *__restrict__ len_out, int n_groups) {
  const int lane = threadIdx.x & 63;
  for (int64_t base = 0; blockIdx.x + base * gridDim.x < n_groups; base += 64) {
    const int64_t gl = blockIdx.x + (base + lane) * gridDim.x;
    bool bad = false;
    if (gl < n_groups) {
      const int last = groups[gl];
      const int start = seq_start[last];
      const int first = group_first ? group_first[gl]
                                    : (last - (kRows - 1) > start ? last - (kRows - 1) : start);
      for (int t = first; t <= last; ++t) bad |= len_out[t] < 0;
    }
    uint64_t m = __ballot(bad);
    while (m != 0u) {
      const int i = __builtin_ctzll(m);
      m &= m - 1u;
      __syncthreads();  // the previous group is done with the LDS
      indexer_group<NMT, D>(q, k, w, seq_start, causal_len, gpos, groups, group_first, H, K,
                            idx_out, len_out, static_cast<int>(blockIdx.x + (base + i) * gridDim.x),
                            false);
    }
  }
}

template <int NMT, int D>
hipError_t launch(const uint16_t *q, const uint16_t *k, const float *w, const IndexerRows &r,
                  int32_t H, int32_t K, int32_t *idx, int32_t *len, hipStream_t s) {
  const size_t smem = sizeof(IndexerSmem<D>);
  auto kern = indexer_topk_kernel<NMT, D>;
  auto redo = indexer_topk_redo_kernel<NMT, D>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(smem));
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(redo),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
  if (e != hipSuccess) return e;
  DSA_LAUNCH("indexer_topk", kern, dim3(r.n_groups), dim3(kThreads), smem, s, q, k, w,
             r.seq_start, r.causal_len, r.gpos, r.groups, r.group_first, H, K, idx, len);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int redo_groups = r.n_groups < kRedoGroups ? r.n_groups : kRedoGroups;
  DSA_LAUNCH("indexer_topk_redo", redo, dim3(redo_groups), dim3(kThreads), smem, s, q, k, w,
             r.seq_start, r.causal_len, r.gpos, r.groups, r.group_first, H, K, idx, len,
             r.n_groups);
  return hipGetLastError();
}

}  // namespace

// k-pool rows: the selected pools (pool coordinates, ascending) -> their keys, then the row's
// incomplete tail pool; one wave per row.
__global__ __launch_bounds__(256) void kpool_expand_kernel(
    const int32_t *__restrict__ pidx, const int32_t *__restrict__ plen,
    const int32_t *__restrict__ pool_start, const int32_t *__restrict__ n_pools,
    const int32_t *__restrict__ key_start, int64_t T, int Kp, int pool,
    int32_t *__restrict__ idx, int32_t *__restrict__ len) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  const int W = Kp * pool + pool - 1;
  const int n = plen[t];
  const int ps = pool_start[t], ks = key_start[t];
  const int P = n_pools[t];
  const int tail = static_cast<int>(t - ks) + 1 - P * pool;  // keys after the last complete pool
  const int32_t *prow = pidx + t * Kp;
  int32_t *row = idx + t * W;
  for (int j = lane; j < W; j += 64) {
    int32_t v = -1;
    if (j < n * pool) {
      v = ks + (prow[j / pool] - ps) * pool + j % pool;
    } else if (j < n * pool + tail) {
      v = ks + P * pool + (j - n * pool);
    }
    row[j] = v;
  }
  if (lane == 0) len[t] = n * pool + tail;
}

hipError_t launch_kpool_expand(const int32_t *pidx, const int32_t *plen,
                               const int32_t *pool_start, const int32_t *n_pools,
                               const int32_t *key_start, int64_t T, int32_t Kp, int32_t pool,
                               int32_t *idx, int32_t *len, hipStream_t s) {
  if (T == 0) return hipSuccess;
  DSA_LAUNCH("kpool_expand", kpool_expand_kernel, dim3(static_cast<unsigned>((T + 3) / 4)),
             dim3(256), 0, s, pidx, plen, pool_start, n_pools, key_start, T, Kp, pool, idx, len);
  return hipGetLastError();
}

hipError_t launch_indexer_topk(const uint16_t *q, const uint16_t *k, const float *w,
                               const IndexerRows &r, int32_t H, int32_t D, int32_t K,
                               int32_t *idx, int32_t *len, hipStream_t s) {
  if (r.n_groups == 0) return hipSuccess;
  const bool two = H > 32;
  if (D == 128) return two ? launch<2, 128>(q, k, w, r, H, K, idx, len, s)
                           : launch<1, 128>(q, k, w, r, H, K, idx, len, s);
  if (D == 64) return two ? launch<2, 64>(q, k, w, r, H, K, idx, len, s)
                          : launch<1, 64>(q, k, w, r, H, K, idx, len, s);
  return hipErrorInvalidValue;
}

}  // namespace dsa
