// THD metadata for packed variable-length batches (NeMo AutoModel cudnn_dsa API reference,
// prepare_cudnn_dsa_packed_metadata / CudnnDsaPackedMetadata: per-query sequence starts and
// real causal lengths, built once and reused by every layer).
//
// One thread per item.  Items [0, T) are query rows: seq_start, causal length L_t, the top-k
// valid length min(K, L_t), and the row's rank in a longest-first order.  Items
// [T, T + n_groups) are indexer work groups (kIdxRowsPerGroup consecutive rows of one
// sequence, aligned to the sequence end); each is written at its rank in decreasing-cost
// order, cost = L of the group's last row.  Ranks are closed-form counts over the B sequences,
// so no sort is needed and the result is deterministic.
#include "dsa_common.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

__device__ __forceinline__ int32_t find_seq(const int32_t *cu, int32_t B, int64_t t) {
  // largest b with cu[b] <= t (zero-length sequences are skipped by taking the largest)
  int32_t lo = 0, hi = B;  // invariant: cu[lo] <= t < cu[hi]
  while (hi - lo > 1) {
    int32_t mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

__global__ void thd_metadata_kernel(const int32_t *__restrict__ cu, int32_t B, int64_t T,
                                    int32_t K, int32_t *__restrict__ seq_start,
                                    int32_t *__restrict__ causal_len,
                                    int32_t *__restrict__ topk_length,
                                    int32_t *__restrict__ row_order, int32_t *__restrict__ groups,
                                    int32_t n_groups) {
  const int64_t item = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  constexpr int32_t G = kIdxRowsPerGroup;
  if (item < T) {
    const int64_t t = item;
    const int32_t b = find_seq(cu, B, t);
    const int32_t start = cu[b];
    const int32_t L = static_cast<int32_t>(t - start + 1);
    seq_start[t] = start;
    causal_len[t] = L;
    topk_length[t] = L < K ? L : K;
    // rank among all rows by decreasing L; ties: lower sequence index first
    int64_t rank = 0;
    for (int32_t bb = 0; bb < B; ++bb) {
      const int32_t len = cu[bb + 1] - cu[bb];
      if (len > L) rank += len - L;
      if (bb < b && len >= L) rank += 1;
    }
    row_order[rank] = static_cast<int32_t>(t);
  } else if (item < T + n_groups) {
    // locate group: sequences contribute ceil(len/G) groups each, in sequence order
    int32_t gid = static_cast<int32_t>(item - T);
    int32_t b = 0;
    for (; b < B; ++b) {
      const int32_t ng = (cu[b + 1] - cu[b] + G - 1) / G;
      if (gid < ng) break;
      gid -= ng;
    }
    const int32_t len_b = cu[b + 1] - cu[b];
    const int32_t cost = len_b - G * gid;  // L of the group's last row, >= 1
    int64_t rank = 0;
    for (int32_t bb = 0; bb < B; ++bb) {
      const int32_t len = cu[bb + 1] - cu[bb];
      if (len > cost) rank += (len - cost + G - 1) / G;
      if (bb < b && len >= cost && (len - cost) % G == 0) rank += 1;
    }
    groups[rank] = cu[b + 1] - 1 - G * gid;
  }
}

}  // namespace

hipError_t launch_thd_metadata(const int32_t *cu, int32_t B, int64_t T, int32_t K,
                               int32_t *seq_start, int32_t *causal_len, int32_t *topk_length,
                               int32_t *row_order, int32_t *groups, int32_t n_groups,
                               hipStream_t s) {
  const int64_t items = T + n_groups;
  if (items == 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (items + threads - 1) / threads;
  DSA_LAUNCH("thd_metadata", thd_metadata_kernel, dim3(static_cast<unsigned>(blocks)), dim3(threads), 0,
                     s, cu, B, T, K, seq_start, causal_len, topk_length, row_order, groups,
                     n_groups);
  return hipGetLastError();
}

}  // namespace dsa
