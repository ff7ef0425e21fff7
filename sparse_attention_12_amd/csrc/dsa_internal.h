// Launchers shared between the kernel translation units and the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

// Benchmark event hooks around every kernel launch (no-ops unless armed through
// dsa_record_kernel_events on the calling thread).
void kernel_begin(hipStream_t s, const char *name);
void kernel_end(hipStream_t s);

// Launch `kern` with the event hooks around it.
#define DSA_LAUNCH(name, kern, grid, block, smem, stream, ...)                   \
  do {                                                                            \
    ::dsa::kernel_begin(stream, name);                                            \
    hipLaunchKernelGGL(kern, grid, block, smem, stream, __VA_ARGS__);             \
    ::dsa::kernel_end(stream);                                                    \
  } while (0)

// Rows of one indexer work group (consecutive query rows of one sequence).
constexpr int kIdxRowsPerGroup = 4;

// Listed rows per work group of the gather probe.
constexpr int64_t kGatherProbeRows = 2048;
hipError_t launch_gather_probe(const uint16_t *table, int32_t width, const int32_t *idx,
                               int64_t n, uint32_t *sink, hipStream_t s);

hipError_t launch_thd_metadata(const int32_t *cu, int32_t B, int64_t T, int32_t K,
                               int32_t *seq_start, int32_t *causal_len, int32_t *topk_length,
                               int32_t *row_order, int32_t *groups, int32_t n_groups,
                               hipStream_t s);

// Query rows of one indexer call (device arrays of the metadata).  gpos / group_first are
// NULL when every row is its own key position (one tensor of queries and keys); otherwise
// gpos[i] is the key position of local row i and group_first[g] the first row of group g.
struct IndexerRows {
  const int32_t *seq_start;   // [T_q] key position of the row's sequence start
  const int32_t *causal_len;  // [T_q] keys of the row (0: padding row)
  const int32_t *gpos;        // [T_q] or NULL
  const int32_t *groups;      // [n_groups] last row of each group
  const int32_t *group_first; // [n_groups] or NULL
  int32_t n_groups;
};

hipError_t launch_indexer_topk(const uint16_t *q, const uint16_t *k, const float *w,
                               const IndexerRows &r, int32_t H, int32_t D, int32_t K,
                               int32_t *idx, int32_t *len, hipStream_t s);

// k-pool rows: pool selection (pidx [T, Kp] pool coordinates, plen [T]) -> key indices
// idx [T, Kp * pool + pool - 1] and lengths, appending each row's incomplete tail pool.
hipError_t launch_kpool_expand(const int32_t *pidx, const int32_t *plen,
                               const int32_t *pool_start, const int32_t *n_pools,
                               const int32_t *key_start, int64_t T, int32_t Kp, int32_t pool,
                               int32_t *idx, int32_t *len, hipStream_t s);

hipError_t launch_sparse_mla_fwd(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                                 const int32_t *topk_length, int64_t T_q, int32_t H,
                                 int32_t D_qk, int32_t K, float scale, uint16_t *out, float *lse,
                                 hipStream_t s);

// Buffers of one backward pass (the key-gradient staging and its counting sort).
struct BwdPassBuffers {
  int32_t *off;     // [T_kv + 1] per latent row: contribution count, then list offset
  int32_t *cursor;  // [T_kv]
  int32_t *list;    // [rows_per_pass * K] pair ids grouped by latent row
  uint32_t *stage;  // [rows_per_pass * K] staged contribution rows of bwd_stage_row_bytes each
};

// Bytes of one staged key-gradient contribution row: D_qk signed 16-bit mantissas, then 16
// exponent bytes (one per block of D_qk / 16 channels).
constexpr size_t bwd_stage_row_bytes(int32_t D_qk) { return static_cast<size_t>(D_qk) * 2 + 16; }

// Backward workspace carved from the caller's buffer.  With two pass buffers the reduction of
// pass p runs on a helper stream while pass p + 1 computes on the caller's stream.
struct BwdWorkspace {
  float *delta;           // [T_q, H]
  int32_t *flag;          // debug index check
  uint32_t *vmax;         // largest |kv| (bf16 magnitude bits), for the fp16 operand scales
  BwdPassBuffers buf[2];
  int nbuf;               // 1 or 2
  int64_t rows_per_pass;  // query rows per pass (>= 1)
};

hipError_t launch_sparse_mla_bwd(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                                 const int32_t *topk_length, const uint16_t *out,
                                 const float *lse, const uint16_t *dout, int64_t T_q,
                                 int64_t T_kv, int32_t H, int32_t D_qk, int32_t K, float scale,
                                 uint16_t *dq, float *dkv, bool accumulate,
                                 const BwdWorkspace &ws, hipStream_t s,
                                 float *kl_target = nullptr);

// Counting sort of the (query, slot) pairs of query rows [row0, row0 + rows) by key row, and
// the per-key-row sum of their staged contributions into dst [n_rows, D] (D = 128: the indexer
// key gradient); the staging kernel counts each key row's pairs into bb.off after count_zero.
hipError_t launch_pair_count_zero(int64_t n_rows, const BwdPassBuffers &bb, hipStream_t s);
hipError_t launch_pair_sort(const int32_t *idx, const int32_t *topk_length, int64_t row0,
                            int64_t rows, int64_t n_rows, int32_t K, const BwdPassBuffers &bb,
                            hipStream_t s);
hipError_t launch_pair_reduce(int32_t D, int64_t n_rows, const BwdPassBuffers &bb, float *dst,
                              hipStream_t s);
hipError_t launch_fill_zero(float *p, int64_t n, hipStream_t s);

// Indexer KL loss: the attention target (score recompute) and the indexer backward over the
// pass buffers (see dsa.h).
hipError_t launch_indexer_kl_target(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                                    const int32_t *topk_length, const float *lse, int64_t T_q,
                                    int32_t H, int32_t D_qk, int32_t K, float scale,
                                    float *target, hipStream_t s);
hipError_t launch_indexer_kl_bwd(const uint16_t *q_idx, const uint16_t *k_idx, const float *w,
                                 const int32_t *idx, const int32_t *topk_length,
                                 const float *target, int64_t T_q, int64_t T_kv, int32_t H_i,
                                 int32_t K, float grad, float *loss, uint16_t *dq_idx, float *dw,
                                 float *dk_idx, bool accumulate, const BwdPassBuffers &bb,
                                 int64_t rows_per_pass, hipStream_t s);

// Fixed device scratch of the allocation-free backward, per GPU (bytes), and the device address
// of the calling thread's current GPU's copy (looked up on first use per device).
constexpr size_t kNoAllocScratchBytes = static_cast<size_t>(256) << 20;
constexpr int kMaxDevices = 64;
hipError_t noalloc_scratch(void **ptr);

// Attention sink: the forward epilogue (out, lse rescaled in place) and the sink gradient.
hipError_t launch_sink_fwd(const float *sink, int64_t T_q, int32_t H, int32_t D_v,
                           uint16_t *out, float *lse, hipStream_t s);
hipError_t launch_sink_bwd(const float *sink, const float *lse, const uint16_t *out,
                           const uint16_t *dout, int64_t T_q, int32_t H, int32_t D_v,
                           float *dsink, bool accumulate, hipStream_t s);

hipError_t launch_check_indices(const int32_t *idx, const int32_t *topk_length, int64_t T_q,
                                int32_t K, int64_t T_kv, int32_t *bad_flag, hipStream_t s);

}  // namespace dsa
