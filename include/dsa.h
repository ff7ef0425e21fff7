/*
 * dsa.h -- C ABI of libdsa: the DeepSeek Sparse Attention (DSA) hot path on
 * AMD Instinct MI355X (gfx950).
 *
 * Two stages:
 *   1. the lightning indexer, which scores every causal key of each query and
 *      keeps the k best per query (NVIDIA "Accelerating GLM-5.2 Long-Context
 *      Training with cuDNN Fused DSA Kernels ...", section "How DSA works";
 *      NeMo AutoModel cudnn_dsa API reference, cudnn_indexer_topk);
 *   2. absorbed sparse MLA, where all heads of a query attend one gathered set
 *      of latent rows, forward and backward (same page, "Why DSA needs fused
 *      kernels"; API reference cudnn_sparse_attention and
 *      _CudnnSparseAttention.forward / .backward).
 *
 * Conventions shared by every call
 *   - All tensor arguments are DEVICE pointers to contiguous row-major
 *     buffers owned by the caller, aligned to 16 bytes.  bf16 tensors are
 *     passed as uint16_t* holding the bf16 bit patterns.  The library never
 *     allocates or frees device memory: scratch space comes from a caller
 *     buffer sized by the matching *_workspace_size() query.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on it and returns; results are valid once the stream has
 *     executed the work.  The single exception is dsa_prepare_thd_metadata,
 *     which synchronises once to read the sequence offsets.
 *   - Every call returns a dsa_status, and on error a message for the calling
 *     thread is available from dsa_last_error().  An error found by the
 *     argument checks returns before anything is enqueued.  A HIP error from a
 *     launch can come after earlier kernels of the same call were enqueued
 *     (the backward's passes): the call's outputs are then undefined.
 *     Argument checks never read device memory (no hidden synchronisation);
 *     index CONTENTS are trusted: an index outside [0, T_kv) other than -1 is
 *     undefined behaviour unless DSA_DEBUG_CHECK_INDICES is set in `flags`.
 *   - Outputs that depend on floating-point summation order: O, LSE and dq are
 *     bitwise reproducible run to run.  dkv is not: each latent row's
 *     contributions are summed in fp32 in the order of a list that device
 *     atomics build, so dkv is reproducible only up to summation order.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_VALUE = 1, /* shape, size, alignment or value out of range */
  DSA_ERR_UNSUPPORTED = 2,   /* device is not gfx950, or the combination is not built */
  DSA_ERR_WORKSPACE = 3,     /* workspace pointer missing or smaller than required */
  DSA_ERR_HIP = 4            /* a HIP runtime call failed (message carries its text) */
} dsa_status;

/* Flags for dsa_sparse_mla_bwd. */
#define DSA_BWD_ACCUMULATE_DKV 0x1u   /* add into dkv instead of overwriting it */
#define DSA_DEBUG_CHECK_INDICES 0x100u /* validate index contents on the device
                                          (adds one synchronisation); debugging only */

/* Message describing the last error returned on the calling thread ("" if none). */
const char *dsa_last_error(void);

/* 1 if `device` is an AMD gfx950 GPU this library was built for, else 0. */
int dsa_device_supported(int device);

/* Largest top-k width the indexer accepts (GLM-5.2's fixed selection width:
 * cudnn_dsa API reference, _validate_topk / _MAX_TOPK). */
#define DSA_MAX_INDEXER_TOPK 2048

/* --------------------------------------------------------------------------
 * THD metadata (API reference: prepare_cudnn_dsa_packed_metadata -- per-query
 * starts and real causal lengths of a packed variable-length batch, built once
 * with one device-to-host synchronisation and reused by every indexer and
 * attention layer; CudnnDsaPackedMetadata).
 * ------------------------------------------------------------------------ */
typedef struct dsa_thd_metadata {
  /* device arrays inside the caller's workspace, valid while it lives */
  int32_t *seq_start;   /* [T]  first token of the row's sequence            */
  int32_t *causal_len;  /* [T]  L_t = t - seq_start[t] + 1 keys (s <= t)     */
  int32_t *topk_length; /* [T]  min(K, L_t)                                  */
  int32_t *row_order;   /* [T]  query rows ordered by decreasing L_t (work schedule) */
  int32_t *groups;      /* [n_groups] indexer work groups: last row of each run of up to 4
                           consecutive rows of one sequence, ordered by decreasing cost */
  /* host values */
  int64_t T;            /* total tokens (= cu_seqlens[B])                    */
  int32_t B;            /* number of sequences                               */
  int32_t K;            /* top-k width the lengths were computed for         */
  int32_t max_seqlen;   /* longest sequence                                  */
  int32_t all_rows_nonempty; /* 1 when every row has at least one valid slot */
  int64_t total_pairs;  /* sum_t L_t   (causal query-key pairs)              */
  int64_t total_valid;  /* sum_t min(K, L_t)                                  */
  int32_t n_groups;     /* sum over sequences of ceil(length / 4)             */
  /* local query rows (dsa_prepare_local_metadata); NULL / T otherwise            */
  int32_t *gpos;        /* [T]  key-tensor coordinate of each local query row  */
  int32_t *group_first; /* [n_groups] first row of each indexer work group     */
  int64_t total_key_tokens; /* rows of the key tensors (k_idx, kv)            */
  /* k-pool rows (dsa_prepare_kpool_metadata); NULL / 0 otherwise                */
  int32_t *key_start;   /* [T]  first token of the row's sequence               */
  int32_t pool;         /* keys per pool                                        */
} dsa_thd_metadata;

/* Bytes of workspace the metadata for T tokens needs. */
size_t dsa_thd_metadata_workspace_size(int64_t T);

/* Builds `md` from cu_seqlens (device int32 [B+1], cumulative sequence
 * lengths: cu[0] = 0, non-decreasing, cu[B] = T; zero-length sequences are
 * allowed).  K in [1, 2048] is the width topk_length is clipped to.  Copies
 * cu_seqlens to the host and synchronises `stream` once; everything else runs
 * on the stream.  Errors: DSA_ERR_INVALID_VALUE for bad B/T/K or offsets;
 * DSA_ERR_WORKSPACE if ws is NULL or ws_bytes too small. */
int dsa_prepare_thd_metadata(const int32_t *cu_seqlens, int32_t B, int64_t T, int32_t K,
                             void *ws, size_t ws_bytes, dsa_thd_metadata *md, void *stream);

/* Local query rows against gathered global keys (API reference
 * prepare_cudnn_dsa_packed_metadata: query_indices are global padded-storage
 * coordinates of the local query rows, cu_seqlens_padded the padded storage
 * boundaries, padding_mask the local padding rows; cudnn_indexer_topk then
 * returns indices in global padded-storage coordinates).
 *   cu_seqlens        device int32 [B+1], real lengths (cu[0] = 0, non-decreasing)
 *   cu_seqlens_padded device int32 [B+1] or NULL (= cu_seqlens); each padded
 *                     sequence at least as long as the real one, cu_pad[B] <= T_k
 *   query_indices     device int32 [T_q] or NULL (identity: T_q = cu_pad[B])
 *   padding_mask      device uint8 [T_q] or NULL; nonzero marks a padding row
 * Local row i with coordinate p lies in sequence b (cu_pad[b] <= p <
 * cu_pad[b+1]) at position pos = p - cu_pad[b]; it is real when pos < cu[b+1]
 * - cu[b] and it is not masked, and then sees the keys cu_pad[b] .. p
 * (causal_len = pos + 1); a padding row has causal_len 0, and the indexer
 * gives it len 0 and -1 everywhere.  The metadata feeds dsa_indexer_topk with
 * q_idx / w of T_q rows and k_idx of T_k rows.  Reads its inputs on the host
 * and synchronises `stream` twice (inputs, then the upload of the tables).
 * Errors: DSA_ERR_INVALID_VALUE for bad sizes, offsets or coordinates;
 * DSA_ERR_WORKSPACE if ws is NULL or smaller than
 * dsa_local_metadata_workspace_size(T_q). */
size_t dsa_local_metadata_workspace_size(int64_t T_q);
int dsa_prepare_local_metadata(const int32_t *cu_seqlens, const int32_t *cu_seqlens_padded,
                               const int32_t *query_indices, const uint8_t *padding_mask,
                               int32_t B, int64_t T_q, int64_t T_k, int32_t K, void *ws,
                               size_t ws_bytes, dsa_thd_metadata *md, void *stream);

/* --------------------------------------------------------------------------
 * k-pool indexer (SkyRL PR 2388, "Why": GLM-5.3-Flash selects keys by pools
 * and adds the still-incomplete pool at the end of the query, which is why its
 * top-k width is 2048 + 3 = 2051).  The pool selection is not spelled out on the page.
 * Reading implemented: the keys of every sequence form pools of `pool`
 * consecutive keys from the sequence start, and the caller supplies one
 * indexer key per complete pool, k_pool [T_pool, D_i] bf16 with sequence b's
 * pools from row cp[b] = sum over b' < b of floor(len_b' / pool).  Query row
 * t of sequence b (position pos = t - cu[b]) sees the P = floor((pos + 1) /
 * pool) pools ending at or before t, scores pool i as
 *     I(t,i) = sum_h w[t,h] * max(0, q_idx[t,h] . k_pool[cp[b] + i])
 * (as dsa_indexer_topk, ties to the lower pool), keeps the n = min(K_pools, P)
 * best and writes their keys in ascending order, then the incomplete tail
 * pool's keys cu[b] + pool P .. t (at most pool - 1); idx [T, W] with
 * W = K_pools * pool + pool - 1, -1 after len = pool n + (pos + 1 - pool P).
 *
 * dsa_prepare_kpool_metadata: rows, pool coordinates and indexer work groups
 * (rows that see the same pools) from cu_seqlens (device int32 [B+1]; one
 * synchronisation to read it, one after the upload of the tables); fills md
 * (md->total_key_tokens = T_pool, md->pool, md->key_start).  1 <= pool <= 16,
 * 1 <= K_pools <= 2048.
 * dsa_kpool_indexer_topk: q_idx [T, H_i, D_i], k_pool [T_pool, D_i], w [T, H_i]
 * with that metadata (limits of dsa_indexer_topk) -> idx, len; workspace of
 * dsa_kpool_indexer_topk_workspace_size(T, K_pools) bytes (the pool
 * selection before it is expanded to keys).
 * ------------------------------------------------------------------------ */
size_t dsa_kpool_metadata_workspace_size(int64_t T);
int dsa_prepare_kpool_metadata(const int32_t *cu_seqlens, int32_t B, int64_t T, int32_t pool,
                               int32_t K_pools, void *ws, size_t ws_bytes, dsa_thd_metadata *md,
                               void *stream);
size_t dsa_kpool_indexer_topk_workspace_size(int64_t T, int32_t K_pools);
int dsa_kpool_indexer_topk(const uint16_t *q_idx, const uint16_t *k_pool, const float *w,
                           const dsa_thd_metadata *md, int32_t H_i, int32_t D_i, int32_t K_pools,
                           int32_t *idx, int32_t *len, void *ws, size_t ws_bytes, void *stream);

/* --------------------------------------------------------------------------
 * Lightning indexer + top-k (GLM-5.2 page, "How DSA works": the indexer rates
 * how relevant each key is to a query and hands the k best keys on;
 * API reference cudnn_indexer_topk and _compact_and_sort_indices).
 *
 * Score of query row t and key s of the same sequence with s <= t:
 *     I(t,s) = sum_h w[t,h] * max(0, sum_d q_idx[t,h,d] * k_idx[s,d])
 * computed with bf16 products accumulated in fp32; ReLU, weighting and the
 * head sum are fp32.  The weights are used exactly as given (the caller owns
 * the 1/sqrt(H) and 1/sqrt(D) scaling, cudnn_indexer_topk head_weights).
 *
 * Output for row t: the n = min(K, L_t) keys with the largest I (equal scores:
 * lower position first), written as ascending global row positions in
 * idx[t, 0:n], idx[t, n:K] = -1, len[t] = n.  No score matrix is stored.
 * The call enqueues two kernels on the stream: the second recomputes the rows
 * for which the first one's speculative candidate threshold proved too high
 * (between the two, such a row holds len = -1); both outputs are final once
 * the call's work on the stream has finished.
 *
 *   q_idx [T, H_i, D_i] bf16   k_idx [T, D_i] bf16   w [T, H_i] fp32
 * (with metadata from dsa_prepare_local_metadata: q_idx, w, idx and len have
 * T = md->T local rows, k_idx has md->total_key_tokens rows, and indices are
 * key-tensor coordinates)
 *   idx   [T, K] int32 (out)   len [T] int32 (out)
 * Supported: 1 <= H_i <= 64, D_i in {64, 128}, 1 <= K <= 2048,
 * T <= INT32_MAX - 4096 (DSA_ERR_INVALID_VALUE otherwise).
 * ------------------------------------------------------------------------ */
size_t dsa_indexer_topk_workspace_size(int64_t T, int32_t H_i, int32_t D_i, int32_t K);
int dsa_indexer_topk(const uint16_t *q_idx, const uint16_t *k_idx, const float *w,
                     const dsa_thd_metadata *md, int32_t H_i, int32_t D_i, int32_t K,
                     int32_t *idx, int32_t *len, void *ws, size_t ws_bytes, void *stream);

/* --------------------------------------------------------------------------
 * Absorbed sparse MLA forward (API reference cudnn_sparse_attention and
 * _CudnnSparseAttention.forward; SkyRL PR 2388 "Why"/"Change" for the NoPE
 * width 512 and top-k widths that are not a multiple of 64).
 *
 * For query row t and head h, the valid slots are j < (topk_length ?
 * topk_length[t] : K) with idx[t,j] != -1.  With logits
 * z_j = scale * <q[t,h,0:D_qk], kv[idx[t,j], 0:D_qk]>:
 *     lse[t,h] = log sum_j exp(z_j)                      (natural log)
 *     out[t,h] = sum_j exp(z_j - lse[t,h]) * kv[idx[t,j], 0:D_v]
 * A row with no valid slot gives out = 0 and lse = -inf.
 *
 *   q   [T_q, H, D_qk] bf16     kv [T_kv, D_qk] bf16 (one latent row per key)
 *   idx [T_q, K] int32          topk_length [T_q] int32 or NULL
 *   out [T_q, H, D_v] bf16 (out)   lse [T_q, H] fp32 (out)
 * `scale` is applied unchanged.  Supported: 1 <= H <= 64, D_qk in {512, 576},
 * D_v = 512, 1 <= K <= 4096, T_kv >= 1 whenever T_q > 0, and kv below 4 GiB
 * (T_kv * D_qk * 2 <= 2^32 - 1; latent rows are addressed with 32-bit byte
 * offsets).  Anything else returns DSA_ERR_INVALID_VALUE.  When topk_length is
 * given the prefix must hold valid indices (it is read without checking for -1
 * beyond the -1 test).
 * ------------------------------------------------------------------------ */
int dsa_sparse_mla_fwd(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                       const int32_t *topk_length, int64_t T_q, int64_t T_kv, int32_t H,
                       int32_t D_qk, int32_t D_v, int32_t K, float scale, uint16_t *out,
                       float *lse, void *stream);

/* --------------------------------------------------------------------------
 * Absorbed sparse MLA backward (API reference _CudnnSparseAttention.backward:
 * gradients for the query [T_q, H, 576] and the latent rows; SkyRL PR 2423
 * "Summary": query chunks are independent and their key gradients sum).
 *
 * With P_j = exp(z_j - lse), dP_j = <dout[t,h], kv[s_j, 0:D_v]>,
 * Delta = <dout[t,h], out[t,h]> (from the bf16 `out` given), and
 * dZ_j = P_j (dP_j - Delta):
 *     dq[t,h,0:D_qk]   = scale * sum_j dZ_j kv[s_j, 0:D_qk]
 *     dkv[s_j, 0:D_qk] += scale * dZ_j q[t,h,0:D_qk]   (over all h, t)
 *     dkv[s_j, 0:D_v]  += P_j dout[t,h]
 *
 *   out, lse: the forward's outputs; dout [T_q, H, D_v] bf16
 *   dq  [T_q, H, D_qk] bf16 (out)   dkv [T_kv, D_qk] fp32 (out / accumulated)
 * flags: DSA_BWD_ACCUMULATE_DKV adds into dkv (query-chunked execution);
 * without it dkv is overwritten.  Same shape limits as dsa_sparse_mla_fwd.
 *
 * Workspace (caller-owned device memory, contents need not be initialised):
 * the key gradient is formed by staging one contribution row of D_qk values
 * per (query, valid slot) as 16-bit block floating point (blocks of D_qk / 16
 * channels sharing a power-of-two scale: error <= 2^-15 of the block's largest
 * magnitude; 2 * D_qk + 16 bytes per row), and summing each latent row's
 * contributions in fp32 after a counting sort, so no atomics touch dkv.  The query rows are
 * processed in passes of R rows, R being as large as ws_bytes allows:
 * dsa_sparse_mla_bwd_workspace_size(..., rows_per_pass) gives the bytes for
 * passes of rows_per_pass rows (<= 0: all T_q rows in one pass, about
 * T_q * K * (2 * D_qk + 20) bytes).  Several passes use two staging buffers:
 * the reduction of pass p then runs on a helper stream of the library (one per
 * calling thread and device, created on first use and kept) while pass p + 1
 * computes on `stream`, which waits for the helper before the call's work
 * ends.  Any ws_bytes of at least the size for rows_per_pass = 1 works; less
 * returns DSA_ERR_WORKSPACE.
 * ------------------------------------------------------------------------ */
size_t dsa_sparse_mla_bwd_workspace_size(int64_t T_q, int64_t T_kv, int32_t H, int32_t D_qk,
                                         int32_t K, int64_t rows_per_pass);
int dsa_sparse_mla_bwd(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                       const int32_t *topk_length, const uint16_t *out, const float *lse,
                       const uint16_t *dout, int64_t T_q, int64_t T_kv, int32_t H,
                       int32_t D_qk, int32_t D_v, int32_t K, float scale, uint16_t *dq,
                       float *dkv, uint32_t flags, void *ws, size_t ws_bytes, void *stream);

/* --------------------------------------------------------------------------
 * Indexer training loss (GLM-5.2 page, "How DSA works": an extra KL loss pulls
 * the indexer's score distribution toward that of the main attention, and it
 * is trained on a graph of its own; "GLM-5.2 training
 * results": sparse formulation, coefficient 0.001, computed with a
 * score-recompute step and an indexer backward; "cuDNN fused DSA kernels").
 * The pages give no formula.  Reading implemented, for query row t with the
 * attention's valid slots j (idx[t,j] != -1, j < topk_length) and key rows s_j:
 *   target  p(j) = sum_h P[t,h,j] / sum_j' sum_h P[t,h,j'], P = exp(z - lse)
 *           (the attention probabilities, recomputed; no gradient)
 *   indexer u(j) = softmax over j of I(t, s_j)   (I as for dsa_indexer_topk)
 *   loss[t] = sum_j p(j) (log p(j) - log u(j))        (KL(p || u))
 * The caller applies the loss coefficient (0.001 on the page) and any
 * normalisation through `grad`, the gradient of its loss with respect to
 * sum_t loss[t]; then dI(t,j) = grad (u(j) - p(j)) and
 *   dw[t,h]     = sum_j dI max(0, d_thj),      d_thj = q_idx[t,h] . k_idx[s_j]
 *   dq_idx[t,h] = sum_j dI w[t,h] [d_thj > 0] k_idx[s_j]
 *   dk_idx[s]  += sum over (t,j) with s_j = s of sum_h dI w[t,h] [d_thj > 0] q_idx[t,h]
 *
 * dsa_indexer_kl_target: target [T_q, K] fp32 (0 at invalid slots and for rows
 * without a valid slot) from q, kv, idx, topk_length and the forward's lse
 * (with a sink, lse' of the sink forward: the sink's mass is then left out and
 * the target renormalised over the slots).  Arguments and limits as
 * dsa_sparse_mla_fwd.
 *
 * dsa_indexer_kl_bwd: from q_idx [T_q, H_i, 128] bf16, k_idx [T_kv, 128] bf16
 * (the key rows of kv), w [T_q, H_i] fp32, idx / topk_length as for attention
 * and the target: loss [T_q] fp32, dq_idx [T_q, H_i, 128] bf16, dw [T_q, H_i]
 * fp32 (overwritten) and dk_idx [T_kv, 128] fp32 (overwritten, or added into
 * with DSA_BWD_ACCUMULATE_DKV).  The key gradient is staged per (query, slot)
 * as for dsa_sparse_mla_bwd (16-bit block floating point rows) and summed per
 * key row after a counting sort; it is reproducible up to summation order.
 * Workspace: dsa_indexer_kl_bwd_workspace_size(..., rows_per_pass) bytes for
 * passes of rows_per_pass query rows (<= 0: one pass); any ws_bytes of at
 * least the size for one row works, larger ones take fewer passes.
 * Supported: 1 <= H_i <= 64, D_i = 128, 1 <= K <= 4096, finite grad.
 * ------------------------------------------------------------------------ */
int dsa_indexer_kl_target(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                          const int32_t *topk_length, const float *lse, int64_t T_q,
                          int64_t T_kv, int32_t H, int32_t D_qk, int32_t K, float scale,
                          float *target, void *stream);
/* The fused KL-score path: dsa_sparse_mla_bwd that also writes the target of
 * dsa_indexer_kl_target (target [T_q, K] fp32, not NULL when T_q > 0), summed
 * over heads from the probabilities the backward recomputes anyway (staged in
 * fp16: relative error about 2^-12 per term).  Arguments, workspace and errors
 * otherwise as dsa_sparse_mla_bwd. */
int dsa_sparse_mla_bwd_kl_target(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                                 const int32_t *topk_length, const uint16_t *out,
                                 const float *lse, const uint16_t *dout, int64_t T_q,
                                 int64_t T_kv, int32_t H, int32_t D_qk, int32_t D_v, int32_t K,
                                 float scale, uint16_t *dq, float *dkv, float *target,
                                 uint32_t flags, void *ws, size_t ws_bytes, void *stream);
size_t dsa_indexer_kl_bwd_workspace_size(int64_t T_q, int64_t T_kv, int32_t K,
                                         int64_t rows_per_pass);
int dsa_indexer_kl_bwd(const uint16_t *q_idx, const uint16_t *k_idx, const float *w,
                       const int32_t *idx, const int32_t *topk_length, const float *target,
                       int64_t T_q, int64_t T_kv, int32_t H_i, int32_t D_i, int32_t K,
                       float grad, float *loss, uint16_t *dq_idx, float *dw, float *dk_idx,
                       uint32_t flags, void *ws, size_t ws_bytes, void *stream);

/* --------------------------------------------------------------------------
 * Allocation-free backward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Arguments, results and errors as dsa_sparse_mla_bwd, without
 * the workspace: the library uses a fixed scratch array in its code object
 * (dsa_sparse_mla_bwd_noalloc_scratch_bytes(), 256 MiB), of which every GPU
 * that loads the library holds its own copy until the process ends.  The
 * first call on a device looks up that device's copy (hipGetSymbolAddress);
 * no call allocates or frees device memory.  The query rows are processed in
 * passes of as many rows as the scratch holds (one staging buffer, all on
 * `stream`; no helper stream), so large problems take many passes.  Sizes
 * whose Delta [T_q, H] and one row's staging do not fit the scratch return
 * DSA_ERR_INVALID_VALUE with the bytes needed.  Every call on one GPU shares
 * that GPU's scratch: calls that overlap in time on one GPU (two streams, two
 * threads) race and give undefined results.  The scratch keeps the last
 * call's contents; every part the kernels read is written or cleared by the
 * same call first.
 * ------------------------------------------------------------------------ */
size_t dsa_sparse_mla_bwd_noalloc_scratch_bytes(void);
int dsa_sparse_mla_bwd_noalloc(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                               const int32_t *topk_length, const uint16_t *out, const float *lse,
                               const uint16_t *dout, int64_t T_q, int64_t T_kv, int32_t H,
                               int32_t D_qk, int32_t D_v, int32_t K, float scale, uint16_t *dq,
                               float *dkv, uint32_t flags, void *stream);

/* --------------------------------------------------------------------------
 * Attention sink (API reference _pad_attention_heads: a per-head sink [H] is
 * padded together with the query heads; the page does not state its
 * arithmetic).  Reading taken: sink[h] is one more logit of head h whose
 * value vector is zero, so it enters only the softmax denominator:
 *     lse'[t,h] = log(sum_j exp(z_j) + exp(sink[h]))
 *     out'[t,h] = sum_j exp(z_j - lse'[t,h]) kv[s_j, 0:D_v]
 * A row with no valid slot gives out' = 0, lse' = sink[h]; sink = -inf is
 * no sink.
 *
 * dsa_sparse_mla_fwd_sink: arguments, layout and errors as
 * dsa_sparse_mla_fwd, plus sink [H] fp32 (device, not NULL when T_q > 0).
 * It runs the forward and then rescales out and lse in place (an exact
 * identity: lse' = logaddexp(lse, sink), out' = out exp(lse - lse')), so
 * out is read and written once more.
 *
 * dsa_sparse_mla_bwd_sink: arguments, layout, workspace and errors as
 * dsa_sparse_mla_bwd, where out / lse are the sink forward's out' / lse',
 * plus sink [H] fp32 and dsink [H] fp32 (device, not NULL).  dq and dkv are
 * those of the attention with the sink, and
 *     dsink[h] = -sum_t exp(sink[h] - lse'[t,h]) <dout[t,h], out'[t,h]>
 * (the sink's probability times the gradient of its zero value).  With
 * DSA_BWD_ACCUMULATE_DKV, dsink is added into as well; otherwise it is
 * overwritten.  dsink is reproducible up to the order of its fp32 sums.
 * ------------------------------------------------------------------------ */
int dsa_sparse_mla_fwd_sink(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                            const int32_t *topk_length, int64_t T_q, int64_t T_kv, int32_t H,
                            int32_t D_qk, int32_t D_v, int32_t K, float scale, const float *sink,
                            uint16_t *out, float *lse, void *stream);
int dsa_sparse_mla_bwd_sink(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                            const int32_t *topk_length, const uint16_t *out, const float *lse,
                            const uint16_t *dout, int64_t T_q, int64_t T_kv, int32_t H,
                            int32_t D_qk, int32_t D_v, int32_t K, float scale, const float *sink,
                            uint16_t *dq, float *dkv, float *dsink, uint32_t flags, void *ws,
                            size_t ws_bytes, void *stream);

/* --------------------------------------------------------------------------
 * Benchmark support (changes no result).  While armed, every kernel the library
 * enqueues records slots[i].start on its stream just before the kernel and
 * slots[i].stop just after it, and sets slots[i].name to a static string naming
 * the kernel, for i = 0, 1, ... < n_slots; *n_used counts the slots filled
 * (kernels beyond n_slots are not recorded).  start/stop are hipEvent_t handles
 * created by the caller with timing enabled.  Call with slots = NULL to disarm.
 * The state is per calling thread.  Returns DSA_ERR_INVALID_VALUE if n_slots < 0
 * or n_used is NULL while slots is not.
 * ------------------------------------------------------------------------ */
typedef struct dsa_kernel_timing {
  void *start;      /* hipEvent_t */
  void *stop;       /* hipEvent_t */
  const char *name; /* set by the library */
} dsa_kernel_timing;

int dsa_record_kernel_events(dsa_kernel_timing *slots, int n_slots, int *n_used);

/* --------------------------------------------------------------------------
 * Benchmark support: gather ceiling (not a step of the method; it measures the
 * memory path of the attention kernels' latent-row gathers, one row per valid
 * top-k slot, GLM-5.2 page "Why DSA needs fused kernels").  Streams the rows
 * idx[0 .. n) of table [rows, width] bf16 through LDS in tiles of 32 rows with
 * the attention kernels' direct loads, tile layout and buffering, and computes
 * nothing with them but one checksum word per work group of 2048 listed rows:
 * sink[g] = XOR over the 32-row tiles c of the group and the 256 threads l of the
 * four 32-bit words of the 16-byte piece at byte 16 l of tile c as laid out in
 * LDS (tile row l / (width/8), row chunk (l mod (width/8)) XOR swizzle(row), the
 * swizzle of the attention kernels' tiles).  A row index of -1 (or a slot beyond
 * n in a group's last tile) loads row 0.
 *   table [rows, width] bf16, 16-byte aligned, width in {512, 576},
 *   rows * width * 2 < 4 GiB; idx [n] int32, entries in [0, rows) or -1 (index
 *   contents are trusted); sink [dsa_gather_probe_groups(n)] uint32 (out).
 * Errors: DSA_ERR_INVALID_VALUE for bad sizes or NULL / misaligned pointers.
 * ------------------------------------------------------------------------ */
int64_t dsa_gather_probe_groups(int64_t n);
int dsa_gather_probe(const uint16_t *table, int64_t rows, int32_t width, const int32_t *idx,
                     int64_t n, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H_ */
