/*
 * dsa_oracle.c -- plain CPU oracle for the DeepSeek Sparse Attention hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; it exists so that tests/, the smoke check and the CPU
 * baseline leg of the benchmark can check the HIP kernels against an
 * obviously correct definition.  It shares no code, header or table with the
 * HIP library.
 *
 * Every quantity is computed from its definition, in double precision, with
 * no blocking, fusion or reordering: bf16 inputs are widened exactly to
 * double, products and sums are formed in double, and results are returned
 * in double.  Rows are independent, so the only parallelism is an OpenMP
 * loop over query rows.
 *
 * Sources (web pages; cited by title and section):
 *   [GLM52]  NVIDIA "Accelerating GLM-5.2 Long-Context Training with cuDNN
 *            Fused DSA Kernels and THD-Packed Context Parallelism using
 *            Megatron Bridge", sections "How DSA works" and "Why DSA needs
 *            fused kernels".
 *   [API]    NeMo AutoModel API reference, module
 *            nemo_automodel.components.models.glm_moe_dsa.kernels.cudnn_dsa:
 *            entries prepare_cudnn_dsa_packed_metadata, cudnn_indexer_topk,
 *            _compact_and_sort_indices, cudnn_sparse_attention,
 *            _CudnnSparseAttention.forward / .backward.
 *   [PR2388] SkyRL PR 2388 (GLM-5.3-Flash NoPE sparse MLA), "Why", "Change".
 *   [PR2423] SkyRL PR 2423 (query-chunked sparse attention), "Summary".
 *
 * The indexer score itself is not written out on the pages ([GLM52] "How DSA
 * works" only describes the indexer as rating how relevant each key is to a query);
 * the reading taken is
 *     I(t,s) = sum_h w[t,h] * max(0, sum_d q[t,h,d] * k[s,d]),
 * with the head weights used exactly as handed over ([API] cudnn_indexer_topk,
 * head_weights: the caller owns the 1/sqrt(H) and 1/sqrt(D) scaling).
 *
 * Parity status: every function below is pinned by tests in tests/ against
 * brute force, closed forms, library routines or finite differences.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL -1
#define ORACLE_ENOMEM -2

static double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* ------------------------------------------------------------------------ */
/* THD metadata ([API] prepare_cudnn_dsa_packed_metadata: per-query starts   */
/* and real causal lengths from cumulative sequence offsets).                */
/* ------------------------------------------------------------------------ */

/* Validates cu_seqlens (starts at 0, non-decreasing, ends at T) and returns
 * for every token t of sequence b: seq_start[t] = cu[b], causal_len[t] =
 * t - cu[b] + 1 (keys s with cu[b] <= s <= t, diagonal included) and
 * topk_len[t] = min(K, causal_len[t]).  *max_seqlen is the longest sequence and
 * *all_rows_nonempty is 1 when every row has at least one key (always true
 * for a causal row that includes itself; 1 also for T == 0). */
int oracle_thd_metadata(const int32_t *cu, int32_t B, int64_t T, int32_t K,
                        int32_t *seq_start, int32_t *causal_len, int32_t *topk_len,
                        int32_t *max_seqlen, int32_t *all_rows_nonempty) {
  if (B < 1 || T < 0 || K < 1) return ORACLE_EINVAL;
  if (cu[0] != 0 || (int64_t)cu[B] != T) return ORACLE_EINVAL;
  int32_t mx = 0;
  for (int32_t b = 0; b < B; ++b) {
    if (cu[b + 1] < cu[b]) return ORACLE_EINVAL;
    int32_t len = cu[b + 1] - cu[b];
    if (len > mx) mx = len;
    for (int32_t t = cu[b]; t < cu[b + 1]; ++t) {
      seq_start[t] = cu[b];
      causal_len[t] = t - cu[b] + 1;
      topk_len[t] = causal_len[t] < K ? causal_len[t] : K;
    }
  }
  *max_seqlen = mx;
  *all_rows_nonempty = 1;
  for (int64_t t = 0; t < T; ++t)
    if (causal_len[t] <= 0) *all_rows_nonempty = 0;
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Lightning indexer score and per-row top-k ([GLM52] "How DSA works";       */
/* [API] cudnn_indexer_topk, _compact_and_sort_indices).                      */
/* ------------------------------------------------------------------------ */

/* One score I(t,s) in double; q and w hold query rows starting at global row q_row0. */
static double indexer_score_rows(const uint16_t *q, const uint16_t *k, const float *w, int32_t H,
                                 int32_t D, int64_t q_row0, int64_t t, int64_t s) {
  double total = 0.0;
  for (int32_t h = 0; h < H; ++h) {
    double dot = 0.0;
    const uint16_t *qr = q + ((size_t)(t - q_row0) * H + h) * D;
    const uint16_t *kr = k + (size_t)s * D;
    for (int32_t d = 0; d < D; ++d) dot += bf16_to_double(qr[d]) * bf16_to_double(kr[d]);
    double relu = dot > 0.0 ? dot : 0.0;
    total += (double)w[(size_t)(t - q_row0) * H + h] * relu;
  }
  return total + 0.0; /* folds a -0.0 sum to +0.0 */
}

double oracle_indexer_score(const uint16_t *q, const uint16_t *k, const float *w,
                            int32_t H, int32_t D, int64_t t, int64_t s) {
  return indexer_score_rows(q, k, w, H, D, 0, t, s);
}

typedef struct {
  double score;
  int32_t pos;
} scored_key;

/* Ranking: higher score first; equal scores -> lower key position first. */
static int by_rank(const void *a, const void *b) {
  const scored_key *x = (const scored_key *)a, *y = (const scored_key *)b;
  if (x->score > y->score) return -1;
  if (x->score < y->score) return 1;
  return (x->pos > y->pos) - (x->pos < y->pos);
}

static int by_pos(const void *a, const void *b) {
  const scored_key *x = (const scored_key *)a, *y = (const scored_key *)b;
  return (x->pos > y->pos) - (x->pos < y->pos);
}

/* For query rows [row_begin, row_end): score every causal key of the row's
 * own sequence, keep the n = min(K, L_t) best (ties -> lower position), and
 * write them as a compact ascending prefix of global key positions followed
 * by -1 ([API] _compact_and_sort_indices "canonicalize ... return valid
 * lengths").  idx_out is [(row_end-row_begin) x K], len_out is
 * [row_end-row_begin].  kth_score (nullable) receives the n-th best score of
 * each row (the selection threshold).  q and w hold the query rows from global row q_row0
 * on (0 for full arrays; row_begin when only the selected rows are passed). */
int oracle_indexer_topk_rows(const uint16_t *q, const uint16_t *k, const float *w,
                             const int32_t *cu, int32_t B, int64_t T, int32_t H, int32_t D,
                             int32_t K, int64_t row_begin, int64_t row_end, int64_t q_row0,
                             int32_t *idx_out, int32_t *len_out, double *kth_score) {
  if (B < 1 || H < 1 || D < 1 || K < 1 || row_begin < 0 || row_end > T || row_begin > row_end)
    return ORACLE_EINVAL;
  if (cu[0] != 0 || (int64_t)cu[B] != T) return ORACLE_EINVAL;
  for (int32_t b = 0; b < B; ++b)
    if (cu[b + 1] < cu[b]) return ORACLE_EINVAL;
  int err = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t t = row_begin; t < row_end; ++t) {
    int32_t b = 0;
    while (!(cu[b] <= t && t < cu[b + 1])) ++b;
    int64_t start = cu[b];
    int64_t L = t - start + 1;
    scored_key *keys = (scored_key *)malloc(sizeof(scored_key) * (size_t)L);
    if (!keys) {
#pragma omp atomic write
      err = ORACLE_ENOMEM;
      continue;
    }
    for (int64_t s = start; s <= t; ++s) {
      keys[s - start].score = indexer_score_rows(q, k, w, H, D, q_row0, t, s);
      keys[s - start].pos = (int32_t)s;
    }
    qsort(keys, (size_t)L, sizeof(scored_key), by_rank);
    int64_t n = L < K ? L : K;
    if (kth_score) kth_score[t - row_begin] = keys[n - 1].score;
    qsort(keys, (size_t)n, sizeof(scored_key), by_pos);
    int32_t *row = idx_out + (size_t)(t - row_begin) * K;
    for (int64_t j = 0; j < K; ++j) row[j] = j < n ? keys[j].pos : -1;
    len_out[t - row_begin] = (int32_t)n;
    free(keys);
  }
  return err;
}

int oracle_indexer_topk(const uint16_t *q, const uint16_t *k, const float *w,
                        const int32_t *cu, int32_t B, int64_t T, int32_t H, int32_t D,
                        int32_t K, int64_t row_begin, int64_t row_end, int32_t *idx_out,
                        int32_t *len_out, double *kth_score) {
  return oracle_indexer_topk_rows(q, k, w, cu, B, T, H, D, K, row_begin, row_end, 0, idx_out,
                                  len_out, kth_score);
}

/* Local query rows against gathered global keys ([API]
 * prepare_cudnn_dsa_packed_metadata and cudnn_indexer_topk: query_indices
 * hold the global padded-storage coordinate of each local query row,
 * cu_seqlens_padded the padded storage boundaries of the sequences (absent:
 * cu_seqlens), cu_seqlens their real lengths, padding_mask the local padding
 * rows; indices come back in global padded-storage coordinates).  For local
 * row i with coordinate p = qidx[i] (i itself when qidx is NULL): the sequence
 * b has cu_pad[b] <= p < cu_pad[b+1], the row's position is pos = p -
 * cu_pad[b], and the row is real when pos < cu[b+1] - cu[b] and pmask[i] is
 * 0.  A real row scores the keys s = cu_pad[b] .. p (q and w row i, k row s)
 * and keeps the n = min(K, pos + 1) best as above; any other row gets len 0
 * and -1 everywhere.  q and w are [T_q x ...], k is [T_k x D]. */
int oracle_indexer_topk_local(const uint16_t *q, const uint16_t *k, const float *w,
                              const int32_t *cu, const int32_t *cu_pad, const int32_t *qidx,
                              const uint8_t *pmask, int32_t B, int64_t T_q, int64_t T_k,
                              int32_t H, int32_t D, int32_t K, int32_t *idx_out,
                              int32_t *len_out) {
  if (B < 1 || H < 1 || D < 1 || K < 1 || T_q < 0 || T_k < 0) return ORACLE_EINVAL;
  if (!cu_pad) cu_pad = cu;
  if (cu[0] != 0 || cu_pad[0] != 0 || cu_pad[B] > T_k) return ORACLE_EINVAL;
  for (int32_t b = 0; b < B; ++b)
    if (cu[b + 1] < cu[b] || cu_pad[b + 1] - cu_pad[b] < cu[b + 1] - cu[b]) return ORACLE_EINVAL;
  int err = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < T_q; ++i) {
    int32_t *row = idx_out + (size_t)i * K;
    for (int32_t j = 0; j < K; ++j) row[j] = -1;
    len_out[i] = 0;
    int64_t p = qidx ? qidx[i] : i;
    if (p < 0 || p >= cu_pad[B]) {
#pragma omp atomic write
      err = ORACLE_EINVAL;
      continue;
    }
    int32_t b = B - 1;
    while (cu_pad[b] > p) --b;  /* the last sequence starting at or before p */
    int64_t start = cu_pad[b], pos = p - start;
    if (pos >= cu[b + 1] - cu[b] || (pmask && pmask[i])) continue;
    int64_t L = pos + 1;
    scored_key *keys = (scored_key *)malloc(sizeof(scored_key) * (size_t)L);
    if (!keys) {
#pragma omp atomic write
      err = ORACLE_ENOMEM;
      continue;
    }
    for (int64_t s = start; s <= p; ++s) {
      keys[s - start].score = indexer_score_rows(q, k, w, H, D, 0, i, s);
      keys[s - start].pos = (int32_t)s;
    }
    qsort(keys, (size_t)L, sizeof(scored_key), by_rank);
    int64_t n = L < K ? L : K;
    qsort(keys, (size_t)n, sizeof(scored_key), by_pos);
    for (int64_t j = 0; j < n; ++j) row[j] = keys[j].pos;
    len_out[i] = (int32_t)n;
    free(keys);
  }
  return err;
}

/* ------------------------------------------------------------------------ */
/* Absorbed sparse MLA ([GLM52] "Why DSA needs fused kernels": all heads of  */
/* a query share one top-k set, MQA-style; [API] cudnn_sparse_attention:     */
/* q [T_q,H,576] = 512 latent + 64 rope, kv_latent [T_kv,1,576], values are   */
/* the first 512 channels, -1 slots are invalid, topk_length limits the row   */
/* to a valid prefix, softmax_scale is applied unchanged; [PR2388] NoPE      */
/* width 512 with value = the same 512 channels).                            */
/* ------------------------------------------------------------------------ */

/* Valid slots of one row: j < (topk_length ? topk_length[t] : K) and
 * idx[t,j] != -1.  Returns the count, or -1 if an index is out of range. */
static int64_t row_slots(const int32_t *idx, const int32_t *topk_length, int64_t t, int32_t K,
                         int64_t T_kv, int32_t *slots) {
  int64_t lim = K;
  if (topk_length) {
    lim = topk_length[t];
    if (lim < 0 || lim > K) return -1;
  }
  int64_t n = 0;
  for (int64_t j = 0; j < lim; ++j) {
    int32_t s = idx[(size_t)t * K + j];
    if (s == -1) continue;
    if (s < 0 || s >= T_kv) return -1;
    slots[n++] = s;
  }
  return n;
}

/* Softmax statistics and output of one (t,h): logits z_j = scale *
 * <q[t,h,:Dqk], kv[s_j,:Dqk]>, lse = log sum_j exp(z_j) (natural log), and
 * out = sum_j exp(z_j - lse) * kv[s_j,:Dv].  An empty row gives out = 0 and
 * lse = -inf.  z receives the logits.
 *
 * Attention sink ([API] _pad_attention_heads pads a per-head sink [H] with
 * the query heads; its arithmetic is not written on the pages).  Reading
 * taken: the sink is one more logit `sink` per head whose value vector is
 * zero, so it enters only the softmax denominator:
 *   lse = log(sum_j exp(z_j) + exp(sink)),  out = sum_j exp(z_j - lse) kv[s_j,:Dv].
 * With no valid slot, lse = sink and out = 0; sink = -inf is no sink. */
static void attend_one(const uint16_t *q, const uint16_t *kv, const int32_t *slots, int64_t n,
                       int64_t t, int32_t h, int32_t H, int32_t Dqk, int32_t Dv, double scale,
                       const double *sink, double *z, double *out, double *lse) {
  const uint16_t *qr = q + ((size_t)t * H + h) * Dqk;
  const double sk = sink ? sink[h] : -INFINITY;
  for (int32_t c = 0; c < Dv; ++c) out[c] = 0.0;
  if (n == 0) {
    *lse = sk;
    return;
  }
  double m = sk;
  for (int64_t j = 0; j < n; ++j) {
    const uint16_t *kr = kv + (size_t)slots[j] * Dqk;
    double dot = 0.0;
    for (int32_t d = 0; d < Dqk; ++d) dot += bf16_to_double(qr[d]) * bf16_to_double(kr[d]);
    z[j] = scale * dot;
    if (z[j] > m) m = z[j];
  }
  double sum = 0.0;
  for (int64_t j = 0; j < n; ++j) sum += exp(z[j] - m);
  if (sink) sum += exp(sk - m);
  *lse = m + log(sum);
  for (int64_t j = 0; j < n; ++j) {
    double p = exp(z[j] - *lse);
    const uint16_t *kr = kv + (size_t)slots[j] * Dqk;
    for (int32_t c = 0; c < Dv; ++c) out[c] += p * bf16_to_double(kr[c]);
  }
}

/* Forward for query rows [row_begin, row_end).  out is [(rows) x H x Dv],
 * lse is [(rows) x H], both double, row-relative. */
int oracle_sparse_mla_fwd(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                          const int32_t *topk_length, int64_t T_q, int64_t T_kv, int32_t H,
                          int32_t Dqk, int32_t Dv, int32_t K, double scale, const double *sink,
                          int64_t row_begin, int64_t row_end, double *out, double *lse) {
  if (H < 1 || Dqk < 1 || Dv < 1 || Dv > Dqk || K < 1 || row_begin < 0 || row_end > T_q ||
      row_begin > row_end)
    return ORACLE_EINVAL;
  int err = ORACLE_OK;
#pragma omp parallel
  {
    int32_t *slots = (int32_t *)malloc(sizeof(int32_t) * (size_t)K);
    double *z = (double *)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(dynamic, 4)
    for (int64_t t = row_begin; t < row_end; ++t) {
      if (!slots || !z) {
#pragma omp atomic write
        err = ORACLE_ENOMEM;
        continue;
      }
      int64_t n = row_slots(idx, topk_length, t, K, T_kv, slots);
      if (n < 0) {
#pragma omp atomic write
        err = ORACLE_EINVAL;
        continue;
      }
      for (int32_t h = 0; h < H; ++h) {
        size_t r = (size_t)(t - row_begin) * H + h;
        attend_one(q, kv, slots, n, t, h, H, Dqk, Dv, scale, sink, z, out + r * Dv, lse + r);
      }
    }
    free(slots);
    free(z);
  }
  return err;
}

/* Backward for query rows [row_begin, row_end) ([API] _CudnnSparseAttention
 * .backward: gradients for the query [T_q,H,576] and the gathered latent
 * rows; [PR2423] "Summary": key gradients of independent query chunks sum).
 *
 * The row's own forward is recomputed here in double.  With P_j =
 * exp(z_j - lse), dP_j = <dO[t,h], kv[s_j,:Dv]>, Delta = <dO[t,h], O[t,h]>,
 * dZ_j = P_j (dP_j - Delta):
 *   dq[t,h,:Dqk]   = scale * sum_j dZ_j kv[s_j,:Dqk]
 *   dkv[s_j,:Dqk] += scale * dZ_j q[t,h,:Dqk]      (summed over h and t)
 *   dkv[s_j,:Dv]  += P_j dO[t,h,:]
 * dq is [(rows) x H x Dqk] (row-relative); dkv is the full [T_kv x Dqk]
 * buffer and is accumulated into (the caller zeroes it).  dkv of a key row is
 * complete only when every query row that selects it is inside the range.
 *
 * With a sink (see attend_one), P_j and Delta use the sink's lse and output;
 * the sink's own probability is P_s = exp(sink - lse) and its value is zero,
 * so its logit gradient is P_s (0 - Delta):
 *   dsink[h] += -exp(sink[h] - lse[t,h]) * Delta[t,h]     (summed over t)
 * accumulated into dsink [H] (the caller zeroes it). */
int oracle_sparse_mla_bwd(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                          const int32_t *topk_length, const uint16_t *dout, int64_t T_q,
                          int64_t T_kv, int32_t H, int32_t Dqk, int32_t Dv, int32_t K,
                          double scale, const double *sink, int64_t row_begin, int64_t row_end,
                          double *dq, double *dkv, double *dsink) {
  if (H < 1 || Dqk < 1 || Dv < 1 || Dv > Dqk || K < 1 || row_begin < 0 || row_end > T_q ||
      row_begin > row_end || (sink && !dsink))
    return ORACLE_EINVAL;
  int err = ORACLE_OK;
#pragma omp parallel
  {
    int32_t *slots = (int32_t *)malloc(sizeof(int32_t) * (size_t)K);
    double *z = (double *)malloc(sizeof(double) * (size_t)K);
    double *o = (double *)malloc(sizeof(double) * (size_t)Dv);
    double *dsk = (double *)malloc(sizeof(double) * (size_t)H); /* this row's dsink terms */
    /* this row's contribution to dkv, one Dqk vector per valid slot */
    double *contrib = (double *)malloc(sizeof(double) * (size_t)K * Dqk);
    /* rows add their contributions into dkv in row order, so dkv does not
     * depend on the thread count or scheduling */
#pragma omp for schedule(dynamic, 1) ordered
    for (int64_t t = row_begin; t < row_end; ++t) {
      int64_t n = (!slots || !z || !o || !contrib || !dsk)
                      ? -2 : row_slots(idx, topk_length, t, K, T_kv, slots);
      if (n < 0) {
#pragma omp atomic write
        err = n == -2 ? ORACLE_ENOMEM : ORACLE_EINVAL;
#pragma omp ordered
        {}
        continue;
      }
      memset(contrib, 0, sizeof(double) * (size_t)n * Dqk);
      for (int32_t h = 0; h < H; ++h) {
        double lse;
        attend_one(q, kv, slots, n, t, h, H, Dqk, Dv, scale, sink, z, o, &lse);
        const uint16_t *qr = q + ((size_t)t * H + h) * Dqk;
        const uint16_t *dor = dout + ((size_t)t * H + h) * Dv;
        double *dqr = dq + ((size_t)(t - row_begin) * H + h) * Dqk;
        for (int32_t d = 0; d < Dqk; ++d) dqr[d] = 0.0;
        double delta = 0.0;
        for (int32_t c = 0; c < Dv; ++c) delta += bf16_to_double(dor[c]) * o[c];
        dsk[h] = sink ? -exp(sink[h] - lse) * delta : 0.0;
        for (int64_t j = 0; j < n; ++j) {
          const uint16_t *kr = kv + (size_t)slots[j] * Dqk;
          double p = exp(z[j] - lse);
          double dp = 0.0;
          for (int32_t c = 0; c < Dv; ++c) dp += bf16_to_double(dor[c]) * bf16_to_double(kr[c]);
          double dz = p * (dp - delta);
          double *cj = contrib + (size_t)j * Dqk;
          for (int32_t d = 0; d < Dqk; ++d) {
            dqr[d] += scale * dz * bf16_to_double(kr[d]);
            cj[d] += scale * dz * bf16_to_double(qr[d]);
          }
          for (int32_t c = 0; c < Dv; ++c) cj[c] += p * bf16_to_double(dor[c]);
        }
      }
#pragma omp ordered
      {
        for (int64_t j = 0; j < n; ++j) {
          double *dst = dkv + (size_t)slots[j] * Dqk;
          const double *cj = contrib + (size_t)j * Dqk;
          for (int32_t d = 0; d < Dqk; ++d) dst[d] += cj[d];
        }
        if (sink)
          for (int32_t h = 0; h < H; ++h) dsink[h] += dsk[h];
      }
    }
    free(slots);
    free(z);
    free(o);
    free(contrib);
    free(dsk);
  }
  return err;
}

/* ------------------------------------------------------------------------ */
/* Indexer training loss ([GLM52] "How DSA works": an extra KL loss pulls the */
/* indexer's score distribution toward the main attention's, on a graph of   */
/* its own; "GLM-5.2 training results": sparse formulation, coefficient      */
/* 0.001; "cuDNN fused DSA kernels": a score-recompute kernel feeds the      */
/* loss).                                                                     */
/* ------------------------------------------------------------------------ */

/* The loss formula is not written on the pages.  Reading taken, for query
 * row t with valid slots j (as for attention) and key rows s_j:
 *   target   p_t(j) = sum_h P[t,h,j] / sum_j' sum_h P[t,h,j'],  with P the main
 *            attention's probabilities exp(z_thj - lse[t,h]) recomputed from
 *            q, kv and the row's own lse (sink: see attend_one; its mass is
 *            not part of the target, which is renormalised over the slots);
 *   indexer  u_t(j) = exp(I(t,s_j)) / sum_j' exp(I(t,s_j'))  (I as above);
 *   loss_t = sum_j p_t(j) (log p_t(j) - log u_t(j))  (KL(p || u), 0 log 0 = 0).
 * The target carries no gradient.  With upstream gradient g of sum_t loss_t:
 *   dI(t,j)     = g (u_t(j) - p_t(j))
 *   dw[t,h]     = sum_j dI(t,j) max(0, d_thj),      d_thj = <q_idx[t,h], k_idx[s_j]>
 *   dq_idx[t,h] = sum_j dI(t,j) w[t,h] [d_thj > 0] k_idx[s_j]
 *   dk_idx[s]  += sum over (t,j) with s_j = s of sum_h dI(t,j) w[t,h] [d_thj > 0] q_idx[t,h]
 * (the derivative of max(0, x) at 0 is taken as 0).  A row with no valid slot
 * has target 0, loss 0 and no gradient.
 *
 * For query rows [row_begin, row_end): target [(rows) x K] (0 at invalid
 * slots), loss [rows], dq_idx [(rows) x Hi x Di], dw [(rows) x Hi] are
 * row-relative; dk_idx [T_kv x Di] is accumulated into (the caller zeroes it)
 * in row order.  k_idx has T_kv rows (the key rows of kv). */
int oracle_indexer_kl(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                      const int32_t *topk_length, int64_t T_q, int64_t T_kv, int32_t H,
                      int32_t Dqk, int32_t K, double scale, const double *sink,
                      const uint16_t *q_idx, const uint16_t *k_idx, const float *w, int32_t Hi,
                      int32_t Di, double g, int64_t row_begin, int64_t row_end, double *target,
                      double *loss, double *dq_idx, double *dw, double *dk_idx) {
  if (H < 1 || Dqk < 1 || K < 1 || Hi < 1 || Di < 1 || row_begin < 0 || row_end > T_q ||
      row_begin > row_end)
    return ORACLE_EINVAL;
  int err = ORACLE_OK;
#pragma omp parallel
  {
    int32_t *slots = (int32_t *)malloc(sizeof(int32_t) * (size_t)K);
    int32_t *where = (int32_t *)malloc(sizeof(int32_t) * (size_t)K); /* slot position j */
    double *z = (double *)malloc(sizeof(double) * (size_t)K);
    double *o = (double *)malloc(sizeof(double) * (size_t)Dqk);
    double *pt = (double *)malloc(sizeof(double) * (size_t)K);
    double *ii = (double *)malloc(sizeof(double) * (size_t)K);
    double *di = (double *)malloc(sizeof(double) * (size_t)K);
    double *dots = (double *)malloc(sizeof(double) * (size_t)K * Hi);
    double *contrib = (double *)malloc(sizeof(double) * (size_t)K * Di);
#pragma omp for schedule(dynamic, 1) ordered
    for (int64_t t = row_begin; t < row_end; ++t) {
      int64_t n = -2;
      if (slots && where && z && o && pt && ii && di && dots && contrib) {
        /* valid slots and their positions j in the row */
        int64_t lim = topk_length ? topk_length[t] : K;
        n = (lim < 0 || lim > K) ? -1 : 0;
        for (int64_t j = 0; n >= 0 && j < lim; ++j) {
          int32_t s = idx[(size_t)t * K + j];
          if (s == -1) continue;
          if (s < 0 || s >= T_kv) { n = -1; break; }
          slots[n] = s;
          where[n++] = (int32_t)j;
        }
      }
      if (n < 0) {
#pragma omp atomic write
        err = n == -2 ? ORACLE_ENOMEM : ORACLE_EINVAL;
#pragma omp ordered
        {}
        continue;
      }
      const size_t r = (size_t)(t - row_begin);
      double *trow = target + r * K;
      for (int32_t j = 0; j < K; ++j) trow[j] = 0.0;
      for (int32_t h = 0; h < Hi; ++h) {
        dw[r * Hi + h] = 0.0;
        for (int32_t d = 0; d < Di; ++d) dq_idx[(r * Hi + h) * Di + d] = 0.0;
      }
      loss[r] = 0.0;
      /* target: head sum of the attention probabilities, renormalised */
      for (int64_t j = 0; j < n; ++j) pt[j] = 0.0;
      for (int32_t h = 0; h < H; ++h) {
        double lse;
        attend_one(q, kv, slots, n, t, h, H, Dqk, 1, scale, sink, z, o, &lse);
        for (int64_t j = 0; j < n; ++j) pt[j] += exp(z[j] - lse);
      }
      double tot = 0.0;
      for (int64_t j = 0; j < n; ++j) tot += pt[j];
      for (int64_t j = 0; j < n; ++j) {
        pt[j] = tot > 0.0 ? pt[j] / tot : 0.0;
        trow[where[j]] = pt[j];
      }
      /* indexer scores on the slots and their log-softmax */
      const uint16_t *qr = q_idx + (size_t)t * Hi * Di;
      const float *wr = w + (size_t)t * Hi;
      double m = -INFINITY;
      for (int64_t j = 0; j < n; ++j) {
        const uint16_t *kr = k_idx + (size_t)slots[j] * Di;
        double score = 0.0;
        for (int32_t h = 0; h < Hi; ++h) {
          double dot = 0.0;
          for (int32_t d = 0; d < Di; ++d)
            dot += bf16_to_double(qr[(size_t)h * Di + d]) * bf16_to_double(kr[d]);
          dots[(size_t)j * Hi + h] = dot;
          score += (double)wr[h] * (dot > 0.0 ? dot : 0.0);
        }
        ii[j] = score;
        if (score > m) m = score;
      }
      double zsum = 0.0;
      for (int64_t j = 0; j < n; ++j) zsum += exp(ii[j] - m);
      const double logz = m + log(zsum);
      double lsum = 0.0;
      for (int64_t j = 0; j < n; ++j) {
        const double logu = ii[j] - logz;
        if (pt[j] > 0.0) lsum += pt[j] * (log(pt[j]) - logu);
        di[j] = g * (exp(logu) - pt[j]);
      }
      loss[r] = lsum;
      /* indexer backward */
      memset(contrib, 0, sizeof(double) * (size_t)n * Di);
      for (int64_t j = 0; j < n; ++j) {
        const uint16_t *kr = k_idx + (size_t)slots[j] * Di;
        double *cj = contrib + (size_t)j * Di;
        for (int32_t h = 0; h < Hi; ++h) {
          const double dot = dots[(size_t)j * Hi + h];
          dw[r * Hi + h] += di[j] * (dot > 0.0 ? dot : 0.0);
          if (!(dot > 0.0)) continue;
          const double gh = di[j] * (double)wr[h];
          double *dqr = dq_idx + (r * Hi + h) * Di;
          for (int32_t d = 0; d < Di; ++d) {
            dqr[d] += gh * bf16_to_double(kr[d]);
            cj[d] += gh * bf16_to_double(qr[(size_t)h * Di + d]);
          }
        }
      }
#pragma omp ordered
      {
        for (int64_t j = 0; j < n; ++j) {
          double *dst = dk_idx + (size_t)slots[j] * Di;
          const double *cj = contrib + (size_t)j * Di;
          for (int32_t d = 0; d < Di; ++d) dst[d] += cj[d];
        }
      }
    }
    free(slots);
    free(where);
    free(z);
    free(o);
    free(pt);
    free(ii);
    free(di);
    free(dots);
    free(contrib);
  }
  return err;
}

/* ------------------------------------------------------------------------ */
/* k-pool indexer ([PR2388] "Why": GLM-5.3-Flash picks keys by pools and adds */
/* the query's still-incomplete last pool, hence top-k width 2048 + 3).      */
/* ------------------------------------------------------------------------ */

/* The pool selection is not spelled out on the pages.  Reading taken: the
 * keys of every sequence form pools of `pool` consecutive keys from the
 * sequence start; the caller supplies one indexer key per complete pool
 * (k_pool rows in sequence order, sequence b's pools from row cp[b] with
 * cp[b] = sum over b' < b of floor(len_b' / pool)).  Query row t of sequence
 * b sees the P = floor((t - cu[b] + 1) / pool) pools that end at or before t,
 * scores pool i as I(t,i) = sum_h w[t,h] max(0, q[t,h] . k_pool[cp[b]+i]),
 * keeps the n = min(K_pools, P) best (ties -> lower pool), and emits their
 * keys in ascending order followed by the incomplete tail pool's keys
 * cu[b] + pool P .. t (at most pool - 1 of them); the rest of the width
 * W = K_pools pool + pool - 1 is -1 and len = pool n + (t - cu[b] + 1 - pool P).
 * pool = 1 is the token-level indexer.  For query rows [row_begin, row_end)
 * (row-relative outputs): idx_out [rows x W], len_out [rows], kth_score
 * (nullable) the n-th best pool score of each row (0 without a pool). */
int oracle_kpool_indexer(const uint16_t *q, const uint16_t *k_pool, const float *w,
                         const int32_t *cu, int32_t B, int64_t T, int32_t H, int32_t D,
                         int32_t pool, int32_t K_pools, int64_t row_begin, int64_t row_end,
                         int32_t *idx_out, int32_t *len_out, double *kth_score) {
  if (B < 1 || H < 1 || D < 1 || pool < 1 || K_pools < 1 || row_begin < 0 || row_end > T ||
      row_begin > row_end)
    return ORACLE_EINVAL;
  if (cu[0] != 0 || (int64_t)cu[B] != T) return ORACLE_EINVAL;
  for (int32_t b = 0; b < B; ++b)
    if (cu[b + 1] < cu[b]) return ORACLE_EINVAL;
  const int64_t W = (int64_t)K_pools * pool + pool - 1;
  int err = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t t = row_begin; t < row_end; ++t) {
    int32_t b = 0;
    int64_t cp = 0; /* first pool row of sequence b */
    while (!(cu[b] <= t && t < cu[b + 1])) {
      cp += (cu[b + 1] - cu[b]) / pool;
      ++b;
    }
    const int64_t start = cu[b], pos = t - start;
    const int64_t P = (pos + 1) / pool;
    int32_t *row = idx_out + (size_t)(t - row_begin) * W;
    for (int64_t j = 0; j < W; ++j) row[j] = -1;
    int64_t n = P < K_pools ? P : K_pools;
    scored_key *pools = P > 0 ? (scored_key *)malloc(sizeof(scored_key) * (size_t)P) : NULL;
    if (P > 0 && !pools) {
#pragma omp atomic write
      err = ORACLE_ENOMEM;
      continue;
    }
    for (int64_t i = 0; i < P; ++i) {
      double total = 0.0;
      for (int32_t h = 0; h < H; ++h) {
        double dot = 0.0;
        const uint16_t *qr = q + ((size_t)t * H + h) * D;
        const uint16_t *kr = k_pool + (size_t)(cp + i) * D;
        for (int32_t d = 0; d < D; ++d) dot += bf16_to_double(qr[d]) * bf16_to_double(kr[d]);
        total += (double)w[(size_t)t * H + h] * (dot > 0.0 ? dot : 0.0);
      }
      pools[i].score = total + 0.0;
      pools[i].pos = (int32_t)i;
    }
    if (kth_score) kth_score[t - row_begin] = 0.0;
    if (P > 0) {
      qsort(pools, (size_t)P, sizeof(scored_key), by_rank);
      if (kth_score) kth_score[t - row_begin] = pools[n - 1].score;
      qsort(pools, (size_t)n, sizeof(scored_key), by_pos);
    }
    int64_t o = 0;
    for (int64_t j = 0; j < n; ++j)
      for (int32_t r = 0; r < pool; ++r) row[o++] = (int32_t)(start + (int64_t)pools[j].pos * pool + r);
    for (int64_t s = start + P * pool; s <= t; ++s) row[o++] = (int32_t)s;
    len_out[t - row_begin] = (int32_t)o;
    free(pools);
  }
  return err;
}
