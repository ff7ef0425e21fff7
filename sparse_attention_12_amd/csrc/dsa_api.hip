// C ABI of libdsa: argument validation, workspace layout, error reporting and launches.
// The contracts are documented in include/dsa.h.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <vector>

#include "../../include/dsa.h"
#include "dsa_common.h"
#include "dsa_internal.h"

namespace {

thread_local std::string g_last_error;

struct TimingState {
  dsa_kernel_timing *slots = nullptr;
  int n_slots = 0;
  int *n_used = nullptr;
  bool open = false;
};
thread_local TimingState g_timing;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char *what) {
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align_up(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

int check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (!dsa_device_supported(dev))
    return fail(DSA_ERR_UNSUPPORTED, "device %d is not an AMD gfx950 GPU", dev);
  return DSA_OK;
}

int32_t n_index_groups(const std::vector<int32_t> &cu) {
  int64_t n = 0;
  for (size_t b = 0; b + 1 < cu.size(); ++b)
    n += (cu[b + 1] - cu[b] + dsa::kIdxRowsPerGroup - 1) / dsa::kIdxRowsPerGroup;
  return static_cast<int32_t>(n);
}

}  // namespace

namespace dsa {

void kernel_begin(hipStream_t s, const char *name) {
  TimingState &st = g_timing;
  st.open = false;
  if (!st.slots || *st.n_used >= st.n_slots) return;
  dsa_kernel_timing &slot = st.slots[*st.n_used];
  slot.name = name;
  // a slot whose start could not be recorded is left unused
  st.open = hipEventRecord(static_cast<hipEvent_t>(slot.start), s) == hipSuccess;
}

void kernel_end(hipStream_t s) {
  TimingState &st = g_timing;
  if (!st.open) return;
  if (hipEventRecord(static_cast<hipEvent_t>(st.slots[*st.n_used].stop), s) == hipSuccess)
    ++*st.n_used;
  st.open = false;
}

}  // namespace dsa

extern "C" {

int dsa_record_kernel_events(dsa_kernel_timing *slots, int n_slots, int *n_used) {
  g_last_error.clear();
  if (slots && (n_slots < 0 || !n_used))
    return fail(DSA_ERR_INVALID_VALUE, "record_kernel_events: bad slot count or counter");
  g_timing.slots = slots;
  g_timing.n_slots = slots ? n_slots : 0;
  g_timing.n_used = slots ? n_used : nullptr;
  g_timing.open = false;
  if (n_used) *n_used = 0;
  return DSA_OK;
}

const char *dsa_last_error(void) { return g_last_error.c_str(); }

int dsa_device_supported(int device) {
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return 0;
  return strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
}

// ---------------------------------------------------------------------------------------
// workspace: seq_start | causal_len | topk_length | row_order | groups   (each 256-B aligned)
size_t dsa_thd_metadata_workspace_size(int64_t T) {
  if (T < 0) return 0;
  const size_t a = align_up(static_cast<size_t>(T) * sizeof(int32_t));
  return 5 * a + 256;
}

int dsa_prepare_thd_metadata(const int32_t *cu_seqlens, int32_t B, int64_t T, int32_t K,
                             void *ws, size_t ws_bytes, dsa_thd_metadata *md, void *stream) {
  g_last_error.clear();
  if (!md) return fail(DSA_ERR_INVALID_VALUE, "prepare_thd_metadata: md is NULL");
  if (B < 1) return fail(DSA_ERR_INVALID_VALUE, "prepare_thd_metadata: B=%d must be >= 1", B);
  if (T < 0 || T > INT32_MAX)
    return fail(DSA_ERR_INVALID_VALUE, "prepare_thd_metadata: T=%lld out of range",
                static_cast<long long>(T));
  if (K < 1 || K > DSA_MAX_INDEXER_TOPK)
    return fail(DSA_ERR_INVALID_VALUE, "prepare_thd_metadata: K=%d not in [1, %d]", K,
                DSA_MAX_INDEXER_TOPK);
  if (!cu_seqlens) return fail(DSA_ERR_INVALID_VALUE, "prepare_thd_metadata: cu_seqlens is NULL");
  const size_t need = dsa_thd_metadata_workspace_size(T);
  if (!ws || ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "prepare_thd_metadata: workspace needs %zu bytes, got %zu",
                need, ws ? ws_bytes : static_cast<size_t>(0));
  if (int rc = check_device()) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);

  // the one synchronisation: read the offsets on the host
  std::vector<int32_t> cu(static_cast<size_t>(B) + 1);
  hipError_t e = hipMemcpyAsync(cu.data(), cu_seqlens, cu.size() * sizeof(int32_t),
                                hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return hip_fail(e, "prepare_thd_metadata: copy of cu_seqlens");
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "prepare_thd_metadata: stream synchronize");
  if (cu[0] != 0) return fail(DSA_ERR_INVALID_VALUE, "cu_seqlens[0]=%d, expected 0", cu[0]);
  int32_t max_len = 0;
  int64_t pairs = 0, valid = 0;
  for (int32_t b = 0; b < B; ++b) {
    if (cu[b + 1] < cu[b])
      return fail(DSA_ERR_INVALID_VALUE, "cu_seqlens decreases at %d (%d > %d)", b, cu[b],
                  cu[b + 1]);
    const int64_t len = cu[b + 1] - cu[b];
    if (len > max_len) max_len = static_cast<int32_t>(len);
    pairs += len * (len + 1) / 2;
    const int64_t full = len < K ? len : K;  // rows 1..full have L <= K
    valid += full * (full + 1) / 2 + (len - full) * K;
  }
  if (cu[B] != T)
    return fail(DSA_ERR_INVALID_VALUE, "cu_seqlens[B]=%d does not match T=%lld", cu[B],
                static_cast<long long>(T));

  char *base = static_cast<char *>(ws);
  const size_t a = align_up(static_cast<size_t>(T) * sizeof(int32_t));
  base = reinterpret_cast<char *>(align_up(reinterpret_cast<uintptr_t>(base)));
  md->seq_start = reinterpret_cast<int32_t *>(base);
  md->causal_len = reinterpret_cast<int32_t *>(base + a);
  md->topk_length = reinterpret_cast<int32_t *>(base + 2 * a);
  md->row_order = reinterpret_cast<int32_t *>(base + 3 * a);
  int32_t *groups = reinterpret_cast<int32_t *>(base + 4 * a);
  md->T = T;
  md->B = B;
  md->K = K;
  md->max_seqlen = max_len;
  md->all_rows_nonempty = 1;  // causal rows always include their own key
  md->total_pairs = pairs;
  md->total_valid = valid;
  const int32_t ng = n_index_groups(cu);
  md->groups = groups;
  md->n_groups = ng;
  md->gpos = nullptr;
  md->group_first = nullptr;
  md->key_start = nullptr;
  md->pool = 0;
  md->total_key_tokens = T;
  e = dsa::launch_thd_metadata(cu_seqlens, B, T, K, md->seq_start, md->causal_len,
                               md->topk_length, md->row_order, groups, ng, s);
  if (e != hipSuccess) return hip_fail(e, "prepare_thd_metadata: launch");
  return DSA_OK;
}

// ---------------------------------------------------------------------------------------
// Local query rows against gathered global keys.  The inputs are read on the host (one
// synchronisation); rows, groups and their order are built there and uploaded into the
// workspace, which takes a second synchronisation so that no host buffer is read after it
// has been released.  workspace: seq_start | causal_len | topk_length | row_order | groups |
// group_first | gpos   (each 256-B aligned)
size_t dsa_local_metadata_workspace_size(int64_t T_q) {
  if (T_q < 0) return 0;
  const size_t a = align_up(static_cast<size_t>(T_q) * sizeof(int32_t));
  return 7 * a + 256;
}

int dsa_prepare_local_metadata(const int32_t *cu_seqlens, const int32_t *cu_seqlens_padded,
                               const int32_t *query_indices, const uint8_t *padding_mask,
                               int32_t B, int64_t T_q, int64_t T_k, int32_t K, void *ws,
                               size_t ws_bytes, dsa_thd_metadata *md, void *stream) {
  g_last_error.clear();
  if (!md) return fail(DSA_ERR_INVALID_VALUE, "prepare_local_metadata: md is NULL");
  if (B < 1) return fail(DSA_ERR_INVALID_VALUE, "prepare_local_metadata: B=%d must be >= 1", B);
  if (T_q < 0 || T_q > INT32_MAX || T_k < 0 || T_k > INT32_MAX)
    return fail(DSA_ERR_INVALID_VALUE, "prepare_local_metadata: T_q=%lld / T_k=%lld out of range",
                static_cast<long long>(T_q), static_cast<long long>(T_k));
  if (K < 1 || K > DSA_MAX_INDEXER_TOPK)
    return fail(DSA_ERR_INVALID_VALUE, "prepare_local_metadata: K=%d not in [1, %d]", K,
                DSA_MAX_INDEXER_TOPK);
  if (!cu_seqlens)
    return fail(DSA_ERR_INVALID_VALUE, "prepare_local_metadata: cu_seqlens is NULL");
  const size_t need = dsa_local_metadata_workspace_size(T_q);
  if (!ws || ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "prepare_local_metadata: workspace needs %zu bytes, got %zu",
                need, ws ? ws_bytes : static_cast<size_t>(0));
  if (int rc = check_device()) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);

  std::vector<int32_t> cu(static_cast<size_t>(B) + 1), cp(static_cast<size_t>(B) + 1);
  std::vector<int32_t> gp(static_cast<size_t>(T_q));
  std::vector<uint8_t> pm(padding_mask ? static_cast<size_t>(T_q) : 0);
  hipError_t e = hipMemcpyAsync(cu.data(), cu_seqlens, cu.size() * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess && cu_seqlens_padded)
    e = hipMemcpyAsync(cp.data(), cu_seqlens_padded, cp.size() * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess && query_indices && T_q > 0)
    e = hipMemcpyAsync(gp.data(), query_indices, gp.size() * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess && padding_mask && T_q > 0)
    e = hipMemcpyAsync(pm.data(), padding_mask, pm.size(), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "prepare_local_metadata: copy of the inputs");
  if (!cu_seqlens_padded) cp = cu;
  if (cu[0] != 0 || cp[0] != 0)
    return fail(DSA_ERR_INVALID_VALUE, "prepare_local_metadata: offsets must start at 0");
  for (int32_t b = 0; b < B; ++b) {
    if (cu[b + 1] < cu[b] || cp[b + 1] < cp[b])
      return fail(DSA_ERR_INVALID_VALUE, "prepare_local_metadata: offsets decrease at %d", b);
    if (cp[b + 1] - cp[b] < cu[b + 1] - cu[b])
      return fail(DSA_ERR_INVALID_VALUE,
                  "prepare_local_metadata: padded sequence %d shorter than its real length", b);
  }
  if (cp[B] > T_k)
    return fail(DSA_ERR_INVALID_VALUE, "prepare_local_metadata: offsets end at %d > T_k=%lld",
                cp[B], static_cast<long long>(T_k));
  if (!query_indices) {
    if (T_q != cp[B])
      return fail(DSA_ERR_INVALID_VALUE,
                  "prepare_local_metadata: without query_indices T_q must equal %d", cp[B]);
    for (int64_t i = 0; i < T_q; ++i) gp[i] = static_cast<int32_t>(i);
  }
  // rows
  const size_t n = static_cast<size_t>(T_q);
  std::vector<int32_t> start(n), clen(n), tlen(n);
  int32_t max_len = 0;
  int64_t pairs = 0, valid = 0;
  bool nonempty = true;
  for (size_t i = 0; i < n; ++i) {
    const int32_t p = gp[i];
    if (p < 0 || p >= cp[B])
      return fail(DSA_ERR_INVALID_VALUE, "prepare_local_metadata: query_indices[%zu]=%d outside "
                  "[0, %d)", i, p, cp[B]);
    const int32_t b = static_cast<int32_t>(std::upper_bound(cp.begin(), cp.end(), p) -
                                           cp.begin()) - 1;
    const int32_t pos = p - cp[b];
    const bool real = pos < cu[b + 1] - cu[b] && !(padding_mask && pm[i]);
    start[i] = cp[b];
    clen[i] = real ? pos + 1 : 0;
    tlen[i] = std::min(clen[i], K);
    max_len = std::max(max_len, clen[i]);
    pairs += clen[i];
    valid += tlen[i];
    nonempty = nonempty && real;
  }
  // groups: runs of up to kIdxRowsPerGroup real rows, consecutive in both row and key
  // position inside one sequence, cut so that each run ends a group; padding rows alone
  std::vector<int32_t> glast, gfirst;
  for (size_t i = 0; i < n;) {
    size_t j = i;
    if (clen[i] > 0)
      while (j + 1 < n && clen[j + 1] > 0 && start[j + 1] == start[i] && gp[j + 1] == gp[j] + 1)
        ++j;
    // rows i..j form one run: groups end at j, j - 4, ...
    for (int64_t last = static_cast<int64_t>(j); last >= static_cast<int64_t>(i);
         last -= dsa::kIdxRowsPerGroup) {
      glast.push_back(static_cast<int32_t>(last));
      gfirst.push_back(static_cast<int32_t>(
          std::max<int64_t>(last - (dsa::kIdxRowsPerGroup - 1), static_cast<int64_t>(i))));
    }
    i = j + 1;
  }
  // longest first (cost = keys of the last row), ties in row order
  std::vector<int32_t> gorder(glast.size());
  for (size_t g = 0; g < gorder.size(); ++g) gorder[g] = static_cast<int32_t>(g);
  std::stable_sort(gorder.begin(), gorder.end(), [&](int32_t a, int32_t b2) {
    return clen[glast[a]] > clen[glast[b2]];
  });
  std::vector<int32_t> groups(glast.size()), group_first(glast.size());
  for (size_t g = 0; g < gorder.size(); ++g) {
    groups[g] = glast[gorder[g]];
    group_first[g] = gfirst[gorder[g]];
  }
  std::vector<int32_t> order(n);
  for (size_t i = 0; i < n; ++i) order[i] = static_cast<int32_t>(i);
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t a, int32_t b2) { return clen[a] > clen[b2]; });

  char *base = reinterpret_cast<char *>(align_up(reinterpret_cast<uintptr_t>(ws)));
  const size_t a = align_up(n * sizeof(int32_t));
  md->seq_start = reinterpret_cast<int32_t *>(base);
  md->causal_len = reinterpret_cast<int32_t *>(base + a);
  md->topk_length = reinterpret_cast<int32_t *>(base + 2 * a);
  md->row_order = reinterpret_cast<int32_t *>(base + 3 * a);
  md->groups = reinterpret_cast<int32_t *>(base + 4 * a);
  md->group_first = reinterpret_cast<int32_t *>(base + 5 * a);
  md->gpos = reinterpret_cast<int32_t *>(base + 6 * a);
  md->T = T_q;
  md->B = B;
  md->K = K;
  md->max_seqlen = max_len;
  md->all_rows_nonempty = nonempty ? 1 : 0;
  md->total_pairs = pairs;
  md->total_valid = valid;
  md->n_groups = static_cast<int32_t>(groups.size());
  md->total_key_tokens = T_k;
  md->key_start = nullptr;
  md->pool = 0;
  const std::pair<int32_t *, const std::vector<int32_t> *> up[] = {
      {md->seq_start, &start}, {md->causal_len, &clen}, {md->topk_length, &tlen},
      {md->row_order, &order}, {md->groups, &groups}, {md->group_first, &group_first},
      {md->gpos, &gp}};
  for (const auto &u : up)
    if (!u.second->empty()) {
      e = hipMemcpyAsync(u.first, u.second->data(), u.second->size() * 4, hipMemcpyHostToDevice,
                         s);
      if (e != hipSuccess) return hip_fail(e, "prepare_local_metadata: upload");
    }
  e = hipStreamSynchronize(s);  // the host vectors are released on return
  if (e != hipSuccess) return hip_fail(e, "prepare_local_metadata: stream synchronize");
  return DSA_OK;
}

// ---------------------------------------------------------------------------------------
// k-pool rows.  workspace: seq_start (pool coordinate of the sequence's first pool) |
// causal_len (complete pools the row sees) | topk_length | row_order | groups | group_first |
// gpos (pool coordinate of the row's last complete pool) | key_start (each 256-B aligned)
size_t dsa_kpool_metadata_workspace_size(int64_t T) {
  if (T < 0) return 0;
  const size_t a = align_up(static_cast<size_t>(T) * sizeof(int32_t));
  return 8 * a + 256;
}

int dsa_prepare_kpool_metadata(const int32_t *cu_seqlens, int32_t B, int64_t T, int32_t pool,
                               int32_t K_pools, void *ws, size_t ws_bytes, dsa_thd_metadata *md,
                               void *stream) {
  g_last_error.clear();
  const char *who = "prepare_kpool_metadata";
  if (!md) return fail(DSA_ERR_INVALID_VALUE, "%s: md is NULL", who);
  if (B < 1) return fail(DSA_ERR_INVALID_VALUE, "%s: B=%d must be >= 1", who, B);
  if (T < 0 || T > INT32_MAX - 4096)
    return fail(DSA_ERR_INVALID_VALUE, "%s: T=%lld out of range", who, static_cast<long long>(T));
  if (pool < 1 || pool > 16) return fail(DSA_ERR_INVALID_VALUE, "%s: pool=%d not in [1, 16]", who, pool);
  if (K_pools < 1 || K_pools > DSA_MAX_INDEXER_TOPK)
    return fail(DSA_ERR_INVALID_VALUE, "%s: K_pools=%d not in [1, %d]", who, K_pools,
                DSA_MAX_INDEXER_TOPK);
  if (!cu_seqlens) return fail(DSA_ERR_INVALID_VALUE, "%s: cu_seqlens is NULL", who);
  const size_t need = dsa_kpool_metadata_workspace_size(T);
  if (!ws || ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "%s: workspace needs %zu bytes, got %zu", who, need,
                ws ? ws_bytes : static_cast<size_t>(0));
  if (int rc = check_device()) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  std::vector<int32_t> cu(static_cast<size_t>(B) + 1);
  hipError_t e = hipMemcpyAsync(cu.data(), cu_seqlens, cu.size() * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "prepare_kpool_metadata: copy of cu_seqlens");
  if (cu[0] != 0 || static_cast<int64_t>(cu[B]) != T)
    return fail(DSA_ERR_INVALID_VALUE, "%s: cu_seqlens must run from 0 to T=%lld", who,
                static_cast<long long>(T));
  for (int32_t b = 0; b < B; ++b)
    if (cu[b + 1] < cu[b]) return fail(DSA_ERR_INVALID_VALUE, "%s: offsets decrease at %d", who, b);
  const size_t n = static_cast<size_t>(T);
  std::vector<int32_t> start(n), clen(n), tlen(n), gp(n), kst(n);
  std::vector<int32_t> glast, gfirst;
  int64_t cp = 0, pairs = 0, valid = 0;
  int32_t max_len = 0;
  for (int32_t b = 0; b < B; ++b) {
    const int32_t s0 = cu[b], s1 = cu[b + 1];
    for (int32_t t = s0; t < s1; ++t) {
      const int32_t P = (t - s0 + 1) / pool;
      start[t] = static_cast<int32_t>(cp);
      clen[t] = P;
      tlen[t] = std::min(P, K_pools);
      gp[t] = static_cast<int32_t>(cp) + P - 1;
      kst[t] = s0;
      pairs += P;
      valid += tlen[t];
      max_len = std::max(max_len, P);
    }
    // work groups: consecutive rows that see the same pools, at most kIdxRowsPerGroup each
    for (int32_t t = s0; t < s1;) {
      int32_t u = t;
      while (u + 1 < s1 && clen[u + 1] == clen[t] && u + 1 - t < dsa::kIdxRowsPerGroup) ++u;
      glast.push_back(u);
      gfirst.push_back(t);
      t = u + 1;
    }
    cp += (s1 - s0) / pool;
  }
  if (cp > INT32_MAX - 4096) return fail(DSA_ERR_INVALID_VALUE, "%s: too many pools", who);
  std::vector<int32_t> gorder(glast.size());
  for (size_t g = 0; g < gorder.size(); ++g) gorder[g] = static_cast<int32_t>(g);
  std::stable_sort(gorder.begin(), gorder.end(), [&](int32_t a, int32_t b2) {
    return clen[glast[a]] > clen[glast[b2]];
  });
  std::vector<int32_t> groups(glast.size()), group_first(glast.size());
  for (size_t g = 0; g < gorder.size(); ++g) {
    groups[g] = glast[gorder[g]];
    group_first[g] = gfirst[gorder[g]];
  }
  std::vector<int32_t> order(n);
  for (size_t i = 0; i < n; ++i) order[i] = static_cast<int32_t>(i);
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t a, int32_t b2) { return clen[a] > clen[b2]; });
  char *base = reinterpret_cast<char *>(align_up(reinterpret_cast<uintptr_t>(ws)));
  const size_t a = align_up(n * sizeof(int32_t));
  md->seq_start = reinterpret_cast<int32_t *>(base);
  md->causal_len = reinterpret_cast<int32_t *>(base + a);
  md->topk_length = reinterpret_cast<int32_t *>(base + 2 * a);
  md->row_order = reinterpret_cast<int32_t *>(base + 3 * a);
  md->groups = reinterpret_cast<int32_t *>(base + 4 * a);
  md->group_first = reinterpret_cast<int32_t *>(base + 5 * a);
  md->gpos = reinterpret_cast<int32_t *>(base + 6 * a);
  md->key_start = reinterpret_cast<int32_t *>(base + 7 * a);
  md->T = T;
  md->B = B;
  md->K = K_pools;
  md->max_seqlen = max_len;
  md->all_rows_nonempty = 1;
  md->total_pairs = pairs;
  md->total_valid = valid;
  md->n_groups = static_cast<int32_t>(groups.size());
  md->total_key_tokens = cp;
  md->pool = pool;
  const std::pair<int32_t *, const std::vector<int32_t> *> up[] = {
      {md->seq_start, &start}, {md->causal_len, &clen}, {md->topk_length, &tlen},
      {md->row_order, &order}, {md->groups, &groups}, {md->group_first, &group_first},
      {md->gpos, &gp}, {md->key_start, &kst}};
  for (const auto &u : up)
    if (!u.second->empty()) {
      e = hipMemcpyAsync(u.first, u.second->data(), u.second->size() * 4, hipMemcpyHostToDevice,
                         s);
      if (e != hipSuccess) return hip_fail(e, "prepare_kpool_metadata: upload");
    }
  e = hipStreamSynchronize(s);  // the host vectors are released on return
  if (e != hipSuccess) return hip_fail(e, "prepare_kpool_metadata: stream synchronize");
  return DSA_OK;
}

size_t dsa_kpool_indexer_topk_workspace_size(int64_t T, int32_t K_pools) {
  if (T < 0 || K_pools < 1) return 0;
  return align_up(static_cast<size_t>(T) * static_cast<size_t>(K_pools) * sizeof(int32_t)) +
         align_up(static_cast<size_t>(T) * sizeof(int32_t)) + 256;
}

// ---------------------------------------------------------------------------------------
size_t dsa_indexer_topk_workspace_size(int64_t T, int32_t H_i, int32_t D_i, int32_t K) {
  (void)T;
  (void)H_i;
  (void)D_i;
  (void)K;
  return 0;  // the candidate buffers live in LDS
}

int dsa_indexer_topk(const uint16_t *q_idx, const uint16_t *k_idx, const float *w,
                     const dsa_thd_metadata *md, int32_t H_i, int32_t D_i, int32_t K,
                     int32_t *idx, int32_t *len, void *ws, size_t ws_bytes, void *stream) {
  g_last_error.clear();
  (void)ws;
  (void)ws_bytes;
  if (!md || (md->T > 0 && (!md->seq_start || !md->groups)))
    return fail(DSA_ERR_INVALID_VALUE, "indexer_topk: metadata missing");
  if (md->pool > 0)
    return fail(DSA_ERR_INVALID_VALUE,
                "indexer_topk: k-pool metadata; use dsa_kpool_indexer_topk");
  if (H_i < 1 || H_i > 64)
    return fail(DSA_ERR_INVALID_VALUE, "indexer_topk: H_i=%d not in [1, 64]", H_i);
  if (D_i != 64 && D_i != 128)
    return fail(DSA_ERR_INVALID_VALUE, "indexer_topk: D_i=%d must be 64 or 128", D_i);
  if (K < 1 || K > DSA_MAX_INDEXER_TOPK)
    return fail(DSA_ERR_INVALID_VALUE, "indexer_topk: K=%d not in [1, %d]", K,
                DSA_MAX_INDEXER_TOPK);
  const int64_t T = md->T;
  if (T == 0) return DSA_OK;
  // key positions are 32-bit inside the kernel, including a few tiles of look-ahead
  const int64_t Tmax = std::max<int64_t>(T, md->total_key_tokens);
  if (Tmax > INT32_MAX - 4096)
    return fail(DSA_ERR_INVALID_VALUE, "indexer_topk: T=%lld exceeds %d",
                static_cast<long long>(Tmax), INT32_MAX - 4096);
  if (!q_idx || !k_idx || !w || !idx || !len)
    return fail(DSA_ERR_INVALID_VALUE, "indexer_topk: NULL tensor pointer");
  if (!aligned16(q_idx) || !aligned16(k_idx))
    return fail(DSA_ERR_INVALID_VALUE, "indexer_topk: q_idx/k_idx must be 16-byte aligned");
  if (int rc = check_device()) return rc;
  dsa::IndexerRows rows;
  rows.seq_start = md->seq_start;
  rows.causal_len = md->causal_len;
  rows.gpos = md->gpos;
  rows.groups = md->groups;
  rows.group_first = md->group_first;
  rows.n_groups = md->n_groups;
  hipError_t e = dsa::launch_indexer_topk(q_idx, k_idx, w, rows, H_i, D_i, K, idx, len,
                                          static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "indexer_topk: launch");
  return DSA_OK;
}

int dsa_kpool_indexer_topk(const uint16_t *q_idx, const uint16_t *k_pool, const float *w,
                           const dsa_thd_metadata *md, int32_t H_i, int32_t D_i, int32_t K_pools,
                           int32_t *idx, int32_t *len, void *ws, size_t ws_bytes, void *stream) {
  g_last_error.clear();
  const char *who = "kpool_indexer_topk";
  if (!md || md->pool < 1 || (md->T > 0 && (!md->seq_start || !md->groups || !md->key_start)))
    return fail(DSA_ERR_INVALID_VALUE, "%s: k-pool metadata missing", who);
  if (K_pools != md->K)
    return fail(DSA_ERR_INVALID_VALUE, "%s: K_pools=%d differs from the metadata's %d", who,
                K_pools, md->K);
  if (H_i < 1 || H_i > 64) return fail(DSA_ERR_INVALID_VALUE, "%s: H_i=%d not in [1, 64]", who, H_i);
  if (D_i != 64 && D_i != 128)
    return fail(DSA_ERR_INVALID_VALUE, "%s: D_i=%d must be 64 or 128", who, D_i);
  const int64_t T = md->T;
  if (T == 0) return DSA_OK;
  const size_t need = dsa_kpool_indexer_topk_workspace_size(T, K_pools);
  if (!ws || ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "%s: workspace needs %zu bytes, got %zu", who, need,
                ws ? ws_bytes : static_cast<size_t>(0));
  if (!q_idx || !w || !idx || !len || (md->total_key_tokens > 0 && !k_pool))
    return fail(DSA_ERR_INVALID_VALUE, "%s: NULL tensor pointer", who);
  if (!aligned16(q_idx) || !aligned16(k_pool))
    return fail(DSA_ERR_INVALID_VALUE, "%s: q_idx/k_pool must be 16-byte aligned", who);
  if (int rc = check_device()) return rc;
  char *p = reinterpret_cast<char *>(align_up(reinterpret_cast<uintptr_t>(ws)));
  int32_t *pidx = reinterpret_cast<int32_t *>(p);
  int32_t *plen = reinterpret_cast<int32_t *>(
      p + align_up(static_cast<size_t>(T) * static_cast<size_t>(K_pools) * sizeof(int32_t)));
  hipStream_t s = static_cast<hipStream_t>(stream);
  dsa::IndexerRows rows;
  rows.seq_start = md->seq_start;
  rows.causal_len = md->causal_len;
  rows.gpos = md->gpos;
  rows.groups = md->groups;
  rows.group_first = md->group_first;
  rows.n_groups = md->n_groups;
  // rows without a complete pool get len 0 from the indexer without reading k_pool
  hipError_t e = dsa::launch_indexer_topk(q_idx, k_pool, w, rows, H_i, D_i, K_pools, pidx, plen,
                                          s);
  if (e == hipSuccess)
    e = dsa::launch_kpool_expand(pidx, plen, md->seq_start, md->causal_len, md->key_start, T,
                                 K_pools, md->pool, idx, len, s);
  if (e != hipSuccess) return hip_fail(e, "kpool_indexer_topk: launch");
  return DSA_OK;
}

// ---------------------------------------------------------------------------------------
static int check_attention_args(const char *who, const uint16_t *q, const uint16_t *kv,
                                const int32_t *idx, int64_t T_q, int64_t T_kv, int32_t H,
                                int32_t D_qk, int32_t D_v, int32_t K, float scale, int32_t max_h) {
  if (T_q < 0 || T_kv < 0 || T_q > INT32_MAX || T_kv > INT32_MAX)
    return fail(DSA_ERR_INVALID_VALUE, "%s: T_q=%lld / T_kv=%lld out of range", who,
                static_cast<long long>(T_q), static_cast<long long>(T_kv));
  if (H < 1 || H > max_h)
    return fail(DSA_ERR_INVALID_VALUE, "%s: H=%d not in [1, %d]", who, H, max_h);
  if (D_qk != 576 && D_qk != 512)
    return fail(DSA_ERR_INVALID_VALUE, "%s: D_qk=%d must be 576 or 512", who, D_qk);
  if (D_v != 512) return fail(DSA_ERR_INVALID_VALUE, "%s: D_v=%d must be 512", who, D_v);
  if (K < 1) return fail(DSA_ERR_INVALID_VALUE, "%s: K=%d must be >= 1", who, K);
  if (!(scale > 0.0f) || scale != scale || scale == INFINITY)
    return fail(DSA_ERR_INVALID_VALUE, "%s: scale must be a positive finite number", who);
  if (T_q > 0 && T_kv < 1)
    return fail(DSA_ERR_INVALID_VALUE, "%s: T_kv must be >= 1 when T_q > 0", who);
  // latent rows are addressed with 32-bit byte offsets from kv
  if (T_kv * static_cast<int64_t>(D_qk) * 2 > static_cast<int64_t>(UINT32_MAX))
    return fail(DSA_ERR_INVALID_VALUE, "%s: kv [%lld, %d] exceeds 4 GiB", who,
                static_cast<long long>(T_kv), D_qk);
  if (T_q > 0 && (!q || !idx || !kv))
    return fail(DSA_ERR_INVALID_VALUE, "%s: NULL tensor pointer", who);
  if (!aligned16(q) || !aligned16(kv))
    return fail(DSA_ERR_INVALID_VALUE, "%s: q/kv must be 16-byte aligned", who);
  return DSA_OK;
}

// Debug-only validation of index contents; `flag` is 4 bytes of caller workspace.
static int debug_check_indices(const int32_t *idx, const int32_t *topk_length, int64_t T_q,
                               int32_t K, int64_t T_kv, int32_t *flag, hipStream_t s) {
  int32_t bad = 0;
  hipError_t e = dsa::launch_check_indices(idx, topk_length, T_q, K, T_kv, flag, s);
  if (e == hipSuccess) e = hipMemcpyAsync(&bad, flag, sizeof bad, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "debug index check");
  if (bad) return fail(DSA_ERR_INVALID_VALUE, "index or topk_length out of range");
  return DSA_OK;
}

int dsa_sparse_mla_fwd(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                       const int32_t *topk_length, int64_t T_q, int64_t T_kv, int32_t H,
                       int32_t D_qk, int32_t D_v, int32_t K, float scale, uint16_t *out,
                       float *lse, void *stream) {
  g_last_error.clear();
  if (int rc = check_attention_args("sparse_mla_fwd", q, kv, idx, T_q, T_kv, H, D_qk, D_v, K,
                                    scale, 64))
    return rc;
  if (K > 4096) return fail(DSA_ERR_INVALID_VALUE, "sparse_mla_fwd: K=%d exceeds 4096", K);
  if (T_q > 0 && (!out || !lse))
    return fail(DSA_ERR_INVALID_VALUE, "sparse_mla_fwd: NULL output pointer");
  if (int rc = check_device()) return rc;
  hipError_t e = dsa::launch_sparse_mla_fwd(q, kv, idx, topk_length, T_q, H, D_qk, K, scale, out,
                                            lse, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "sparse_mla_fwd: launch");
  return DSA_OK;
}

// Backward workspace layout: delta [T_q, H] fp32 | debug flag and largest |kv| | then one or two pass buffers,
// each off [T_kv + 1] | cursor [T_kv] | list [R * K] int32 | stage [R * K] rows of
// bwd_stage_row_bytes(D_qk); every segment 256-byte aligned.  One buffer when a single pass
// covers every query row; otherwise two, so that a pass's reduction overlaps the next pass's
// compute.
static size_t bwd_fixed_bytes(int64_t T_q, int32_t H) {
  return align_up(static_cast<size_t>(T_q) * static_cast<size_t>(H) * sizeof(float)) + 256 +
         256 /* base alignment */;
}

static size_t bwd_pass_bytes(int64_t rows, int64_t T_kv, int32_t D_qk, int32_t K) {
  const size_t pairs = static_cast<size_t>(rows) * static_cast<size_t>(K);
  return align_up(static_cast<size_t>(T_kv + 1) * sizeof(int32_t)) +
         align_up(static_cast<size_t>(T_kv) * sizeof(int32_t)) + align_up(pairs * sizeof(int32_t)) +
         align_up(pairs * dsa::bwd_stage_row_bytes(D_qk));
}

static size_t bwd_total_bytes(int64_t T_q, int64_t T_kv, int32_t H, int32_t D_qk, int32_t K,
                              int64_t R) {
  const int nbuf = R < T_q ? 2 : 1;
  return bwd_fixed_bytes(T_q, H) + nbuf * bwd_pass_bytes(std::max<int64_t>(R, 1), T_kv, D_qk, K);
}

size_t dsa_sparse_mla_bwd_workspace_size(int64_t T_q, int64_t T_kv, int32_t H, int32_t D_qk,
                                         int32_t K, int64_t rows_per_pass) {
  if (T_q < 0 || T_kv < 0 || H < 0 || D_qk < 0 || K < 1) return 0;
  int64_t R = rows_per_pass <= 0 || rows_per_pass > T_q ? T_q : rows_per_pass;
  R = std::min<int64_t>(R, INT32_MAX / K);
  return bwd_total_bytes(T_q, T_kv, H, D_qk, K, std::max<int64_t>(R, 1));
}

// Argument checks, pass planning, workspace carving and launch of the backward.  With
// two_buffers false every pass uses one staging buffer on the caller's stream (no helper
// stream), and a workspace that holds less than one row per pass is reported as `small_code`.
static int bwd_run(const char *who, const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                   const int32_t *topk_length, const uint16_t *out, const float *lse,
                   const uint16_t *dout, int64_t T_q, int64_t T_kv, int32_t H, int32_t D_qk,
                   int32_t D_v, int32_t K, float scale, uint16_t *dq, float *dkv, uint32_t flags,
                   void *ws, size_t ws_bytes, bool two_buffers, int small_code, void *stream,
                   float *kl_target = nullptr) {
  if (int rc = check_attention_args(who, q, kv, idx, T_q, T_kv, H, D_qk, D_v, K, scale, 64))
    return rc;
  if (K > 4096) return fail(DSA_ERR_INVALID_VALUE, "%s: K=%d exceeds 4096", who, K);
  if (flags & ~(DSA_BWD_ACCUMULATE_DKV | DSA_DEBUG_CHECK_INDICES))
    return fail(DSA_ERR_INVALID_VALUE, "%s: unknown flags 0x%x", who, flags);
  if (T_q > 0 && (!out || !lse || !dout || !dq))
    return fail(DSA_ERR_INVALID_VALUE, "%s: NULL tensor pointer", who);
  if (T_kv > 0 && !dkv) return fail(DSA_ERR_INVALID_VALUE, "%s: dkv is NULL", who);
  if (!aligned16(out) || !aligned16(dout) || !aligned16(dkv))
    return fail(DSA_ERR_INVALID_VALUE, "%s: out/dout/dkv must be 16-byte aligned", who);
  // rows per pass: all of them in one buffer if the workspace holds that, else as many as two
  // buffers hold, else as many as one buffer holds (pair ids are int32)
  const int64_t R_max = std::min<int64_t>(T_q, INT32_MAX / K);
  const size_t need = bwd_fixed_bytes(T_q, H) + bwd_pass_bytes(1, T_kv, D_qk, K);
  if (T_q > 0 && (!ws || ws_bytes < need))
    return fail(small_code, "%s: workspace needs at least %zu bytes, got %zu", who, need,
                ws ? ws_bytes : static_cast<size_t>(0));
  int64_t R = 0;
  int nbuf = 1;
  if (T_q > 0) {
    const size_t fixed = bwd_fixed_bytes(T_q, H);
    const size_t per_row = static_cast<size_t>(K) * (dsa::bwd_stage_row_bytes(D_qk) + 4);
    auto largest = [&](int nb) -> int64_t {  // rows per pass that nb buffers hold (0: none)
      const size_t base = fixed + nb * bwd_pass_bytes(0, T_kv, D_qk, K);
      if (ws_bytes <= base) return 0;
      int64_t r = std::min<int64_t>(R_max, static_cast<int64_t>((ws_bytes - base) / (nb * per_row)));
      while (r > 0 && fixed + nb * bwd_pass_bytes(r, T_kv, D_qk, K) > ws_bytes) --r;  // slack
      return r;
    };
    if (R_max == T_q && fixed + bwd_pass_bytes(T_q, T_kv, D_qk, K) <= ws_bytes) {
      R = T_q;
    } else if (two_buffers && (R = largest(2)) >= 1) {
      nbuf = 2;
    } else {
      R = std::max<int64_t>(largest(1), 1);
    }
    if (R >= T_q) nbuf = 1;
  }
  if (int rc = check_device()) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char *p = reinterpret_cast<char *>(align_up(reinterpret_cast<uintptr_t>(ws)));
  dsa::BwdWorkspace w;
  w.delta = reinterpret_cast<float *>(p);
  p += align_up(static_cast<size_t>(T_q) * static_cast<size_t>(H) * sizeof(float));
  w.flag = reinterpret_cast<int32_t *>(p);
  w.vmax = reinterpret_cast<uint32_t *>(p + 64);
  p += 256;
  w.nbuf = nbuf;
  for (int b = 0; b < 2; ++b) {
    dsa::BwdPassBuffers &bb = w.buf[b];
    if (b >= nbuf) {
      bb = w.buf[0];
      continue;
    }
    bb.off = reinterpret_cast<int32_t *>(p);
    p += align_up(static_cast<size_t>(T_kv + 1) * sizeof(int32_t));
    bb.cursor = reinterpret_cast<int32_t *>(p);
    p += align_up(static_cast<size_t>(T_kv) * sizeof(int32_t));
    bb.list = reinterpret_cast<int32_t *>(p);
    p += align_up(static_cast<size_t>(R) * static_cast<size_t>(K) * sizeof(int32_t));
    bb.stage = reinterpret_cast<uint32_t *>(p);
    p += align_up(static_cast<size_t>(R) * static_cast<size_t>(K) *
                  dsa::bwd_stage_row_bytes(D_qk));
  }
  w.rows_per_pass = R;
  if ((flags & DSA_DEBUG_CHECK_INDICES) && T_q > 0)
    if (int rc = debug_check_indices(idx, topk_length, T_q, K, T_kv, w.flag, s)) return rc;
  hipError_t e = dsa::launch_sparse_mla_bwd(q, kv, idx, topk_length, out, lse, dout, T_q, T_kv,
                                            H, D_qk, K, scale, dq, dkv,
                                            (flags & DSA_BWD_ACCUMULATE_DKV) != 0, w, s,
                                            kl_target);
  if (e != hipSuccess) {
    char what[64];
    snprintf(what, sizeof what, "%s: launch", who);
    return hip_fail(e, what);
  }
  return DSA_OK;
}

int dsa_sparse_mla_bwd(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                       const int32_t *topk_length, const uint16_t *out, const float *lse,
                       const uint16_t *dout, int64_t T_q, int64_t T_kv, int32_t H,
                       int32_t D_qk, int32_t D_v, int32_t K, float scale, uint16_t *dq,
                       float *dkv, uint32_t flags, void *ws, size_t ws_bytes, void *stream) {
  g_last_error.clear();
  return bwd_run("sparse_mla_bwd", q, kv, idx, topk_length, out, lse, dout, T_q, T_kv, H, D_qk,
                 D_v, K, scale, dq, dkv, flags, ws, ws_bytes, true, DSA_ERR_WORKSPACE, stream);
}

// ---------------------------------------------------------------------------------------
// Indexer KL loss.  kl_bwd workspace: off [T_kv + 1] | cursor [T_kv] | list [R * K] | stage
// [R * K] rows of bwd_stage_row_bytes(128), every segment 256-byte aligned.
static size_t kl_pass_bytes(int64_t rows, int64_t T_kv, int32_t K) {
  const size_t pairs = static_cast<size_t>(rows) * static_cast<size_t>(K);
  return 256 + align_up(static_cast<size_t>(T_kv + 1) * sizeof(int32_t)) +
         align_up(static_cast<size_t>(T_kv) * sizeof(int32_t)) + align_up(pairs * sizeof(int32_t)) +
         align_up(pairs * dsa::bwd_stage_row_bytes(128));
}

size_t dsa_indexer_kl_bwd_workspace_size(int64_t T_q, int64_t T_kv, int32_t K,
                                         int64_t rows_per_pass) {
  if (T_q < 0 || T_kv < 0 || K < 1) return 0;
  int64_t R = rows_per_pass <= 0 || rows_per_pass > T_q ? T_q : rows_per_pass;
  R = std::min<int64_t>(R, INT32_MAX / K);
  return kl_pass_bytes(std::max<int64_t>(R, 1), T_kv, K);
}

int dsa_indexer_kl_target(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                          const int32_t *topk_length, const float *lse, int64_t T_q,
                          int64_t T_kv, int32_t H, int32_t D_qk, int32_t K, float scale,
                          float *target, void *stream) {
  g_last_error.clear();
  const char *who = "indexer_kl_target";
  if (int rc = check_attention_args(who, q, kv, idx, T_q, T_kv, H, D_qk, 512, K, scale, 64))
    return rc;
  if (K > 4096) return fail(DSA_ERR_INVALID_VALUE, "%s: K=%d exceeds 4096", who, K);
  if (T_q > 0 && (!lse || !target))
    return fail(DSA_ERR_INVALID_VALUE, "%s: NULL lse or target", who);
  if (int rc = check_device()) return rc;
  hipError_t e = dsa::launch_indexer_kl_target(q, kv, idx, topk_length, lse, T_q, H, D_qk, K,
                                               scale, target, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "indexer_kl_target: launch");
  return DSA_OK;
}

int dsa_indexer_kl_bwd(const uint16_t *q_idx, const uint16_t *k_idx, const float *w,
                       const int32_t *idx, const int32_t *topk_length, const float *target,
                       int64_t T_q, int64_t T_kv, int32_t H_i, int32_t D_i, int32_t K,
                       float grad, float *loss, uint16_t *dq_idx, float *dw, float *dk_idx,
                       uint32_t flags, void *ws, size_t ws_bytes, void *stream) {
  g_last_error.clear();
  const char *who = "indexer_kl_bwd";
  if (T_q < 0 || T_kv < 0 || T_q > INT32_MAX || T_kv > INT32_MAX)
    return fail(DSA_ERR_INVALID_VALUE, "%s: T_q / T_kv out of range", who);
  if (H_i < 1 || H_i > 64) return fail(DSA_ERR_INVALID_VALUE, "%s: H_i=%d not in [1, 64]", who, H_i);
  if (D_i != 128) return fail(DSA_ERR_INVALID_VALUE, "%s: D_i=%d must be 128", who, D_i);
  if (K < 1 || K > 4096) return fail(DSA_ERR_INVALID_VALUE, "%s: K=%d not in [1, 4096]", who, K);
  if (!(grad == grad) || grad == INFINITY || grad == -INFINITY)
    return fail(DSA_ERR_INVALID_VALUE, "%s: grad must be finite", who);
  if (flags & ~DSA_BWD_ACCUMULATE_DKV)
    return fail(DSA_ERR_INVALID_VALUE, "%s: unknown flags 0x%x", who, flags);
  if (T_q > 0 && T_kv < 1)
    return fail(DSA_ERR_INVALID_VALUE, "%s: T_kv must be >= 1 when T_q > 0", who);
  if (T_kv * static_cast<int64_t>(D_i) * 2 > static_cast<int64_t>(UINT32_MAX))
    return fail(DSA_ERR_INVALID_VALUE, "%s: k_idx exceeds 4 GiB", who);
  if (T_q > 0 && (!q_idx || !k_idx || !w || !idx || !target || !loss || !dq_idx || !dw))
    return fail(DSA_ERR_INVALID_VALUE, "%s: NULL tensor pointer", who);
  if (T_kv > 0 && !dk_idx) return fail(DSA_ERR_INVALID_VALUE, "%s: dk_idx is NULL", who);
  if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(dq_idx) || !aligned16(dk_idx))
    return fail(DSA_ERR_INVALID_VALUE, "%s: q_idx/k_idx/dq_idx/dk_idx must be 16-byte aligned",
                who);
  const size_t need = kl_pass_bytes(1, T_kv, K);
  if (T_q > 0 && (!ws || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "%s: workspace needs at least %zu bytes, got %zu", who, need,
                ws ? ws_bytes : static_cast<size_t>(0));
  int64_t R = 1;
  if (T_q > 0) {
    const int64_t R_max = std::min<int64_t>(T_q, INT32_MAX / K);
    const size_t per_row = static_cast<size_t>(K) * (dsa::bwd_stage_row_bytes(128) + 4);
    R = std::min<int64_t>(R_max, static_cast<int64_t>((ws_bytes - kl_pass_bytes(0, T_kv, K)) /
                                                      per_row) + 1);
    while (R > 1 && kl_pass_bytes(R, T_kv, K) > ws_bytes) --R;
  }
  if (int rc = check_device()) return rc;
  dsa::BwdPassBuffers bb;
  char *p = reinterpret_cast<char *>(align_up(reinterpret_cast<uintptr_t>(ws)));
  bb.off = reinterpret_cast<int32_t *>(p);
  p += align_up(static_cast<size_t>(T_kv + 1) * sizeof(int32_t));
  bb.cursor = reinterpret_cast<int32_t *>(p);
  p += align_up(static_cast<size_t>(T_kv) * sizeof(int32_t));
  bb.list = reinterpret_cast<int32_t *>(p);
  p += align_up(static_cast<size_t>(R) * static_cast<size_t>(K) * sizeof(int32_t));
  bb.stage = reinterpret_cast<uint32_t *>(p);
  hipError_t e = dsa::launch_indexer_kl_bwd(
      q_idx, k_idx, w, idx, topk_length, target, T_q, T_kv, H_i, K, grad, loss, dq_idx, dw,
      dk_idx, (flags & DSA_BWD_ACCUMULATE_DKV) != 0, bb, R, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "indexer_kl_bwd: launch");
  return DSA_OK;
}

int dsa_sparse_mla_bwd_kl_target(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                                 const int32_t *topk_length, const uint16_t *out,
                                 const float *lse, const uint16_t *dout, int64_t T_q,
                                 int64_t T_kv, int32_t H, int32_t D_qk, int32_t D_v, int32_t K,
                                 float scale, uint16_t *dq, float *dkv, float *target,
                                 uint32_t flags, void *ws, size_t ws_bytes, void *stream) {
  g_last_error.clear();
  if (T_q > 0 && !target)
    return fail(DSA_ERR_INVALID_VALUE, "sparse_mla_bwd_kl_target: target is NULL");
  return bwd_run("sparse_mla_bwd_kl_target", q, kv, idx, topk_length, out, lse, dout, T_q, T_kv,
                 H, D_qk, D_v, K, scale, dq, dkv, flags, ws, ws_bytes, true, DSA_ERR_WORKSPACE,
                 stream, target);
}

int64_t dsa_gather_probe_groups(int64_t n) {
  return n <= 0 ? 0 : (n + dsa::kGatherProbeRows - 1) / dsa::kGatherProbeRows;
}

int dsa_gather_probe(const uint16_t *table, int64_t rows, int32_t width, const int32_t *idx,
                     int64_t n, uint32_t *sink, void *stream) {
  g_last_error.clear();
  if (width != 512 && width != 576)
    return fail(DSA_ERR_INVALID_VALUE, "gather_probe: width=%d not in {512, 576}", width);
  if (rows < 1 || rows * static_cast<int64_t>(width) * 2 > static_cast<int64_t>(UINT32_MAX))
    return fail(DSA_ERR_INVALID_VALUE, "gather_probe: rows=%lld out of range",
                static_cast<long long>(rows));
  if (n < 0 || dsa_gather_probe_groups(n) > INT32_MAX)
    return fail(DSA_ERR_INVALID_VALUE, "gather_probe: n=%lld out of range",
                static_cast<long long>(n));
  if (n > 0 && (!table || !idx || !sink))
    return fail(DSA_ERR_INVALID_VALUE, "gather_probe: NULL pointer");
  if (!aligned16(table)) return fail(DSA_ERR_INVALID_VALUE, "gather_probe: table not 16-byte aligned");
  if (int rc = check_device()) return rc;
  hipError_t e = dsa::launch_gather_probe(table, width, idx, n, sink,
                                          static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gather_probe: launch");
  return DSA_OK;
}

size_t dsa_sparse_mla_bwd_noalloc_scratch_bytes(void) { return dsa::kNoAllocScratchBytes; }

int dsa_sparse_mla_bwd_noalloc(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                               const int32_t *topk_length, const uint16_t *out, const float *lse,
                               const uint16_t *dout, int64_t T_q, int64_t T_kv, int32_t H,
                               int32_t D_qk, int32_t D_v, int32_t K, float scale, uint16_t *dq,
                               float *dkv, uint32_t flags, void *stream) {
  g_last_error.clear();
  const char *who = "sparse_mla_bwd_noalloc";
  if (int rc = check_attention_args(who, q, kv, idx, T_q, T_kv, H, D_qk, D_v, K, scale, 64))
    return rc;
  // sizes the scratch cannot hold are rejected before the device is touched
  if (T_q > 0 && K <= 4096) {
    const size_t need = bwd_fixed_bytes(T_q, H) + bwd_pass_bytes(1, T_kv, D_qk, K);
    if (need > dsa::kNoAllocScratchBytes)
      return fail(DSA_ERR_INVALID_VALUE,
                  "%s: these sizes need at least %zu bytes of scratch; the library's scratch "
                  "holds %zu",
                  who, need, dsa::kNoAllocScratchBytes);
  }
  void *ws = nullptr;
  if (T_q > 0) {
    if (int rc = check_device()) return rc;
    hipError_t e = dsa::noalloc_scratch(&ws);
    if (e != hipSuccess) return hip_fail(e, "sparse_mla_bwd_noalloc: scratch address");
  }
  return bwd_run(who, q, kv, idx, topk_length, out, lse, dout, T_q, T_kv, H, D_qk, D_v, K, scale,
                 dq, dkv, flags, ws, dsa::kNoAllocScratchBytes, false, DSA_ERR_INVALID_VALUE,
                 stream);
}

// ---------------------------------------------------------------------------------------
int dsa_sparse_mla_fwd_sink(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                            const int32_t *topk_length, int64_t T_q, int64_t T_kv, int32_t H,
                            int32_t D_qk, int32_t D_v, int32_t K, float scale, const float *sink,
                            uint16_t *out, float *lse, void *stream) {
  g_last_error.clear();
  if (T_q > 0 && !sink) return fail(DSA_ERR_INVALID_VALUE, "sparse_mla_fwd_sink: sink is NULL");
  if (!aligned16(out))
    return fail(DSA_ERR_INVALID_VALUE, "sparse_mla_fwd_sink: out must be 16-byte aligned");
  if (int rc = dsa_sparse_mla_fwd(q, kv, idx, topk_length, T_q, T_kv, H, D_qk, D_v, K, scale, out,
                                  lse, stream))
    return rc;
  hipError_t e = dsa::launch_sink_fwd(sink, T_q, H, D_v, out, lse,
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "sparse_mla_fwd_sink: launch");
  return DSA_OK;
}

int dsa_sparse_mla_bwd_sink(const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                            const int32_t *topk_length, const uint16_t *out, const float *lse,
                            const uint16_t *dout, int64_t T_q, int64_t T_kv, int32_t H,
                            int32_t D_qk, int32_t D_v, int32_t K, float scale, const float *sink,
                            uint16_t *dq, float *dkv, float *dsink, uint32_t flags, void *ws,
                            size_t ws_bytes, void *stream) {
  g_last_error.clear();
  if (!sink || !dsink)
    return fail(DSA_ERR_INVALID_VALUE, "sparse_mla_bwd_sink: sink and dsink must not be NULL");
  if (int rc = dsa_sparse_mla_bwd(q, kv, idx, topk_length, out, lse, dout, T_q, T_kv, H, D_qk,
                                  D_v, K, scale, dq, dkv, flags, ws, ws_bytes, stream))
    return rc;
  hipError_t e = dsa::launch_sink_bwd(sink, lse, out, dout, T_q, H, D_v, dsink,
                                      (flags & DSA_BWD_ACCUMULATE_DKV) != 0,
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "sparse_mla_bwd_sink: launch");
  return DSA_OK;
}

}  // extern "C"
