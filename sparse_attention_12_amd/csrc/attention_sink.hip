// Attention sink for sparse MLA (NeMo AutoModel cudnn_dsa API reference, _pad_attention_heads:
// a per-head sink [H] travels with the query heads; its arithmetic is not on the page).  The
// reading taken is one extra logit sink[h] per head whose value vector is zero, so it enters
// only the softmax denominator:
//   lse'[t,h] = log(exp(lse[t,h]) + exp(sink[h])),   out'[t,h,:] = out[t,h,:] exp(lse - lse'),
// where (out, lse) is the attention without the sink.  This is exact, so the sink is applied
// as an epilogue of the forward: one pass over the [T, H, D_v] output.
//
// Backward: P and Delta = dO . out' computed from the sink's (out', lse') already give dq and
// dkv (the sink's zero value adds nothing to dP); the sink's own logit gradient is
//   dsink[h] = -sum_t exp(sink[h] - lse'[t,h]) * Delta[t,h].
#include <math.h>

#include <algorithm>

#include "dsa_common.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kWaves = 4;
constexpr int kFwdRows = 4;  // (t, h) rows per wave in the forward epilogue

// logaddexp(a, b) in fp32 for a, b in [-inf, +inf) (both -inf: -inf).
__device__ __forceinline__ float log_add_exp(float a, float b) {
  const float m = fmaxf(a, b);
  if (m == -INFINITY) return -INFINITY;
  return m + log1pf(expf(-fabsf(a - b)));
}

// Rows of D_v = 512 bf16 outputs (one 16-byte piece per lane), kFwdRows consecutive (t, h)
// rows per wave: the wave loads all of its pieces first, then rescales and stores them in
// place; lane j < kFwdRows replaces lse of row j.
__global__ __launch_bounds__(64 * kWaves) void sink_fwd_kernel(const float *__restrict__ sink,
                                                               int64_t rows, int H,
                                                               uint16_t *__restrict__ out,
                                                               float *__restrict__ lse) {
  constexpr int Dv = 512;
  const int lane = threadIdx.x & 63;
  const int64_t r0 = (static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6)) * kFwdRows;
  if (r0 >= rows) return;
  const int n = static_cast<int>(min<int64_t>(kFwdRows, rows - r0));
  u32x4 v[kFwdRows];
  float f[kFwdRows];
#pragma unroll
  for (int j = 0; j < kFwdRows; ++j)
    if (j < n) v[j] = *reinterpret_cast<const u32x4 *>(out + (r0 + j) * Dv + lane * 8);
  float l2_mine = 0.0f;
#pragma unroll
  for (int j = 0; j < kFwdRows; ++j) {
    const float l = j < n ? lse[r0 + j] : 0.0f;
    const float l2 = log_add_exp(l, sink[(r0 + j) % H]);
    f[j] = l == -INFINITY ? 0.0f : expf(l - l2);  // empty row: the output stays 0
    if (lane == j) l2_mine = l2;
  }
#pragma unroll
  for (int j = 0; j < kFwdRows; ++j) {
    if (j >= n) break;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      v[j][w] = pack_bf16x2(__uint_as_float(v[j][w] << 16) * f[j],
                            __uint_as_float(v[j][w] & 0xFFFF0000u) * f[j]);
    *reinterpret_cast<u32x4 *>(out + (r0 + j) * Dv + lane * 8) = v[j];
  }
  if (lane < n) lse[r0 + lane] = l2_mine;
}

// dsink[h] += -sum_t exp(sink[h] - lse[t,h]) (dO[t,h] . out[t,h]): waves stride over the
// (t, h) rows and add their terms into per-head LDS sums; each block then adds its sums to
// dsink with one atomic per head (the result depends on the summation order only).
__global__ __launch_bounds__(64 * kWaves) void sink_bwd_kernel(const float *__restrict__ sink,
                                                               const float *__restrict__ lse,
                                                               const uint16_t *__restrict__ out,
                                                               const uint16_t *__restrict__ dout,
                                                               int64_t rows, int H,
                                                               float *__restrict__ dsink) {
  constexpr int Dv = 512;
  __shared__ float acc[64];
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 64) acc[threadIdx.x] = 0.0f;
  __syncthreads();
  // two rows per trip (D_v = 512: one 16-byte piece of out and of dout per lane and row),
  // their four loads issued together
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kWaves * 2;
  for (int64_t r = (static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6)) * 2; r < rows;
       r += stride) {
    const bool two = r + 1 < rows;
    const u32x4 o0 = *reinterpret_cast<const u32x4 *>(out + r * Dv + lane * 8);
    const u32x4 d0 = *reinterpret_cast<const u32x4 *>(dout + r * Dv + lane * 8);
    u32x4 o1 = {0u, 0u, 0u, 0u}, d1 = {0u, 0u, 0u, 0u};
    if (two) {
      o1 = *reinterpret_cast<const u32x4 *>(out + (r + 1) * Dv + lane * 8);
      d1 = *reinterpret_cast<const u32x4 *>(dout + (r + 1) * Dv + lane * 8);
    }
    float dot0 = 0.0f, dot1 = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      dot0 = fmaf(__uint_as_float(o0[w] << 16), __uint_as_float(d0[w] << 16), dot0);
      dot0 = fmaf(__uint_as_float(o0[w] & 0xFFFF0000u), __uint_as_float(d0[w] & 0xFFFF0000u),
                  dot0);
      dot1 = fmaf(__uint_as_float(o1[w] << 16), __uint_as_float(d1[w] << 16), dot1);
      dot1 = fmaf(__uint_as_float(o1[w] & 0xFFFF0000u), __uint_as_float(d1[w] & 0xFFFF0000u),
                  dot1);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      dot0 += __shfl_xor(dot0, off, 64);
      dot1 += __shfl_xor(dot1, off, 64);
    }
    if (lane < 2 && (lane == 0 || two)) {
      const int64_t rr = r + lane;
      const int h = static_cast<int>(rr % H);
      const float l = lse[rr];
      // lse = -inf only when the row is empty and the sink is -inf: no term
      const float p = l == -INFINITY ? 0.0f : expf(sink[h] - l);
      atomicAdd(&acc[h], -p * (lane == 0 ? dot0 : dot1));
    }
  }
  __syncthreads();
  if (threadIdx.x < H) atomicAdd(&dsink[threadIdx.x], acc[threadIdx.x]);
}

__global__ void sink_zero_kernel(float *__restrict__ p, int n) {
  if (static_cast<int>(threadIdx.x) < n) p[threadIdx.x] = 0.0f;
}

}  // namespace

hipError_t launch_sink_fwd(const float *sink, int64_t T_q, int32_t H, int32_t D_v,
                           uint16_t *out, float *lse, hipStream_t s) {
  if (D_v != 512) return hipErrorInvalidValue;
  const int64_t rows = T_q * H;
  if (rows == 0) return hipSuccess;
  const int64_t blocks = (rows + kWaves * kFwdRows - 1) / (kWaves * kFwdRows);
  DSA_LAUNCH("sink_fwd", sink_fwd_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(64 * kWaves),
             0, s, sink, rows, H, out, lse);
  return hipGetLastError();
}

hipError_t launch_sink_bwd(const float *sink, const float *lse, const uint16_t *out,
                           const uint16_t *dout, int64_t T_q, int32_t H, int32_t D_v,
                           float *dsink, bool accumulate, hipStream_t s) {
  if (D_v != 512) return hipErrorInvalidValue;
  if (!accumulate) DSA_LAUNCH("sink_zero", sink_zero_kernel, dim3(1), dim3(64), 0, s, dsink, H);
  const int64_t rows = T_q * H;
  if (rows > 0) {
    // enough blocks to keep HBM busy; each block then adds H partial sums
    const int64_t blocks = std::min<int64_t>((rows + 2 * kWaves - 1) / (2 * kWaves), 2048);
    DSA_LAUNCH("sink_bwd", sink_bwd_kernel, dim3(static_cast<uint32_t>(blocks)),
               dim3(64 * kWaves), 0, s, sink, lse, out, dout, rows, H, dsink);
  }
  return hipGetLastError();
}

}  // namespace dsa
