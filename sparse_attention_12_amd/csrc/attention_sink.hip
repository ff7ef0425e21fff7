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

constexpr int kWaves = 4;  // one (t, h) row per wave

// logaddexp(a, b) in fp32 for a, b in [-inf, +inf) (both -inf: -inf).
__device__ __forceinline__ float log_add_exp(float a, float b) {
  const float m = fmaxf(a, b);
  if (m == -INFINITY) return -INFINITY;
  return m + log1pf(expf(-fabsf(a - b)));
}

// Rows of D_v bf16 outputs, one wave per (t, h) row: each lane rescales 16-byte pieces in
// place; lane 0 replaces lse.
__global__ __launch_bounds__(64 * kWaves) void sink_fwd_kernel(const float *__restrict__ sink,
                                                               int64_t rows, int H, int Dv,
                                                               uint16_t *__restrict__ out,
                                                               float *__restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int h = static_cast<int>(r % H);
  const float l = lse[r];
  const float l2 = log_add_exp(l, sink[h]);
  const float f = l == -INFINITY ? 0.0f : expf(l - l2);  // empty row: the output stays 0
  uint16_t *o = out + r * Dv;
  for (int c = lane * 8; c < Dv; c += 64 * 8) {
    u32x4 v = *reinterpret_cast<const u32x4 *>(o + c);
#pragma unroll
    for (int w = 0; w < 4; ++w)
      v[w] = pack_bf16x2(__uint_as_float(v[w] << 16) * f,
                         __uint_as_float(v[w] & 0xFFFF0000u) * f);
    *reinterpret_cast<u32x4 *>(o + c) = v;
  }
  if (lane == 0) lse[r] = l2;
}

// dsink[h] += -sum_t exp(sink[h] - lse[t,h]) (dO[t,h] . out[t,h]): waves stride over the
// (t, h) rows and add their terms into per-head LDS sums; each block then adds its sums to
// dsink with one atomic per head (the result depends on the summation order only).
__global__ __launch_bounds__(64 * kWaves) void sink_bwd_kernel(const float *__restrict__ sink,
                                                               const float *__restrict__ lse,
                                                               const uint16_t *__restrict__ out,
                                                               const uint16_t *__restrict__ dout,
                                                               int64_t rows, int H, int Dv,
                                                               float *__restrict__ dsink) {
  __shared__ float acc[64];
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 64) acc[threadIdx.x] = 0.0f;
  __syncthreads();
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kWaves;
  for (int64_t r = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6); r < rows;
       r += stride) {
    const uint16_t *o = out + r * Dv;
    const uint16_t *d = dout + r * Dv;
    float dot = 0.0f;
    for (int c = lane * 8; c < Dv; c += 64 * 8) {
      const u32x4 ov = *reinterpret_cast<const u32x4 *>(o + c);
      const u32x4 dv = *reinterpret_cast<const u32x4 *>(d + c);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        dot = fmaf(__uint_as_float(ov[w] << 16), __uint_as_float(dv[w] << 16), dot);
        dot = fmaf(__uint_as_float(ov[w] & 0xFFFF0000u), __uint_as_float(dv[w] & 0xFFFF0000u),
                   dot);
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) dot += __shfl_xor(dot, off, 64);
    if (lane == 0) {
      const int h = static_cast<int>(r % H);
      const float l = lse[r];
      // lse = -inf only when the row is empty and the sink is -inf: no term
      const float p = l == -INFINITY ? 0.0f : expf(sink[h] - l);
      atomicAdd(&acc[h], -p * dot);
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
  const int64_t rows = T_q * H;
  if (rows == 0) return hipSuccess;
  const int64_t blocks = (rows + kWaves - 1) / kWaves;
  DSA_LAUNCH("sink_fwd", sink_fwd_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(64 * kWaves),
             0, s, sink, rows, H, D_v, out, lse);
  return hipGetLastError();
}

hipError_t launch_sink_bwd(const float *sink, const float *lse, const uint16_t *out,
                           const uint16_t *dout, int64_t T_q, int32_t H, int32_t D_v,
                           float *dsink, bool accumulate, hipStream_t s) {
  if (!accumulate) DSA_LAUNCH("sink_zero", sink_zero_kernel, dim3(1), dim3(64), 0, s, dsink, H);
  const int64_t rows = T_q * H;
  if (rows > 0) {
    // enough blocks to keep HBM busy; each block then adds H partial sums
    const int64_t blocks = std::min<int64_t>((rows + kWaves - 1) / kWaves, 2048);
    DSA_LAUNCH("sink_bwd", sink_bwd_kernel, dim3(static_cast<uint32_t>(blocks)),
               dim3(64 * kWaves), 0, s, sink, lse, out, dout, rows, H, D_v, dsink);
  }
  return hipGetLastError();
}

}  // namespace dsa
