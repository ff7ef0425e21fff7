// Gather ceiling of the latent-row tiles.  Not a step of the method: a measurement of the memory
// path that the attention kernels' gathers take (the pages' forward and backward read one
// latent row per valid top-k slot, NVIDIA GLM-5.2 cuDNN DSA page, "Why DSA needs fused
// kernels").  A work group streams kProbeRows listed rows of a latent table through LDS in
// tiles of 32 rows with the same direct 16-byte global->LDS loads, tile layout and buffering
// as the attention kernels (TileStream, three tiles in flight), and does nothing with them but
// fold one 16-byte piece per lane and tile into a checksum, so that its time is the time of
// the gathers alone.
#include "dsa_common.h"
#include "dsa_internal.h"
#include "tile.h"

namespace dsa {
namespace {

constexpr int kProbeWaves = 4;
constexpr int kProbeNBuf = 4;

template <int DQK>
__global__ __launch_bounds__(kProbeWaves * 64) void gather_probe_kernel(
    const uint16_t *__restrict__ table, const int32_t *__restrict__ idx, int64_t n,
    uint32_t *__restrict__ sink) {
  using TL = Tile<DQK>;
  using TS = TileStream<DQK, kProbeWaves, kProbeNBuf>;
  extern __shared__ __align__(16) unsigned char smem[];
  int32_t *slot_rows = reinterpret_cast<int32_t *>(smem + kProbeNBuf * TL::kBytes);
  __shared__ uint32_t part[kProbeWaves];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t b = static_cast<int64_t>(blockIdx.x) * kGatherProbeRows;
  const int cnt = static_cast<int>(n - b < kGatherProbeRows ? n - b : kGatherProbeRows);
  const int nch = (cnt + TL::kSlots - 1) / TL::kSlots;
  for (int j = threadIdx.x; j < nch * TL::kSlots; j += kProbeWaves * 64)
    slot_rows[j] = j < cnt ? idx[b + j] : -1;  // -1: row 0 is loaded
  __syncthreads();
  TS ts;
  ts.init(smem, wave);
  for (int c = 0; c < kProbeNBuf - 1; ++c)
    if (c < nch) ts.issue(c, table, slot_rows);
  uint32_t x = 0u;
  for (int c = 0; c < nch; ++c) {
    TS::acquire(c, nch);  // tile c complete; every wave is done with tile c - 1
    if (c + kProbeNBuf - 1 < nch) ts.issue(c + kProbeNBuf - 1, table, slot_rows);
    const u32x4 v = *reinterpret_cast<const u32x4 *>(smem + (c % kProbeNBuf) * TL::kBytes +
                                                     threadIdx.x * 16);
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), off, 64));
  if (lane == 0) part[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

template <int DQK>
hipError_t launch(const uint16_t *table, const int32_t *idx, int64_t n, uint32_t *sink,
                  hipStream_t s) {
  const size_t smem = static_cast<size_t>(kProbeNBuf) * Tile<DQK>::kBytes +
                      kGatherProbeRows * sizeof(int32_t);
  auto kern = gather_probe_kernel<DQK>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(smem));
  if (e != hipSuccess) return e;
  const int64_t groups = (n + kGatherProbeRows - 1) / kGatherProbeRows;
  DSA_LAUNCH("gather_probe", kern, dim3(static_cast<unsigned>(groups)), dim3(kProbeWaves * 64),
             smem, s, table, idx, n, sink);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gather_probe(const uint16_t *table, int32_t width, const int32_t *idx,
                               int64_t n, uint32_t *sink, hipStream_t s) {
  if (n == 0) return hipSuccess;
  return width == 576 ? launch<576>(table, idx, n, sink, s) : launch<512>(table, idx, n, sink, s);
}

}  // namespace dsa
