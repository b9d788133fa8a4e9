// Read-only HBM probes: the practical read ceiling that the decode kernels are
// compared with.  Pattern 0 streams a buffer contiguously; pattern 1 reads
// whole 4 KiB tiles in a caller-given order, the access pattern of a paged
// K/V cache whose (page, head) tiles are scattered over the pool.  Both use
// non-temporal loads, as the decode kernels do for their once-read K/V.
// Pattern 2 reads 2 KiB tiles: the (page, head) tile of 8-bit K or V at
// head_dim 128.
// Every load's data feeds a data-dependent store, so no load can be removed.
#include "attn_internal.h"
#include "common.h"

namespace pa {

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeWgPerCu = 2;   // the best of 1-16 in a sweep on MI355X, for both patterns
constexpr uint32_t kNever = 0x9E3779B9u;   // a sum the data would have to hit exactly

__global__ __launch_bounds__(kProbeThreads) void probe_contig(const u32x4 *src, size_t n16,
                                                              uint32_t *sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 v0 = ld16_nt(src + i), v1 = ld16_nt(src + i + stride);
    const u32x4 v2 = ld16_nt(src + i + 2 * stride), v3 = ld16_nt(src + i + 3 * stride);
    acc ^= v0 ^ v1 ^ v2 ^ v3;
  }
  for (; i < n16; i += stride) acc ^= ld16_nt(src + i);
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == kNever) *sink = x;
}

// one wave per tile of TILE bytes (TILE / 1 KiB instructions of 64 lanes x
// 16 B), four tiles in flight
template <int TILE>
__global__ __launch_bounds__(kProbeThreads) void probe_tiles(const char *pool, const int32_t *order,
                                                             int ntiles, uint32_t *sink) {
  constexpr int kDepth = 4;
  constexpr int NC = TILE / 1024;
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int nwaves = (gridDim.x * blockDim.x) >> 6;
  u32x4 acc = {0u, 0u, 0u, 0u};
  int t = wave;
  for (; t + (kDepth - 1) * nwaves < ntiles; t += kDepth * nwaves) {
    u32x4 v[kDepth][NC];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      const char *a = pool + (size_t)order[t + d * nwaves] * TILE + lane * 16;
#pragma unroll
      for (int c = 0; c < NC; ++c) v[d][c] = ld16_nt(a + c * 1024);
    }
#pragma unroll
    for (int d = 0; d < kDepth; ++d)
#pragma unroll
      for (int c = 0; c < NC; ++c) acc ^= v[d][c];
  }
  for (; t < ntiles; t += nwaves) {
    const char *a = pool + (size_t)order[t] * TILE + lane * 16;
#pragma unroll
    for (int c = 0; c < NC; ++c) acc ^= ld16_nt(a + c * 1024);
  }
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == kNever) *sink = x;
}

}  // namespace

hipError_t launch_read_probe(const void *buf, size_t bytes, int pattern, const int32_t *order,
                             uint32_t *sink, int num_cus, hipStream_t s) {
  const dim3 grid(num_cus * kProbeWgPerCu), block(kProbeThreads);
  if (pattern == 0)
    hipLaunchKernelGGL(probe_contig, grid, block, 0, s, reinterpret_cast<const u32x4 *>(buf),
                       bytes / 16, sink);
  else if (pattern == 1)
    hipLaunchKernelGGL(probe_tiles<4096>, grid, block, 0, s, reinterpret_cast<const char *>(buf),
                       order, (int)(bytes / 4096), sink);
  else
    hipLaunchKernelGGL(probe_tiles<2048>, grid, block, 0, s, reinterpret_cast<const char *>(buf),
                       order, (int)(bytes / 2048), sink);
  return hipGetLastError();
}

}  // namespace pa
