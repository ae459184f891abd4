// Streaming-read probe: reads a buffer once with 16-byte loads, 8 in flight per
// thread, and folds it into per-workgroup checksums.  A measurement helper, not a
// step of the method: its bandwidth is the ceiling the step kernels' achieved HBM
// bandwidth is compared with (PowerInfer page, Problem: batch-1 decode is bound by
// reading the weights).
#include "sfx_common.hpp"
#include "sfx_launch.hpp"

namespace sfx {
namespace {

constexpr int kProbeThreads = 512;
constexpr int kProbeBlocks = 2048;
constexpr int kProbeU = 8;

__global__ __launch_bounds__(kProbeThreads) void k_stream_read(const uint8_t* __restrict__ buf, size_t n16,
                                                               uint32_t* __restrict__ out) {
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  uint32_t acc = 0;
  for (size_t i0 = (size_t)blockIdx.x * kProbeThreads + threadIdx.x; i0 < n16; i0 += stride * kProbeU) {
    Raw<16> v[kProbeU];
#pragma unroll
    for (int u = 0; u < kProbeU; ++u) {
      const size_t i = i0 + (size_t)u * stride;
      v[u] = load_raw<16>(buf + (i < n16 ? i : n16 - 1) * 16);
    }
#pragma unroll
    for (int u = 0; u < kProbeU; ++u) acc ^= v[u].w[0] ^ v[u].w[1] ^ v[u].w[2] ^ v[u].w[3];
  }
  for (int o = kWave / 2; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, kWave);
  if ((threadIdx.x & (kWave - 1)) == 0) out[(size_t)blockIdx.x * (kProbeThreads / kWave) + (threadIdx.x >> 6)] = acc;
}

}  // namespace

size_t stream_read_out_words() { return (size_t)kProbeBlocks * (kProbeThreads / kWave); }

hipError_t launch_stream_read(hipStream_t s, const void* buf, size_t nbytes, uint32_t* out) {
  k_stream_read<<<dim3(kProbeBlocks), dim3(kProbeThreads), 0, s>>>((const uint8_t*)buf, nbytes / 16, out);
  return hipGetLastError();
}

}  // namespace sfx
