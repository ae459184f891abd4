// Dense FFN step on the sparse kernels (PowerInfer page, Implementation: long
// inputs switch to dense GPU computation in the prefill stage; KAIROX page, Future
// work: choosing sparse or dense kernels online from the batch).  Every neuron is
// listed, so the gathered up and down kernels stream every row: the same products,
// activations and fixed-order sums as the sparse step with an all-ones mask, and no
// predictor.
#include "sfx_common.hpp"
#include "sfx_launch.hpp"

namespace sfx {
namespace {

__global__ __launch_bounds__(kBlock) void k_iota(int32_t* __restrict__ idx, int32_t* __restrict__ count, int f) {
  const int i = blockIdx.x * kBlock + threadIdx.x;
  if (i < f) idx[i] = i;
  if (i == 0) count[0] = f;
}

size_t up256(size_t n) { return (n + 255) & ~(size_t)255; }

}  // namespace

// Workspace: identity list [f] | count | the down kernel's workspace.
size_t dense_ws_bytes(int wdt, int B, int d, int f) {
  return up256((size_t)f * 4) + 256 + down_ws_bytes(wdt, B, d, f);
}

hipError_t launch_dense(hipStream_t s, int wdt, int act, int B, int d, int f, const void* x, const void* Wa,
                        const void* Wa_s, const float* ba, const void* Wl, const void* Wl_s, const void* Wd,
                        const void* Wd_s, float* hact, float* y, void* ws) {
  uint8_t* base = (uint8_t*)ws;
  int32_t* idx = (int32_t*)base;
  int32_t* count = (int32_t*)(base + up256((size_t)f * 4));
  void* dws = base + up256((size_t)f * 4) + 256;
  k_iota<<<dim3((f + kBlock - 1) / kBlock), dim3(kBlock), 0, s>>>(idx, count, f);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_up(s, wdt, act, B, d, f, x, Wa, Wa_s, ba, Wl, Wl_s, idx, count, f, hact);
  if (e != hipSuccess) return e;
  return launch_down(s, wdt, B, d, f, Wd, Wd_s, idx, count, f, hact, y, dws);
}

}  // namespace sfx
