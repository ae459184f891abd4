// Threshold and compaction: active = score >= t per token, union over the batch,
// ascending index list of the union (PowerInfer page, Method, hybrid-execution
// pseudocode; Paper vs code, predictor threshold: a neuron whose score is below the
// threshold is skipped).
//
// One kernel.  Every workgroup turns 256 neurons x B tokens into mask words with
// wave ballots (one 64-bit ballot = two 32-bit words = two groups of 32 neurons)
// and ORs the tokens into the union word.  The last workgroup to finish (a ticket
// in the workspace) prefix-sums the popcounts of all union words and writes the
// index list and the count.  Nothing leaves the device.
#include "sfx_common.hpp"
#include "sfx_launch.hpp"

namespace sfx {
namespace {

constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void k_compact(const float* __restrict__ scores, int B, int f,
                                                          float t, uint32_t* __restrict__ tok_bits,
                                                          uint32_t* __restrict__ union_bits,
                                                          int32_t* __restrict__ idx,
                                                          int32_t* __restrict__ count,
                                                          uint32_t* __restrict__ ticket) {
  __shared__ uint32_t s_pref[kScanThreads];
  __shared__ int s_last;
  const int W = (f + 31) >> 5;
  const int lane = threadIdx.x & (kWave - 1);
  const int n = blockIdx.x * kScanThreads + threadIdx.x;
  const int w0 = n >> 5;  // word of this lane's neuron; lanes 0 and 32 write words w0
  uint64_t uni = 0;
  for (int b = 0; b < B; ++b) {
    const bool m = (n < f) && (scores[(size_t)b * f + n] >= t);  // NaN compares false
    const uint64_t bal = __ballot(m);
    uni |= bal;
    if (tok_bits != nullptr && (lane == 0 || lane == 32) && w0 < W)
      tok_bits[(size_t)b * W + w0] = (uint32_t)(lane == 0 ? bal : (bal >> 32));
  }
  if ((lane == 0 || lane == 32) && w0 < W) union_bits[w0] = (uint32_t)(lane == 0 ? uni : (uni >> 32));

  // Publish the union words, then take a ticket.
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = atomicAdd(ticket, 1u);
    s_last = (prev == gridDim.x - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  // Last workgroup: exclusive scan of popcounts over all W words.
  const int per = (W + kScanThreads - 1) / kScanThreads;  // words per thread
  const int wb = threadIdx.x * per;
  uint32_t cnt = 0;
  for (int i = 0; i < per; ++i)
    if (wb + i < W) cnt += __popc(__hip_atomic_load(union_bits + wb + i, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT));
  s_pref[threadIdx.x] = cnt;
  __syncthreads();
  // Hillis-Steele inclusive scan in LDS.
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const uint32_t v = threadIdx.x >= off ? s_pref[threadIdx.x - off] : 0u;
    __syncthreads();
    s_pref[threadIdx.x] += v;
    __syncthreads();
  }
  uint32_t pos = s_pref[threadIdx.x] - cnt;
  for (int i = 0; i < per; ++i) {
    if (wb + i >= W) break;
    uint32_t word = __hip_atomic_load(union_bits + wb + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    while (word) {
      const int bit = __builtin_ctz(word);
      idx[pos++] = ((wb + i) << 5) + bit;
      word &= word - 1;
    }
  }
  if (threadIdx.x == kScanThreads - 1) {
    *count = (int32_t)s_pref[kScanThreads - 1];
    *ticket = 0u;  // ready for the next call
  }
}

}  // namespace

size_t compact_ws_bytes(int B, int f) {
  (void)B; (void)f;
  return 256;
}

hipError_t launch_compact(hipStream_t s, int B, int f, const float* scores, float t,
                          uint32_t* tok_bits, uint32_t* union_bits, int32_t* idx, int kmax,
                          int32_t* count, void* ws) {
  (void)kmax;
  const int blocks = (f + kScanThreads - 1) / kScanThreads;
  k_compact<<<dim3(blocks), dim3(kScanThreads), 0, s>>>(scores, B, f, t, tok_bits, union_bits, idx,
                                                        count, (uint32_t*)ws);
  return hipGetLastError();
}

}  // namespace sfx
