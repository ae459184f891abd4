// Threshold and compaction: active = score >= t per token, union over the batch,
// ascending index list of the union (PowerInfer page, Method, hybrid-execution
// pseudocode; Paper vs code, predictor threshold: a neuron whose score is below the
// threshold is skipped).
//
// One kernel.  Every workgroup turns 1024 neurons x B tokens into mask words with
// wave ballots (one 64-bit ballot = two 32-bit words = two groups of 32 neurons)
// and ORs the tokens into the union word, which it writes through to the
// coherence point.  The last workgroup to take a ticket prefix-sums the popcounts
// of all union words and writes the index list and the count.  Nothing leaves the
// device.
#include "sfx_common.hpp"
#include "sfx_launch.hpp"

namespace sfx {
namespace {

constexpr int kT = 1024;
constexpr int kWaves = kT / kWave;

// Exclusive prefix sum of one value per thread over a 1024-thread block; also
// returns the block total.  Wave-level shuffle scan, then a scan of the 16 wave
// totals.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_tot, uint32_t& total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  uint32_t inc = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t n = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += n;
  }
  if (lane == kWave - 1) s_tot[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    uint32_t t = lane < kWaves ? s_tot[lane] : 0u;
#pragma unroll
    for (int o = 1; o < kWaves; o <<= 1) {
      const uint32_t n = __shfl_up(t, o, kWave);
      if (lane >= o) t += n;
    }
    if (lane < kWaves) s_tot[kWaves + lane] = t;   // inclusive wave prefix
  }
  __syncthreads();
  total = s_tot[2 * kWaves - 1];
  const uint32_t before = wave > 0 ? s_tot[kWaves + wave - 1] : 0u;
  return before + inc - v;
}

__global__ __launch_bounds__(kT) void k_compact(const float* __restrict__ scores, int B, int f, float t,
                                                uint32_t* __restrict__ tok_bits, uint32_t* __restrict__ union_bits,
                                                int32_t* __restrict__ idx, int32_t* __restrict__ count,
                                                uint32_t* __restrict__ ticket) {
  __shared__ uint32_t s_tot[2 * kWaves];
  __shared__ int s_last;
  const int W = (f + 31) >> 5;
  const int lane = threadIdx.x & (kWave - 1);
  const int n = blockIdx.x * kT + threadIdx.x;
  const int w0 = n >> 5;  // lanes 0 and 32 own words w0
  uint64_t uni = 0;
  const int nc = min(n, f - 1);
  for (int b0 = 0; b0 < B; b0 += 8) {
    float v[8];   // eight tokens' scores in flight together (clamped, not branched on)
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = scores[(size_t)min(b0 + q, B - 1) * f + nc];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (b0 + q < B) {
        const bool m = (n < f) && (v[q] >= t);  // NaN compares false
        const uint64_t bal = __ballot(m);
        uni |= bal;
        if (tok_bits != nullptr && (lane == 0 || lane == 32) && w0 < W)
          tok_bits[(size_t)(b0 + q) * W + w0] = (uint32_t)(lane == 0 ? bal : (bal >> 32));
      }
    }
  }
  if ((lane == 0 || lane == 32) && w0 < W) store_through(union_bits + w0, (uint32_t)(lane == 0 ? uni : (uni >> 32)));

  wait_memory();
  __syncthreads();
  if (threadIdx.x == 0) s_last = (take_ticket(ticket) == gridDim.x - 1);
  __syncthreads();
  if (!s_last) return;
  acquire_agent();

  // Last workgroup: exclusive scan of popcounts over all W words, `per`
  // consecutive words per thread.
  const int per = (W + kT - 1) / kT;
  const int wb = threadIdx.x * per;
  uint32_t cnt = 0;
  for (int i = 0; i < per; ++i)
    if (wb + i < W) cnt += __popc(union_bits[wb + i]);
  uint32_t total;
  uint32_t pos = block_exclusive_scan(cnt, s_tot, total);
  for (int i = 0; i < per; ++i) {
    if (wb + i >= W) break;
    uint32_t word = union_bits[wb + i];
    while (word) {
      idx[pos++] = ((wb + i) << 5) + __builtin_ctz(word);
      word &= word - 1;
    }
  }
  if (threadIdx.x == 0) {
    *count = (int32_t)total;
    *ticket = 0u;  // ready for the next call
  }
}

}  // namespace

size_t compact_ws_bytes(int B, int f) {
  (void)B; (void)f;
  return 256;
}

hipError_t launch_compact(hipStream_t s, int B, int f, const float* scores, float t, uint32_t* tok_bits,
                          uint32_t* union_bits, int32_t* idx, int kmax, int32_t* count, void* ws) {
  (void)kmax;
  const int blocks = (f + kT - 1) / kT;
  k_compact<<<dim3(blocks), dim3(kT), 0, s>>>(scores, B, f, t, tok_bits, union_bits, idx, count, (uint32_t*)ws);
  return hipGetLastError();
}

}  // namespace sfx
