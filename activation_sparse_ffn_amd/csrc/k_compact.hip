// Threshold and compaction: active = score >= t per token, union over the batch,
// ascending index list of the union (PowerInfer page, Method, hybrid-execution
// pseudocode; Paper vs code, predictor threshold: a neuron whose score is below the
// threshold is skipped).
//
// One kernel.  Every workgroup takes 1024 neurons and turns them x B tokens into
// mask words with wave ballots (one 64-bit ballot = two 32-bit words = two groups
// of 32 neurons), ORing the tokens into the union words.  Its active count goes
// out as one word (count + 1, never zero); it reads the words of the workgroups
// before it (one batch of loads, re-polled while any is still zero) and every
// active neuron's thread writes it at prefix + rank, so the whole grid writes the
// list in rank order (the last workgroup writing the whole list alone, one
// scattered store per set bit, took 4-12 us).  Count words carry the call's epoch
// (a 16-bit call counter in the workspace) instead of being cleared: the last
// workgroup, which has seen every count and so knows every workgroup has read the
// counter, advances it.  (A closing ticket whose last taker cleared the words cost a
// store wait and an atomic round trip per call, about 2 us of the 8 at the OPT-30B
// shape.)  Nothing leaves the device.
// A workgroup waits only for workgroups of lower index, which publish before they
// wait themselves; workgroups are dispatched in index order, so those are running
// or done (the wait is bounded all the same).
#include "sfx_common.hpp"
#include "sfx_launch.hpp"

namespace sfx {
namespace {

constexpr int kT = 1024;
constexpr int kWaves = kT / kWave;
constexpr int kSpin = 1 << 20;

__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ctl: [0] epoch of the last call (16 bits), [1] error (nonzero: a count word did
// not arrive in time); cnt: one word per workgroup, epoch << 16 | (count + 1).
__global__ __launch_bounds__(kT) void k_compact(const float* __restrict__ scores, int B, int f, float t,
                                                uint32_t* __restrict__ tok_bits, uint32_t* __restrict__ union_bits,
                                                int32_t* __restrict__ idx, int32_t* __restrict__ count,
                                                uint32_t* __restrict__ ctl, uint32_t* __restrict__ cnt) {
  __shared__ uint32_t s_wc[kWaves];
  __shared__ uint32_t s_red[kWaves];
  const int W = (f + 31) >> 5;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int n = blockIdx.x * kT + threadIdx.x;
  const int w0 = n >> 5;  // lanes 0 and 32 own words w0
  const uint32_t ep = (ld_agent(ctl) + 1u) & 0xffffu;   // this call's epoch
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
  if ((lane == 0 || lane == 32) && w0 < W) union_bits[w0] = (uint32_t)(lane == 0 ? uni : (uni >> 32));

  // This workgroup's count and this wave's offset within it.
  if (lane == 0) s_wc[wave] = (uint32_t)__popcll(uni);
  __syncthreads();
  uint32_t woff = 0, btot = 0;
#pragma unroll
  for (int v = 0; v < kWaves; ++v) {
    const uint32_t c = s_wc[v];
    btot += c;
    woff += v < wave ? c : 0u;
  }
  if (threadIdx.x == 0) store_through(cnt + blockIdx.x, (ep << 16) | (btot + 1u));

  // Counts of the workgroups before this one: thread j reads workgroup j's word.
  uint32_t part = 0;
  for (int j0 = 0; j0 < (int)blockIdx.x; j0 += kT) {
    const int j = j0 + (int)threadIdx.x;
    const bool mine = j < (int)blockIdx.x;
    uint32_t c = ld_agent(cnt + (mine ? j : 0));
    for (int spins = 0; mine && (c >> 16) != ep; ++spins) {
      if (spins > kSpin) {
        store_through(ctl + 1, 1u);
        break;
      }
      c = ld_agent(cnt + j);
    }
    if (mine && (c >> 16) == ep) part += (c & 0xffffu) - 1u;
  }
  part = (uint32_t)wave_sum_i32((int)part, lane);
  if (lane == 0) s_red[wave] = part;
  __syncthreads();
  uint32_t prefix = 0;
#pragma unroll
  for (int v = 0; v < kWaves; ++v) prefix += s_red[v];

  if ((uni >> lane) & 1ull) {
    const uint32_t below = (uint32_t)__popcll(uni & ((1ull << lane) - 1ull));
    idx[prefix + woff + below] = n;
  }
  // the last workgroup: every count seen (the __syncthreads above ended its polls),
  // so every workgroup has read the epoch; the next call takes the next one
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) {
    *count = (int32_t)(prefix + btot);
    store_through(ctl, ep);
  }
}

size_t cnt_offset() { return 256; }

}  // namespace

// control words | one count word per workgroup of 1024 neurons
size_t compact_ws_bytes(int B, int f) {
  (void)B;
  const size_t blocks = ((size_t)f + kT - 1) / kT;
  return cnt_offset() + ((blocks * 4 + 255) & ~(size_t)255);
}

hipError_t launch_compact(hipStream_t s, int B, int f, const float* scores, float t, uint32_t* tok_bits,
                          uint32_t* union_bits, int32_t* idx, int kmax, int32_t* count, void* ws) {
  (void)kmax;
  const int blocks = (f + kT - 1) / kT;
  uint32_t* ctl = (uint32_t*)ws;
  uint32_t* cnt = (uint32_t*)((uint8_t*)ws + cnt_offset());
  k_compact<<<dim3(blocks), dim3(kT), 0, s>>>(scores, B, f, t, tok_bits, union_bits, idx, count, ctl, cnt);
  return hipGetLastError();
}

}  // namespace sfx
