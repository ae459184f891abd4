// Temporal activation momentum over groups of 32 neurons (KAIROX page, Core method:
// item 3, decisions per group with at most 1024 groups per layer so that a GPU
// sort stays cheap; item 4, the TAM score, accumulated when the group is active
// and decayed by lambda when not, candidates above tau = (1 - lambda) + eps, the
// best candidates fill the capacity; item 6, entering / leaving sets by XOR/AND).
//
// One 1024-thread workgroup per layer: thread g updates group g's score, builds a
// 64-bit key (score bits << 32 | ~g) for candidates (score >= 0, so the bits order
// like the values), a bitonic sort ranks the keys (score descending, then group id
// ascending; in-wave stages on registers, wider ones in LDS), and the first
// min(K, #candidates) become the hot set.
//
// The same ranking also serves a reload rule without memory (the Top-K reload the
// KAIROX page compares TAM with, Experiments: strategies and ablations): the key is
// the number of the group's neurons active in this step's union mask, every group
// with at least one is a candidate, and no score is kept.
#include "sfx_common.hpp"
#include "sfx_launch.hpp"

namespace sfx {
namespace {

constexpr int kT = 1024;

template <bool kNow>
__global__ __launch_bounds__(kT) void k_tam(int G, const uint32_t* __restrict__ union_bits, float lambda,
                                            float tau, int K, float* __restrict__ score,
                                            uint32_t* __restrict__ hot_bits, uint32_t* __restrict__ entered,
                                            uint32_t* __restrict__ left, int32_t* __restrict__ topk,
                                            int32_t* __restrict__ topk_count) {
  __shared__ unsigned long long s_key[kT];
  __shared__ uint32_t s_hot[kT / 32];
  const int l = blockIdx.x;
  const int g = threadIdx.x;
  const int HW = (G + 31) >> 5;
  const float one_minus = 1.0f - lambda;

  unsigned long long key = 0ull;
  int cand = 0;
  if (g < G && kNow) {
    const uint32_t n = (uint32_t)__popc(union_bits[(size_t)l * G + g]);
    if (n > 0u) {
      cand = 1;
      key = ((unsigned long long)n << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)g);
    }
  } else if (g < G) {
    const float a = union_bits[(size_t)l * G + g] != 0u ? 1.0f : 0.0f;
    float s = score[(size_t)l * G + g];
    s = fmaf(lambda, s, one_minus * a);
    score[(size_t)l * G + g] = s;
    if (s > tau) {
      cand = 1;
      key = ((unsigned long long)__float_as_uint(s) << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)g);
    }
  }
  if (g < kT / 32) s_hot[g] = 0u;
  const int ncand = __syncthreads_count(cand);

  // Bitonic sort of the first NP >= G keys, descending.  Exchanges between lanes
  // of one wave (distance < 64) run on registers with shuffles; only the wider
  // distances go through LDS, one barrier each.
  int NP = 1;
  while (NP < G) NP <<= 1;
  for (int k = 2; k <= NP; k <<= 1) {
    const bool desc = (g & k) == 0;
    int j = k >> 1;
    if (j >= kWave) {
      s_key[g] = key;
      __syncthreads();
      for (; j >= kWave; j >>= 1) {
        const int p = g ^ j;
        if (p > g) {
          const unsigned long long a = s_key[g], b = s_key[p];
          if (desc ? (a < b) : (a > b)) {
            s_key[g] = b;
            s_key[p] = a;
          }
        }
        __syncthreads();
      }
      key = s_key[g];
    }
    for (; j > 0; j >>= 1) {
      const uint32_t lo = __shfl_xor((uint32_t)key, j, kWave);
      const uint32_t hi = __shfl_xor((uint32_t)(key >> 32), j, kWave);
      const unsigned long long b = ((unsigned long long)hi << 32) | lo;
      const bool lower = (g & j) == 0;        // lower index keeps the larger key when descending
      key = (lower == desc) ? (key > b ? key : b) : (key < b ? key : b);
    }
  }
  s_key[g] = key;
  __syncthreads();

  const int kk = ncand < K ? ncand : K;
  if (g < K) {
    int32_t id = -1;
    if (g < kk) {
      id = (int32_t)(0xFFFFFFFFu - (uint32_t)(s_key[g] & 0xFFFFFFFFull));
      atomicOr(&s_hot[id >> 5], 1u << (id & 31));
    }
    topk[(size_t)l * K + g] = id;
  }
  __syncthreads();
  if (g < HW) {
    const uint32_t now = s_hot[g];
    const uint32_t prev = hot_bits[(size_t)l * HW + g];
    entered[(size_t)l * HW + g] = now & ~prev;
    left[(size_t)l * HW + g] = prev & ~now;
    hot_bits[(size_t)l * HW + g] = now;
  }
  if (g == 0) topk_count[l] = kk;
}

}  // namespace

size_t tam_ws_bytes(int G, int K) {
  (void)G; (void)K;
  return 0;
}

hipError_t launch_tam(hipStream_t s, int L, int G, const uint32_t* union_bits, float lambda, float eps,
                      int K, float* score, uint32_t* hot_bits, uint32_t* entered, uint32_t* left,
                      int32_t* topk, int32_t* topk_count) {
  const float tau = (1.0f - lambda) + eps;
  k_tam<false><<<dim3(L), dim3(kT), 0, s>>>(G, union_bits, lambda, tau, K, score, hot_bits, entered, left, topk,
                                            topk_count);
  return hipGetLastError();
}

hipError_t launch_topk_now(hipStream_t s, int L, int G, const uint32_t* union_bits, int K, uint32_t* hot_bits,
                           uint32_t* entered, uint32_t* left, int32_t* topk, int32_t* topk_count) {
  k_tam<true><<<dim3(L), dim3(kT), 0, s>>>(G, union_bits, 0.f, 0.f, K, nullptr, hot_bits, entered, left, topk,
                                           topk_count);
  return hipGetLastError();
}

}  // namespace sfx
