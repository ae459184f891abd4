// Offline calibration of a layer (PowerInfer page, Method: offline profiling counts
// how often each neuron is active on calibration inputs, and the neuron table maps
// the stored order to the model's; KAIROX page, Core method, item 1: co-active
// neurons are reordered into contiguous groups; per-layer threshold of the
// predictor: Paper vs code, predictor threshold).  Nothing here runs in the
// decode step; the step reads the thresholds and the reordered weights.
//
//   k_count_active   counts[i] += number of tokens whose mask holds neuron i
//   k_sel_*          exact k-th smallest of n fp32 values (radix select on the
//                    order-preserving 32-bit key, 8 bits per pass, four passes)
//   k_group_sum + k_rank   hot-first order: rank of every neuron under
//                    (group count desc, group id asc, neuron count desc, slot asc)
//   k_gather_rows    dst row r = src row idx[r] (applies the order to a matrix)
#include "sfx_common.hpp"
#include "sfx_launch.hpp"

namespace sfx {
namespace {

constexpr int kCB = 256;

__global__ __launch_bounds__(kCB) void k_count_active(int B, int f, const uint32_t* __restrict__ tok_bits,
                                                      int32_t* __restrict__ counts) {
  const int i = blockIdx.x * kCB + threadIdx.x;
  if (i >= f) return;
  const int W = (f + 31) >> 5;
  int c = 0;
  for (int b = 0; b < B; ++b) c += (int)((tok_bits[(size_t)b * W + (i >> 5)] >> (i & 31)) & 1u);
  counts[i] += c;
}

// ---------------------------------------------------------------- radix select
// Key: sign bit clear (>= +0) -> bits | 0x80000000, else ~bits, so keys order like
// the values (with -0 below +0).  State words: [0] prefix, [1] mask, [2] rank still
// to skip inside the prefix; histogram at word 64.
constexpr int kSelHist = 64;

__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__global__ __launch_bounds__(kCB) void k_sel_init(uint32_t* __restrict__ ws, uint32_t k) {
  const int t = threadIdx.x;
  ws[kSelHist + t] = 0u;
  if (t == 0) {
    ws[0] = 0u;
    ws[1] = 0u;
    ws[2] = k;
  }
}

__global__ __launch_bounds__(kCB) void k_sel_hist(size_t n, const float* __restrict__ v, uint32_t* __restrict__ ws,
                                                  int shift) {
  __shared__ uint32_t h[256];
  const int t = threadIdx.x;
  h[t] = 0u;
  __syncthreads();
  const uint32_t prefix = ws[0], mask = ws[1];
  for (size_t i = (size_t)blockIdx.x * kCB + t; i < n; i += (size_t)gridDim.x * kCB) {
    const uint32_t key = order_key(v[i]);
    if ((key & mask) == prefix) atomicAdd(&h[(key >> shift) & 255u], 1u);
  }
  __syncthreads();
  if (h[t]) atomicAdd(&ws[kSelHist + t], h[t]);
}

// One workgroup: find the bin that holds the remaining rank, extend the prefix,
// clear the histogram for the next pass; after the last pass write the value.
__global__ __launch_bounds__(kCB) void k_sel_pick(uint32_t* __restrict__ ws, int shift, float* __restrict__ out) {
  __shared__ uint32_t c[256];
  const int t = threadIdx.x;
  const uint32_t own = ws[kSelHist + t];
  c[t] = own;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {              // inclusive scan
    const uint32_t a = t >= o ? c[t - o] : 0u;
    __syncthreads();
    c[t] += a;
    __syncthreads();
  }
  const uint32_t rank = ws[2];
  const uint32_t before = c[t] - own;
  __syncthreads();                                  // every thread has read ws[2]
  if (own > 0u && before <= rank && rank < c[t]) {  // exactly one bin holds the rank
    const uint32_t prefix = ws[0] | ((uint32_t)t << shift);
    ws[0] = prefix;
    ws[1] |= 255u << shift;
    ws[2] = rank - before;
    if (shift == 0) out[0] = key_value(prefix);
  }
  ws[kSelHist + t] = 0u;
}

// ---------------------------------------------------------------- hot-first order
__global__ __launch_bounds__(kCB) void k_fill_zero(int32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * kCB + threadIdx.x;
  if (i < n) p[i] = 0;
}

__global__ __launch_bounds__(kCB) void k_group_sum(int f, const int32_t* __restrict__ counts,
                                                   const int32_t* __restrict__ group, int32_t* __restrict__ gsum) {
  const int i = blockIdx.x * kCB + threadIdx.x;
  if (i >= f) return;
  const int g = group[i];
  if (g >= 0 && g < f) atomicAdd(&gsum[g], counts[i]);
}

struct Key2 {
  unsigned long long hi, lo;
};

__device__ __forceinline__ Key2 order_key2(int i, int f, const int32_t* counts, const int32_t* group,
                                           const int32_t* gsum) {
  const uint32_t nc = (uint32_t)max(counts[i], 0);
  uint32_t gc = nc, gid = (uint32_t)i;
  if (group) {
    const int g = group[i];
    gid = (g >= 0 && g < f) ? (uint32_t)g : 0xFFFFFFFFu;
    gc = (g >= 0 && g < f) ? (uint32_t)max(gsum[g], 0) : 0u;
  }
  Key2 k;
  k.hi = ((unsigned long long)gc << 32) | (unsigned long long)(0xFFFFFFFFu - gid);
  k.lo = ((unsigned long long)nc << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)i);
  return k;
}

constexpr int kRankTile = 1024;

// rank_i = number of neurons whose key is larger (keys are distinct: the slot is
// part of them); perm[rank_i] = i.
__global__ __launch_bounds__(kCB) void k_rank(int f, const int32_t* __restrict__ counts,
                                              const int32_t* __restrict__ group, const int32_t* __restrict__ gsum,
                                              int32_t* __restrict__ perm) {
  __shared__ unsigned long long s_hi[kRankTile], s_lo[kRankTile];
  const int i = blockIdx.x * kCB + threadIdx.x;
  Key2 me{0ull, 0ull};
  if (i < f) me = order_key2(i, f, counts, group, gsum);
  int rank = 0;
  for (int j0 = 0; j0 < f; j0 += kRankTile) {
    const int nj = min(kRankTile, f - j0);
    __syncthreads();
    for (int q = threadIdx.x; q < nj; q += kCB) {
      const Key2 k = order_key2(j0 + q, f, counts, group, gsum);
      s_hi[q] = k.hi;
      s_lo[q] = k.lo;
    }
    __syncthreads();
    for (int q = 0; q < nj; ++q) {
      const unsigned long long hi = s_hi[q], lo = s_lo[q];
      rank += (hi > me.hi || (hi == me.hi && lo > me.lo)) ? 1 : 0;
    }
  }
  if (i < f) perm[rank] = i;
}

// ---------------------------------------------------------------- row gather
template <int W>
__global__ __launch_bounds__(kCB) void k_gather_rows(int n_dst, int n_src, size_t words_per_row,
                                                     const uint8_t* __restrict__ src,
                                                     const int32_t* __restrict__ idx, uint8_t* __restrict__ dst) {
  const size_t total = (size_t)n_dst * words_per_row;
  for (size_t w = (size_t)blockIdx.x * kCB + threadIdx.x; w < total; w += (size_t)gridDim.x * kCB) {
    const size_t r = w / words_per_row, c = w - r * words_per_row;
    const int s = idx[r];
    if (s < 0 || s >= n_src) continue;
    *reinterpret_cast<Raw<W>*>(dst + w * W) = load_raw<W>(src + ((size_t)s * words_per_row + c) * W);
  }
}

int grid_for(size_t items, int per_cu) {
  const int cus = device_cu_count();
  const size_t cap = (size_t)(cus > 0 ? cus : 256) * per_cu;
  const size_t need = (items + kCB - 1) / kCB;
  return (int)(need < cap ? (need > 0 ? need : 1) : cap);
}

}  // namespace

size_t select_ws_bytes() { return (size_t)(kSelHist + 256) * 4; }

hipError_t launch_count_active(hipStream_t s, int B, int f, const uint32_t* tok_bits, int32_t* counts) {
  k_count_active<<<dim3((f + kCB - 1) / kCB), dim3(kCB), 0, s>>>(B, f, tok_bits, counts);
  return hipGetLastError();
}

hipError_t launch_select_kth(hipStream_t s, size_t n, const float* v, size_t k, float* out, void* ws) {
  uint32_t* w = (uint32_t*)ws;
  k_sel_init<<<dim3(1), dim3(kCB), 0, s>>>(w, (uint32_t)k);
  const int grid = grid_for(n, 8);
  for (int shift = 24; shift >= 0; shift -= 8) {
    k_sel_hist<<<dim3(grid), dim3(kCB), 0, s>>>(n, v, w, shift);
    k_sel_pick<<<dim3(1), dim3(kCB), 0, s>>>(w, shift, out);
  }
  return hipGetLastError();
}

size_t order_ws_bytes(int f) { return ((size_t)f * 4 + 255) & ~(size_t)255; }

hipError_t launch_hot_first_order(hipStream_t s, int f, const int32_t* counts, const int32_t* group, int32_t* perm,
                                  void* ws) {
  int32_t* gsum = (int32_t*)ws;
  const int nb = (f + kCB - 1) / kCB;
  if (group) {
    k_fill_zero<<<dim3(nb), dim3(kCB), 0, s>>>(gsum, f);
    k_group_sum<<<dim3(nb), dim3(kCB), 0, s>>>(f, counts, group, gsum);
  }
  k_rank<<<dim3(nb), dim3(kCB), 0, s>>>(f, counts, group, group ? gsum : nullptr, perm);
  return hipGetLastError();
}

hipError_t launch_gather_rows(hipStream_t s, int n_dst, int n_src, size_t row_bytes, const void* src,
                              const int32_t* idx, void* dst) {
  const bool wide = (row_bytes % 16 == 0) && (((uintptr_t)src | (uintptr_t)dst) % 16 == 0);
  if (wide) {
    const size_t wpr = row_bytes / 16;
    k_gather_rows<16><<<dim3(grid_for((size_t)n_dst * wpr, 16)), dim3(kCB), 0, s>>>(
        n_dst, n_src, wpr, (const uint8_t*)src, idx, (uint8_t*)dst);
  } else {
    const size_t wpr = row_bytes / 4;
    k_gather_rows<4><<<dim3(grid_for((size_t)n_dst * wpr, 16)), dim3(kCB), 0, s>>>(
        n_dst, n_src, wpr, (const uint8_t*)src, idx, (uint8_t*)dst);
  }
  return hipGetLastError();
}

}  // namespace sfx
