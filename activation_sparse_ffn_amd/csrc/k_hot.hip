// Hot region: the groups TAM keeps hot, copied into a contiguous region of K
// group slots per layer (KAIROX page, Core method, items 3 and 4: decisions and
// transfers are per group of 32 co-activated neurons stored together; the groups
// with the highest momentum fill the capacity; item 6: the hot set changes by set
// differences, and only entering groups are transferred).  On one GPU every layer
// already sits in HBM, so the transfer becomes a copy into the hot region and its
// bytes per step measure the churn a CPU-GPU system would pay as reloads.
//
// sfx_hot_assign (one workgroup per layer, G <= 1024, K <= 1024):
//   1. every leaving group g frees its slot:  group_of[slot_of[g]] = -1, slot_of[g] = -1
//   2. free slots, ascending:  F = [s : group_of[s] == -1]
//   3. entering groups, ascending, take them in order:  slot_of[E_i] = F_i,
//      group_of[F_i] = E_i, and (E_i, F_i) is copy i of the layer.
// copy step: copy i of layer l moves group_bytes bytes of each matrix m from
//   src[l][m] + E_i * group_bytes to dst[l][m] + F_i * group_bytes.
#include "sfx_common.hpp"
#include "sfx_launch.hpp"

namespace sfx {
namespace {

constexpr int kHT = 1024;

__global__ __launch_bounds__(kHT) void k_hot_assign(int G, int K, const uint32_t* __restrict__ entered,
                                                    const uint32_t* __restrict__ left,
                                                    int32_t* __restrict__ slot_of, int32_t* __restrict__ group_of,
                                                    int32_t* __restrict__ copies, int32_t* __restrict__ ncopies) {
  __shared__ uint32_t s_cnt[kHT / kWave];
  __shared__ int32_t s_free[kHT];
  const int l = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1), wave = t >> 6;
  const int HW = (G + 31) >> 5;
  const uint32_t* en = entered + (size_t)l * HW;
  const uint32_t* lf = left + (size_t)l * HW;
  int32_t* so = slot_of + (size_t)l * G;
  int32_t* go = group_of + (size_t)l * K;
  // 1. leaving groups free their slots (distinct groups hold distinct slots)
  if (t < G && ((lf[t >> 5] >> (t & 31)) & 1u)) {
    const int s = so[t];
    if (s >= 0 && s < K) go[s] = -1;
    so[t] = -1;
  }
  __syncthreads();
  // 2. free slots, ascending: ballot + prefix over the waves
  const bool fr = t < K && go[t] < 0;
  const uint64_t bf = __ballot(fr);
  if (lane == 0) s_cnt[wave] = (uint32_t)__popcll(bf);
  __syncthreads();
  uint32_t before = 0, nfree = 0;
  for (int v = 0; v < kHT / kWave; ++v) {
    const uint32_t c = s_cnt[v];
    if (v < wave) before += c;
    nfree += c;
  }
  if (fr) s_free[before + __popcll(bf & ((1ull << lane) - 1ull))] = t;
  __syncthreads();
  // 3. entering groups, ascending, take the free slots in order
  const bool ent = t < G && ((en[t >> 5] >> (t & 31)) & 1u);
  const uint64_t be = __ballot(ent);
  __syncthreads();                                      // s_cnt reused
  if (lane == 0) s_cnt[wave] = (uint32_t)__popcll(be);
  __syncthreads();
  uint32_t eb = 0, etot = 0;
  for (int v = 0; v < kHT / kWave; ++v) {
    const uint32_t c = s_cnt[v];
    if (v < wave) eb += c;
    etot += c;
  }
  if (ent) {
    const int i = (int)(eb + __popcll(be & ((1ull << lane) - 1ull)));
    const int s = i < (int)nfree ? s_free[i] : -1;      // a hot set of at most K groups always fits
    so[t] = s;
    if (s >= 0) {
      go[s] = t;
      copies[((size_t)l * K + i) * 2] = t;
      copies[((size_t)l * K + i) * 2 + 1] = s;
    }
  }
  if (t == 0) ncopies[l] = (int32_t)(etot < nfree ? etot : nfree);
}

// Copy kernel: work item w = (copy j, chunk c), with j running over the copies of
// all layers in layer order (an exclusive prefix of ncopies in LDS) and c over the
// 16 KB chunks of the group's rows in every matrix (matrix m owns chunks
// [chunk_off[m], chunk_off[m + 1])).  Each thread moves up to four 16-byte words of
// a chunk, so all loads of a chunk are in flight together; the grid strides over
// the items.
constexpr int kCT = 256;
constexpr int kLPT = kHotMaxLayers / kCT;        // layers per thread in the prefix

__global__ __launch_bounds__(kCT) void k_hot_copy(int L, int K, HotMats mats, const void* const* __restrict__ src,
                                                  void* const* __restrict__ dst, const int32_t* __restrict__ copies,
                                                  const int32_t* __restrict__ ncopies) {
  __shared__ int32_t s_pre[kHotMaxLayers + 1];
  __shared__ int32_t s_part[kCT];
  const int t = threadIdx.x;
  int loc[kLPT], run = 0;
#pragma unroll
  for (int q = 0; q < kLPT; ++q) {
    const int l = t * kLPT + q;
    loc[q] = l < L ? ncopies[l] : 0;
    run += loc[q];
  }
  s_part[t] = run;
  __syncthreads();
  for (int o = 1; o < kCT; o <<= 1) {              // inclusive scan of the per-thread sums
    const int v = t >= o ? s_part[t - o] : 0;
    __syncthreads();
    s_part[t] += v;
    __syncthreads();
  }
  int pre = s_part[t] - run;
#pragma unroll
  for (int q = 0; q < kLPT; ++q) {
    s_pre[t * kLPT + q] = pre;
    pre += loc[q];
  }
  if (t == kCT - 1) s_pre[kHotMaxLayers] = pre;
  __syncthreads();
  const int C = mats.chunk_off[mats.n];
  const int64_t items = (int64_t)s_pre[kHotMaxLayers] * C;
  for (int64_t w = blockIdx.x; w < items; w += gridDim.x) {
    const int j = (int)(w / C), c = (int)(w - (int64_t)j * C);
    int lo = 0, hi = L - 1;                         // last layer l with s_pre[l] <= j
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pre[mid] <= j) lo = mid; else hi = mid - 1;
    }
    const int l = lo, i = j - s_pre[l];
    int m = 0;
    while (c >= mats.chunk_off[m + 1]) ++m;
    const size_t gb = mats.group_bytes[m];
    const size_t off = (size_t)(c - mats.chunk_off[m]) * kHotChunk;
    const size_t n16 = (gb - off < (size_t)kHotChunk ? gb - off : (size_t)kHotChunk) / 16;
    const size_t u = (size_t)l * K + i;
    const size_t g = (size_t)copies[u * 2], sl = (size_t)copies[u * 2 + 1];
    const uint8_t* a = (const uint8_t*)src[(size_t)l * mats.n + m] + g * gb + off;
    uint8_t* b = (uint8_t*)dst[(size_t)l * mats.n + m] + sl * gb + off;
    Raw<16> v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const size_t e = (size_t)t + (size_t)q * kCT;
      v[q] = load_raw<16>(a + (e < n16 ? e : 0) * 16);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const size_t e = (size_t)t + (size_t)q * kCT;
      if (e < n16) *reinterpret_cast<Raw<16>*>(b + e * 16) = v[q];
    }
  }
}

static_assert(kHotChunk == kCT * 4 * 16, "one chunk is four 16-byte words per thread");
static_assert(kHotMaxLayers % kCT == 0, "layer prefix split evenly over the threads");

}  // namespace

hipError_t launch_hot_assign(hipStream_t s, int L, int G, int K, const uint32_t* entered, const uint32_t* left,
                             int32_t* slot_of, int32_t* group_of, int32_t* copies, int32_t* ncopies) {
  k_hot_assign<<<dim3(L), dim3(kHT), 0, s>>>(G, K, entered, left, slot_of, group_of, copies, ncopies);
  return hipGetLastError();
}

hipError_t launch_hot_copy(hipStream_t s, int L, int K, const HotMats& mats, const void* const* src,
                           void* const* dst, const int32_t* copies, const int32_t* ncopies) {
  const int cus = device_cu_count();
  const int grid = (cus > 0 ? cus : 256) * 8;
  k_hot_copy<<<dim3(grid), dim3(kCT), 0, s>>>(L, K, mats, src, dst, copies, ncopies);
  return hipGetLastError();
}

}  // namespace sfx
