// Gathered up / gate rows on the matrix cores for B >= 3 tokens (PowerInfer page,
// Method, neuron-aware operators of §5.4: only the rows of active neurons are read;
// Paper vs code, activation functions: ReLU, ReGLU and squared ReLU).
//
//   hact[j][b] = max(Wa[idx_j] . x_b + ba[idx_j], 0)                 ReLU
//   hact[j][b] = max(Wa[idx_j] . x_b + ba[idx_j], 0) * (Wl[idx_j] . x_b)   ReGLU
//   hact[j][b] = max(Wa[idx_j] . x_b + ba[idx_j], 0)^2                    squared ReLU
//
// From 3 tokens on every row byte feeds >= 3 multiply-adds and the per-row input
// re-reads of the vector kernel dominate (pad tokens of the 16-token tile cost
// nothing measurable: the kernel is bound by memory); here the gathered rows are the A operand
// of v_mfma_f32_16x16x32 (16 list entries x 32 columns: lane l reads 16 bytes of
// row l % 16, columns 8 (l / 16) ..) and the tokens are the B operand (lane l reads
// 16 bytes of token l % 16), both straight from memory with no transposition.
// fp16 / bf16 products are exact in fp32, so only the summation order differs from
// the vector kernel.
//
// Workgroup = one tile of MT x 16 list entries; its 8 waves take interleaved
// 32-column steps (U steps in flight per wave), add their partial tiles in LDS in
// wave order, and apply bias and activation in registers.  A persistent grid
// strides over the tiles of the device-resident count.
#include "sfx_launch.hpp"
#include "sfx_mfma.hpp"

namespace sfx {
namespace {

constexpr int kUW = 8;          // waves per workgroup
constexpr int kUpBlocksPerCU = 2;

template <class T, int NT, int MT, bool REGLU>
__global__ __launch_bounds__(kUW * kWave) void k_up_mfma(const uint8_t* __restrict__ x,
                                                        const uint8_t* __restrict__ Wa,
                                                        const float* __restrict__ ba,
                                                        const uint8_t* __restrict__ Wl,
                                                        const int32_t* __restrict__ idx,
                                                        const int32_t* __restrict__ count, int kmax, int B,
                                                        int d, int f, float* __restrict__ hact,
                                                        int square) {
  constexpr int NA = REGLU ? 2 : 1;
  constexpr int kUU = NT == 1 ? 8 : 4;          // 32-column steps per wave in flight (8 spills at 64 tokens)
  __shared__ f32x4 s_acc[kUW - 1][NA][MT][NT][kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int k = min(*count, kmax);
  const int nsteps = (d + 31) >> 5;
  const int kq = (lane >> 4) * 8;               // this lane's 8 columns within a step
  const size_t rb = (size_t)d * 2;
  const uint8_t* xr[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) xr[n] = x + (size_t)min(n * 16 + (lane & 15), B - 1) * rb;

  for (int tile = blockIdx.x; tile * MT * 16 < k; tile += gridDim.x) {
    const int j0 = tile * MT * 16;
    // Row of this lane in each 16-entry sub-tile (clamped to the list; an index
    // out of [0, f) reads row 0 and its outputs are written as 0).
    const uint8_t* ar[MT];
    const uint8_t* lr[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      int i = idx[min(j0 + m * 16 + (lane & 15), k - 1)];
      if ((unsigned)i >= (unsigned)f) i = 0;
      ar[m] = Wa + (size_t)i * rb;
      lr[m] = REGLU ? Wl + (size_t)i * rb : nullptr;
    }
    f32x4 acc[NA][MT][NT];
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[a][m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int s0 = wave; s0 < nsteps; s0 += kUW * kUU) {
      // Every load of the batch is issued before the first product; columns past
      // d are read clamped and zeroed after the load.
      Raw<16> wa[kUU][MT], wl[kUU][MT], xv[kUU][NT];
#pragma unroll
      for (int u = 0; u < kUU; ++u) {
        const int c = (s0 + u * kUW) * 32 + kq;
        const size_t off = (size_t)min(c, d - 8) * 2;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          wa[u][m] = load_raw<16>(ar[m] + off);
          if (REGLU) wl[u][m] = load_raw<16>(lr[m] + off);
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) xv[u][n] = load_raw<16>(xr[n] + off);
      }
      __builtin_amdgcn_sched_barrier(0);   // keep the scheduler from interleaving loads and products
#pragma unroll
      for (int u = 0; u < kUU; ++u) {
        const int c = (s0 + u * kUW) * 32 + kq;
        if (c >= d) {
#pragma unroll
          for (int n = 0; n < NT; ++n) xv[u][n] = zero16();
        }
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            acc[0][m][n] = Mma<T>::run(wa[u][m], xv[u][n], acc[0][m][n]);
            if (REGLU) acc[NA - 1][m][n] = Mma<T>::run(wl[u][m], xv[u][n], acc[NA - 1][m][n]);
          }
      }
    }

    // Partial tiles of waves 1..7 to LDS; wave 0 adds them in wave order and
    // finishes the tile.
    if (wave > 0) {
#pragma unroll
      for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int n = 0; n < NT; ++n) s_acc[wave - 1][a][m][n][lane] = acc[a][m][n];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll 1
      for (int v = 0; v < kUW - 1; ++v)
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
          for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int n = 0; n < NT; ++n) acc[a][m][n] += s_acc[v][a][m][n][lane];
      // D layout: lane l holds entries 4 (l / 16) + e of the sub-tile for token l % 16.
      int ie[MT][4];
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) ie[m][e] = idx[min(j0 + m * 16 + (lane >> 4) * 4 + e, k - 1)];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = j0 + m * 16 + (lane >> 4) * 4 + e;
          const int i = ie[m][e];
          const bool ok = (unsigned)i < (unsigned)f;
          const float bias = (ok && ba != nullptr) ? ba[ok ? i : 0] : 0.f;
          if (j < k) {
#pragma unroll
            for (int n = 0; n < NT; ++n) {
              const int b = n * 16 + (lane & 15);
              if (b < B) {
                float h = ok ? fmaxf(acc[0][m][n][e] + bias, 0.f) : 0.f;
                if (REGLU) h *= acc[NA - 1][m][n][e];
                if (square) h *= h;
                hact[(size_t)j * B + b] = h;
              }
            }
          }
        }
      }
    }
    __syncthreads();
  }
}

template <class T, int NT, int MT>
hipError_t run(hipStream_t s, int act, int B, int d, int f, const void* x, const void* Wa, const float* ba,
               const void* Wl, const int32_t* idx, const int32_t* count, int kmax, float* hact) {
  const int tiles = (kmax + MT * 16 - 1) / (MT * 16);
  const int cus = device_cu_count();
  const int cap = (cus > 0 ? cus : 256) * kUpBlocksPerCU;
  dim3 g(tiles < cap ? (tiles > 0 ? tiles : 1) : cap), blk(kUW * kWave);
  if (act == 1)
    k_up_mfma<T, NT, MT, true><<<g, blk, 0, s>>>((const uint8_t*)x, (const uint8_t*)Wa, ba, (const uint8_t*)Wl,
                                                  idx, count, kmax, B, d, f, hact, 0);
  else
    k_up_mfma<T, NT, MT, false><<<g, blk, 0, s>>>((const uint8_t*)x, (const uint8_t*)Wa, ba, nullptr, idx,
                                                   count, kmax, B, d, f, hact, act == 2 ? 1 : 0);
  return hipGetLastError();
}

template <class T>
hipError_t dispatch(hipStream_t s, int act, int B, int d, int f, const void* x, const void* Wa, const float* ba,
                    const void* Wl, const int32_t* idx, const int32_t* count, int kmax, float* hact) {
  if (B <= 16) return run<T, 1, 1>(s, act, B, d, f, x, Wa, ba, Wl, idx, count, kmax, hact);
  if (B <= 32) return run<T, 2, 2>(s, act, B, d, f, x, Wa, ba, Wl, idx, count, kmax, hact);
  // 64 tokens: two row sub-tiles per step halve the input reads per row byte
  // (Falcon-40B shape: 262 -> 167 us); below that taller tiles measured slower.
  return run<T, 4, 2>(s, act, B, d, f, x, Wa, ba, Wl, idx, count, kmax, hact);
}

}  // namespace

bool up_mfma_eligible(int wdt, int B, int d) {
  return (wdt == DT_F16 || wdt == DT_BF16) && B >= 3 && B <= 64 && d >= 8;   // as down: from 3 tokens
}

hipError_t launch_up_mfma(hipStream_t s, int wdt, int act, int B, int d, int f, const void* x, const void* Wa,
                          const float* ba, const void* Wl, const int32_t* idx, const int32_t* count, int kmax,
                          float* hact) {
  if (wdt == DT_F16) return dispatch<TF16>(s, act, B, d, f, x, Wa, ba, Wl, idx, count, kmax, hact);
  return dispatch<TBF16>(s, act, B, d, f, x, Wa, ba, Wl, idx, count, kmax, hact);
}

}  // namespace sfx
