// Gathered up / gate rows of the active neurons (PowerInfer page, Method, neuron-
// aware operators of §5.4: the operator reads only the rows of neurons marked
// active; Paper vs code, activation functions: ReLU, ReGLU and squared ReLU).
//
//   hact[j][b] = act(Wa[idx_j] . x_b + ba[idx_j])        ReLU
//   hact[j][b] = max(Wa[idx_j] . x_b + ba[idx_j], 0) * (Wl[idx_j] . x_b)   ReGLU
//   hact[j][b] = max(Wa[idx_j] . x_b + ba[idx_j], 0)^2                    squared ReLU
// (squared ReLU runs the ReLU instantiations with a wave-uniform `square` flag)
//
// A persistent grid of waves strides over the device-resident count; each wave
// reads whole rows with coalesced 16-byte loads (a row is contiguous), keeps the
// B dot products in registers, reduces them across the wave and applies the bias
// and the activation in registers.  int4 rows are decoded in the kernel: a lane's
// 16-byte load is exactly one group of 32 codes with its one fp16 scale.
#include "sfx_common.hpp"
#include "sfx_launch.hpp"

namespace sfx {

bool up_mfma_eligible(int wdt, int B, int d);
hipError_t launch_up_mfma(hipStream_t s, int wdt, int act, int B, int d, int f, const void* x, const void* Wa,
                          const float* ba, const void* Wl, const int32_t* idx, const int32_t* count, int kmax,
                          float* hact);

namespace {

constexpr int kU = 8;         // 16-byte chunks per lane issued together
constexpr int kBlocksPerCU = 2;

template <class T, int NB, bool REGLU>
__global__ __launch_bounds__(kBlock) void k_up(const uint8_t* __restrict__ x, const uint8_t* __restrict__ Wa,
                                               const float* __restrict__ ba, const uint8_t* __restrict__ Wl,
                                               const int32_t* __restrict__ idx, const int32_t* __restrict__ count,
                                               int kmax, int B, int d, int f, float* __restrict__ hact,
                                               int square) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * kWavesPerBlock;
  const int k = min(*count, kmax);
  const int nchunk = d / T::vec;
  const size_t row_bytes = (size_t)d * T::bytes;

  // The first index is loaded before the count is known (clamped to the list's
  // capacity), and each row's bias is loaded with its row, so no load waits on
  // another that it does not need.
  int i_next = idx[min(wave, kmax - 1)];
  for (int j = wave; j < k; j += nwaves) {
    const int i = i_next;
    i_next = idx[min(j + nwaves, kmax - 1)];
    const bool ok = (unsigned)i < (unsigned)f;
    const float bias = (ok && ba != nullptr) ? ba[ok ? i : 0] : 0.f;
    float za[NB], zl[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) { za[b] = 0.f; zl[b] = 0.f; }
    if (ok) {
      const uint8_t* ra = Wa + (size_t)i * row_bytes;
      const uint8_t* rl = REGLU ? Wl + (size_t)i * row_bytes : nullptr;
      // Every load of a batch is issued before the first is used: chunk indices
      // are clamped instead of branched on (in branches the compiler serialises the
      // input loads, one round trip per chunk).
      constexpr int KB = NB == 1 ? kU : NB == 2 ? 4 : 2;   // row chunks per lane per batch
      constexpr int TG = NB < 4 ? NB : 4;                  // tokens whose input chunks load together
      for (int c0 = 0; c0 < nchunk; c0 += KB * kWave) {
        Raw<16> wa[KB], wl[KB];
#pragma unroll
        for (int u = 0; u < KB; ++u) {
          const int c = min(c0 + u * kWave + lane, nchunk - 1);
          wa[u] = load_raw<16>(ra + (size_t)c * 16);
          if (REGLU) wl[u] = load_raw<16>(rl + (size_t)c * 16);
        }
#pragma unroll
        for (int b0 = 0; b0 < NB; b0 += TG) {
          if (b0 < B) {
            Raw<16> xq[KB][TG];
#pragma unroll
            for (int u = 0; u < KB; ++u) {
              const int c = min(c0 + u * kWave + lane, nchunk - 1);
#pragma unroll
              for (int t = 0; t < TG; ++t) xq[u][t] = load_raw<16>(x + (size_t)min(b0 + t, B - 1) * row_bytes + (size_t)c * 16);
            }
#pragma unroll
            for (int u = 0; u < KB; ++u) {
              if (c0 + u * kWave + lane < nchunk) {
                float af[T::vec], lf[T::vec];
                unpack<T, 4>(wa[u].w, af);
                if (REGLU) unpack<T, 4>(wl[u].w, lf);
#pragma unroll
                for (int t = 0; t < TG; ++t) {
                  if (b0 + t < B) {
                    float xf[T::vec];
                    unpack<T, 4>(xq[u][t].w, xf);
#pragma unroll
                    for (int e = 0; e < T::vec; ++e) {
                      za[b0 + t] = fmaf(af[e], xf[e], za[b0 + t]);
                      if (REGLU) zl[b0 + t] = fmaf(lf[e], xf[e], zl[b0 + t]);
                    }
                  }
                }
              }
            }
          }
        }
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      za[b] = wave_sum(za[b]);
      if (REGLU) zl[b] = wave_sum(zl[b]);
    }
    if (lane == 0) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if (b < B) {
          float a = ok ? fmaxf(za[b] + bias, 0.f) : 0.f;
          if (REGLU) a *= zl[b];
          if (square) a *= a;
          hact[(size_t)j * B + b] = a;
        }
      }
    }
  }
}

// int4 rows: codes [f][d/2] bytes, scales [f][d/32] fp16; x is fp16.
template <int NB, bool REGLU>
__global__ __launch_bounds__(kBlock) void k_up_q4(const uint8_t* __restrict__ x, const uint8_t* __restrict__ Wa,
                                                  const uint16_t* __restrict__ Wa_s, const float* __restrict__ ba,
                                                  const uint8_t* __restrict__ Wl, const uint16_t* __restrict__ Wl_s,
                                                  const int32_t* __restrict__ idx, const int32_t* __restrict__ count,
                                                  int kmax, int B, int d, int f, float* __restrict__ hact,
                                                  int square) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * kWavesPerBlock;
  const int k = min(*count, kmax);
  const int ngroup = d >> 5;                  // 32 columns per group = 16 bytes of codes
  const size_t row_bytes = (size_t)d >> 1;
  const size_t x_bytes = (size_t)d * 2;

  // The first index is loaded before the count is known (clamped to the list's
  // capacity), and each row's bias is loaded with its row, so no load waits on
  // another that it does not need.
  int i_next = idx[min(wave, kmax - 1)];
  for (int j = wave; j < k; j += nwaves) {
    const int i = i_next;
    i_next = idx[min(j + nwaves, kmax - 1)];
    const bool ok = (unsigned)i < (unsigned)f;
    const float bias = (ok && ba != nullptr) ? ba[ok ? i : 0] : 0.f;
    float za[NB], zl[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) { za[b] = 0.f; zl[b] = 0.f; }
    if (ok) {
      // Same batching as the fp16 rows: clamped group indices, every load of a
      // batch in flight before the first decode.
      constexpr int KQ = NB == 1 ? 4 : 2;   // groups per lane per batch
      constexpr int TG = NB == 1 ? 1 : 2;   // tokens whose input groups load together
      const uint8_t* ra = Wa + (size_t)i * row_bytes;
      const uint8_t* rl = REGLU ? Wl + (size_t)i * row_bytes : nullptr;
      for (int g0 = 0; g0 < ngroup; g0 += KQ * kWave) {
        Raw<16> qa[KQ], ql[KQ];
        float sa[KQ], sl[KQ];
#pragma unroll
        for (int u = 0; u < KQ; ++u) {
          const int g = min(g0 + u * kWave + lane, ngroup - 1);
          qa[u] = load_raw<16>(ra + (size_t)g * 16);
          sa[u] = (float)__builtin_bit_cast(_Float16, Wa_s[(size_t)i * ngroup + g]);
          if (REGLU) {
            ql[u] = load_raw<16>(rl + (size_t)g * 16);
            sl[u] = (float)__builtin_bit_cast(_Float16, Wl_s[(size_t)i * ngroup + g]);
          }
        }
#pragma unroll
        for (int b0 = 0; b0 < NB; b0 += TG) {
          if (b0 < B) {
            Raw<16> xq[KQ][TG][4];              // 32 fp16 columns of each token per group
#pragma unroll
            for (int u = 0; u < KQ; ++u) {
              const int g = min(g0 + u * kWave + lane, ngroup - 1);
#pragma unroll
              for (int t = 0; t < TG; ++t) {
                const uint8_t* xg = x + (size_t)min(b0 + t, B - 1) * x_bytes + (size_t)g * 64;
#pragma unroll
                for (int q = 0; q < 4; ++q) xq[u][t][q] = load_raw<16>(xg + q * 16);
              }
            }
#pragma unroll
            for (int u = 0; u < KQ; ++u) {
              if (g0 + u * kWave + lane < ngroup) {
#pragma unroll
                for (int t = 0; t < TG; ++t) {
                  if (b0 + t < B) {
                    float pa = 0.f, pl = 0.f;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {       // 4 words of codes = 32 columns
                      float xf[8];
                      unpack<TF16, 4>(xq[u][t][q].w, xf);
                      const uint32_t wa = qa[u].w[q];
#pragma unroll
                      for (int e = 0; e < 8; ++e) {
                        const float c = (float)((int32_t)(wa << (28 - 4 * e)) >> 28);
                        pa = fmaf(c, xf[e], pa);
                      }
                      if (REGLU) {
                        const uint32_t wl = ql[u].w[q];
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                          const float c = (float)((int32_t)(wl << (28 - 4 * e)) >> 28);
                          pl = fmaf(c, xf[e], pl);
                        }
                      }
                    }
                    za[b0 + t] = fmaf(sa[u], pa, za[b0 + t]);
                    if (REGLU) zl[b0 + t] = fmaf(sl[u], pl, zl[b0 + t]);
                  }
                }
              }
            }
          }
        }
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      za[b] = wave_sum(za[b]);
      if (REGLU) zl[b] = wave_sum(zl[b]);
    }
    if (lane == 0) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if (b < B) {
          float a = ok ? fmaxf(za[b] + bias, 0.f) : 0.f;
          if (REGLU) a *= zl[b];
          if (square) a *= a;
          hact[(size_t)j * B + b] = a;
        }
      }
    }
  }
}

int grid_blocks(int kmax) {
  const int cus = device_cu_count();
  const int cap = (cus > 0 ? cus : 256) * kBlocksPerCU;
  const int need = (kmax + kWavesPerBlock - 1) / kWavesPerBlock;
  return need < cap ? (need > 0 ? need : 1) : cap;
}

template <class T, int NB>
hipError_t run(hipStream_t s, int act, int B, int d, int f, const void* x, const void* Wa,
               const float* ba, const void* Wl, const int32_t* idx, const int32_t* count, int kmax,
               float* hact) {
  dim3 g(grid_blocks(kmax)), blk(kBlock);
  if (act == 1)
    k_up<T, NB, true><<<g, blk, 0, s>>>((const uint8_t*)x, (const uint8_t*)Wa, ba, (const uint8_t*)Wl, idx,
                                         count, kmax, B, d, f, hact, 0);
  else
    k_up<T, NB, false><<<g, blk, 0, s>>>((const uint8_t*)x, (const uint8_t*)Wa, ba, nullptr, idx, count,
                                          kmax, B, d, f, hact, act == 2 ? 1 : 0);
  return hipGetLastError();
}

template <int NB>
hipError_t run_q4(hipStream_t s, int act, int B, int d, int f, const void* x, const void* Wa,
                  const void* Wa_s, const float* ba, const void* Wl, const void* Wl_s,
                  const int32_t* idx, const int32_t* count, int kmax, float* hact) {
  dim3 g(grid_blocks(kmax)), blk(kBlock);
  if (act == 1)
    k_up_q4<NB, true><<<g, blk, 0, s>>>((const uint8_t*)x, (const uint8_t*)Wa, (const uint16_t*)Wa_s, ba,
                                         (const uint8_t*)Wl, (const uint16_t*)Wl_s, idx, count, kmax, B, d,
                                         f, hact, 0);
  else
    k_up_q4<NB, false><<<g, blk, 0, s>>>((const uint8_t*)x, (const uint8_t*)Wa, (const uint16_t*)Wa_s, ba,
                                          nullptr, nullptr, idx, count, kmax, B, d, f, hact, act == 2 ? 1 : 0);
  return hipGetLastError();
}

template <class T>
hipError_t dispatch(hipStream_t s, int act, int B, int d, int f, const void* x, const void* Wa,
                    const float* ba, const void* Wl, const int32_t* idx, const int32_t* count, int kmax,
                    float* hact) {
  switch (nb_class(B)) {
    case 1: return run<T, 1>(s, act, B, d, f, x, Wa, ba, Wl, idx, count, kmax, hact);
    case 2: return run<T, 2>(s, act, B, d, f, x, Wa, ba, Wl, idx, count, kmax, hact);
    case 4: return run<T, 4>(s, act, B, d, f, x, Wa, ba, Wl, idx, count, kmax, hact);
    case 8: return run<T, 8>(s, act, B, d, f, x, Wa, ba, Wl, idx, count, kmax, hact);
    case 16: return run<T, 16>(s, act, B, d, f, x, Wa, ba, Wl, idx, count, kmax, hact);
    case 32: return run<T, 32>(s, act, B, d, f, x, Wa, ba, Wl, idx, count, kmax, hact);
    default: return run<T, 64>(s, act, B, d, f, x, Wa, ba, Wl, idx, count, kmax, hact);
  }
}

}  // namespace

bool up_supported(int wdt, int act, int B) {
  (void)act;
  if (wdt == DT_Q4) return B <= 16;
  return true;
}

hipError_t launch_up(hipStream_t s, int wdt, int act, int B, int d, int f, const void* x,
                     const void* Wa, const void* Wa_s, const float* ba, const void* Wl,
                     const void* Wl_s, const int32_t* idx, const int32_t* count, int kmax,
                     float* hact) {
  if (up_mfma_eligible(wdt, B, d)) return launch_up_mfma(s, wdt, act, B, d, f, x, Wa, ba, Wl, idx, count, kmax, hact);
  switch (wdt) {
    case DT_F32: return dispatch<TF32>(s, act, B, d, f, x, Wa, ba, Wl, idx, count, kmax, hact);
    case DT_F16: return dispatch<TF16>(s, act, B, d, f, x, Wa, ba, Wl, idx, count, kmax, hact);
    case DT_BF16: return dispatch<TBF16>(s, act, B, d, f, x, Wa, ba, Wl, idx, count, kmax, hact);
    case DT_Q4:
      switch (nb_class(B)) {
        case 1: return run_q4<1>(s, act, B, d, f, x, Wa, Wa_s, ba, Wl, Wl_s, idx, count, kmax, hact);
        case 2: return run_q4<2>(s, act, B, d, f, x, Wa, Wa_s, ba, Wl, Wl_s, idx, count, kmax, hact);
        case 4: return run_q4<4>(s, act, B, d, f, x, Wa, Wa_s, ba, Wl, Wl_s, idx, count, kmax, hact);
        case 8: return run_q4<8>(s, act, B, d, f, x, Wa, Wa_s, ba, Wl, Wl_s, idx, count, kmax, hact);
        default: return run_q4<16>(s, act, B, d, f, x, Wa, Wa_s, ba, Wl, Wl_s, idx, count, kmax, hact);
      }
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sfx
