// Per-layer predictor on the matrix cores for B >= 16 tokens (PowerInfer page,
// Method, per-layer predictor of §5.1).  From 16 tokens on, each predictor weight
// feeds >= 16 multiply-adds and the two layers are dense contractions:
//
//   layer 1   hidden[b][j] = max(sum_c W1[j][c] x[b][c], 0)       W1, x: fp16 / bf16
//   layer 2   scores[b][i] = sum_j W2[i][j] hidden[b][j]           hidden: fp32
//
// Both use v_mfma_f32_16x16x32 (A = 16 weight rows x 32 k, B = 32 k x 16 tokens,
// fp32 accumulation).  Layer 2 must not round the fp32 hidden to the weight type,
// so it is split into exact pieces that the matrix cores multiply separately:
// fp16 weights: hidden = hi + 2^-11 lo with hi = fp16(v), lo = fp16((v - hi) 2^11)
// (22 significant bits, lo scaled so it does not fall into fp16 subnormals);
// bf16 weights: hidden = hi + mid + lo, three bf16 terms (24 bits, exact for
// normal values).  Products of two 16-bit values are exact in fp32 (sfx_mfma.hpp).
#include "sfx_launch.hpp"
#include "sfx_mfma.hpp"

namespace sfx {
namespace {

// ------------------------------------------------------------------ layer 1
// Workgroup = one tile of 16 W1 rows; its 8 waves take interleaved 32-wide k
// steps; partial tiles are added in wave order in LDS.
constexpr int kHW = 8;

template <class T, int NT>
__global__ __launch_bounds__(kHW * kWave) void k_hidden_mfma(const uint8_t* __restrict__ x,
                                                            const uint8_t* __restrict__ W1,
                                                            float* __restrict__ hid, int B, int d, int h) {
  __shared__ f32x4 s_acc[kHW][NT][kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int row0 = blockIdx.x * 16;
  const int r = row0 + (lane & 15);
  const int kq = (lane >> 4) * 8;
  const int nsteps = (d + 31) / 32;
  f32x4 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr int U = 4;
  for (int s0 = wave; s0 < nsteps; s0 += kHW * U) {
    Raw<16> a[U], bx[U][NT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (s0 + u * kHW) * 32 + kq;
      const bool kin = (s0 + u * kHW) < nsteps && k < d;
      a[u] = (kin && r < h) ? load_raw<16>(W1 + ((size_t)r * d + k) * 2) : zero16();
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const int tok = n * 16 + (lane & 15);
        bx[u][n] = (kin && tok < B) ? load_raw<16>(x + ((size_t)tok * d + k) * 2) : zero16();
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[n] = Mma<T>::run(a[u], bx[u][n], acc[n]);
  }
#pragma unroll
  for (int n = 0; n < NT; ++n) s_acc[wave][n][lane] = acc[n];
  __syncthreads();
  if (wave < NT) {
    const int n = wave;
    f32x4 t = s_acc[0][n][lane];
    for (int v = 1; v < kHW; ++v) t += s_acc[v][n][lane];
    const int tok = n * 16 + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = row0 + (lane >> 4) * 4 + i;
      if (tok < B && row < h) hid[(size_t)tok * h + row] = fmaxf(t[i], 0.f);
    }
  }
}

// ------------------------------------------------------------------ layer 2
// Workgroup = 8 waves x one 16-row tile of W2 each (128 rows); the fp32 hidden of
// all tokens is split into 16-bit pieces in LDS, KC columns at a time.
constexpr int kSW = 8;
constexpr int kKC = 256;                 // k columns per LDS chunk
constexpr int kPad = 8;                  // halves of padding per token row (bank spread)
constexpr int kStride = kKC + kPad;

template <class T, int NT>
__global__ __launch_bounds__(kSW * kWave) void k_scores_mfma(const uint8_t* __restrict__ W2,
                                                            const float* __restrict__ hid,
                                                            float* __restrict__ scores, int B, int h, int f) {
  constexpr int NP = Split<T>::pieces;
  __shared__ __attribute__((aligned(16))) uint16_t s_h[NP][NT * 16][kStride];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int row0 = blockIdx.x * (kSW * 16) + wave * 16;
  const int r = row0 + (lane & 15);
  const int kq = (lane >> 4) * 8;
  f32x4 acc[NP == 2 ? 2 : 1][NT];
#pragma unroll
  for (int p = 0; p < (NP == 2 ? 2 : 1); ++p)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[p][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int kc = 0; kc < h; kc += kKC) {
    // issue this chunk's W2 loads first; they stream while the hidden is split
    Raw<16> a[kKC / 32];
#pragma unroll
    for (int s = 0; s < kKC / 32; ++s) {
      const int k = kc + s * 32 + kq;
      a[s] = (r < f && k < h) ? load_raw<16>(W2 + ((size_t)r * h + k) * 2) : zero16();
    }
    __syncthreads();                        // previous chunk's pieces are consumed
    for (int i = tid; i < NT * 16 * kKC; i += kSW * kWave) {
      const int tok = i / kKC, j = i - tok * kKC;
      const float v = (tok < B && kc + j < h) ? hid[(size_t)tok * h + kc + j] : 0.f;
      uint16_t pc[NP];
      Split<T>::run(v, pc);
#pragma unroll
      for (int p = 0; p < NP; ++p) s_h[p][tok][j] = pc[p];
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kKC / 32; ++s) {
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const int tok = n * 16 + (lane & 15);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const Raw<16> b = *reinterpret_cast<const Raw<16>*>(&s_h[p][tok][s * 32 + kq]);
          const int ai = NP == 2 ? p : 0;
          acc[ai][n] = Mma<T>::run(a[s], b, acc[ai][n]);
        }
      }
    }
  }
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int tok = n * 16 + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = row0 + (lane >> 4) * 4 + i;
      float v = acc[0][n][i];
      if (NP == 2) v += acc[NP == 2 ? 1 : 0][n][i] * (1.0f / 2048.0f);
      if (tok < B && row < f) scores[(size_t)tok * f + row] = v;
    }
  }
}

template <class T, int NT>
hipError_t run(hipStream_t s, int B, int d, int h, int f, const void* x, const void* W1, const void* W2,
               float* hid, float* scores) {
  k_hidden_mfma<T, NT><<<dim3((h + 15) / 16), dim3(kHW * kWave), 0, s>>>((const uint8_t*)x, (const uint8_t*)W1,
                                                                           hid, B, d, h);
  k_scores_mfma<T, NT><<<dim3((f + kSW * 16 - 1) / (kSW * 16)), dim3(kSW * kWave), 0, s>>>(
      (const uint8_t*)W2, hid, scores, B, h, f);
  return hipGetLastError();
}

template <class T>
hipError_t dispatch(hipStream_t s, int B, int d, int h, int f, const void* x, const void* W1, const void* W2,
                    float* hid, float* scores) {
  if (B <= 16) return run<T, 1>(s, B, d, h, f, x, W1, W2, hid, scores);
  if (B <= 32) return run<T, 2>(s, B, d, h, f, x, W1, W2, hid, scores);
  return run<T, 4>(s, B, d, h, f, x, W1, W2, hid, scores);
}

}  // namespace

bool pred_mfma_eligible(int wdt, int B, int h, int f) {
  (void)h; (void)f;
  return (wdt == DT_F16 || wdt == DT_BF16) && B >= 16 && B <= 64;
}

hipError_t launch_pred_mfma(hipStream_t s, int wdt, int B, int d, int h, int f, const void* x, const void* W1,
                            const void* W2, float* hid, float* scores) {
  if (wdt == DT_F16) return dispatch<TF16>(s, B, d, h, f, x, W1, W2, hid, scores);
  return dispatch<TBF16>(s, B, d, h, f, x, W1, W2, hid, scores);
}

}  // namespace sfx
