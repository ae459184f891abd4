// Per-layer MLP predictor with int4 weights (PowerInfer page, Method, per-layer
// predictor of §5.1; Pitfalls: the predictors' size, which for the OPT-30B-shaped
// layer is most of the bytes a batch-1 step reads):
//
//   hidden_b = max(W1 x_b, 0),  scores_b = W2 hidden_b,   W = q * s
//
// W1: codes [h][d/2] + scales [h][d/32], W2: codes [f][h/2] + scales [f][h/32] (the
// library's planar int4 layout: column 2c in the low nibble of byte c, two's
// complement in [-8, 7], one fp16 scale per 32 consecutive columns).  x is fp16 and
// the hidden stays fp32.  Each lane's 16-byte load is one group of 32 codes; its
// partial sum over the group is taken on the codes and multiplied by the group's
// scale once (w = q s is exact in fp32, so only the summation order differs from
// the dequantised product).
#include "sfx_common.hpp"
#include "sfx_launch.hpp"

namespace sfx {
namespace {

__device__ __forceinline__ float code(uint32_t word, int e) { return (float)((int32_t)(word << (28 - 4 * e)) >> 28); }
__device__ __forceinline__ float scale_of(const uint16_t* s, size_t i) {
  return (float)__builtin_bit_cast(_Float16, s[i]);
}

// hidden[b][row] = max(W1[row] . x_b, 0); one wave per row, KQ groups per lane in flight.
template <int NB>
__global__ __launch_bounds__(kBlock) void k_pred_hidden_q4(const uint8_t* __restrict__ x,
                                                           const uint8_t* __restrict__ W1,
                                                           const uint16_t* __restrict__ W1_s,
                                                           float* __restrict__ hid, int B, int d, int h) {
  const int lane = threadIdx.x & (kWave - 1);
  const int row = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (row >= h) return;
  const int ngroup = d >> 5;
  const uint8_t* rq = W1 + (size_t)row * (d >> 1);
  const size_t x_bytes = (size_t)d * 2;
  constexpr int KQ = NB == 1 ? 4 : 2;
  constexpr int TG = NB == 1 ? 1 : 2;
  float acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = 0.f;
  for (int g0 = 0; g0 < ngroup; g0 += KQ * kWave) {
    Raw<16> q[KQ];
    float sc[KQ];
#pragma unroll
    for (int u = 0; u < KQ; ++u) {
      const int g = min(g0 + u * kWave + lane, ngroup - 1);
      q[u] = load_raw<16>(rq + (size_t)g * 16);
      sc[u] = scale_of(W1_s, (size_t)row * ngroup + g);
    }
#pragma unroll
    for (int b0 = 0; b0 < NB; b0 += TG) {
      if (b0 < B) {
        Raw<16> xq[KQ][TG][4];
#pragma unroll
        for (int u = 0; u < KQ; ++u) {
          const int g = min(g0 + u * kWave + lane, ngroup - 1);
#pragma unroll
          for (int t = 0; t < TG; ++t) {
            const uint8_t* xg = x + (size_t)min(b0 + t, B - 1) * x_bytes + (size_t)g * 64;
#pragma unroll
            for (int k = 0; k < 4; ++k) xq[u][t][k] = load_raw<16>(xg + k * 16);
          }
        }
#pragma unroll
        for (int u = 0; u < KQ; ++u) {
          if (g0 + u * kWave + lane < ngroup) {
#pragma unroll
            for (int t = 0; t < TG; ++t) {
              if (b0 + t < B) {
                float pa = 0.f;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                  float xf[8];
                  unpack<TF16, 4>(xq[u][t][k].w, xf);
#pragma unroll
                  for (int e = 0; e < 8; ++e) pa = fmaf(code(q[u].w[k], e), xf[e], pa);
                }
                acc[b0 + t] = fmaf(sc[u], pa, acc[b0 + t]);
              }
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = wave_sum(acc[b]);
  if (lane == 0) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
      if (b < B) hid[(size_t)b * h + row] = fmaxf(acc[b], 0.f);
  }
}

// scores[b][i] = W2[i] . hidden_b; each wave owns R consecutive rows; one group of
// 32 codes per lane and row in flight with the 32 hidden values it meets.
template <int NB, int R>
__global__ __launch_bounds__(kBlock) void k_pred_scores_q4(const uint8_t* __restrict__ W2,
                                                           const uint16_t* __restrict__ W2_s,
                                                           const float* __restrict__ hid,
                                                           float* __restrict__ scores, int B, int h, int f) {
  const int lane = threadIdx.x & (kWave - 1);
  const int row0 = (blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6)) * R;
  if (row0 >= f) return;
  const int ngroup = h >> 5;
  const size_t row_bytes = (size_t)h >> 1;
  float acc[R][NB];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[r][b] = 0.f;
  for (int g0 = 0; g0 < ngroup; g0 += kWave) {
    const int g = min(g0 + lane, ngroup - 1);
    Raw<16> q[R];
    float sc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = min(row0 + r, f - 1);
      q[r] = load_raw<16>(W2 + (size_t)row * row_bytes + (size_t)g * 16);
      sc[r] = scale_of(W2_s, (size_t)row * ngroup + g);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b < B) {
        Raw<16> hq[8];                         // 32 fp32 hidden values of the group
#pragma unroll
        for (int k = 0; k < 8; ++k) hq[k] = load_raw<16>(hid + (size_t)b * h + (size_t)g * 32 + k * 4);
        if (g0 + lane < ngroup) {
#pragma unroll
          for (int r = 0; r < R; ++r) {
            float p = 0.f;
#pragma unroll
            for (int k = 0; k < 4; ++k)      // code word k = columns 8k .. 8k+7
#pragma unroll
              for (int e = 0; e < 8; ++e)
                p = fmaf(code(q[r].w[k], e), __uint_as_float(hq[(8 * k + e) >> 2].w[(8 * k + e) & 3]), p);
            acc[r][b] = fmaf(sc[r], p, acc[r][b]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[r][b] = wave_sum(acc[r][b]);
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int b = 0; b < NB; ++b)
        if (b < B && row0 + r < f) scores[(size_t)b * f + row0 + r] = acc[r][b];
  }
}

template <int NB>
hipError_t run(hipStream_t s, int B, int d, int h, int f, const void* x, const void* W1, const void* W1_s,
               const void* W2, const void* W2_s, float* scores, float* hid) {
  dim3 blk(kBlock);
  k_pred_hidden_q4<NB><<<dim3((h + kWavesPerBlock - 1) / kWavesPerBlock), blk, 0, s>>>(
      (const uint8_t*)x, (const uint8_t*)W1, (const uint16_t*)W1_s, hid, B, d, h);
  constexpr int R = NB == 1 ? 4 : NB == 2 ? 2 : 1;
  const int rows_per_block = kWavesPerBlock * R;
  k_pred_scores_q4<NB, R><<<dim3((f + rows_per_block - 1) / rows_per_block), blk, 0, s>>>(
      (const uint8_t*)W2, (const uint16_t*)W2_s, hid, scores, B, h, f);
  return hipGetLastError();
}

}  // namespace

// Workspace: the predictor's control line (256 bytes, unused here), then the fp32
// hidden [B][h] -- the layout sfx_predict_ws(SFX_Q4G32, ...) sizes.
hipError_t launch_predict_q4(hipStream_t s, int B, int d, int h, int f, const void* x, const void* W1,
                             const void* W1_s, const void* W2, const void* W2_s, float* scores, void* ws) {
  float* hid = (float*)((uint8_t*)ws + 256);
  switch (nb_class(B)) {
    case 1: return run<1>(s, B, d, h, f, x, W1, W1_s, W2, W2_s, scores, hid);
    case 2: return run<2>(s, B, d, h, f, x, W1, W1_s, W2, W2_s, scores, hid);
    case 4: return run<4>(s, B, d, h, f, x, W1, W1_s, W2, W2_s, scores, hid);
    case 8: return run<8>(s, B, d, h, f, x, W1, W1_s, W2, W2_s, scores, hid);
    case 16: return run<16>(s, B, d, h, f, x, W1, W1_s, W2, W2_s, scores, hid);
    case 32: return run<32>(s, B, d, h, f, x, W1, W1_s, W2, W2_s, scores, hid);
    default: return run<64>(s, B, d, h, f, x, W1, W1_s, W2, W2_s, scores, hid);
  }
}

}  // namespace sfx
