// Per-layer MLP predictor: scores_b = W2 max(W1 x_b, 0)
// (PowerInfer page, Method, per-layer predictor of §5.1: one hidden layer with ReLU,
// one score per FFN neuron).
//
// At small batch both layers are HBM streams of the weights: every weight byte is
// read once and feeds B multiply-adds.  Layer 1 gives one wave per hidden row;
// layer 2 gives each wave R rows of W2, so a lane keeps R 16-byte loads in flight
// per chunk.  The hidden vector is kept in fp32 (workspace), never rounded to the
// weight type.  From B = 3 on (fp16 / bf16) both layers are dense contractions
// and run on the matrix cores (k_predict_mfma.hip).
#include "sfx_common.hpp"
#include "sfx_launch.hpp"

namespace sfx {

hipError_t launch_pred_mfma(hipStream_t s, int wdt, int B, int d, int h, int f, const void* x, const void* W1,
                            const void* W2, void* ws, float* scores, uint32_t* range_flag);
bool pred_mfma_eligible(int wdt, int B, int h, int f);
size_t pred_mfma_ws_bytes(int wdt, int B, int h);

namespace {

constexpr int kU = 8;  // 16-byte chunks per lane issued together

// hidden[b][row] = max(W1[row] . x_b, 0); one wave per row.
template <class T, int NB>
__global__ __launch_bounds__(kBlock) void k_pred_hidden(const uint8_t* __restrict__ x,
                                                        const uint8_t* __restrict__ W1,
                                                        float* __restrict__ hid, int B, int d, int h) {
  const int lane = threadIdx.x & (kWave - 1);
  const int row = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (row >= h) return;
  const int nchunk = d / T::vec;
  const size_t row_bytes = (size_t)d * T::bytes;
  const uint8_t* wrow = W1 + (size_t)row * row_bytes;
  float acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = 0.f;

  // Chunk indices are clamped, not branched on, so every load of a batch is in
  // flight before the first is used (loads under per-chunk branches are issued
  // one round trip at a time).
  constexpr int KB = NB == 1 ? kU : NB == 2 ? 4 : 2;   // row chunks per lane per batch
  constexpr int TG = NB < 4 ? NB : 4;                  // tokens whose input chunks load together
  for (int c0 = 0; c0 < nchunk; c0 += KB * kWave) {
    Raw<16> w[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) w[u] = load_raw<16>(wrow + (size_t)min(c0 + u * kWave + lane, nchunk - 1) * 16);
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
            float wf[T::vec];
            unpack<T, 4>(w[u].w, wf);
#pragma unroll
            for (int t = 0; t < TG; ++t) {
              if (b0 + t < B) {
                float xf[T::vec];
                unpack<T, 4>(xq[u][t].w, xf);
#pragma unroll
                for (int e = 0; e < T::vec; ++e) acc[b0 + t] = fmaf(wf[e], xf[e], acc[b0 + t]);
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

// scores[b][i] = W2[i] . hidden_b; each wave owns R consecutive rows.
template <class T, int NB, int R>
__global__ __launch_bounds__(kBlock) void k_pred_scores(const uint8_t* __restrict__ W2,
                                                        const float* __restrict__ hid,
                                                        float* __restrict__ scores, int B, int h, int f) {
  const int lane = threadIdx.x & (kWave - 1);
  const int row0 = (blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6)) * R;
  if (row0 >= f) return;
  const int nchunk = h / T::vec;
  const size_t row_bytes = (size_t)h * T::bytes;
  float acc[R][NB];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[r][b] = 0.f;

  // Rows past f and chunks past the row end are clamped, not branched on, so the
  // R x KC weight loads of a batch and the hidden loads are all in flight together.
  constexpr int KC = R >= 4 ? 2 : 4;                  // chunks per lane per batch
  for (int c0 = 0; c0 < nchunk; c0 += KC * kWave) {
    Raw<16> w[KC][R];
#pragma unroll
    for (int u = 0; u < KC; ++u) {
      const int c = min(c0 + u * kWave + lane, nchunk - 1);
#pragma unroll
      for (int r = 0; r < R; ++r) w[u][r] = load_raw<16>(W2 + (size_t)min(row0 + r, f - 1) * row_bytes + (size_t)c * 16);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b < B) {
        Raw<16> hq[KC][T::vec / 4];
#pragma unroll
        for (int u = 0; u < KC; ++u) {
          const int c = min(c0 + u * kWave + lane, nchunk - 1);
#pragma unroll
          for (int e = 0; e < T::vec / 4; ++e) hq[u][e] = load_raw<16>(hid + (size_t)b * h + (size_t)c * T::vec + e * 4);
        }
#pragma unroll
        for (int u = 0; u < KC; ++u) {
          if (c0 + u * kWave + lane < nchunk) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
              float wf[T::vec];
              unpack<T, 4>(w[u][r].w, wf);
#pragma unroll
              for (int e = 0; e < T::vec; ++e) acc[r][b] = fmaf(wf[e], __uint_as_float(hq[u][e / 4].w[e % 4]), acc[r][b]);
            }
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

template <class T, int NB>
hipError_t run(hipStream_t s, int B, int d, int h, int f, const void* x, const void* W1,
               const void* W2, float* scores, float* hid, bool mfma, int wdt, uint32_t* range_flag) {
  if (mfma) return launch_pred_mfma(s, wdt, B, d, h, f, x, W1, W2, hid, scores, range_flag);   // hid = the pieces buffer
  dim3 blk(kBlock);
  k_pred_hidden<T, NB><<<dim3((h + kWavesPerBlock - 1) / kWavesPerBlock), blk, 0, s>>>(
      (const uint8_t*)x, (const uint8_t*)W1, hid, B, d, h);
  constexpr int R = NB == 1 ? 4 : NB == 2 ? 2 : 1;
  const int rows_per_block = kWavesPerBlock * R;
  k_pred_scores<T, NB, R><<<dim3((f + rows_per_block - 1) / rows_per_block), blk, 0, s>>>(
      (const uint8_t*)W2, hid, scores, B, h, f);
  return hipGetLastError();
}

template <class T>
hipError_t dispatch_nb(hipStream_t s, int B, int d, int h, int f, const void* x, const void* W1,
                       const void* W2, float* scores, float* hid, bool mfma, int wdt, uint32_t* flag) {
  switch (nb_class(B)) {
    case 1: return run<T, 1>(s, B, d, h, f, x, W1, W2, scores, hid, mfma, wdt, flag);
    case 2: return run<T, 2>(s, B, d, h, f, x, W1, W2, scores, hid, mfma, wdt, flag);
    case 4: return run<T, 4>(s, B, d, h, f, x, W1, W2, scores, hid, mfma, wdt, flag);
    case 8: return run<T, 8>(s, B, d, h, f, x, W1, W2, scores, hid, mfma, wdt, flag);
    case 16: return run<T, 16>(s, B, d, h, f, x, W1, W2, scores, hid, mfma, wdt, flag);
    case 32: return run<T, 32>(s, B, d, h, f, x, W1, W2, scores, hid, mfma, wdt, flag);
    default: return run<T, 64>(s, B, d, h, f, x, W1, W2, scores, hid, mfma, wdt, flag);
  }
}

}  // namespace

// control line (word 0: sticky fp16-range flag of the matrix-core path) | the fp32
// hidden [B][h] (vector path) or the pieces, tickets and partial tiles (matrix cores)
constexpr size_t kCtlBytes = 256;

size_t predict_ws_bytes(int wdt, int B, int d, int h, int f) {
  (void)d;
  size_t hid = (size_t)B * h * sizeof(float);
  if (pred_mfma_eligible(wdt, B, h, f)) hid = pred_mfma_ws_bytes(wdt, B, h);
  return kCtlBytes + ((hid + 255) & ~(size_t)255);
}

hipError_t launch_predict(hipStream_t s, int wdt, int B, int d, int h, int f, const void* x,
                          const void* W1, const void* W2, float* scores, void* ws) {
  uint32_t* flag = (uint32_t*)ws;
  float* hid = (float*)((uint8_t*)ws + kCtlBytes);
  const bool mfma = pred_mfma_eligible(wdt, B, h, f);
  switch (wdt) {
    case DT_F32: return dispatch_nb<TF32>(s, B, d, h, f, x, W1, W2, scores, hid, mfma, wdt, flag);
    case DT_F16: return dispatch_nb<TF16>(s, B, d, h, f, x, W1, W2, scores, hid, mfma, wdt, flag);
    case DT_BF16: return dispatch_nb<TBF16>(s, B, d, h, f, x, W1, W2, scores, hid, mfma, wdt, flag);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sfx
