// Per-layer predictor on the matrix cores for B >= 3 tokens (PowerInfer page,
// Method, per-layer predictor of §5.1).  From 3 tokens on, each predictor weight
// feeds >= 3 multiply-adds and the two layers are dense contractions:
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
//
// Layer 1 writes the pieces once, already in layer 2's B-operand layout
// (hp[piece][token][hidden row], 16-bit), so layer 2 copies them into LDS with
// plain 16-byte loads and stores and reads its B fragments from there.
#include "sfx_launch.hpp"
#include "sfx_mfma.hpp"

namespace sfx {
namespace {

// ------------------------------------------------------------------ layer 1
// Workgroup = one tile of 16 W1 rows and one of S equal parts of the d walk; its
// 16 waves take interleaved 32-wide k steps (kHU in flight each); every wave's
// partial tile goes to LDS, and wave n adds token tile n's partials in wave order.
// With S > 1 (fewer row tiles than compute units) each part stores its tile
// write-through and takes the tile's ticket; the last part to arrive reads the S
// tiles with agent-scope loads, adds them in part order, resets the ticket and
// goes on as the only part would: ReLU, split, store the pieces (pad tokens past B
// store 0).
constexpr int kHW = 16;
constexpr int kHU = 4;
constexpr int kPredCUs = 256;   // split the d walk until the tiles reach this many workgroups
constexpr int kMaxSplit = 4;

__device__ __forceinline__ unsigned long long ld_agent64(const void* p) {
  return __hip_atomic_load(reinterpret_cast<const unsigned long long*>(p), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

int hidden_split(int h) {
  const int tiles = (h + 15) / 16;
  const int S = kPredCUs / tiles;
  return S < 1 ? 1 : S > kMaxSplit ? kMaxSplit : S;
}

template <class T, int NT>
__global__ __launch_bounds__(kHW * kWave) void k_hidden_mfma(const uint8_t* __restrict__ x,
                                                            const uint8_t* __restrict__ W1,
                                                            uint16_t* __restrict__ hp, int B, int d, int h,
                                                            int S, float* __restrict__ part,
                                                            uint32_t* __restrict__ tickets,
                                                            uint32_t* __restrict__ range_flag) {
  constexpr int NP = Split<T>::pieces;
  __shared__ f32x4 s_acc[kHW][NT][kWave];
  __shared__ int s_last;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int tiles = (h + 15) >> 4;
  const int tile = blockIdx.x % tiles;
  const int sp = blockIdx.x / tiles;            // part of the d walk
  const int row0 = tile * 16;
  const int r = min(row0 + (lane & 15), h - 1);      // rows past h read row h - 1, never stored
  const int kq = (lane >> 4) * 8;
  const int nsteps = (d + 31) >> 5;
  const uint8_t* ar = W1 + (size_t)r * d * 2;
  const uint8_t* xr[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) xr[n] = x + (size_t)min(n * 16 + (lane & 15), B - 1) * d * 2;
  f32x4 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int sb = (int)((long long)nsteps * sp / S);
  const int se = (int)((long long)nsteps * (sp + 1) / S);
  for (int s0 = sb + wave; s0 < se; s0 += kHW * kHU) {
    Raw<16> a[kHU], bx[kHU][NT];
#pragma unroll
    for (int u = 0; u < kHU; ++u) {
      // a step of the next part re-reads this wave's first step (a cache hit)
      const int st = s0 + u * kHW < se ? s0 + u * kHW : s0;
      const size_t off = (size_t)min(st * 32 + kq, d - 8) * 2;
      a[u] = load_raw<16>(ar + off);
#pragma unroll
      for (int n = 0; n < NT; ++n) bx[u][n] = load_raw<16>(xr[n] + off);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kHU; ++u) {
      // steps of the next part and columns past d add nothing
      if (s0 + u * kHW >= se || (s0 + u * kHW) * 32 + kq >= d) a[u] = zero16();
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[n] = Mma<T>::run(a[u], bx[u][n], acc[n]);
    }
  }
#pragma unroll
  for (int n = 0; n < NT; ++n) s_acc[wave][n][lane] = acc[n];
  __syncthreads();
  f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
  if (wave < NT) {
    t = s_acc[0][wave][lane];
    for (int v = 1; v < kHW; ++v) t += s_acc[v][wave][lane];
  }
  if (S > 1) {
    // part tile [tile][sp][n][lane] (16 bytes per lane)
    auto slot = [&](int q) { return part + (((size_t)tile * S + q) * NT + wave) * kWave * 4 + lane * 4; };
    if (wave < NT) {
      store_through2(slot(sp), t[0], t[1]);
      store_through2(slot(sp) + 2, t[2], t[3]);
    }
    wait_memory();
    __syncthreads();
    if (threadIdx.x == 0) s_last = (take_ticket(tickets + tile) == (uint32_t)(S - 1));
    __syncthreads();
    if (!s_last) return;
    if (threadIdx.x == 0) tickets[tile] = 0u;   // ready for the next call
    if (wave < NT) {
      unsigned long long v[kMaxSplit][2];
#pragma unroll
      for (int q = 0; q < kMaxSplit; ++q) {
        const float* pq = slot(min(q, S - 1));
        v[q][0] = ld_agent64(pq);
        v[q][1] = ld_agent64(pq + 2);
      }
      t = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < kMaxSplit; ++q)
        if (q < S) {
          t[0] += __uint_as_float((uint32_t)v[q][0]);
          t[1] += __uint_as_float((uint32_t)(v[q][0] >> 32));
          t[2] += __uint_as_float((uint32_t)v[q][1]);
          t[3] += __uint_as_float((uint32_t)(v[q][1] >> 32));
        }
    }
  }
  if (wave < NT) {
    const int n = wave;
    // D layout: lane l holds rows 4 (l / 16) + i of the tile for token l % 16.
    const int tok = n * 16 + (lane & 15);
    const size_t tstride = (size_t)NT * 16 * h;   // one piece plane
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = row0 + (lane >> 4) * 4 + i;
      if (row < h) {
        uint16_t pc[NP];
        const float hv = tok < B ? fmaxf(t[i], 0.f) : 0.f;
        // fp16 pieces: a hidden value past the fp16 range has no finite leading
        // piece; the call's scores are then wrong, so the sticky flag records it
        if (Split<T>::max_finite > 0.f && !(hv <= Split<T>::max_finite)) store_through(range_flag, 1u);
        Split<T>::run(hv, pc);
#pragma unroll
        for (int p = 0; p < NP; ++p) hp[p * tstride + (size_t)tok * h + row] = pc[p];
      }
    }
  }
}

// ------------------------------------------------------------------ layer 2
// Each wave owns one tile of 16 W2 rows and walks the h columns in 32-wide steps,
// kSU steps in flight: one 16-byte W2 load per lane and step (16 steps measured
// 9% faster than 4 on the Falcon-40B shape; issuing the first batch before the
// staging barrier measured slower).  The pieces (the B
// operand, shared by every wave) are staged in LDS, KC columns at a time, by the
// whole workgroup: read from memory by every wave at every step they tripled the
// load requests and halved the W2 stream.  With fewer than 256 workgroups of 8
// row tiles (small f), two waves share a row tile (wpt = 2), taking alternate
// batches of steps; the second adds its tile to the first through LDS.
constexpr int kSWB = 8;   // waves per workgroup
constexpr int kSU = 16;

template <class T, int NT>
struct ScoreTile {
  static constexpr int NP = Split<T>::pieces;
  static constexpr int rows = NP * NT * 16;                       // piece rows in LDS
  static constexpr int KC = rows <= 32 ? 2048 : rows <= 64 ? 1024 : rows <= 128 ? 512 : 256;   // columns per stage
  static constexpr int KS = KC + 8;                               // halves per LDS row (16-byte skew)
};

template <class T, int NT>
__global__ __launch_bounds__(kSWB * kWave) void k_scores_mfma(const uint8_t* __restrict__ W2,
                                                             const uint16_t* __restrict__ hp,
                                                             float* __restrict__ scores, int B, int h, int f,
                                                             int wpt) {
  using G = ScoreTile<T, NT>;
  constexpr int NP = G::NP;
  constexpr int NACC = Split<T>::accumulators;
  constexpr int KC = G::KC, KS = G::KS, NR = G::rows;
  __shared__ __attribute__((aligned(16))) uint16_t s_p[NR * KS];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = wave % wpt;                  // this wave's share of the tile's steps
  const int row0 = (blockIdx.x * (kSWB / wpt) + wave / wpt) * 16;
  const bool active = row0 < f;                 // no early exit: the workgroup stages together
  const int r = min(row0 + (lane & 15), f - 1);
  const int kq = (lane >> 4) * 8;
  const uint8_t* ar = W2 + (size_t)r * h * 2;
  const size_t tstride = (size_t)NT * 16 * h;
  f32x4 acc[NACC][NT];
#pragma unroll
  for (int q = 0; q < NACC; ++q)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[q][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int kc = 0; kc < h; kc += KC) {
    const int cw = min(KC, h - kc);            // a multiple of 8: rows span multiples of 16 bytes
    // stage piece rows (piece p, token t) columns [kc, kc + cw): 16 bytes per item,
    // every item of a thread loaded before the first is stored
    __syncthreads();                           // the previous stage is consumed
    {
      constexpr int IPT = (NR * (KC / 8) + kSWB * kWave - 1) / (kSWB * kWave);
      const int per_row = cw >> 3, items = NR * per_row;
      Raw<16> v[IPT];
#pragma unroll
      for (int q = 0; q < IPT; ++q) {
        const int i = min(tid + q * kSWB * kWave, items - 1);
        const int pr = i / per_row, c8 = i - pr * per_row;
        const int p = pr / (NT * 16), t = pr - p * (NT * 16);
        v[q] = load_raw<16>(hp + p * tstride + (size_t)t * h + kc + c8 * 8);
      }
#pragma unroll
      for (int q = 0; q < IPT; ++q) {
        const int i = tid + q * kSWB * kWave;
        if (i < items) {
          const int pr = i / per_row, c8 = i - pr * per_row;
          *reinterpret_cast<Raw<16>*>(s_p + pr * KS + c8 * 8) = v[q];
        }
      }
    }
    __syncthreads();
    if (active) {
      const int nst = (cw + 31) >> 5;
      for (int s0 = half * kSU; s0 < nst; s0 += wpt * kSU) {
        Raw<16> a[kSU];
#pragma unroll
        for (int u = 0; u < kSU; ++u) {
          const int c = min(kc + (s0 + u) * 32 + kq, h - 8);
          a[u] = load_raw<16>(ar + (size_t)c * 2);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kSU; ++u) {
          const int cl = (s0 + u) * 32 + kq;    // column within the stage
          if (cl >= cw) a[u] = zero16();       // past the stage (or past h): adds nothing
          const int clc = min(cl, cw - 8);     // read a staged column there (finite, times zero)
#pragma unroll
          for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int p = 0; p < NP; ++p) {
              const Raw<16> bv = *reinterpret_cast<const Raw<16>*>(s_p + (p * NT * 16 + n * 16 + (lane & 15)) * KS + clc);
              const int q = NACC == 1 ? 0 : p;
              acc[q][n] = Mma<T>::run(a[u], bv, acc[q][n]);
            }
        }
      }
    }
  }
  if (wpt > 1) {
    // the staged pieces are consumed: the second wave of each tile parks its
    // partial tile where they were, the first adds it
    f32x4* s_red = reinterpret_cast<f32x4*>(s_p);
    const int slot = (wave / wpt) * NACC * NT;
    __syncthreads();
    if (half == 1) {
#pragma unroll
      for (int q = 0; q < NACC; ++q)
#pragma unroll
        for (int n = 0; n < NT; ++n) s_red[(slot + q * NT + n) * kWave + lane] = acc[q][n];
    }
    __syncthreads();
    if (half == 1) return;
#pragma unroll
    for (int q = 0; q < NACC; ++q)
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[q][n] += s_red[(slot + q * NT + n) * kWave + lane];
  }
  if (!active) return;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int tok = n * 16 + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = row0 + (lane >> 4) * 4 + i;
      const float v = Split<T>::combine(acc[0][n][i], acc[NACC - 1][n][i]);
      if (tok < B && row < f) scores[(size_t)tok * f + row] = v;
    }
  }
}

template <class T, int NT>
hipError_t run(hipStream_t s, int B, int d, int h, int f, const void* x, const void* W1, const void* W2,
               uint16_t* hp, float* scores, float* part, uint32_t* tickets, uint32_t* range_flag) {
  const int S = hidden_split(h);
  k_hidden_mfma<T, NT><<<dim3(((h + 15) / 16) * S), dim3(kHW * kWave), 0, s>>>(
      (const uint8_t*)x, (const uint8_t*)W1, hp, B, d, h, S, part, tickets, range_flag);
  const int rtiles = (f + 15) / 16;
  const int wpt = (rtiles + kSWB - 1) / kSWB < kPredCUs ? 2 : 1;
  const int per_wg = kSWB / wpt;
  k_scores_mfma<T, NT><<<dim3((rtiles + per_wg - 1) / per_wg), dim3(kSWB * kWave), 0, s>>>(
      (const uint8_t*)W2, hp, scores, B, h, f, wpt);
  return hipGetLastError();
}

template <class T>
hipError_t dispatch(hipStream_t s, int B, int d, int h, int f, const void* x, const void* W1, const void* W2,
                    uint16_t* hp, float* scores, float* part, uint32_t* tickets, uint32_t* range_flag) {
  if (B <= 16) return run<T, 1>(s, B, d, h, f, x, W1, W2, hp, scores, part, tickets, range_flag);
  if (B <= 32) return run<T, 2>(s, B, d, h, f, x, W1, W2, hp, scores, part, tickets, range_flag);
  return run<T, 4>(s, B, d, h, f, x, W1, W2, hp, scores, part, tickets, range_flag);
}

size_t up256(size_t n) { return (n + 255) & ~(size_t)255; }
int token_tiles(int B) { return B <= 16 ? 1 : B <= 32 ? 2 : 4; }

}  // namespace

bool pred_mfma_eligible(int wdt, int B, int h, int f) {
  (void)h; (void)f;
  return (wdt == DT_F16 || wdt == DT_BF16) && B >= 3 && B <= 64;   // as down: from 3 tokens
}

// Pieces (pieces x 16 token-tile rows x h halves) | with S > 1 parts of the d
// walk: one ticket per row tile | S partial tiles per row tile (fp32).
size_t pred_mfma_ws_bytes(int wdt, int B, int h) {
  const int np = wdt == DT_BF16 ? Split<TBF16>::pieces : Split<TF16>::pieces;
  const int nt = token_tiles(B);
  const int tiles = (h + 15) / 16, S = hidden_split(h);
  size_t n = up256((size_t)np * nt * 16 * h * sizeof(uint16_t));
  if (S > 1) n += up256((size_t)tiles * 4) + (size_t)S * tiles * nt * 16 * 16 * sizeof(float);
  return n;
}

hipError_t launch_pred_mfma(hipStream_t s, int wdt, int B, int d, int h, int f, const void* x, const void* W1,
                            const void* W2, void* ws, float* scores, uint32_t* range_flag) {
  const int np = wdt == DT_BF16 ? Split<TBF16>::pieces : Split<TF16>::pieces;
  const int tiles = (h + 15) / 16;
  uint8_t* base = (uint8_t*)ws;
  uint16_t* hp = (uint16_t*)base;
  const size_t off_t = up256((size_t)np * token_tiles(B) * 16 * h * sizeof(uint16_t));
  uint32_t* tickets = (uint32_t*)(base + off_t);
  float* part = (float*)(base + off_t + up256((size_t)tiles * 4));
  if (wdt == DT_F16) return dispatch<TF16>(s, B, d, h, f, x, W1, W2, hp, scores, part, tickets, range_flag);
  return dispatch<TBF16>(s, B, d, h, f, x, W1, W2, hp, scores, part, tickets, range_flag);
}

}  // namespace sfx
