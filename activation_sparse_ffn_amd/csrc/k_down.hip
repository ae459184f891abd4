// Gathered neuron-major down rows (PowerInfer page, Method: hybrid-execution
// pseudocode, y is the sum of the active neurons' contributions; neuron-aware
// operators of §5.4, each block owns a disjoint set of neurons).
//
//   y[b][:] = sum_{j < count} hact[j][b] * Wd[idx_j][:]
//
// Grid = S neuron slices x T column tiles.  Workgroup (s, t) reads the tile-t
// segment (64 lanes x LW bytes, contiguous) of list rows s, s + S, s + 2S, ...
// (the slice), with their indices and activations staged in LDS, accumulates
// B x CPL fp32 sums per lane, adds its four waves in LDS in a fixed order and
// writes one partial tile.  The last workgroup of a tile to finish (ticket in the
// workspace) adds the S partials in slice order and writes y: no atomics on data,
// and y is the same bit for bit on every run.
#include <atomic>
#include <mutex>

#include "sfx_common.hpp"
#include "sfx_launch.hpp"
#include "sfx_mfma.hpp"

namespace sfx {
namespace {

constexpr int kTargetBlocks = 256;
constexpr int kMaxSlices = 64;

// Decoded columns of one lane's segment.
template <class T, int LW>
struct Seg {
  static constexpr int cpl = LW / T::bytes;
  __device__ static void decode(const Raw<LW>& r, const uint16_t*, int, float* o) { unpack<T, LW / 4>(r.w, o); }
};
struct TQ4 { static constexpr int bytes = 0; };
template <int LW>
struct Seg<TQ4, LW> {
  static constexpr int cpl = LW * 2;
  // Codes only: the group's fp16 scale is applied to hact by the caller.
  __device__ static void decode(const Raw<LW>& r, const uint16_t*, int, float* o) {
#pragma unroll
    for (int q = 0; q < LW / 4; ++q)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[q * 8 + e] = (float)((int32_t)(r.w[q] << (28 - 4 * e)) >> 28);
  }
};

template <class T>
struct RowGeom {
  __device__ static size_t row_bytes(int d) { return (size_t)d * T::bytes; }
  __device__ static size_t col_byte(int col) { return (size_t)col * T::bytes; }
};
template <>
struct RowGeom<TQ4> {
  __device__ static size_t row_bytes(int d) { return (size_t)d >> 1; }
  __device__ static size_t col_byte(int col) { return (size_t)col >> 1; }
};

// Called by every thread of a workgroup after its partial tile has been stored
// (agent-scope stores).  The last workgroup of the tile to take the ticket adds
// the S partials in slice order and writes y.  Each thread owns 4 consecutive
// columns of one token and keeps up to 32 partial loads in flight.
__device__ __forceinline__ void finish_tile(const float* __restrict__ part, uint32_t* __restrict__ tickets,
                                            float* __restrict__ y, int B, int d, int S, int ntiles, int tile,
                                            int TW) {
  __shared__ int s_last;
  wait_memory();
  __syncthreads();
  if (threadIdx.x == 0) s_last = (take_ticket(tickets + tile) == (uint32_t)(S - 1));
  __syncthreads();
  if (!s_last) return;
  acquire_agent();

  for (int e = threadIdx.x; e < B * (TW / 4); e += kBlock) {
    const int b = e / (TW / 4);
    const int cc = (e - b * (TW / 4)) * 4;
    const int col = tile * TW + cc;
    if (col >= d) continue;
    float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = 0; s0 < S; s0 += 32) {
      float4 v[32];
#pragma unroll
      for (int u = 0; u < 32; ++u)
        v[u] = *reinterpret_cast<const float4*>(part + ((size_t)(min(s0 + u, S - 1) * ntiles + tile) * B + b) * TW + cc);
#pragma unroll
      for (int u = 0; u < 32; ++u)
        if (s0 + u < S) { sum.x += v[u].x; sum.y += v[u].y; sum.z += v[u].z; sum.w += v[u].w; }
    }
    float* yo = y + (size_t)b * d + col;
    yo[0] = sum.x;
    if (col + 1 < d) yo[1] = sum.y;
    if (col + 2 < d) yo[2] = sum.z;
    if (col + 3 < d) yo[3] = sum.w;
  }
  if (threadIdx.x == 0) tickets[tile] = 0u;
}

template <class T, int NB, int LW>
__global__ __launch_bounds__(kBlock) void k_down(const uint8_t* __restrict__ Wd, const uint16_t* __restrict__ Wd_s,
                                                 const int32_t* __restrict__ idx, const int32_t* __restrict__ count,
                                                 int kmax, const float* __restrict__ hact, int B, int d, int f,
                                                 float* __restrict__ y, float* __restrict__ part,
                                                 uint32_t* __restrict__ tickets, int S, int ntiles) {
  constexpr int CPL = Seg<T, LW>::cpl;
  constexpr int TW = kWave * CPL;
  constexpr bool Q4 = T::bytes == 0;
  constexpr int kRowsInFlight = 16;                   // rows per wave whose segments load together
  constexpr int CH = kWavesPerBlock * kRowsInFlight;  // rows per staged chunk
  __shared__ float s_red[kWavesPerBlock - 1][NB][TW];
  __shared__ float s_h[CH * NB];
  __shared__ int s_idx[CH];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int tile = blockIdx.x % ntiles;
  const int slice = blockIdx.x / ntiles;
  const int k = min(*count, kmax);
  const int col0 = tile * TW + lane * CPL;
  const bool valid = col0 < d;
  const size_t rb = RowGeom<T>::row_bytes(d);
  const size_t cb = RowGeom<T>::col_byte(valid ? col0 : 0);  // lanes past d read column 0, never store
  const int ngroup = d >> 5;

  float acc[NB][CPL];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[b][c] = 0.f;

  // Slice s takes rows j = s, s + S, s + 2S, ... (CH of them per chunk), so the
  // first chunk's index and activation loads do not depend on the count and go
  // out together with it.  Rows past the count are skipped; loads past kmax are
  // clamped (idx and hact hold kmax rows).
  int m = 0;
  do {
    const int jr = slice + S * m * CH;  // row of chunk entry 0; entry r is jr + S * r
    {
      constexpr int HQ = (CH * NB + kBlock - 1) / kBlock;
      const int jt = jr + S * min((int)threadIdx.x, CH - 1);
      const int it = idx[min(jt, kmax - 1)];          // issued with the activation loads
      float hv[HQ];
#pragma unroll
      for (int q = 0; q < HQ; ++q) {
        const int e = min((int)threadIdx.x + q * kBlock, CH * NB - 1);
        const int j = jr + S * (e / NB);
        hv[q] = hact[(size_t)min(j, kmax - 1) * B + min(e % NB, B - 1)];
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < HQ; ++q) {
        const int e = threadIdx.x + q * kBlock;
        if (e < CH * NB) s_h[e] = hv[q];
      }
      if (threadIdx.x < CH) s_idx[threadIdx.x] = (jt >= k || (unsigned)it >= (unsigned)f) ? -1 : it;
    }
    __syncthreads();

    // Entry r of the chunk goes to wave r mod 4; every segment load is issued
    // before the first is used (skipped entries read row 0).
    Raw<LW> w[kRowsInFlight];
    float sc[kRowsInFlight];
    int rowi[kRowsInFlight];
#pragma unroll
    for (int u = 0; u < kRowsInFlight; ++u) {
      const int i = s_idx[wave + u * kWavesPerBlock];
      rowi[u] = i;
      const size_t ir = (size_t)(i < 0 ? 0 : i);
      w[u] = load_raw<LW>(Wd + ir * rb + cb);
      if (Q4) sc[u] = (float)__builtin_bit_cast(_Float16, Wd_s[ir * ngroup + ((valid ? col0 : 0) >> 5)]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kRowsInFlight; ++u) {
      if (rowi[u] >= 0) {
        const int r = wave + u * kWavesPerBlock;
        float wf[CPL];
        Seg<T, LW>::decode(w[u], nullptr, 0, wf);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          if (b < B) {
            float hv = s_h[r * NB + b];
            if (Q4) hv *= sc[u];
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[b][c] = fmaf(hv, wf[c], acc[b][c]);
          }
        }
      }
    }
    __syncthreads();
  } while (slice + S * (++m) * CH < k);

  // Combine the four waves in LDS: wave 0 + wave 1 + wave 2 + wave 3, in that order.
  if (wave > 0) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int c = 0; c < CPL; ++c) s_red[wave - 1][b][lane * CPL + c] = acc[b][c];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int v = 0; v < kWavesPerBlock - 1; ++v)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[b][c] += s_red[v][b][lane * CPL + c];
    if (valid) {
      if (S == 1) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
          if (b < B)
#pragma unroll
            for (int c = 0; c < CPL; ++c)
              if (col0 + c < d) y[(size_t)b * d + col0 + c] = acc[b][c];
      } else {
        float* p = part + ((size_t)(slice * ntiles + tile) * B) * TW;
#pragma unroll
        for (int b = 0; b < NB; ++b)
          if (b < B) {
            if constexpr (CPL % 2 == 0) {
#pragma unroll
              for (int c = 0; c < CPL; c += 2)
                store_through2(p + (size_t)b * TW + lane * CPL + c, acc[b][c], acc[b][c + 1]);
            } else {
#pragma unroll
              for (int c = 0; c < CPL; ++c) store_through(p + (size_t)b * TW + lane * CPL + c, acc[b][c]);
            }
          }
      }
    }
  }
  if (S == 1) return;

  finish_tile(part, tickets, y, B, d, S, ntiles, tile, TW);
}


// ------------------------------------------------------------------ B <= 2, 16-bit rows
// Column tiles without partial sums: workgroup t owns columns [CW t, CW t + CW) of
// y and reads that segment of every listed row (CW / 8 lanes per row, 256 / (CW /
// 8) row slots per workgroup, kCU rows per slot in flight), so y is written by its
// owner after a fixed-order sum over the slots: two dependent round trips
// (indices and activations, then the row segments) instead of the slices' five
// (plus write-through partials, a ticket and the last workgroup's reduction).
// Tiles are numbered so that the four tiles sharing a 128-byte line of a row run
// on one XCD (workgroups are dispatched round-robin over the 8 XCDs).
// CW = 16 columns (32-byte segments) up to d = 4096; 32 columns (64-byte segments,
// half as many workgroups) above.
template <class T, int NB, int CW>
__global__ __launch_bounds__(kBlock) void k_down_cols(const uint8_t* __restrict__ Wd,
                                                      const int32_t* __restrict__ idx,
                                                      const int32_t* __restrict__ count, int kmax,
                                                      const float* __restrict__ hact, int B, int d, int f,
                                                      float* __restrict__ y, int ntiles) {
  constexpr int kLPR = CW / 8;            // lanes per row
  constexpr int kColSlots = kBlock / kLPR;
  constexpr int kCU = NB == 1 ? 16 : 8;   // rows per slot in flight
  constexpr int kColW = CW;
  __shared__ float s_sum[kWavesPerBlock][kLPR][NB][8];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int w = blockIdx.x, P = gridDim.x;
  const int tile = (P % 8 == 0 && P == ntiles) ? (w & 7) * (P >> 3) + (w >> 3) : w;
  const int half = threadIdx.x & (kLPR - 1);
  const int slot = threadIdx.x / kLPR;
  const int col = tile * kColW + half * 8;
  const bool cok = col < d;
  const size_t rb = (size_t)d * 2;
  const size_t cb = (size_t)(cok ? col : 0) * 2;
  const int k = min(*count, kmax);
  float acc[NB][8];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[b][e] = 0.f;
  for (int r0 = slot; r0 < k; r0 += kColSlots * kCU) {
    int nid[kCU];
    float hv[kCU][NB];
#pragma unroll
    for (int u = 0; u < kCU; ++u) {
      const int r = min(r0 + u * kColSlots, k - 1);
      nid[u] = idx[r];
#pragma unroll
      for (int b = 0; b < NB; ++b) hv[u][b] = hact[(size_t)r * B + min(b, B - 1)];
    }
    Raw<16> wv[kCU];
#pragma unroll
    for (int u = 0; u < kCU; ++u) {
      const int i = (unsigned)nid[u] < (unsigned)f ? nid[u] : 0;
      wv[u] = load_raw<16>(Wd + (size_t)i * rb + cb);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kCU; ++u) {
      if (r0 + u * kColSlots < k && (unsigned)nid[u] < (unsigned)f) {
        float wf[8];
        unpack<T, 4>(wv[u].w, wf);
#pragma unroll
        for (int b = 0; b < NB; ++b)
          if (b < B) {
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[b][e] = fmaf(hv[u][b], wf[e], acc[b][e]);
          }
      }
    }
  }
  // sum the slots: lanes of one column chunk within the wave (fixed butterfly
  // over the lane bits above the chunk), then the four waves in order
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = acc[b][e];
      if constexpr (kLPR <= 1) v += __uint_as_float(lane_xor_u32<1>(__float_as_uint(v), lane));
      if constexpr (kLPR <= 2) v += __uint_as_float(lane_xor_u32<2>(__float_as_uint(v), lane));
      if constexpr (kLPR <= 4) v += __uint_as_float(lane_xor_u32<4>(__float_as_uint(v), lane));
      if constexpr (kLPR <= 8) v += __uint_as_float(lane_xor_u32<8>(__float_as_uint(v), lane));
      v += __uint_as_float(lane_xor_u32<16>(__float_as_uint(v), lane));
      v += __uint_as_float(lane_xor_u32<32>(__float_as_uint(v), lane));
      acc[b][e] = v;
    }
  if (lane < kLPR) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int e = 0; e < 8; ++e) s_sum[wave][lane][b][e] = acc[b][e];
  }
  __syncthreads();
  if (threadIdx.x < kLPR * NB * 8) {
    const int hh = threadIdx.x / (NB * 8), rem = threadIdx.x % (NB * 8), b = rem / 8, e = rem % 8;
    const int c = tile * kColW + hh * 8 + e;
    if (b < B && c < d) {
      float t = 0.f;
#pragma unroll
      for (int v = 0; v < kWavesPerBlock; ++v) t += s_sum[v][hh][b][e];
      y[(size_t)b * d + c] = t;
    }
  }
}

// ------------------------------------------------------------------ B <= 2, int4 rows
// The column-tile kernel for int4 g32 rows: workgroup t owns the 32 columns of group
// t (16 bytes of codes and one fp16 scale per row), one lane per row, kCU rows per
// lane in flight; the scale folds into the activation (q s h as q (s h): only the
// rounding order differs from the decoded product).  No partial sums: indices and
// activations, then codes and scales, two dependent round trips (the slice kernel
// also wrote and re-read 2 MB of partial tiles per call at the OPT-30B shape).
template <int NB>
__global__ __launch_bounds__(kBlock) void k_down_cols_q4(const uint8_t* __restrict__ Wd,
                                                         const uint16_t* __restrict__ Wd_s,
                                                         const int32_t* __restrict__ idx,
                                                         const int32_t* __restrict__ count, int kmax,
                                                         const float* __restrict__ hact, int B, int d, int f,
                                                         float* __restrict__ y, int ntiles) {
  constexpr int kCU = NB == 1 ? 16 : 8;   // rows per lane in flight
  constexpr int V = 32 * NB;              // sums per lane: 32 columns x NB tokens
  __shared__ float s_sum[kWavesPerBlock][V];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int w = blockIdx.x, P = gridDim.x;
  const int tile = (P % 8 == 0 && P == ntiles) ? (w & 7) * (P >> 3) + (w >> 3) : w;
  const size_t rb = (size_t)d >> 1;       // code bytes per row
  const int ng = d >> 5;                  // scales per row
  const int k = min(*count, kmax);
  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.f;
  for (int r0 = threadIdx.x; r0 < k; r0 += kBlock * kCU) {
    int nid[kCU];
    float hv[kCU][NB];
#pragma unroll
    for (int u = 0; u < kCU; ++u) {
      const int r = min(r0 + u * kBlock, k - 1);
      nid[u] = idx[r];
#pragma unroll
      for (int b = 0; b < NB; ++b) hv[u][b] = hact[(size_t)r * B + min(b, B - 1)];
    }
    Raw<16> wv[kCU];
    uint16_t sc[kCU];
#pragma unroll
    for (int u = 0; u < kCU; ++u) {
      const int i = (unsigned)nid[u] < (unsigned)f ? nid[u] : 0;
      wv[u] = load_raw<16>(Wd + (size_t)i * rb + (size_t)tile * 16);
      sc[u] = Wd_s[(size_t)i * ng + tile];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kCU; ++u) {
      if (r0 + u * kBlock < k && (unsigned)nid[u] < (unsigned)f) {
        const float s = (float)__builtin_bit_cast(_Float16, sc[u]);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          if (b < B) {
            const float hs = hv[u][b] * s;
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
              for (int e = 0; e < 8; ++e)
                acc[b * 32 + q * 8 + e] =
                    fmaf((float)((int32_t)(wv[u].w[q] << (28 - 4 * e)) >> 28), hs, acc[b * 32 + q * 8 + e]);
          }
        }
      }
    }
  }
  // sum over the 64 lanes of each wave (halving exchanges), then the four waves in
  // order: lane L ends with sum index L >> (6 - log2 V)
  const float v = wave_reduce_multi<V>(acc);
  if ((lane & (kWave / V - 1)) == 0) s_sum[wave][lane >> (6 - ilog2c(V))] = v;
  __syncthreads();
  if (threadIdx.x < V) {
    const int b = threadIdx.x >> 5, c = tile * 32 + (threadIdx.x & 31);
    if (b < B && c < d) {
      float t = 0.f;
#pragma unroll
      for (int vv = 0; vv < kWavesPerBlock; ++vv) t += s_sum[vv][threadIdx.x];
      y[(size_t)b * d + c] = t;
    }
  }
}

// ------------------------------------------------------------------ B >= 3
// From 3 tokens on the products run on the matrix cores: v_mfma_f32_16x16x4_f32
// (fp32 operands, so the fp32 activations are used as they are and the 16-bit
// weights convert exactly).  A = 16 column slots x 4 list entries: lane l reads 16
// bytes (8 consecutive columns) of entry l / 16's row at column slot l % 16, which
// gives the A operand of 8 products, one per column of the slot; B = 4 list
// entries x 16 tokens, lane l holding the activation of entry l / 16 for token
// l % 16.  A tile is 128 columns (16 slots x 8) by all tokens.  Grid, slices,
// partial tiles and the fixed-order final sum are those of the kernel above;
// a slice takes groups of 4 list entries g = s, s + S, ..., its four waves every
// fourth of them, in batches of U groups: while a batch is multiplied the next
// batch's rows and the batch after that's indices and activations are loading.
// Up to 32 tokens the batch is sized so that two waves fit on each SIMD (one wave
// per SIMD left the matrix cores idle while it waited for rows).
constexpr int kMfmaTW = 128;

template <class T, int NT>
__global__ __launch_bounds__(kBlock, NT <= 2 ? 2 : 1) void k_down_mfma(const uint8_t* __restrict__ Wd,
                                                      const int32_t* __restrict__ idx,
                                                      const int32_t* __restrict__ count, int kmax,
                                                      const float* __restrict__ hact, int B, int d, int f,
                                                      float* __restrict__ y, float* __restrict__ part,
                                                      uint32_t* __restrict__ tickets, int S, int ntiles) {
  constexpr int TW = kMfmaTW;
  constexpr int U = NT <= 1 ? 8 : NT <= 2 ? 4 : 2;
  __shared__ f32x4 s_red[kWavesPerBlock - 1][8][NT][kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tile = blockIdx.x % ntiles;
  const int slice = blockIdx.x / ntiles;
  const int k = min(*count, kmax);
  const int ng = (k + 3) >> 2;
  const int r = lane >> 4;                        // list entry of this lane within a group
  const int col = tile * TW + 8 * (lane & 15);    // first of this lane's 8 columns
  const bool cvalid = col < d;
  const size_t rb = (size_t)d * 2;
  const size_t cb = (size_t)(cvalid ? col : 0) * 2;

  f32x4 acc[8][NT];
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[e][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Software pipeline over batches of U groups.  Metadata of a batch (list entry,
  // index, activations: raw clamped loads) goes out two batches ahead and its rows
  // one batch ahead, in the order M(i+2), W(i+1) before batch i is multiplied, so
  // the in-order memory counter lets the products of batch i start while W(i+1)
  // and M(i+2) are still in flight.
  struct Meta { int j[U], i[U]; float h[U][NT]; };
  auto load_meta = [&](Meta& m, int t0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long long g = (long long)slice + (long long)S * (t0 + 4 * u);
      const int j = (int)min(g * 4 + r, (long long)kmax);   // kmax marks "past the list"
      const int jc = min(j, kmax - 1);
      m.j[u] = j;
      m.i[u] = idx[jc];
#pragma unroll
      for (int n = 0; n < NT; ++n) m.h[u][n] = hact[(size_t)jc * B + min(n * 16 + (lane & 15), B - 1)];
    }
  };
  // Validity of a batch: rows past the count or out of [0, f) multiply as zeros
  // (their A and B operands are zero) and load row 0.
  auto settle = [&](const Meta& m, int (&iv)[U], float (&hv)[U][NT], Raw<16> (&w)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = m.j[u] < k && (unsigned)m.i[u] < (unsigned)f;
      iv[u] = ok ? m.i[u] : -1;
#pragma unroll
      for (int n = 0; n < NT; ++n) hv[u][n] = (ok && n * 16 + (lane & 15) < B) ? m.h[u][n] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = load_raw<16>(Wd + (size_t)(iv[u] < 0 ? 0 : iv[u]) * rb + cb);
  };

  auto multiply = [&](const int (&iv)[U], const float (&hv)[U][NT], const Raw<16> (&w)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float a[8];
      unpack<T, 4>(w[u].w, a);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float ae = iv[u] < 0 ? 0.f : a[e];
#pragma unroll
        for (int n = 0; n < NT; ++n)
          acc[e][n] = __builtin_amdgcn_mfma_f32_16x16x4f32(ae, hv[u][n], acc[e][n], 0, 0, 0);
      }
    }
  };
  // Two register sets used in turn (no copies between batches: a copy of a loaded
  // register would wait for its load).
  Meta mA, mB;
  int ivA[U], ivB[U];
  float hvA[U][NT], hvB[U][NT];
  Raw<16> wA[U], wB[U];
  load_meta(mA, wave);
  load_meta(mB, wave + 4 * U);
  settle(mA, ivA, hvA, wA);
  // Batches go in pairs with no exit between them (a load behind a conditional
  // exit would be moved down to its use); a batch past the list multiplies zeros.
  for (int t0 = wave; slice + (long long)S * t0 < ng; t0 += 8 * U) {
    load_meta(mA, t0 + 8 * U);
    settle(mB, ivB, hvB, wB);
    __builtin_amdgcn_sched_barrier(0);
    multiply(ivA, hvA, wA);
    __builtin_amdgcn_sched_barrier(0);
    load_meta(mB, t0 + 12 * U);
    settle(mA, ivA, hvA, wA);
    __builtin_amdgcn_sched_barrier(0);
    multiply(ivB, hvB, wB);
    __builtin_amdgcn_sched_barrier(0);
  }

  // Waves 1..3 to LDS; wave 0 adds them in wave order.  D layout: lane l holds
  // slots 4 (l / 16) + i for token l % 16; slot m, product e is column 8 m + e.
  if (wave > 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int n = 0; n < NT; ++n) s_red[wave - 1][e][n][lane] = acc[e][n];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll 1
    for (int v = 0; v < kWavesPerBlock - 1; ++v)
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[e][n] += s_red[v][e][n][lane];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int b = n * 16 + (lane & 15);
      if (b >= B) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = tile * TW + 8 * (4 * r + i);     // 8 consecutive columns c .. c + 7
        if (c >= d) continue;
        const float4 lo = make_float4(acc[0][n][i], acc[1][n][i], acc[2][n][i], acc[3][n][i]);
        const float4 hi = make_float4(acc[4][n][i], acc[5][n][i], acc[6][n][i], acc[7][n][i]);
        if (S == 1) {
          float4* yo = reinterpret_cast<float4*>(y + (size_t)b * d + c);
          yo[0] = lo;
          yo[1] = hi;
        } else {
          float* p = part + ((size_t)(slice * ntiles + tile) * B + b) * TW + (c - tile * TW);
          store_through2(p + 0, lo.x, lo.y);
          store_through2(p + 2, lo.z, lo.w);
          store_through2(p + 4, hi.x, hi.y);
          store_through2(p + 6, hi.z, hi.w);
        }
      }
    }
  }
  (void)cvalid;
  if (S == 1) return;
  finish_tile(part, tickets, y, B, d, S, ntiles, tile, TW);
}

// Load width (bytes per lane per row) for a storage type and token class: keep
// NB x CPL accumulators per lane at <= 64 (<= 128 for int4 at B = 16).  Tiles stay
// at <= 512 columns: the last workgroup of a tile reads S partial tiles, and wide
// tiles (few tiles, many slices) made that one workgroup read ~0.5 MB.
template <class T>
constexpr int lw_for(int nb) {
  return T::bytes == 0 ? 4   // 8 int4 columns per lane: 512-column tiles, as for 16-bit rows
                       : (nb * (16 / T::bytes) <= 64 ? 16 : nb * (8 / T::bytes) <= 64 ? 8 : 4);
}

struct Plan { int lw, cpl, tw, ntiles, S; bool mfma; };

// 16-bit rows at 1-2 tokens take the column-tile kernel (no workspace).
bool cols_eligible(int B) { return B <= 2; }

// From 3 tokens on (measured, separate calls, all three matrix-core kernels against
// the vector ones: LLaMA2-7B shape 3 tokens 67.5 -> 56.7 us per layer-step, 4 tokens
// 76.2 -> 58.9, OPT-6.7B shape 3 tokens 68.3 -> 53.0; at 2 tokens every vector kernel
// was faster, LLaMA2-7B 48.9 against 54.4, at 1 token 35.8 against 49.7).
bool down_mfma_eligible(int wdt, int B) { return (wdt == DT_F16 || wdt == DT_BF16) && B >= 3 && B <= 64; }

Plan plan_for(int wdt, int B, int d, int kmax) {
  if (down_mfma_eligible(wdt, B)) {
    Plan p;
    p.mfma = true;
    p.lw = 16;
    p.cpl = 8;
    p.tw = kMfmaTW;
    p.ntiles = (d + p.tw - 1) / p.tw;
    int S = 2 * kTargetBlocks / p.ntiles;
    // 8 slices measured best on 32 and 64 column tiles (LLaMA2-7B shape at 8 tokens:
    // 16 slices 24.7 us, 8: 21.4; Falcon-40B shape: 4 slices 50.0 / 131.4 us at 8 /
    // 32 tokens, 8: 48.5 / 125.6, 16: 59.8 / 141.4): beyond that the fixed-order
    // sum of the partial tiles costs more than the shorter walks save.
    if (p.ntiles >= 32 && S > 8) S = 8;
    if (S > kMaxSlices) S = kMaxSlices;
    const int groups = (kmax + 3) / 4;
    const int cap = (groups + kWavesPerBlock - 1) / kWavesPerBlock;   // >= one group per wave
    if (S > cap) S = cap;
    if (S < 1) S = 1;
    p.S = S;
    return p;
  }
  const int nb = nb_class(B);
  int lw = 16, cpl = 4;
  switch (wdt) {
    case DT_F32: lw = lw_for<TF32>(nb); cpl = lw / 4; break;
    case DT_F16: lw = lw_for<TF16>(nb); cpl = lw / 2; break;
    case DT_BF16: lw = lw_for<TBF16>(nb); cpl = lw / 2; break;
    default: lw = lw_for<TQ4>(nb); cpl = lw * 2; break;
  }
  Plan p;
  p.mfma = false;
  p.lw = lw;
  p.cpl = cpl;
  p.tw = kWave * cpl;
  p.ntiles = (d + p.tw - 1) / p.tw;
  int S = kTargetBlocks / p.ntiles;
  if (S > kMaxSlices) S = kMaxSlices;
  const int rows_cap = (kmax + kWavesPerBlock - 1) / kWavesPerBlock;  // >= 4 rows per slice
  if (S > rows_cap) S = rows_cap;
  if (S < 1) S = 1;
  p.S = S;
  return p;
}

template <class T, int NB>
hipError_t run(hipStream_t s, const Plan& p, int B, int d, int f, const void* Wd, const void* Wd_s,
               const int32_t* idx, const int32_t* count, int kmax, const float* hact, float* y, void* ws) {
  constexpr int LW = lw_for<T>(NB);
  uint32_t* tickets = (uint32_t*)ws;
  const size_t tick_bytes = ((size_t)p.ntiles * 4 + 255) & ~(size_t)255;
  float* part = (float*)((uint8_t*)ws + tick_bytes);
  k_down<T, NB, LW><<<dim3(p.S * p.ntiles), dim3(kBlock), 0, s>>>(
      (const uint8_t*)Wd, (const uint16_t*)Wd_s, idx, count, kmax, hact, B, d, f, y, part, tickets, p.S,
      p.ntiles);
  return hipGetLastError();
}

template <class T, int NT>
hipError_t run_mfma(hipStream_t s, const Plan& p, int B, int d, int f, const void* Wd, const int32_t* idx,
                    const int32_t* count, int kmax, const float* hact, float* y, void* ws) {
  uint32_t* tickets = (uint32_t*)ws;
  const size_t tick_bytes = ((size_t)p.ntiles * 4 + 255) & ~(size_t)255;
  float* part = (float*)((uint8_t*)ws + tick_bytes);
  k_down_mfma<T, NT><<<dim3(p.S * p.ntiles), dim3(kBlock), 0, s>>>((const uint8_t*)Wd, idx, count, kmax, hact, B,
                                                                   d, f, y, part, tickets, p.S, p.ntiles);
  return hipGetLastError();
}

template <class T>
hipError_t dispatch(hipStream_t s, const Plan& p, int B, int d, int f, const void* Wd, const void* Wd_s,
                    const int32_t* idx, const int32_t* count, int kmax, const float* hact, float* y, void* ws) {
  if constexpr (T::bytes == 2) {
    if (cols_eligible(B)) {
      const bool wide = d > 4096;
      const int cw = wide ? 32 : 16;
      const int ntiles = (d + cw - 1) / cw;
      const uint8_t* W = (const uint8_t*)Wd;
      if (B == 1) {
        if (wide) k_down_cols<T, 1, 32><<<dim3(ntiles), dim3(kBlock), 0, s>>>(W, idx, count, kmax, hact, B, d, f, y, ntiles);
        else k_down_cols<T, 1, 16><<<dim3(ntiles), dim3(kBlock), 0, s>>>(W, idx, count, kmax, hact, B, d, f, y, ntiles);
      } else {
        if (wide) k_down_cols<T, 2, 32><<<dim3(ntiles), dim3(kBlock), 0, s>>>(W, idx, count, kmax, hact, B, d, f, y, ntiles);
        else k_down_cols<T, 2, 16><<<dim3(ntiles), dim3(kBlock), 0, s>>>(W, idx, count, kmax, hact, B, d, f, y, ntiles);
      }
      return hipGetLastError();
    }
    if (p.mfma) {
      if (B <= 16) return run_mfma<T, 1>(s, p, B, d, f, Wd, idx, count, kmax, hact, y, ws);
      if (B <= 32) return run_mfma<T, 2>(s, p, B, d, f, Wd, idx, count, kmax, hact, y, ws);
      return run_mfma<T, 4>(s, p, B, d, f, Wd, idx, count, kmax, hact, y, ws);
    }
  }
  switch (nb_class(B)) {
    case 1: return run<T, 1>(s, p, B, d, f, Wd, Wd_s, idx, count, kmax, hact, y, ws);
    case 2: return run<T, 2>(s, p, B, d, f, Wd, Wd_s, idx, count, kmax, hact, y, ws);
    case 4: return run<T, 4>(s, p, B, d, f, Wd, Wd_s, idx, count, kmax, hact, y, ws);
    case 8: return run<T, 8>(s, p, B, d, f, Wd, Wd_s, idx, count, kmax, hact, y, ws);
    case 16: return run<T, 16>(s, p, B, d, f, Wd, Wd_s, idx, count, kmax, hact, y, ws);
    case 32: return run<T, 32>(s, p, B, d, f, Wd, Wd_s, idx, count, kmax, hact, y, ws);
    default: return run<T, 64>(s, p, B, d, f, Wd, Wd_s, idx, count, kmax, hact, y, ws);
  }
}

}  // namespace

bool down_supported(int wdt, int B) { return wdt != DT_Q4 || B <= 16; }

size_t down_ws_bytes(int wdt, int B, int d, int kmax) {
  const Plan p = plan_for(wdt, B, d, kmax);
  const size_t tick_bytes = ((size_t)p.ntiles * 4 + 255) & ~(size_t)255;
  const size_t part = p.S > 1 ? (size_t)p.S * p.ntiles * B * p.tw * sizeof(float) : 0;
  return tick_bytes + ((part + 255) & ~(size_t)255);
}

hipError_t launch_down(hipStream_t s, int wdt, int B, int d, int f, const void* Wd, const void* Wd_s,
                       const int32_t* idx, const int32_t* count, int kmax, const float* hact, float* y,
                       void* ws) {
  const Plan p = plan_for(wdt, B, d, kmax);
  switch (wdt) {
    case DT_F32: return dispatch<TF32>(s, p, B, d, f, Wd, Wd_s, idx, count, kmax, hact, y, ws);
    case DT_F16: return dispatch<TF16>(s, p, B, d, f, Wd, Wd_s, idx, count, kmax, hact, y, ws);
    case DT_BF16: return dispatch<TBF16>(s, p, B, d, f, Wd, Wd_s, idx, count, kmax, hact, y, ws);
    case DT_Q4:
      if (cols_eligible(B)) {
        const int ntiles = d / 32;
        const uint8_t* W = (const uint8_t*)Wd;
        const uint16_t* S = (const uint16_t*)Wd_s;
        if (B == 1) k_down_cols_q4<1><<<dim3(ntiles), dim3(kBlock), 0, s>>>(W, S, idx, count, kmax, hact, B, d, f, y, ntiles);
        else k_down_cols_q4<2><<<dim3(ntiles), dim3(kBlock), 0, s>>>(W, S, idx, count, kmax, hact, B, d, f, y, ntiles);
        return hipGetLastError();
      }
      switch (nb_class(B)) {
        case 1: return run<TQ4, 1>(s, p, B, d, f, Wd, Wd_s, idx, count, kmax, hact, y, ws);
        case 2: return run<TQ4, 2>(s, p, B, d, f, Wd, Wd_s, idx, count, kmax, hact, y, ws);
        case 4: return run<TQ4, 4>(s, p, B, d, f, Wd, Wd_s, idx, count, kmax, hact, y, ws);
        case 8: return run<TQ4, 8>(s, p, B, d, f, Wd, Wd_s, idx, count, kmax, hact, y, ws);
        default: return run<TQ4, 16>(s, p, B, d, f, Wd, Wd_s, idx, count, kmax, hact, y, ws);
      }
    default: return hipErrorInvalidValue;
  }
}

// ------------------------------------------------------------------ static scratch
// Workspace of sfx_sparse_down_noalloc: a file-scope device array, one copy per GPU
// the library runs on, held until the process ends.  Its device address is looked
// up once per device (with that device current) and kept; host code uses only that
// address, never the array's name.  The ticket words at its start are zero when the
// module loads and every call leaves them at zero (the last workgroup of each
// column tile resets its ticket), so each call starts from cleared tickets.
static __device__ __align__(256) uint8_t scratch[kDownScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t down_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr) return e != hipSuccess ? e : hipErrorInvalidSymbol;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace sfx
