// Fused multi-layer step: for every layer in order, predict -> compact -> sparse up
// -> sparse down, in one persistent kernel (PowerInfer page, Method: per-layer
// predictor, hybrid-execution pseudocode, neuron-aware operators; KAIROX page, Core
// method, item 3: neurons stored in contiguous groups of 32).
//
// One workgroup of 512 threads per compute unit, all resident; phases are separated
// by grid barriers (per-workgroup arrival flags polled by workgroup 0, which then
// releases a `go` word; every wait is bounded and sets an error word instead of
// hanging).  Data one workgroup hands to another (hidden, union words, idx, hact)
// is written with agent-scope atomic stores and read with agent-scope atomic loads,
// so no barrier needs a cache write-back.  Per layer:
//
//   A  hidden rows owned round-robin (row r -> workgroup r mod P), W1 chunks and x
//      in registers, fp32 dot products, relu.  Meanwhile the workgroup's W2 rows
//      (mask words g = w, w + P, ...: 32 rows each) stream straight into LDS with
//      16-byte global->LDS loads.                                          barrier
//   B  scores of the owned rows from LDS (or from HBM when the rows do not fit),
//      threshold, per-token and union mask words.                          barrier
//   C  every workgroup scans the union popcounts (the list itself lands in LDS);
//      workgroup w takes active ranks [w k / P, (w+1) k / P) -- an even split of
//      the work whatever the mask looks like -- writes idx, gathers its up (and
//      gate) rows, applies bias and ReLU / ReGLU and hands hact over.       barrier
//   D  down by column tiles: workgroup w owns d/P columns (rounded to 8) of y and
//      reads that segment of every active row, so y needs no partial sums and no
//      atomics; the reduction order is fixed, so y is bitwise reproducible.
//      Tiles are mapped so workgroups sharing a 128-byte line of Wd run on one XCD.
//                                                                           barrier
#pragma once
#include "sfx_common.hpp"
#include "sfx_step.hpp"

namespace sfx {
namespace step {

constexpr int kNT = 512;                 // threads per workgroup
constexpr int kNW = kNT / kWave;         // 8 waves
constexpr int kLds = 163840;             // gfx950 LDS per compute unit
constexpr int kW2Bytes = 131072;         // LDS region for the W2 rows
constexpr int kRedFloats = 1024;         // reduction scratch
constexpr int kXBytes = kLds - kW2Bytes - kRedFloats * 4 - 768;
constexpr int kMaxWords = 1024;          // f <= 32768
constexpr int kPrefBytes = (kMaxWords + 8) * 4;
constexpr int kNidCap = (kXBytes - kPrefBytes) / 4;
constexpr int kSpin = 1 << 20;

__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_agent(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Grid barrier.  Threads that wrote handed-over data must have waited for those
// stores (wait_memory) before calling; thread 0 then raises the workgroup's flag
// to `target`.  Readers fetch handed-over data with agent-scope atomic loads issued
// in batches (no cache invalidation: a per-workgroup agent acquire is serialised
// across the device).  Workgroup 0 polls all flags and
// raises `go`; the others poll `go`.  Bounded: on timeout the error word is set and
// the workgroup continues, and once the error word is set no later barrier waits
// (outputs are then undefined; nothing hangs).
__device__ __forceinline__ void grid_barrier(const StepParams& p, uint32_t target) {
  __syncthreads();
  if (threadIdx.x == 0) store_through(p.flags + blockIdx.x, target);
  if (blockIdx.x == 0) {
    int spins = 0;
    while (true) {
      int ok = 1;
      for (int i = threadIdx.x; i < (int)gridDim.x; i += kNT) ok &= ((int)(ld_agent(p.flags + i) - target) >= 0);
      const int bad = threadIdx.x == 0 && ld_agent(p.err) != 0u;
      const int all_ok = __syncthreads_and(ok);
      if (all_ok || __syncthreads_or(bad)) break;
      if (++spins > kSpin) {
        if (threadIdx.x == 0) store_through(p.err, 1u);
        break;
      }
    }
    if (threadIdx.x == 0) store_through(p.go, target);
  } else if (threadIdx.x == 0) {
    int spins = 0;
    while ((int)(ld_agent(p.go) - target) < 0) {
      if (ld_agent(p.err) != 0u) break;
      if (++spins > kSpin) {
        store_through(p.err, 2u);
        break;
      }
    }
  }
  __syncthreads();
}

template <class T>
__device__ __forceinline__ void dot_chunk(const uint32_t* w, const uint32_t* x, float& acc) {
  float wf[8], xf[8];
  unpack<T, 4>(w, wf);
  unpack<T, 4>(x, xf);
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = fmaf(wf[e], xf[e], acc);
}

// Workgroups are dispatched round-robin over the 8 XCDs, so tiles
// [x P/8, (x+1) P/8) go to the workgroups of XCD x and neighbouring tiles (which
// share cache lines of Wd) stay in one L2.
__device__ __forceinline__ int tile_of(int w, int P) {
  if ((P & 7) != 0) return w;
  return (w & 7) * (P >> 3) + (w >> 3);
}

// Lane L of a wave holds, after wave_reduce_multi<V>, the total of value index
// L >> (6 - log2 V); lanes with (L mod 64/V) == 0 hold distinct indices.
template <int V>
__device__ __forceinline__ bool reduce_owner(int lane) { return (lane & ((kWave / V) - 1)) == 0; }
template <int V>
__device__ __forceinline__ int reduce_index(int lane) { return lane >> (6 - ilog2c(V)); }

// T: TF16 or TBF16.  NB: token class.  DL: 1 for d <= 4096, 2 for d <= 8192.
template <class T, int NB, bool REGLU, int DL>
__global__ __launch_bounds__(kNT, 1) void k_step(StepParams p) {
  constexpr int kU = 8 * DL;              // 16-byte chunks per lane of a d-row
  constexpr int TB = NB < 4 ? NB : 4;     // tokens per pass in phase B
  constexpr int kUP = (REGLU || NB >= 4) ? 4 : kU;   // up-row chunks per lane loaded together
  constexpr int kRD = NB >= 4 ? 8 : 16;   // down rows per lane loaded together
  __shared__ __attribute__((aligned(16))) uint8_t s_w2[kW2Bytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_x[kXBytes];
  __shared__ __attribute__((aligned(16))) float s_red[kRedFloats];
  __shared__ uint32_t s_words[64];
  __shared__ uint32_t s_wt[kNW];
  uint32_t* s_pref = reinterpret_cast<uint32_t*>(s_x);
  int32_t* s_nid = reinterpret_cast<int32_t*>(s_x + kPrefBytes);

  uint32_t epoch = ld_agent(p.flags + blockIdx.x);
  for (int l = 0; l < p.L; ++l) {
    // Re-derived per layer behind opaque copies, so per-thread offsets are not
    // hoisted out of the layer loop (that would keep every phase's values live).
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & (kWave - 1);
    const int wave = tid >> 6;
    int w = blockIdx.x;
    asm volatile("" : "+s"(w));
    const int P = gridDim.x;
    const int B = p.B, d = p.d, h = p.h, f = p.f, W = p.W;
    const int nch1 = d / 8;        // 16-byte chunks per W1 / Wa / Wd row
    const int nch2 = h / 8;        // 16-byte chunks per W2 row
    const size_t rb1 = (size_t)d * 2, rb2 = (size_t)h * 2;

    // Phase-A geometry: rows w + P s (s < nr1) of W1, wpr waves per row.
    const int nr1 = p.nr1;
    const int wpr = kNW / nr1;
    const int a_slot = wave / wpr;
    const int a_part = wave - a_slot * wpr;
    const int a_row = w + P * a_slot;
    const bool a_active = a_slot < nr1 && a_row < h;
    const int a_stride = wpr * kWave;
    // Phase-B geometry: owned mask words w + P m, m < nw2.
    const int nw2 = w < W ? (W - w + P - 1) / P : 0;
    const int rows2 = nw2 * 32;
    const bool w2_lds = p.w2_lds != 0;
    // Phase-D geometry.
    const int nct = p.cw / 8;
    const int c0 = tile_of(w, P) * p.cw;
    const int d_j = wave % nct;
    const int d_rr = (wave / nct) * kWave + lane;
    const int d_rs = (kNW / nct) * kWave;
    const int d_col = c0 + d_j * 8;
    const bool d_ok = d_col < d;

    const LayerDesc& Ld = p.layers[l];
    const uint8_t* x = (const uint8_t*)Ld.x;
    const uint8_t* W2 = (const uint8_t*)Ld.W2;

    // ---------------------------------------------------------------- phase A
    Raw<16> w1r[kU];
    if (a_active) {
      const uint8_t* row = (const uint8_t*)Ld.W1 + (size_t)a_row * rb1;
#pragma unroll
      for (int m = 0; m < kU; ++m) {
        const int c = a_part * kWave + lane + m * a_stride;
        if (c < nch1) w1r[m] = load_raw<16>(row + (size_t)c * 16);
      }
    }
    {
      float acc[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[b] = 0.f;
      if (a_active) {
#pragma unroll
        for (int m = 0; m < kU; ++m) {
          const int c = a_part * kWave + lane + m * a_stride;
          if (c < nch1) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
              if (b < B) {
                Raw<16> xv = load_raw<16>(x + (size_t)b * rb1 + (size_t)c * 16);
                dot_chunk<T>(w1r[m].w, xv.w, acc[b]);
              }
          }
        }
      }
      const float v = wave_reduce_multi<NB>(acc);
      if (reduce_owner<NB>(lane)) s_red[wave * NB + reduce_index<NB>(lane)] = v;
      __syncthreads();
      if (tid < nr1 * B) {
        const int slot = tid / B, b = tid - slot * B;
        const int row = w + P * slot;
        if (row < h) {
          float s = 0.f;
          for (int q = 0; q < wpr; ++q) s += s_red[(slot * wpr + q) * NB + b];
          store_through(p.hid + (size_t)b * h + row, fmaxf(s, 0.f));
        }
        wait_memory();
      }
    }
    // The W2 rows go to LDS while the grid waits at the barrier (issued after the
    // hidden stores: memory waits on this GPU count loads and stores in order).
    if (w2_lds) {
      // the owned W2 rows -> LDS, row-major, 16 bytes per lane
      const int items = rows2 * nch2;
      for (int i0 = wave * kWave; i0 < items; i0 += kNT) {
        const int i = i0 + lane;
        if (i < items) {
          const int q = i / nch2;
          const int c = i - q * nch2;
          int row = 32 * (w + P * (q >> 5)) + (q & 31);
          if (row >= f) row = f - 1;     // rows past f are loaded but never used
          __builtin_amdgcn_global_load_lds((const void*)(W2 + (size_t)row * rb2 + (size_t)c * 16),
                                           (__attribute__((address_space(3))) void*)(s_w2 + (size_t)i0 * 16), 16, 0,
                                           0);
        }
      }
    }
    grid_barrier(p, ++epoch);

    // ---------------------------------------------------------------- phase B
    if (w2_lds) {
      wait_memory();
      __syncthreads();
    }
    {
      float* s_hid = w2_lds ? reinterpret_cast<float*>(s_x) : reinterpret_cast<float*>(s_w2);
      float* s_sc = s_red;                     // [rows2][NB]
      for (int b0 = 0; b0 < B; b0 += TB) {
        const int tb = min(TB, B - b0);
        for (int i0 = tid; i0 < tb * h; i0 += 8 * kNT) {
          float hvv[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * kNT;
            hvv[u] = i < tb * h ? ld_agent(p.hid + (size_t)b0 * h + i) : 0.f;
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * kNT;
            if (i < tb * h) s_hid[i] = hvv[u];
          }
        }
        __syncthreads();
        for (int q0 = wave; q0 < rows2; q0 += kNW * 8) {
          float a2[8 * TB];
#pragma unroll
          for (int i = 0; i < 8 * TB; ++i) a2[i] = 0.f;
          for (int c = lane; c < nch2; c += kWave) {
            float hv[TB][8];
#pragma unroll
            for (int b = 0; b < TB; ++b) {
              const float4* hp = reinterpret_cast<const float4*>(s_hid + (b < tb ? b : 0) * h + c * 8);
              const float4 u0 = hp[0], u1 = hp[1];
              hv[b][0] = u0.x; hv[b][1] = u0.y; hv[b][2] = u0.z; hv[b][3] = u0.w;
              hv[b][4] = u1.x; hv[b][5] = u1.y; hv[b][6] = u1.z; hv[b][7] = u1.w;
            }
#pragma unroll
            for (int r = 0; r < 8; ++r) {
              const int q = q0 + r * kNW;
              if (q < rows2) {
                Raw<16> wv;
                if (w2_lds) {
                  wv = *reinterpret_cast<const Raw<16>*>(s_w2 + ((size_t)q * nch2 + c) * 16);
                } else {
                  const int row = 32 * (w + P * (q >> 5)) + (q & 31);
                  if (row < f) wv = load_raw<16>(W2 + (size_t)row * rb2 + (size_t)c * 16);
                  else wv.w[0] = wv.w[1] = wv.w[2] = wv.w[3] = 0u;
                }
                float wf[8];
                unpack<T, 4>(wv.w, wf);
#pragma unroll
                for (int b = 0; b < TB; ++b)
#pragma unroll
                  for (int e = 0; e < 8; ++e) a2[r * TB + b] = fmaf(wf[e], hv[b][e], a2[r * TB + b]);
              }
            }
          }
          const float v = wave_reduce_multi<8 * TB>(a2);
          if (reduce_owner<8 * TB>(lane)) {
            const int idx = reduce_index<8 * TB>(lane);
            const int r = idx / TB, b = idx - r * TB;
            const int q = q0 + r * kNW;
            if (q < rows2 && b < tb) s_sc[q * NB + b0 + b] = v;
          }
        }
        __syncthreads();
      }
      // scores out, mask words
      for (int i = tid; i < rows2 * B; i += kNT) {
        const int q = i / B, b = i - q * B;
        const int row = 32 * (w + P * (q >> 5)) + (q & 31);
        if (row < f) Ld.scores[(size_t)b * f + row] = s_sc[q * NB + b];
      }
      if (tid < nw2 * B) {
        const int m = tid / B, b = tid - m * B;
        const int g = w + P * m;
        uint32_t word = 0;
        for (int i = 0; i < 32; ++i) {
          const int row = 32 * g + i;
          if (row < f && s_sc[(32 * m + i) * NB + b] >= Ld.threshold) word |= 1u << i;
        }
        if (Ld.tok_bits != nullptr) Ld.tok_bits[(size_t)b * W + g] = word;
        s_words[m * NB + b] = word;
      }
      __syncthreads();
      if (tid < nw2) {
        uint32_t u = 0;
        for (int b = 0; b < B; ++b) u |= s_words[tid * NB + b];
        store_through(Ld.union_bits + w + P * tid, u);
        wait_memory();
      }
    }
    grid_barrier(p, ++epoch);

    // ---------------------------------------------------------------- phase C
    uint32_t w0 = 0, w1 = 0;
    if (2 * tid < W) w0 = ld_agent(Ld.union_bits + 2 * tid);
    if (2 * tid + 1 < W) w1 = ld_agent(Ld.union_bits + 2 * tid + 1);
    const uint32_t cnt0 = __popc(w0), cnt = cnt0 + __popc(w1);
    uint32_t inc = cnt;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const uint32_t n = __shfl_up(inc, o, kWave);
      if (lane >= o) inc += n;
    }
    if (lane == kWave - 1) s_wt[wave] = inc;
    __syncthreads();
    uint32_t before = 0, total = 0;
#pragma unroll
    for (int v = 0; v < kNW; ++v) {
      const uint32_t t = s_wt[v];
      if (v < wave) before += t;
      total += t;
    }
    const uint32_t base = before + inc - cnt;
    if (2 * tid < W) s_pref[2 * tid] = base;
    if (2 * tid + 1 < W) s_pref[2 * tid + 1] = base + cnt0;
    if (tid == 0) s_pref[W] = total;
    const int k = (int)total;
    const bool in_lds = k <= kNidCap;
    if (in_lds) {
      uint32_t pos = base;
      uint32_t wd = w0;
      while (wd) { s_nid[pos++] = 64 * tid + __builtin_ctz(wd); wd &= wd - 1; }
      wd = w1;
      while (wd) { s_nid[pos++] = 64 * tid + 32 + __builtin_ctz(wd); wd &= wd - 1; }
    }
    if (w == 0 && tid == 0) *Ld.count = k;
    __syncthreads();

    {
      const int r0 = (int)(((long long)k * w) / P);
      const int r1 = (int)(((long long)k * (w + 1)) / P);
      for (int r = r0 + wave; r < r1; r += kNW) {
        int nid;
        if (in_lds) {
          nid = s_nid[r];
        } else {
          int lo = 0, hi = W;                 // s_pref[lo] <= r < s_pref[hi]
          while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if ((int)s_pref[mid] <= r) lo = mid; else hi = mid;
          }
          uint32_t wd = ld_agent(Ld.union_bits + lo);
          for (int s = r - (int)s_pref[lo]; s > 0; --s) wd &= wd - 1;
          nid = 32 * lo + __builtin_ctz(wd);
        }
        if (lane == 0) st_agent(Ld.idx + r, nid);
        const uint8_t* ra = (const uint8_t*)Ld.Wa + (size_t)nid * rb1;
        const uint8_t* rl = REGLU ? (const uint8_t*)Ld.Wl + (size_t)nid * rb1 : nullptr;
        float za[NB], zl[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) { za[b] = 0.f; zl[b] = 0.f; }
#pragma unroll
        for (int u0 = 0; u0 < kU; u0 += kUP) {
          Raw<16> wa[kUP], wl[kUP];
#pragma unroll
          for (int u = 0; u < kUP; ++u) {
            const int c = lane + (u0 + u) * kWave;
            if (c < nch1) {
              wa[u] = load_raw<16>(ra + (size_t)c * 16);
              if (REGLU) wl[u] = load_raw<16>(rl + (size_t)c * 16);
            }
          }
#pragma unroll
          for (int u = 0; u < kUP; ++u) {
            const int c = lane + (u0 + u) * kWave;
            if (c < nch1) {
#pragma unroll
              for (int b = 0; b < NB; ++b)
                if (b < B) {
                  Raw<16> xv = load_raw<16>(x + (size_t)b * rb1 + (size_t)c * 16);
                  dot_chunk<T>(wa[u].w, xv.w, za[b]);
                  if (REGLU) dot_chunk<T>(wl[u].w, xv.w, zl[b]);
                }
            }
          }
        }
        const float bias = Ld.ba != nullptr ? Ld.ba[nid] : 0.f;
        const float ta = wave_reduce_multi<NB>(za);
        float v = fmaxf(ta + bias, 0.f);
        if (REGLU) v *= wave_reduce_multi<NB>(zl);
        if (reduce_owner<NB>(lane)) {
          const int b = reduce_index<NB>(lane);
          if (b < B) store_through(Ld.hact + (size_t)r * B + b, v);
        }
      }
    }
    wait_memory();
    grid_barrier(p, ++epoch);

    // ---------------------------------------------------------------- phase D
    {
      float yacc[NB * 8];
#pragma unroll
      for (int i = 0; i < NB * 8; ++i) yacc[i] = 0.f;
      if (d_ok) {
        const uint8_t* Wd = (const uint8_t*)Ld.Wd;
        for (int rb = d_rr; rb < k; rb += d_rs * kRD) {
          Raw<16> wv[kRD];
          float hv[kRD][NB];
#pragma unroll
          for (int u = 0; u < kRD; ++u) {
            const int r = rb + u * d_rs;
            if (r < k) {
              const int nid = in_lds ? s_nid[r] : ld_agent(Ld.idx + r);
              wv[u] = load_raw<16>(Wd + (size_t)nid * rb1 + (size_t)d_col * 2);
#pragma unroll
              for (int b = 0; b < NB; ++b) hv[u][b] = b < B ? ld_agent(Ld.hact + (size_t)r * B + b) : 0.f;
            }
          }
#pragma unroll
          for (int u = 0; u < kRD; ++u) {
            const int r = rb + u * d_rs;
            if (r < k) {
              float wf[8];
              unpack<T, 4>(wv[u].w, wf);
#pragma unroll
              for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int e = 0; e < 8; ++e) yacc[b * 8 + e] = fmaf(hv[u][b], wf[e], yacc[b * 8 + e]);
            }
          }
        }
      }
      const float v = wave_reduce_multi<NB * 8>(yacc);
      __syncthreads();                                   // s_red was read in phase B
      if (reduce_owner<NB * 8>(lane)) s_red[wave * 64 + reduce_index<NB * 8>(lane)] = v;
      __syncthreads();
      for (int i = tid; i < nct * B * 8; i += kNT) {
        const int j = i / (B * 8);
        const int be = i - j * B * 8;                    // b * 8 + e
        const int col = c0 + j * 8 + (be & 7);
        if (col < d) {
          float s = 0.f;
          for (int wv2 = j; wv2 < kNW; wv2 += nct) s += s_red[wv2 * 64 + be];
          Ld.y[(size_t)(be >> 3) * d + col] = s;
        }
      }
    }
    if (l + 1 < p.L) grid_barrier(p, ++epoch);
  }
}

template <class T, int NB, int DL>
hipError_t run_step(hipStream_t s, const StepParams& p, int act, int P) {
  if (act == 1) k_step<T, NB, true, DL><<<dim3(P), dim3(kNT), 0, s>>>(p);
  else k_step<T, NB, false, DL><<<dim3(P), dim3(kNT), 0, s>>>(p);
  return hipGetLastError();
}

// Built for d <= 4096 and B <= 4 (the register budget of 2 waves per SIMD holds
// every phase without spilling there).
template <class T>
hipError_t dispatch_step(hipStream_t s, const StepParams& p, int act, int P) {
  switch (nb_class(p.B)) {
    case 1: return run_step<T, 1, 1>(s, p, act, P);
    case 2: return run_step<T, 2, 1>(s, p, act, P);
    default: return run_step<T, 4, 1>(s, p, act, P);
  }
}

}  // namespace step
}  // namespace sfx
