// Fused multi-layer step: for every layer in order, predict -> compact -> sparse up
// -> sparse down, in one persistent kernel (PowerInfer page, Method: per-layer
// predictor, hybrid-execution pseudocode, neuron-aware operators; KAIROX page, Core
// method, item 3: neurons stored in contiguous groups of 32).
//
// One workgroup of 512 threads per compute unit, all resident.  Inside a layer,
// data one workgroup hands to others (hidden values, union mask words, hact) is
// written as 64-bit words {layer tag, value} with one agent-scope atomic store each;
// readers poll those words with agent-scope atomic loads until the tag of the
// current layer shows up.  So a hand-off costs one store and one poll, with no
// store-completion wait and no grid barrier.  Between layers a grid barrier
// (arrival flags polled by workgroup 0, which then releases a `go` word) makes the
// layer's y complete before the next layer's input is read.  Every wait is bounded
// and sets an error word instead of hanging.  Per layer:
//
//   A  hidden rows owned round-robin (row r -> workgroup r mod P), W1 chunks and x
//      in registers, fp32 dot products, relu, tagged hidden out.  Then the
//      workgroup's W2 rows (mask words g = w, w + P, ...: 32 rows each) stream
//      straight into LDS with 16-byte global->LDS loads.
//   B  poll the hidden, scores of the owned rows from LDS (or from HBM when the rows
//      do not fit), threshold, per-token and union mask words (union tagged out).
//   C  poll the union words, scan their popcounts (the active list lands in LDS);
//      workgroup w takes active ranks [w k / P, (w+1) k / P) -- an even split of
//      the work whatever the mask looks like -- writes idx, gathers its up (and
//      gate) rows, applies bias and ReLU / ReGLU, tagged hact out.
//   D  down by column tiles: workgroup w owns d/P columns (rounded to 8) of y and
//      reads that segment of every active row (polling each row's hact), so y
//      needs no partial sums and no atomics; the reduction order is fixed, so y is
//      bitwise reproducible.  Tiles are mapped so workgroups sharing a 128-byte
//      line of Wd run on one XCD.                                grid barrier
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
constexpr int kUwBytes = kMaxWords * 4;
constexpr int kNidCap = (kXBytes - kPrefBytes - kUwBytes) / 4;
constexpr int kSpin = 1 << 20;

__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long ld_agent64(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_tagged(unsigned long long* p, uint32_t tag, uint32_t bits) {
  __hip_atomic_store(p, ((unsigned long long)tag << 32) | bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool tag_ok(unsigned long long v, uint32_t tag) { return (uint32_t)(v >> 32) == tag; }

// Poll N tagged words (entries i < n, addresses addr(i)) until all carry `tag`.
// Loads are issued as one batch, then only stale entries are reloaded.  Bounded:
// on timeout (or when another workgroup already failed) the error word is set and
// whatever was read is returned.
template <int N, class Addr>
__device__ __forceinline__ void poll_tagged(unsigned long long (&v)[N], int n, Addr addr, uint32_t tag,
                                            uint32_t* err) {
#pragma unroll
  for (int i = 0; i < N; ++i)
    if (i < n) v[i] = ld_agent64(addr(i));
  for (int spins = 0;; ++spins) {
    bool stale = false;
#pragma unroll
    for (int i = 0; i < N; ++i) stale |= (i < n) && !tag_ok(v[i], tag);
    if (!stale) return;
    if (spins > kSpin || ((spins & 255) == 255 && ld_agent(err) != 0u)) {
      store_through(err, 3u);
      return;
    }
    // back off: thousands of waves re-reading uncached words would otherwise
    // crowd out the loads that do the work
    __builtin_amdgcn_s_sleep(2);
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (i < n && !tag_ok(v[i], tag)) v[i] = ld_agent64(addr(i));
  }
}

// Grid barrier between layers.  Thread 0 raises the workgroup's flag to `target`;
// workgroup 0 polls all flags and raises `go`; the others poll `go`.  Bounded:
// on timeout the error word is set, and once it is set no later wait spins.
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
      __builtin_amdgcn_s_sleep(1);
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

// Neuron of active rank r from the union words and their prefix (both in LDS).
__device__ __forceinline__ int rank_to_neuron(int r, const uint32_t* s_pref, const uint32_t* s_uw, int W) {
  int lo = 0, hi = W;                   // s_pref[lo] <= r < s_pref[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((int)s_pref[mid] <= r) lo = mid; else hi = mid;
  }
  uint32_t wd = s_uw[lo];
  for (int s = r - (int)s_pref[lo]; s > 0; --s) wd &= wd - 1;
  return 32 * lo + __builtin_ctz(wd);
}

// T: TF16 or TBF16.  NB: token class (1, 2, 4).  DL: 1 for d <= 4096.
template <class T, int NB, bool REGLU, int DL>
__global__ __launch_bounds__(kNT, 1) void k_step(StepParams p) {
  constexpr int kU = 8 * DL;              // 16-byte chunks per lane of a d-row
  constexpr int TB = NB < 4 ? NB : 4;     // tokens per pass in phase B
  constexpr int kUP = (REGLU || NB >= 4) ? 4 : kU;   // up-row chunks per lane loaded together
  constexpr int kRD = 8 / NB;             // down rows per lane loaded together
  __shared__ __attribute__((aligned(16))) uint8_t s_w2[kW2Bytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_x[kXBytes];
  __shared__ __attribute__((aligned(16))) float s_red[kRedFloats];
  __shared__ uint32_t s_words[64];
  __shared__ uint32_t s_wt[kNW];
  uint32_t* s_pref = reinterpret_cast<uint32_t*>(s_x);
  uint32_t* s_uw = reinterpret_cast<uint32_t*>(s_x + kPrefBytes);
  int32_t* s_nid = reinterpret_cast<int32_t*>(s_x + kPrefBytes + kUwBytes);

  const uint32_t e0 = ld_agent(p.flags + blockIdx.x);
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
    const uint32_t tag = e0 + (uint32_t)l + 1u;

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
    {
      Raw<16> w1r[kU];
      if (a_active) {
        const uint8_t* row = (const uint8_t*)Ld.W1 + (size_t)a_row * rb1;
#pragma unroll
        for (int m = 0; m < kU; ++m) {
          const int c = a_part * kWave + lane + m * a_stride;
          if (c < nch1) w1r[m] = load_raw<16>(row + (size_t)c * 16);
        }
      }
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
          st_tagged(p.hid + (size_t)b * h + row, tag, __float_as_uint(fmaxf(s, 0.f)));
        }
      }
    }
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

    // ---------------------------------------------------------------- phase B
    {
      float* s_hid = w2_lds ? reinterpret_cast<float*>(s_x) : reinterpret_cast<float*>(s_w2);
      float* s_sc = s_red;                     // [rows2][NB]
      if (w2_lds) {
        wait_memory();                         // this thread's LDS rows have landed
      }
      for (int b0 = 0; b0 < B; b0 += TB) {
        const int tb = min(TB, B - b0);
        __syncthreads();                       // previous use of s_hid / s_w2 done
        for (int i0 = tid; i0 < tb * h; i0 += 8 * kNT) {
          unsigned long long hw[8];
          const int n = min(8, (tb * h - i0 + kNT - 1) / kNT);
          poll_tagged<8>(hw, n, [&](int u) { return p.hid + (size_t)b0 * h + i0 + u * kNT; }, tag, p.err);
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (u < n) s_hid[i0 + u * kNT] = __uint_as_float((uint32_t)hw[u]);
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
      }
      __syncthreads();
      // mask words by wave ballots (lane = row of a 64-row pair of words), then the
      // union goes out tagged, then the scores
      for (int m0 = 2 * wave; m0 < nw2; m0 += 2 * kNW) {
        const int m = m0 + (lane >> 5);
        const int g = w + P * m;
        const int row = 32 * g + (lane & 31);
        const bool in = m < nw2 && row < f;
        const float thr = Ld.threshold;
        for (int b = 0; b < B; ++b) {
          const uint64_t bal = __ballot(in && s_sc[(32 * m + (lane & 31)) * NB + b] >= thr);
          if ((lane & 31) == 0 && m < nw2) {
            const uint32_t word = (uint32_t)(lane == 0 ? bal : (bal >> 32));
            if (Ld.tok_bits != nullptr) Ld.tok_bits[(size_t)b * W + g] = word;
            s_words[m * NB + b] = word;
          }
        }
      }
      __syncthreads();
      if (tid < nw2) {
        uint32_t u = 0;
        for (int b = 0; b < B; ++b) u |= s_words[tid * NB + b];
        const int g = w + P * tid;
        st_tagged(p.uni + g, tag, u);
        Ld.union_bits[g] = u;
      }
      for (int i = tid; i < rows2 * B; i += kNT) {
        const int q = i / B, b = i - q * B;
        const int row = 32 * (w + P * (q >> 5)) + (q & 31);
        if (row < f) Ld.scores[(size_t)b * f + row] = s_sc[q * NB + b];
      }
    }

    // ---------------------------------------------------------------- phase C
    unsigned long long uw[2];
    {
      const int base2 = 2 * tid;
      const int n = base2 + 1 < W ? 2 : (base2 < W ? 1 : 0);
      poll_tagged<2>(uw, n, [&](int u) { return p.uni + base2 + u; }, tag, p.err);
    }
    const uint32_t w0 = 2 * tid < W ? (uint32_t)uw[0] : 0u;
    const uint32_t w1 = 2 * tid + 1 < W ? (uint32_t)uw[1] : 0u;
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
    if (2 * tid < W) { s_pref[2 * tid] = base; s_uw[2 * tid] = w0; }
    if (2 * tid + 1 < W) { s_pref[2 * tid + 1] = base + cnt0; s_uw[2 * tid + 1] = w1; }
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
        const int nid = in_lds ? s_nid[r] : rank_to_neuron(r, s_pref, s_uw, W);
        if (lane == 0) Ld.idx[r] = nid;
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
          if (b < B) {
            st_tagged(p.hact + (size_t)r * B + b, tag, __float_as_uint(v));
            Ld.hact[(size_t)r * B + b] = v;
          }
        }
      }
    }

    // ---------------------------------------------------------------- phase D
    {
      float yacc[NB * 8];
#pragma unroll
      for (int i = 0; i < NB * 8; ++i) yacc[i] = 0.f;
      if (d_ok) {
        const uint8_t* Wd = (const uint8_t*)Ld.Wd;
        for (int rb = d_rr; rb < k; rb += d_rs * kRD) {
          Raw<16> wv[kRD];
#pragma unroll
          for (int u = 0; u < kRD; ++u) {
            const int r = rb + u * d_rs;
            if (r < k) {
              const int nid = in_lds ? s_nid[r] : rank_to_neuron(r, s_pref, s_uw, W);
              wv[u] = load_raw<16>(Wd + (size_t)nid * rb1 + (size_t)d_col * 2);
            }
          }
          unsigned long long hv[kRD * NB];
          const int nrow = min(kRD, (k - rb + d_rs - 1) / d_rs);
          poll_tagged<kRD * NB>(hv, nrow * B,
                                [&](int i) { return p.hact + (size_t)(rb + (i / B) * d_rs) * B + (i % B); }, tag,
                                p.err);
#pragma unroll
          for (int u = 0; u < kRD; ++u) {
            if (u < nrow) {
              float wf[8];
              unpack<T, 4>(wv[u].w, wf);
#pragma unroll
              for (int b = 0; b < NB; ++b)
                if (b < B) {
                  const float hvf = __uint_as_float((uint32_t)hv[u * B + b]);
#pragma unroll
                  for (int e = 0; e < 8; ++e) yacc[b * 8 + e] = fmaf(hvf, wf[e], yacc[b * 8 + e]);
                }
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
    if (l + 1 < p.L) grid_barrier(p, e0 + (uint32_t)l + 1u);
  }
  // Every workgroup ends with its flag at e0 + L, so all flags agree at the next call.
  if (threadIdx.x == 0) store_through(p.flags + blockIdx.x, e0 + (uint32_t)p.L);
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
