// Fused multi-layer step: for every layer in order, predict -> compact -> sparse up
// -> sparse down, in one persistent kernel (PowerInfer page, Method: per-layer
// predictor, hybrid-execution pseudocode, neuron-aware operators; KAIROX page, Core
// method, item 3: neurons stored in contiguous groups of 32).
//
// One workgroup of 512 threads per compute unit, all resident.  Data one workgroup
// hands to the others (hidden values, union mask words, activations) is written as
// 64-bit words {layer tag, value}, one agent-scope atomic store each, in a block of
// its own per producer; readers load those words with agent-scope loads and
// re-poll the ones whose tag is stale.  The grid barrier between layers polls one
// flag per workgroup from the control wave.
// Every wait is bounded and sets an error word instead of hanging.  Per layer:
//
//   A  hidden rows w + P s (one W1 row per wave of waves 0..3, held in registers
//      since the previous layer), input rows staged in LDS, fp32 dot products,
//      relu, tagged hidden out; then this layer's W2 rows (mask words g = w, w + P,
//      ...: 32 rows each) start streaming into LDS (waves 4..6).
//   B  read the hidden, scores of the owned rows from LDS (or from HBM when the
//      rows do not fit), threshold, per-token and union mask words (union tagged
//      out).
//   C  read the union words, scan their popcounts (the active list lands in LDS);
//      workgroup w takes active ranks [w k / P, (w+1) k / P) -- an even split of
//      the work whatever the mask looks like -- writes idx, gathers its up (and
//      gate) rows, applies bias and ReLU / ReGLU, tagged activations out.
//   D  down by column tiles: workgroup w owns 8 or 16 columns of y and reads that
//      segment of every active row, so y needs no partial sums and no atomics;
//      the reduction order is fixed, so y is bitwise reproducible.  Tiles are
//      mapped so workgroups sharing a 128-byte line of Wd run on one XCD.
//                                                                   grid barrier
#pragma once
#include <type_traits>
#include "sfx_common.hpp"
#include "sfx_step.hpp"

namespace sfx {
namespace step {

constexpr int kNT = 512;                 // threads per workgroup
constexpr int kNW = kNT / kWave;         // 8 waves
constexpr int kLds = 163840;             // gfx950 LDS per compute unit
constexpr int kW2Bytes = 131072;         // LDS region for the W2 rows
constexpr int kUpSlot0 = 16384;          // up rows' LDS slots in s_w2 (past the union words)
constexpr int kUpSlot = 8192;            // one slot per wave: a row of d <= 4096 at 2 bytes
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

// Poll N tagged words (entries i with valid(i), addresses addr(i)) until all carry
// `tag`.  Every addr(i), valid or not, must point into the caller's buffer: the
// first loads are issued unconditionally as one batch (loads under per-entry
// branches were each preceded by a wait for all memory, one round trip per word);
// then only stale entries are reloaded.  Bounded: on timeout (or when another
// workgroup already failed) the error word is set and whatever was read is returned.
template <int N, class Valid, class Addr, int SL = 2>
__device__ __forceinline__ void poll_tagged_if(unsigned long long (&v)[N], Valid valid, Addr addr, uint32_t tag,
                                               uint32_t* err) {
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = ld_agent64(addr(i));
  for (int spins = 0;; ++spins) {
    bool stale = false;
#pragma unroll
    for (int i = 0; i < N; ++i) stale |= valid(i) && !tag_ok(v[i], tag);
    if (!stale) return;
    if (spins > kSpin || ((spins & 255) == 255 && ld_agent(err) != 0u)) {
      store_through(err, 3u);
      return;
    }
    // back off: many waves re-reading uncached words would otherwise crowd out
    // the loads that do the work
    __builtin_amdgcn_s_sleep(SL);
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (valid(i) && !tag_ok(v[i], tag)) v[i] = ld_agent64(addr(i));
  }
}
template <int N, class Addr>
__device__ __forceinline__ void poll_tagged(unsigned long long (&v)[N], int n, Addr addr, uint32_t tag,
                                            uint32_t* err) {
  poll_tagged_if<N>(v, [&](int i) { return i < n; }, addr, tag, err);
}

// Workgroup barrier for LDS hand-offs only.  __syncthreads() also orders LDS
// writes still in flight from global->LDS loads, so it waits for every one of them;
// this barrier leaves those streaming (they are waited for explicitly where their
// data is read).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);    // lgkmcnt(0): this wave's LDS accesses are done
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Barrier among some waves of the workgroup only: each arriving wave adds 1 to an
// LDS counter that only grows, and waits until it reaches `target`.  Lets waves that
// are busy issuing a long stream of loads stay out of the way.
__device__ __forceinline__ void lds_wait_at_least(const uint32_t* ctr, uint32_t target, uint32_t* err) {
  for (int spins = 0; __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target; ++spins) {
    if (spins > kSpin) {                  // cannot happen unless a wave skipped its arrival
      if ((threadIdx.x & (kWave - 1)) == 0) store_through(err, 6u);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}
// Arrival on an LDS counter once this wave's LDS accesses are done (no wait).
__device__ __forceinline__ void group_arrive(uint32_t* ctr) {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);    // lgkmcnt(0)
  if ((threadIdx.x & (kWave - 1)) == 0) atomicAdd(ctr, 1u);
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void group_sync(uint32_t* ctr, uint32_t target, uint32_t* err) {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);    // lgkmcnt(0): this wave's LDS accesses are done
  if ((threadIdx.x & (kWave - 1)) == 0) atomicAdd(ctr, 1u);
  lds_wait_at_least(ctr, target, err);
  asm volatile("" ::: "memory");
}

// Hand-off completion flags: one 32-bit word per workgroup and hand-off kind,
// raised to the layer tag once the workgroup has issued all its tagged words of
// that kind.  A consumer waits for all P flags with one wave (P/64 coalesced loads
// per round), then reads the tagged words once; a word that is still stale (its
// store overtaken by the flag) is simply polled again.  Polling every tagged word
// from every workgroup instead would load the memory system with re-reads while
// slower workgroups are still gathering rows.
constexpr int kMaxP = 256;
#ifndef SFX_POLL_SLEEP
#define SFX_POLL_SLEEP 2
#endif
constexpr int kPollSleep = SFX_POLL_SLEEP;   // pause between flag polls, in units of 64 clocks
#ifndef SFX_STEP_POLL_SLEEP
#define SFX_STEP_POLL_SLEEP 2
#endif
constexpr int kStepPS = SFX_STEP_POLL_SLEEP;  // pause between polls of tagged words, x 64 clocks
#ifndef SFX_TLB_WARM
#define SFX_TLB_WARM 1
#endif
constexpr bool kTlbWarm = SFX_TLB_WARM != 0;
// Flags sit kFS words apart: flags sharing a cache line with many writers become
// visible to other compute units much later.
constexpr int kFS = kFlagStride;

// Layer descriptors are read-only for the whole launch: read them through the
// constant address space so they come in on scalar loads.
typedef const LayerDesc __attribute__((address_space(4))) CLayer;
__device__ __forceinline__ void wait_flags(const uint32_t* fl, int P, uint32_t tag, uint32_t* err, uint32_t code) {
  constexpr int N = kMaxP / kWave;
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));           // keep the flag addresses out of the layer loop
  const int lane = tid & (kWave - 1);
  uint32_t v[N];
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const int i = lane + u * kWave;
    v[u] = i < P ? ld_agent(fl + (size_t)i * kFS) : tag;
  }
  for (int spins = 0;; ++spins) {
    bool stale = false;
#pragma unroll
    for (int u = 0; u < N; ++u) stale |= (int)(v[u] - tag) < 0;
    if (__ballot(stale) == 0) return;
    if (spins > kSpin || ((spins & 63) == 63 && ld_agent(err) != 0u)) {
      if (lane == 0) store_through(err, code);
      return;
    }
    __builtin_amdgcn_s_sleep(kPollSleep);
#pragma unroll
    for (int u = 0; u < N; ++u) {
      const int i = lane + u * kWave;
      if (i < P && (int)(v[u] - tag) < 0) v[u] = ld_agent(fl + (size_t)i * kFS);
    }
  }
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

// Wave roles.  A wave's loads and stores complete in issue order, so a wave that
// waits for a flag must have nothing slow in flight ahead of the flag loads:
//   waves 0..3  W1 rows (registers) and phase A;
//   waves 4..6  stream the layer's W2 rows into LDS once phase A has asked for its inputs;
//   wave 7      the control wave: polls the grid-barrier flags;
//   all waves   up rows and down segments.
constexpr int kAW = 4;                   // waves [0, kAW): W1 rows
constexpr int kCW = 7;                   // control wave; waves [kAW, kCW) stream W2
constexpr int kWork = kNW;               // waves [0, kWork) take up and down rows


// Weights of a layer that do not depend on its input, fetched before the layer
// starts (behind the previous layer's barrier): the W1 row of each of waves 0..3
// into registers, and the workgroup's W2 rows (mask words g = w, w + P, ...: 32
// rows each) straight into LDS with 16-byte global->LDS loads.
template <int kU>
__device__ __forceinline__ void prefetch_w1(const StepParams& p, CLayer* Ld, Raw<16> (&w1r)[kU]) {
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int w = blockIdx.x;
  const int P = gridDim.x;
  const int a_row = w + P * wave;
  if (wave < kAW && wave < p.nr1 && a_row < p.h) {
    const uint8_t* row = (const uint8_t*)Ld->W1 + (size_t)a_row * p.d * 2;
    const int nch1 = p.d / 8;
#pragma unroll
    for (int m = 0; m < kU; ++m) {
      const int c = lane + m * kWave;
      if (c < nch1) w1r[m] = load_raw<16>(row + (size_t)c * 16);
    }
  }
}

__device__ __forceinline__ void prefetch_w2(const StepParams& p, CLayer* Ld, uint8_t* s_w2) {
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int w = blockIdx.x;
  const int P = gridDim.x;
  if (wave >= kAW && wave < kCW && p.w2_lds != 0) {
    const uint8_t* W2 = (const uint8_t*)Ld->W2;
    const int nch2 = p.h / 8;
    const size_t rb2 = (size_t)p.h * 2;
    const int nw2 = w < p.W ? (p.W - w + P - 1) / P : 0;
    const int items = nw2 * 32 * nch2;
    // item i = q nch2 + c: chunk c of the workgroup's row q; (q, c) advance by the
    // stride with a carry instead of a division per load, so issuing stays cheap
    constexpr int kStride = (kCW - kAW) * kWave;
    const int i_first = (wave - kAW) * kWave + lane;
    int q = i_first / nch2, c = i_first - q * nch2;
    const int dq = kStride / nch2, dc = kStride - dq * nch2;
#pragma unroll 1
    for (int i0 = (wave - kAW) * kWave; i0 < items; i0 += kStride) {
      if (i0 + lane < items) {
        int row = 32 * (w + P * (q >> 5)) + (q & 31);
        if (row >= p.f) row = p.f - 1;       // rows past f are loaded but never used
        __builtin_amdgcn_global_load_lds((const void*)(W2 + (size_t)row * rb2 + (size_t)c * 16),
                                         (__attribute__((address_space(3))) void*)(s_w2 + (size_t)i0 * 16), 16, 0, 0);
      }
      q += dq;
      c += dc;
      if (c >= nch2) { c -= nch2; ++q; }
    }
  }
}

// The fused step's W2 rows: workgroup w owns rows w + P j (j < nr2), strided over
// the workgroups, so hot-first storage spreads the most active neurons evenly
// over them; own row q lands at s_w2 + q * (h/8) * 16, like prefetch_w2.  Waves
// [wlo, whi) load own rows [q_lo, min(q_hi, nr2)), 16 bytes per lane.
__device__ __forceinline__ void prefetch_w2_rows(const StepParams& p, CLayer* Ld, uint8_t* s_w2, int wlo, int whi,
                                                 int q_lo, int q_hi) {
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int w = blockIdx.x;
  const int P = gridDim.x;
  if (wave >= wlo && wave < whi && p.w2_lds != 0) {
    const uint8_t* W2 = (const uint8_t*)Ld->W2;
    const int nch2 = p.h / 8;
    const size_t rb2 = (size_t)p.h * 2;
    const int nr2 = w < p.f ? (p.f - w + P - 1) / P : 0;
    const int q_end = min(nr2, q_hi);
    const int items = max(q_end - q_lo, 0) * nch2;
    uint8_t* const dst = s_w2 + (size_t)q_lo * nch2 * 16;
    const int stride = (whi - wlo) * kWave;
    const int i_first = (wave - wlo) * kWave + lane;
    int q = i_first / nch2, c = i_first - q * nch2;
    q += q_lo;
    const int dq = stride / nch2, dc = stride - dq * nch2;
#pragma unroll 1
    for (int i0 = (wave - wlo) * kWave; i0 < items; i0 += stride) {
      if (i0 + lane < items) {
        int row = w + P * q;
        if (row >= p.f) row = p.f - 1;       // never: q < nr2
        __builtin_amdgcn_global_load_lds((const void*)(W2 + (size_t)row * rb2 + (size_t)c * 16),
                                         (__attribute__((address_space(3))) void*)(dst + (size_t)i0 * 16), 16, 0, 0);
      }
      q += dq;
      c += dc;
      if (c >= nch2) { c -= nch2; ++q; }
    }
  }
}
// One eighth late since the hidden is polled after the W2 rows land (one token,
// us per layer-step, eighths 2 -> 1: OPT-6.7B shape 21.0 -> 20.6, LLaMA2-7B shape
// 22.95 -> 23.15; 0: 21.5 / 23.9; 4: 21.2 / 22.9).
#ifndef SFX_W2_LATE
#define SFX_W2_LATE 1
#endif
// Own W2 rows [w2_split, nr2) that waves 0..kAW-1 load once their W1 rows are done
// (the last SFX_W2_LATE eighths); waves kAW.. load [0, w2_split) from the start of
// the layer.
__device__ __forceinline__ int w2_split(int f, int P) {
  const int nr2 = (f + P - 1) / P;
  return nr2 - (nr2 * SFX_W2_LATE + 7) / 8;
}

// A layer's input rows [B][d] into s_x by waves 0..kAW-1, 16 bytes per lane
// (B d 2 <= kXBytes).
__device__ __forceinline__ void load_x_lds(const StepParams& p, CLayer* Ld, uint8_t* s_x) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const uint8_t* x = (const uint8_t*)Ld->x;
  const int items = p.B * (p.d / 8);
#pragma unroll 1
  for (int i0 = wave * kWave; i0 < items; i0 += kAW * kWave)
    if (i0 + lane < items)
      __builtin_amdgcn_global_load_lds((const void*)(x + (size_t)(i0 + lane) * 16),
                                       (__attribute__((address_space(3))) void*)(s_x + (size_t)i0 * 16), 16, 0, 0);
}

// One stage of a 32 x 32 bit-matrix transpose held one row per lane (each half
// wave its own matrix): rows L and L ^ s swap the s x s blocks off the diagonal of
// their 2s x 2s block; `hi` marks the columns t with t & s set.
template <int S>
__device__ __forceinline__ uint32_t transpose_step(uint32_t x, int lane, uint32_t hi) {
  const uint32_t y = lane_xor_u32<S>(x, lane);
  return (lane & S) ? ((x & hi) | ((y & hi) >> S)) : ((x & ~hi) | ((y & ~hi) << S));
}

// Own mask words per workgroup (at most) when workgroup w owns rows w + P j.
__device__ __forceinline__ int own_words_max(int f, int P) { return (((f + P - 1) / P) + 31) >> 5; }

// Thread and shape values, re-derived at the start of every phase behind opaque
// copies: values computed once would be hoisted out of the layer loop and kept
// live through every phase.
#define SFX_PHASE_IDS                                                      \
  int tid = threadIdx.x;                                                   \
  asm volatile("" : "+v"(tid));                                            \
  const int lane = tid & (kWave - 1);                                      \
  const int wave = tid >> 6;                                               \
  int w = blockIdx.x;                                                      \
  asm volatile("" : "+s"(w));                                              \
  const int P = gridDim.x;                                                 \
  const int B = p.B, d = p.d, h = p.h, f = p.f, W = p.W;                   \
  const int nch1 = d / 8;        /* 16-byte chunks per W1 / Wa / Wd row */ \
  const int nch2 = h / 8;        /* 16-byte chunks per W2 row */           \
  const size_t rb1 = (size_t)d * 2, rb2 = (size_t)h * 2;                   \
  (void)lane; (void)wave; (void)P; (void)B; (void)d; (void)h; (void)f; (void)W; \
  (void)nch1; (void)nch2; (void)rb1; (void)rb2

// Tile shares of the down phase: layer l's share of workgroup w (tile w / dsplit,
// 64 columns x NB tokens) sits in buffer l mod 2 (summed before the grid barrier of
// layer l, so the next layer's shares never meet unsummed ones).  The tile's first
// workgroup adds its dsplit shares in share order: wave kAW + b takes token b,
// lane = column, entry s of yv = share s.
__device__ __forceinline__ bool tile_y_mine(const StepParams& p) {
  const int b = (int)(threadIdx.x >> 6) - kAW;
  return b >= 0 && b < p.B && blockIdx.x % p.dsplit == 0 && (int)blockIdx.x / p.dsplit < p.dtiles;
}
template <int NB>
__device__ __forceinline__ const unsigned long long* tile_y_addr(const StepParams& p, int lp, int s) {
  const int lane = threadIdx.x & (kWave - 1), b = (int)(threadIdx.x >> 6) - kAW;
  return p.ypart + ((size_t)(lp & 1) * gridDim.x + blockIdx.x + min(s, p.dsplit - 1)) * (64 * NB) + b * 64 + lane;
}
template <int NB>
__device__ __forceinline__ void tile_y_issue(const StepParams& p, int lp, unsigned long long (&yv)[8]) {
  if (!tile_y_mine(p)) return;
#pragma unroll
  for (int s = 0; s < 8; ++s) yv[s] = ld_agent64(tile_y_addr<NB>(p, lp, s));
}
// Checks the tags (stale words are polled again, bounded), adds the shares and
// writes y of layer lp (token kAW - wave, the lane's column).
template <int NB>
__device__ __forceinline__ void tile_y_sum(const StepParams& p, int lp, uint32_t tagp, unsigned long long (&yv)[8]) {
  if (!tile_y_mine(p)) return;
  for (int spins = 0;; ++spins) {
    bool stale = false;
#pragma unroll
    for (int s = 0; s < 8; ++s) stale |= s < p.dsplit && !tag_ok(yv[s], tagp);
    if (!stale) break;
    if (spins > kSpin || ((spins & 255) == 255 && ld_agent(p.err) != 0u)) {
      store_through(p.err, 3u);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
#pragma unroll
    for (int s = 0; s < 8; ++s)
      if (s < p.dsplit && !tag_ok(yv[s], tagp)) yv[s] = ld_agent64(tile_y_addr<NB>(p, lp, s));
  }
  const int col = ((int)blockIdx.x / p.dsplit) * 64 + (int)(threadIdx.x & (kWave - 1));
  const int b = (int)(threadIdx.x >> 6) - kAW;
  if (col < p.d) {
    float sum = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      if (s < p.dsplit) sum += __uint_as_float((uint32_t)yv[s]);
    ((CLayer*)p.layers + lp)->y[(size_t)b * p.d + col] = sum;
  }
}

// T: TF16 or TBF16.  NB: token class (1, 2, 4).  DL: 1 for d <= 4096.
template <class T, int NB, bool REGLU, int DL>
__global__ __launch_bounds__(kNT, 1) void k_step(StepParams p) {
  constexpr int kU = 8 * DL;              // 16-byte chunks per lane of a d-row
  constexpr int TB = NB < 4 ? NB : 4;     // tokens per pass in phase B
  // up-row chunks per lane loaded together (with the input chunks they meet)
  constexpr int kUP = (NB == 1 && !REGLU) ? kU : (NB == 1 || (NB == 2 && !REGLU)) ? 4 : 2;
  constexpr int kRD = 8 / NB;             // down rows per lane loaded together
  constexpr int kRB = TB <= 2 ? 8 : 4;    // score rows per lane per pass
  // own up rows a workgroup takes before the union exchange: two rounds of the
  // waves when a row is one load batch, one round otherwise
  // ReGLU at one token: the Wl row goes through an LDS slot, so a row pair is one
  // load batch as well
  constexpr bool kGluSlot = REGLU && NB == 1;
  constexpr int kHS = 4 * NB;             // tagged hidden words per workgroup, packed
  constexpr int kOwnCap = (kUP == kU || kGluSlot ? 2 : 1) * kWork;
  __shared__ __attribute__((aligned(16))) uint8_t s_w2[kW2Bytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_x[kXBytes];
  __shared__ __attribute__((aligned(16))) float s_red[kRedFloats];
  __shared__ uint32_t s_words[64];
  __shared__ uint32_t s_wt[kNW];
  __shared__ uint32_t s_nosplit;             // = layer tag: a hidden value is outside the fp16 range
  uint32_t* s_pref = reinterpret_cast<uint32_t*>(s_x);
  uint32_t* s_uw = reinterpret_cast<uint32_t*>(s_x + kPrefBytes);
  int32_t* s_nid = reinterpret_cast<int32_t*>(s_x + kPrefBytes + kUwBytes);

  __shared__ uint32_t s_grp;                 // group_sync arrivals of waves 0..3
  if (threadIdx.x == 0) {
    s_grp = 0u;
    s_nosplit = 0u;                          // layer tags start at 1
  }
  lds_barrier();
  const uint32_t e0 = ld_agent(p.fbar + (size_t)blockIdx.x * kFS);
  int k_prev = -1;                           // active neurons of the previous layer
  bool x_from_lds = false;                   // up rows read the input from s_x
  Raw<16> w1r[kU];
  prefetch_w1<kU>(p, (CLayer*)p.layers, w1r);
  prefetch_w2_rows(p, (CLayer*)p.layers, s_w2, kAW, kNW, 0, 1 << 30);
  for (int l = 0; l < p.L; ++l) {
    const uint32_t tag = e0 + (uint32_t)l + 1u;
    CLayer* Ld = (CLayer*)p.layers + l;

    // ---------------------------------------------------------------- phase A
    {
      SFX_PHASE_IDS;
      // row w + P s of W1 in wave s (s < nr1 <= 4)
      const int a_row = w + P * wave;
      const bool a_active = wave < p.nr1 && a_row < h;
      const uint8_t* x = (const uint8_t*)Ld->x;
      // The input rows go to LDS first (waves 0..3, 16 bytes per lane; for layers
      // after the first they were requested during the grid barrier) and only
      // then does this layer's W2 stream start, so they are not queued behind
      // it.  Inputs larger than the staging area are read directly.  Waves 0..3
      // synchronise among themselves (group_sync) so the streaming waves,
      // blocked while their loads issue, hold nobody up.
      const bool x_lds = (size_t)B * rb1 <= (size_t)kXBytes;
      uint8_t* s_xin = s_x;
      const uint32_t g0 = 3u * kAW * (uint32_t)l;      // s_grp arrivals before this layer
      if (wave < kAW) {
        if (x_lds && l == 0) load_x_lds(p, Ld, s_x);
        group_sync(&s_grp, g0 + kAW, p.err);                  // inputs requested
        if (x_lds) wait_memory();
        group_sync(&s_grp, g0 + 2 * kAW, p.err);              // inputs landed
      } else if (l > 0) {
        lds_wait_at_least(&s_grp, g0 + kAW, p.err);
        prefetch_w2_rows(p, Ld, s_w2, kAW, kNW, 0, w2_split(f, P));
      }
      float acc[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[b] = 0.f;
      if (a_active) {
        // The input source is chosen once, outside the loop, and a group's input
        // chunks are all read before the first product (clamped, not branched
        // on): with the choice per chunk every read waited for all memory.
        auto dots = [&](auto from_lds) {
          constexpr bool kL = decltype(from_lds)::value;
          constexpr int MG = NB == 1 ? kU : NB == 2 ? (kU >= 4 ? kU / 2 : kU) : (kU >= 8 ? kU / 4 : kU);
#pragma unroll
          for (int m0 = 0; m0 < kU; m0 += MG) {
            Raw<16> xv[MG][NB];
#pragma unroll
            for (int i = 0; i < MG; ++i) {
              const int c = min(lane + (m0 + i) * kWave, nch1 - 1);
#pragma unroll
              for (int b = 0; b < NB; ++b) {
                const size_t off = (size_t)min(b, B - 1) * rb1 + (size_t)c * 16;
                if constexpr (kL) xv[i][b] = *reinterpret_cast<const Raw<16>*>(s_xin + off);
                else xv[i][b] = load_raw<16>(x + off);
              }
            }
#pragma unroll
            for (int i = 0; i < MG; ++i)
              if (lane + (m0 + i) * kWave < nch1) {
#pragma unroll
                for (int b = 0; b < NB; ++b)
                  if (b < B) dot_chunk<T>(w1r[m0 + i].w, xv[i][b].w, acc[b]);
              }
          }
        };
        if (x_lds) dots(std::true_type{});
        else dots(std::false_type{});
        const float v = wave_reduce_multi<NB>(acc);
        const int b = reduce_index<NB>(lane);
        if (reduce_owner<NB>(lane) && b < B)
          st_tagged(p.hid + (size_t)w * kHS + wave * NB + b, tag, __float_as_uint(fmaxf(v, 0.f)));
      }
      if (wave < kAW) group_sync(&s_grp, g0 + 3 * kAW, p.err);  // inputs read: s_x is reused in phase B
      // the rest of this layer's W2 rows (their waits fall in the scores phase,
      // which needs them anyway)
      if (l > 0) prefetch_w2_rows(p, Ld, s_w2, 0, kAW, w2_split(f, P), 1 << 30);
    }
    // ---------------------------------------------------------------- phase B
    {
      SFX_PHASE_IDS;
      // owned rows w + P j, j < nr2, and their mask words m < nwo (bit j % 32 of
      // word j / 32)
      const int nr2 = w < f ? (f - w + P - 1) / P : 0;
      const int nwo = (nr2 + 31) >> 5;
      const int rows2 = nr2;
      const bool w2_lds = p.w2_lds != 0;
      const uint8_t* W2 = (const uint8_t*)Ld->W2;
      // The hidden goes after the layer's input when both fit in s_x, so the up rows
      // read the input from LDS instead of memory: half the load requests of an up
      // row (one token, OPT-6.7B shape: 22.6 -> 21.4 us per layer-step).
      const size_t x_bytes = (size_t)B * rb1;
      const bool x_keep = w2_lds && x_bytes + (size_t)TB * h * 4 <= (size_t)kXBytes;
      const size_t hid_off = x_keep ? ((x_bytes + 255) & ~(size_t)255) : 0;
      x_from_lds = x_keep;
      float* s_hid = w2_lds ? reinterpret_cast<float*>(s_x + hid_off) : reinterpret_cast<float*>(s_w2);
      float* s_sc = s_red;                     // [rows2][NB]
      // Every wave first waits for its own W2 rows (waves 0..3 for their late share,
      // issued last), so the hidden is polled once the rows have landed, when the
      // other workgroups' hidden words are long out.  Polled from the end of phase A
      // instead, its rounds of loads slowed the W2 stream (one token: 22.9 -> 22.6 us
      // per layer-step at the OPT-6.7B shape, 23.9 -> 23.4 at LLaMA2-7B, with the
      // hidden words packed at 4 NB per workgroup).
      if (w2_lds) wait_memory();
      // waves 0..3 read the hidden: thread o polls the block of workgroup o (rows
      // o + P s, s < nr1, all tokens) and spreads it into s_hid[b][row].  With
      // fp16 W2 rows staged in LDS the hidden goes in as two fp16 pieces instead,
      // hi = fp16(h) and lo = fp16((h - hi) 2^11) (h to about 2^-22 relative, the
      // scaled lo clear of the subnormals), so the scores run on the fp16
      // dot-product instruction with fp32 sums; a hidden value outside the fp16
      // range sends the layer to the fp32 spread and sums instead.
      constexpr int kPT = kAW * kWave;
      constexpr bool kSplitH = std::is_same<T, TF16>::value;
      uint16_t* s_hh = reinterpret_cast<uint16_t*>(s_hid);     // [TB][h] hi
      uint16_t* s_hl = s_hh + (size_t)TB * h;                   // [TB][h] lo * 2^11
      auto spread = [&](bool split_in) {
        if (wave < kAW) {
#pragma unroll 1
          for (int o = tid; o < P; o += kPT) {
            const int ns = o < h ? (h - o + P - 1) / P : 0;
            // block entry s NB + b holds row o + P s, token b
            unsigned long long hw[4 * NB];
            auto valid = [&](int i) { return i / NB < ns && i % NB < B; };
            auto addr = [&](int i) { return p.hid + (size_t)o * kHS + i; };
            poll_tagged_if<4 * NB, decltype(valid), decltype(addr), kStepPS>(hw, valid, addr, tag, p.err);
#pragma unroll
            for (int i = 0; i < 4 * NB; ++i) {
              if (valid(i)) {
                const float v = __uint_as_float((uint32_t)hw[i]);
                const int at = (i % NB) * h + o + P * (i / NB);
                if (split_in) {
                  if (!(fabsf(v) < 65504.f)) s_nosplit = tag;
                  const _Float16 hi = (_Float16)v;
                  const _Float16 lo = (_Float16)((v - (float)hi) * 2048.f);
                  s_hh[at] = __builtin_bit_cast(uint16_t, hi);
                  s_hl[at] = __builtin_bit_cast(uint16_t, lo);
                } else {
                  s_hid[at] = v;
                }
              }
            }
          }
        }
        __syncthreads();
      };
      const bool split_try = kSplitH && w2_lds;
      spread(split_try);
      const bool split = split_try && s_nosplit != tag;
      if (split_try && !split) spread(false);   // the words are still in place: no wait
      // The W2 source is chosen once, outside the loop: with the choice inside it,
      // every row read became its own branch with a full memory wait, one LDS
      // round trip per row.
      auto scores_pass = [&](auto from_lds) {
        constexpr bool kLds = decltype(from_lds)::value;
        constexpr int b0 = 0;
        const int tb = B;
        for (int q0 = wave; q0 < rows2; q0 += kNW * kRB) {
          float a2[kRB * TB];
#pragma unroll
          for (int i = 0; i < kRB * TB; ++i) a2[i] = 0.f;
          for (int c = lane; c < nch2; c += kWave) {
            float hv[TB][8];
#pragma unroll
            for (int b = 0; b < TB; ++b) {
              const float4* hp = reinterpret_cast<const float4*>(s_hid + (b < tb ? b : 0) * h + c * 8);
              const float4 u0 = hp[0], u1 = hp[1];
              hv[b][0] = u0.x; hv[b][1] = u0.y; hv[b][2] = u0.z; hv[b][3] = u0.w;
              hv[b][4] = u1.x; hv[b][5] = u1.y; hv[b][6] = u1.z; hv[b][7] = u1.w;
            }
            // kRB rows per lane, no per-row branches (rows past the end are clamped
            // and their sums dropped), so the kRB TB accumulation chains interleave
            Raw<16> wv[kRB];
#pragma unroll
            for (int r = 0; r < kRB; ++r) {
              const int q = min(q0 + r * kNW, rows2 - 1);
              if constexpr (kLds) {
                wv[r] = *reinterpret_cast<const Raw<16>*>(s_w2 + ((size_t)q * nch2 + c) * 16);
              } else {
                const int row = min(w + P * q, f - 1);
                wv[r] = load_raw<16>(W2 + (size_t)row * rb2 + (size_t)c * 16);
              }
            }
            float wf[kRB][8];
#pragma unroll
            for (int r = 0; r < kRB; ++r) unpack<T, 4>(wv[r].w, wf[r]);
#pragma unroll
            for (int e = 0; e < 8; ++e)
#pragma unroll
              for (int r = 0; r < kRB; ++r)
#pragma unroll
                for (int b = 0; b < TB; ++b) a2[r * TB + b] = fmaf(wf[r][e], hv[b][e], a2[r * TB + b]);
          }
          const float v = wave_reduce_multi<kRB * TB>(a2);
          if (reduce_owner<kRB * TB>(lane)) {
            const int idx = reduce_index<kRB * TB>(lane);
            const int r = idx / TB, b = idx - r * TB;
            const int q = q0 + r * kNW;
            if (q < rows2 && b < tb) s_sc[q * NB + b0 + b] = v;
          }
        }
      };
      // the split hidden against the fp16 rows in LDS: two dot-product sums per
      // row, hi and lo (scaled back by 2^-11 at the end)
      auto scores_pass_split = [&]() {
        const int tb = B;
        for (int q0 = wave; q0 < rows2; q0 += kNW * kRB) {
          float a2[kRB * TB], a3[kRB * TB];
#pragma unroll
          for (int i = 0; i < kRB * TB; ++i) { a2[i] = 0.f; a3[i] = 0.f; }
          for (int c = lane; c < nch2; c += kWave) {
            half2_t hh[TB][4], hl[TB][4];
#pragma unroll
            for (int b = 0; b < TB; ++b) {
              const uint4 u = *reinterpret_cast<const uint4*>(s_hh + (size_t)(b < tb ? b : 0) * h + c * 8);
              const uint4 v = *reinterpret_cast<const uint4*>(s_hl + (size_t)(b < tb ? b : 0) * h + c * 8);
              hh[b][0] = __builtin_bit_cast(half2_t, u.x); hh[b][1] = __builtin_bit_cast(half2_t, u.y);
              hh[b][2] = __builtin_bit_cast(half2_t, u.z); hh[b][3] = __builtin_bit_cast(half2_t, u.w);
              hl[b][0] = __builtin_bit_cast(half2_t, v.x); hl[b][1] = __builtin_bit_cast(half2_t, v.y);
              hl[b][2] = __builtin_bit_cast(half2_t, v.z); hl[b][3] = __builtin_bit_cast(half2_t, v.w);
            }
            Raw<16> wv[kRB];
#pragma unroll
            for (int r = 0; r < kRB; ++r) {
              const int q = min(q0 + r * kNW, rows2 - 1);
              wv[r] = *reinterpret_cast<const Raw<16>*>(s_w2 + ((size_t)q * nch2 + c) * 16);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
              for (int r = 0; r < kRB; ++r) {
                const half2_t wj = __builtin_bit_cast(half2_t, wv[r].w[j]);
#pragma unroll
                for (int b = 0; b < TB; ++b) {
                  a2[r * TB + b] = __builtin_amdgcn_fdot2(wj, hh[b][j], a2[r * TB + b], false);
                  a3[r * TB + b] = __builtin_amdgcn_fdot2(wj, hl[b][j], a3[r * TB + b], false);
                }
              }
          }
#pragma unroll
          for (int i = 0; i < kRB * TB; ++i) a2[i] = fmaf(a3[i], 1.f / 2048.f, a2[i]);
          const float v = wave_reduce_multi<kRB * TB>(a2);
          if (reduce_owner<kRB * TB>(lane)) {
            const int idx = reduce_index<kRB * TB>(lane);
            const int r = idx / TB, b = idx - r * TB;
            const int q = q0 + r * kNW;
            if (q < rows2 && b < tb) s_sc[q * NB + b] = v;
          }
        }
      };
      if (split) scores_pass_split();
      else if (w2_lds) scores_pass(std::true_type{});
      else scores_pass(std::false_type{});
      __syncthreads();
      // own mask words by wave ballots (lane = own row j of a 64-row pair of
      // words), then the union words go out tagged (block words [0, nwm)), the
      // per-token words too when the caller asked for per-token masks (block words
      // nwm (1 + b) + m), then the scores
      for (int m0 = 2 * wave; m0 < nwo; m0 += 2 * kNW) {
        const int m = m0 + (lane >> 5);
        const int j = 32 * m + (lane & 31);
        const bool in = m < nwo && j < nr2;
        const float thr = Ld->threshold;
        for (int b = 0; b < B; ++b) {
          const uint64_t bal = __ballot(in && s_sc[j * NB + b] >= thr);
          if ((lane & 31) == 0 && m < nwo) s_words[m * NB + b] = (uint32_t)(lane == 0 ? bal : (bal >> 32));
        }
      }
      lds_barrier();
      const int nwm = own_words_max(f, P);
      if (tid < nwo) {
        uint32_t u = 0;
        for (int b = 0; b < B; ++b) u |= s_words[tid * NB + b];
        // word-major: word m of owner o at m P + o, so a poll of every owner's words
        // touches nwm P / 16 cache lines rather than one line per owner (OPT-6.7B
        // shape, one token: 21.35 -> 21.0 us per layer-step)
        st_tagged(p.uni + (size_t)tid * P + w, tag, u);
      }
      if (Ld->tok_bits != nullptr && tid < nwo * B) {
        const int m = tid / B, b = tid - m * B;
        st_tagged(p.uni + (size_t)(nwm * (1 + b) + m) * P + w, tag, s_words[m * NB + b]);
      }
      for (int i = tid; i < rows2 * B; i += kNT) {
        const int q = i / B, b = i - q * B;
        const int row = w + P * q;
        if (row < f) Ld->scores[(size_t)b * f + row] = s_sc[q * NB + b];
      }
    }

    // ---------------------------------------------------------------- phase C
    int k;                                     // active neurons of the layer
    bool in_lds;                               // their list fits in LDS (s_nid)
    {
    SFX_PHASE_IDS;
    // One up row: Wa (and Wl) row of neuron nid against the input, bias, activation,
    // out tagged and indexed by neuron.
    const uint8_t* x = (const uint8_t*)Ld->x;
    auto up_row = [&](int nid) {
      if constexpr (kGluSlot) {
        // one load batch: the Wl row into this wave's 8 KB slot of s_w2 (free from
        // the end of the scores to the next layer's W2 rows, past the union words
        // s_raw), the Wa row and the input into registers
        const uint8_t* ra = (const uint8_t*)Ld->Wa + (size_t)nid * rb1;
        const uint8_t* rl = (const uint8_t*)Ld->Wl + (size_t)nid * rb1;
        uint8_t* slot = s_w2 + kUpSlot0 + wave * kUpSlot;
        const float bias = Ld->ba != nullptr ? Ld->ba[nid] : 0.f;
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int c = min(lane + u * kWave, nch1 - 1);
          __builtin_amdgcn_global_load_lds((const void*)(rl + (size_t)c * 16),
                                           (__attribute__((address_space(3))) void*)(slot + u * kWave * 16), 16, 0, 0);
        }
        Raw<16> wa[kU], xq[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int c = min(lane + u * kWave, nch1 - 1);
          wa[u] = load_raw<16>(ra + (size_t)c * 16);
        }
        if (x_from_lds) {
#pragma unroll
          for (int u = 0; u < kU; ++u)
            xq[u] = *reinterpret_cast<const Raw<16>*>(s_x + (size_t)min(lane + u * kWave, nch1 - 1) * 16);
        } else {
#pragma unroll
          for (int u = 0; u < kU; ++u) xq[u] = load_raw<16>(x + (size_t)min(lane + u * kWave, nch1 - 1) * 16);
        }
        wait_memory();                           // registers and the slot
        float za[1] = {0.f}, zl[1] = {0.f};
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          if (lane + u * kWave < nch1) {
            dot_chunk<T>(wa[u].w, xq[u].w, za[0]);
            const Raw<16> wl = *reinterpret_cast<const Raw<16>*>(slot + (u * kWave + lane) * 16);
            dot_chunk<T>(wl.w, xq[u].w, zl[0]);
          }
        }
        const float ta = wave_reduce_multi<1>(za);
        const float v = fmaxf(ta + bias, 0.f) * wave_reduce_multi<1>(zl);
        if (lane == 0) st_tagged(p.hact + (size_t)nid, tag, __float_as_uint(v));
        return;
      }
      const uint8_t* ra = (const uint8_t*)Ld->Wa + (size_t)nid * rb1;
      const uint8_t* rl = REGLU ? (const uint8_t*)Ld->Wl + (size_t)nid * rb1 : nullptr;
      // the bias goes out ahead of the row (loaded after the dot products it
      // was one more round trip per row)
      const float bias = Ld->ba != nullptr ? Ld->ba[nid] : 0.f;
      float za[NB], zl[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) { za[b] = 0.f; zl[b] = 0.f; }
#pragma unroll
      for (int u0 = 0; u0 < kU; u0 += kUP) {
        // every load of the batch is issued before the first is used: chunk
        // indices are clamped instead of branched on, so the compiler keeps
        // them together and waits once
        Raw<16> wa[kUP], wl[kUP], xq[kUP][NB];
#pragma unroll
        for (int u = 0; u < kUP; ++u) {
          const int c = min(lane + (u0 + u) * kWave, nch1 - 1);
          wa[u] = load_raw<16>(ra + (size_t)c * 16);
          if (REGLU) wl[u] = load_raw<16>(rl + (size_t)c * 16);
        }
        if (x_from_lds) {
#pragma unroll
          for (int u = 0; u < kUP; ++u)
#pragma unroll
            for (int b = 0; b < NB; ++b)
              xq[u][b] = *reinterpret_cast<const Raw<16>*>(s_x + (size_t)min(b, B - 1) * rb1 +
                                                           (size_t)min(lane + (u0 + u) * kWave, nch1 - 1) * 16);
        } else {
#pragma unroll
          for (int u = 0; u < kUP; ++u)
#pragma unroll
            for (int b = 0; b < NB; ++b)
              xq[u][b] = load_raw<16>(x + (size_t)min(b, B - 1) * rb1 + (size_t)min(lane + (u0 + u) * kWave, nch1 - 1) * 16);
        }
#pragma unroll
        for (int u = 0; u < kUP; ++u) {
          if (lane + (u0 + u) * kWave < nch1) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
              if (b < B) {
                dot_chunk<T>(wa[u].w, xq[u][b].w, za[b]);
                if (REGLU) dot_chunk<T>(wl[u].w, xq[u][b].w, zl[b]);
              }
          }
        }
      }
      const float ta = wave_reduce_multi<NB>(za);
      float v = fmaxf(ta + bias, 0.f);
      if (REGLU) v *= wave_reduce_multi<NB>(zl);
      if (reduce_owner<NB>(lane)) {
        const int b = reduce_index<NB>(lane);
        if (b < B) st_tagged(p.hact + (size_t)nid * B + b, tag, __float_as_uint(v));
      }
    };
    // Up rows first, for this workgroup's own active neurons: the union bits of its
    // own rows w + P j (mask words still in s_words), so no exchange is waited for;
    // at most `cap` of them: twice the previous layer's even share ceil(k / P), at
    // least one round of the waves and at most kOwnCap (two rounds; kOwnCap for the
    // first layer).  These rows overlap the union exchange; the rows past `cap`
    // are left to the split below, after the union exchange.
    const int cap = k_prev < 0 ? kOwnCap : min(kOwnCap, max(kWork, 2 * ((k_prev + P - 1) / P)));
    const int nwm = own_words_max(f, P);
    {
      const int nr2 = w < f ? (f - w + P - 1) / P : 0;
      const int nwo = (nr2 + 31) >> 5;
      auto own_word = [&](int m) {
        uint32_t u = 0;
        for (int b = 0; b < B; ++b) u |= s_words[m * NB + b];
        return u;
      };
      int own_k = 0;
      for (int m = 0; m < nwo; ++m) own_k += __popc(own_word(m));
      const int own_n = min(own_k, cap);
      auto own_entry = [&](int e) {              // entry e of the own list: word m, its rem-th set bit
        int m = 0, rem = e;
        uint32_t um = own_word(0);
        while (rem >= __popc(um)) { rem -= __popc(um); um = own_word(++m); }
        for (int i = 0; i < rem; ++i) um &= um - 1;
        return w + P * (32 * m + __builtin_ctz(um));
      };
      for (int e = wave; e < own_n; e += kWork) up_row(own_entry(e));
    }
    // thread o polls the union words of owner o into s_raw[o][m] (zero past the
    // owner's words); s_w2 is free from the end of phase B to the next layer
    uint32_t* s_raw = reinterpret_cast<uint32_t*>(s_w2);      // [P][nwm]
#pragma unroll 1
    for (int o = tid; o < P; o += kNT) {
      const int nro = o < f ? (f - o + P - 1) / P : 0;
      const int nw = (nro + 31) >> 5;
#pragma unroll 1
      for (int m0 = 0; m0 < nwm; m0 += 8) {
        unsigned long long uv[8];
        const int n = min(8, nw - m0);
        auto valid = [&](int i) { return i < n; };
        auto addr = [&](int i) { return p.uni + (size_t)(m0 + i) * P + o; };
        poll_tagged_if<8, decltype(valid), decltype(addr), kStepPS>(uv, valid, addr, tag, p.err);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (m0 + i < nwm) s_raw[o * nwm + m0 + i] = i < n ? (uint32_t)uv[i] : 0u;
      }
    }
    lds_barrier();
    // Owner counts, scanned once: c_o (active rows of owner o) and, packed in the
    // same word, the owner's rows past `cap` (taken over by the split below); both
    // fit in 16 bits (k <= f <= 32 kMaxWords).  The exclusive prefix of c_o places
    // owner o's rows at positions [s_opre[o], s_opre[o + 1]) of an owner-major list
    // (owner ascending, then row ascending), which the down phase walks: it needs
    // no transposition or global scan first.
    uint32_t* s_own = reinterpret_cast<uint32_t*>(s_red) + 512;   // [P] own rows done first
    uint32_t* s_ovp = reinterpret_cast<uint32_t*>(s_red);         // [P + 1] overflow prefix
    uint32_t* s_opre = reinterpret_cast<uint32_t*>(s_nid) + kNidCap - (kMaxP + 1);   // [P + 1]
    int32_t* s_onid = s_nid;                                      // owner-major list
    const int onid_cap = kNidCap - (kMaxP + 1);
    {
      uint32_t c = 0, ovc = 0;
      if (tid < P) {
        for (int m = 0; m < nwm; ++m) c += __popc(s_raw[tid * nwm + m]);
        ovc = c > (uint32_t)cap ? c - (uint32_t)cap : 0u;
        s_own[tid] = c - ovc;
      }
      const uint32_t pk = c | (ovc << 16);
      const uint32_t inc = wave_inclusive_scan_u32(pk);
      if (lane == kWave - 1) s_wt[wave] = inc;
      lds_barrier();
      uint32_t before_pk = 0, total_pk = 0;
#pragma unroll
      for (int v = 0; v < kNW; ++v) {
        const uint32_t t = s_wt[v];
        if (v < wave) before_pk += t;
        total_pk += t;
      }
      const uint32_t base_pk = before_pk + inc - pk;
      k = (int)(total_pk & 0xffffu);
      k_prev = k;
      in_lds = k <= onid_cap;
      if (tid < P) {
        s_ovp[tid] = base_pk >> 16;
        s_opre[tid] = base_pk & 0xffffu;
        if (in_lds) {                            // owner tid's rows, ascending
          uint32_t at = base_pk & 0xffffu;
          for (int m = 0; m < nwm; ++m) {
            uint32_t wd = s_raw[tid * nwm + m];
            while (wd) { s_onid[at++] = tid + P * (32 * m + __builtin_ctz(wd)); wd &= wd - 1; }
          }
        }
      }
      if (tid == 0) {
        s_ovp[P] = total_pk >> 16;
        s_opre[P] = total_pk & 0xffffu;
      }
      if (w == 0 && tid == 0) *Ld->count = k;
      lds_barrier();
    }
    // neuron at owner-major position q: from the LDS list, or (long lists) by a
    // search of the owner prefix and a walk over that owner's set bits
    auto pos_to_neuron = [&](int q) -> int {
      if (in_lds) return s_onid[q];
      int lo = 0, hi = P;                        // s_opre[lo] <= q < s_opre[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if ((int)s_opre[mid] <= q) lo = mid; else hi = mid;
      }
      int m = 0, rem = q - (int)s_opre[lo];
      uint32_t um = s_raw[lo * nwm];
      while (rem >= __popc(um)) { rem -= __popc(um); um = s_raw[lo * nwm + (++m)]; }
      for (int i = 0; i < rem; ++i) um &= um - 1;
      return lo + P * (32 * m + __builtin_ctz(um));
    };

    // ---------------------------------------------------------------- phase D
    {
      // Down-phase geometry: workgroup w takes the column tile d_tile = w / dsplit
      // (64 columns: 128 bytes, one line, of every active row) and the positions
      // d_sub + dsplit i of the owner-major list (d_sub = w mod dsplit).  The same
      // bytes read as 32-byte slices of every row took about three times as long:
      // a compute unit keeps only so many line requests in flight.  Lane group
      // j = lane mod 8 reads columns c0 + 8 j; row slot wave * 8 + lane / 8 walks
      // the local positions i.
      const int dsplit = p.dsplit;
      const int d_tile = w / dsplit, d_sub = w - d_tile * dsplit;
      const int d_tiles = p.dtiles;
      const int c0 = d_tile * 64;
      const int d_j = lane & 7;
      const int d_rr = wave * 8 + (lane >> 3);
      const int d_rs = kWork * 8;
      const int d_col = c0 + d_j * 8;
      const bool d_ok = wave < kWork && d_tile < d_tiles && d_col < d;
      const int kl = k > d_sub ? (k - d_sub + dsplit - 1) / dsplit : 0;   // local positions
      const uint8_t* Wd = (const uint8_t*)Ld->Wd;
      Raw<16> wdv[kRD];
      int nid[kRD];
      auto load_wd = [&](int qb) {                 // kRD local positions at a time, qb < kl
        // positions past kl are clamped to kl - 1 (loaded, never used), so the
        // loads are issued back to back without branches
        // at one token (one batch of kRD = 8 rows per lane): the rows this wave needs
        // (wave-uniform: its lowest lane group's count); the rest are not loaded,
        // their neuron set to 0 so every poll address stays valid.  (Measured, us
        // per layer-step: one token 20.55 -> 20.4 / 23.15 -> 22.45 at the OPT-6.7B /
        // LLaMA2-7B shapes; at 3-4 tokens, several batches of kRD = 2, it cost 3 us.)
        const int nu = NB == 1 ? min(kRD, (kl - __builtin_amdgcn_readfirstlane(qb) + d_rs - 1) / d_rs) : kRD;
#pragma unroll
        for (int u = 0; u < kRD; ++u) nid[u] = u < nu ? pos_to_neuron(d_sub + dsplit * min(qb + u * d_rs, kl - 1)) : 0;
#pragma unroll
        for (int u = 0; u < kRD; ++u)
          if (u < nu) wdv[u] = load_raw<16>(Wd + (size_t)nid[u] * rb1 + (size_t)d_col * 2);
      };
      // the workers' first batch goes out before anything else is waited for; the
      // outputs in the standard layout are built while it is in flight
      if (d_ok && d_rr < kl) load_wd(d_rr);

      // The outputs in the standard layout (union words and the list with its
      // activations in rank order) are for the caller only: when this workgroup's
      // positions fit the save area (s_w2 past the raw mask words and the up-row
      // slots, which other waves may still fill with overflow rows while this wave
      // saves; the area is free until the next layer's W2 rows), the down loop keeps
      // (neuron, activation) of every position in LDS and the outputs are built after
      // the grid-barrier flag, while the other workgroups finish; otherwise before
      // the down loop, as the list is read.
      constexpr int kSave0 = kUpSlot0 + (kGluSlot ? kWork * kUpSlot : 0);
      const int save_cap = (kW2Bytes - kSave0) / (4 + 4 * NB);
      const bool late_out = kl <= save_cap;
      int32_t* s_snid = reinterpret_cast<int32_t*>(s_w2 + kSave0);          // [save_cap]
      float* s_shv = reinterpret_cast<float*>(s_w2 + kSave0) + save_cap;    // [save_cap][NB]
      auto std_outputs = [&]() {
      // Union words in the standard layout (bit b of word g = neuron 32 g + b).
        // With P = 64, 128 or 256, the neurons of word g share j = g / (P/32) and
        // belong to owners 32 (g mod P/32) + b.  Lane L holds the mask word c of owner
        // 64 q + L (bits j = 32 c + t); a 32 x 32 bit transpose within each half wave
        // (five exchange stages) leaves in lane t the bits j = 32 c + t of owners
        // 64 q .. + 31 (lanes 0..31) or 64 q + 32 .. + 63 (lanes 32..63): words
        // j P/32 + 2q (+1).
        {
          const int wv = __builtin_amdgcn_readfirstlane(wave);
          const int nq = P >> 6;
          const int nr2m = (f + P - 1) / P;
          for (int it = wv; it < nq * nwm; it += kNW) {
            const int q = it % nq, c = it / nq;
            uint32_t x = s_raw[(64 * q + lane) * nwm + c];
            x = transpose_step<16>(x, lane, 0xFFFF0000u);
            x = transpose_step<8>(x, lane, 0xFF00FF00u);
            x = transpose_step<4>(x, lane, 0xF0F0F0F0u);
            x = transpose_step<2>(x, lane, 0xCCCCCCCCu);
            x = transpose_step<1>(x, lane, 0xAAAAAAAAu);
            const int j = 32 * c + (lane & 31);
            const int g = j * (P >> 5) + 2 * q + (lane >> 5);
            if (j < nr2m && g < W) s_uw[g] = x;
          }
        }
        lds_barrier();
        // outputs of this workgroup: union words g = w + P m and, when asked for, the
        // per-token words (bit b from owner 32 (g mod P/32) + b, one tagged word per lane)
        for (int g = w + P * tid; g < W; g += P * kNT) Ld->union_bits[g] = s_uw[g];
        // prefix of the standard words (the rank of a neuron in the ascending list =
        // s_pref[g] + its set bits below it in word g); thread t owns words [wpt t, +wpt)
        {
          const int wpt = W <= kNT ? 1 : 2;
          const int g0 = wpt * tid;
          const uint32_t cnt0 = g0 < W ? __popc(s_uw[g0]) : 0u;
          const uint32_t cnt = cnt0 + (wpt == 2 && g0 + 1 < W ? __popc(s_uw[g0 + 1]) : 0u);
          const uint32_t inc = wave_inclusive_scan_u32(cnt);
          if (lane == kWave - 1) s_wt[wave] = inc;
          lds_barrier();
          uint32_t before = 0;
#pragma unroll
          for (int v = 0; v < kNW; ++v)
            if (v < wave) before += s_wt[v];
          const uint32_t base = before + inc - cnt;
          if (g0 < W) s_pref[g0] = base;
          if (wpt == 2 && g0 + 1 < W) s_pref[g0 + 1] = base + cnt0;
          if (tid == 0) s_pref[W] = (uint32_t)k;
          lds_barrier();
        }
      };
      if (!late_out) std_outputs();
      // per-token words (read from the owners' tagged words: before the flag)
      if (Ld->tok_bits != nullptr && wave == 0) {
        for (int g = w; g < W; g += P) {
          const int j = g / (P >> 5), c = g - j * (P >> 5);
          for (int b = 0; b < B; ++b) {
            unsigned long long tv[1];
            auto valid = [&](int i) { (void)i; return lane < 32; };
            auto addr = [&](int i) {
              (void)i;
              return p.uni + (size_t)(nwm * (1 + b) + (j >> 5)) * P + 32 * c + (lane & 31);
            };
            poll_tagged_if<1, decltype(valid), decltype(addr), kStepPS>(tv, valid, addr, tag, p.err);
            const uint64_t bal = __ballot(lane < 32 && (((uint32_t)tv[0] >> (j & 31)) & 1u) != 0u);
            if (lane == 0) Ld->tok_bits[(size_t)b * W + g] = (uint32_t)bal;
          }
        }
      }
      // Own entries past `cap` of every workgroup (owner o: the set bits of its own
      // mask words in order, from entry cap on), ranked by owner through the prefix
      // s_ovp, fill the workgroups up to T = ceil(k / P) rows each: workgroup w takes
      // the T - own_w overflow ranks after those of workgroups 0..w-1 (each wave sums
      // the deficits before w itself).  Since P T >= k the deficits cover every
      // overflow rank, and no workgroup does more than max(T, cap) up rows.
      {
        const int nov = (int)s_ovp[P];             // overflow rows of all workgroups
        const int fair = (k + P - 1) / P;          // T
        int dsum = 0;
        for (int o = lane; o < w; o += kWave) dsum += max(fair - (int)s_own[o], 0);
        dsum = wave_sum_i32(dsum, lane);
        const int q0 = min(dsum, nov), q1 = min(dsum + max(fair - (int)s_own[w], 0), nov);
        auto ov_entry = [&](int r) {               // neuron of overflow rank r
          int lo = 0, hi = P;                      // s_ovp[lo] <= r < s_ovp[hi]
          while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if ((int)s_ovp[mid] <= r) lo = mid; else hi = mid;
          }
          int m = 0, rem = cap + (r - (int)s_ovp[lo]);
          uint32_t um = s_raw[lo * nwm];
          while (rem >= __popc(um)) { rem -= __popc(um); um = s_raw[lo * nwm + (++m)]; }
          for (int i = 0; i < rem; ++i) um &= um - 1;
          return lo + P * (32 * m + __builtin_ctz(um));
        };
        // the input is still in s_x unless the standard-layout outputs were built over
        // it (before the down loop) or the owner-major list reaches into it
        x_from_lds = x_from_lds && late_out && (size_t)B * rb1 <= (size_t)(kPrefBytes + kUwBytes);
        for (int r = q0 + wave; r < q1; r += kWork) up_row(ov_entry(r));
      }

      float yacc[NB * 8];
#pragma unroll
      for (int i = 0; i < NB * 8; ++i) yacc[i] = 0.f;
      if (d_ok) {
        for (int qb = d_rr; qb < kl; qb += d_rs * kRD) {
          if (qb != d_rr) load_wd(qb);
          unsigned long long hv[kRD * NB];
          const int nrow = min(kRD, (kl - qb + d_rs - 1) / d_rs);
          // entry u NB + b: activation of position qb + u d_rs, token b
          auto valid = [&](int i) { return i / NB < nrow && i % NB < B; };
          auto addr = [&](int i) { return p.hact + (size_t)nid[i / NB] * B + min(i % NB, B - 1); };
          poll_tagged_if<kRD * NB, decltype(valid), decltype(addr), kStepPS>(hv, valid, addr, tag, p.err);
          // the list and the activations in rank order (outputs): rank r is
          // written by the workgroup whose column tile is r mod the tile count
          if (d_j == 0) {
#pragma unroll
            for (int u = 0; u < kRD; ++u) {
              if (u < nrow) {
                const int n = nid[u];
                if (late_out) {
                  const int i = qb + u * d_rs;
                  s_snid[i] = n;
#pragma unroll
                  for (int b = 0; b < NB; ++b) s_shv[i * NB + b] = __uint_as_float((uint32_t)hv[u * NB + b]);
                } else {
                  const int g = n >> 5;
                  const int r = (int)s_pref[g] + __popc(s_uw[g] & ((1u << (n & 31)) - 1u));
                  if (r % d_tiles == d_tile) {
                    Ld->idx[r] = n;
#pragma unroll
                    for (int b = 0; b < NB; ++b)
                      if (b < B) Ld->hact[(size_t)r * B + b] = __uint_as_float((uint32_t)hv[u * NB + b]);
                  }
                }
              }
            }
          }
#pragma unroll
          for (int u = 0; u < kRD; ++u) {
            if (u < nrow) {
              float wf[8];
              unpack<T, 4>(wdv[u].w, wf);
#pragma unroll
              for (int b = 0; b < NB; ++b)
                if (b < B) {
                  const float hvf = __uint_as_float((uint32_t)hv[u * NB + b]);
#pragma unroll
                  for (int e = 0; e < 8; ++e) yacc[b * 8 + e] = fmaf(hvf, wf[e], yacc[b * 8 + e]);
                }
            }
          }
        }
      }
      // Sum over the 8 row slots of each wave (lane L ends with column
      // 8 (L mod 8) + L / 8 of the tile, per token), then over the worker waves in a
      // fixed order: this workgroup's share of the tile, handed over tagged; the
      // tile's first workgroup adds the dsplit shares (tile_y_sum) before the grid
      // barrier.
      float vb[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        float t8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) t8[e] = yacc[b * 8 + e];
        vb[b] = wave_reduce_multi_groups<8, 8>(t8);
      }
      lds_barrier();                                     // every wave is past its rows: s_x is free
      float* s_part = reinterpret_cast<float*>(s_x);     // [kNW][NB][64]
      {
        const int colL = 8 * (lane & 7) + (lane >> 3);
#pragma unroll
        for (int b = 0; b < NB; ++b) s_part[(wave * NB + b) * 64 + colL] = vb[b];
      }
      lds_barrier();
      // written by waves kAW + b (their next full memory wait is in the scores
      // phase; wave 0's comes as soon as the next layer's inputs are requested)
      if (d_tile < d_tiles && wave >= kAW && wave - kAW < B) {
        const int col = lane, b = wave - kAW;
        float sum = 0.f;
        for (int wv2 = 0; wv2 < kWork; ++wv2) sum += s_part[(wv2 * NB + b) * 64 + col];
        st_tagged(p.ypart + ((size_t)(l & 1) * P + w) * (64 * NB) + b * 64 + col, tag, __float_as_uint(sum));
      }
      // The tile's first workgroup adds the dsplit shares and writes y before it
      // raises its flag, so y of this layer is complete when the grid barrier
      // passes (the order a real model imposes: the next layer's input follows
      // from y).
      {
        unsigned long long yv[8];
        tile_y_issue<NB>(p, l, yv);
        tile_y_sum<NB>(p, l, tag, yv);
      }
      // Grid barrier, first half: the flag goes up once every wave is done with the
      // layer's exchanges (and y of this workgroup's tile is written).
      lds_barrier();
      if (l + 1 < p.L && tid == 0) store_through(p.fbar + (size_t)w * kFS, tag);
      if (late_out) {
        std_outputs();
        if (d_tile < d_tiles) {
          for (int i = tid; i < kl; i += kNT) {
            const int n = s_snid[i], g = n >> 5;
            const int r = (int)s_pref[g] + __popc(s_uw[g] & ((1u << (n & 31)) - 1u));
            if (r % d_tiles == d_tile) {
              Ld->idx[r] = n;
              for (int b = 0; b < B; ++b) Ld->hact[(size_t)r * B + b] = s_shv[i * NB + b];
            }
          }
        }
        lds_barrier();                           // s_x is the next layer's input area
      }
    }
    }                                          // phases C and D
    if (l + 1 < p.L) {
      // grid barrier, second half: every workgroup has raised its flag (end of
      // phase D) and waits for all flags
      SFX_PHASE_IDS;
      prefetch_w1<kU>(p, (CLayer*)p.layers + l + 1, w1r);
      // the next layer's input (in place since the launch) goes to LDS now: s_x is
      // free once every wave has passed the last LDS barrier of phase D
      if (wave < kAW && (size_t)B * rb1 <= (size_t)kXBytes) load_x_lds(p, (CLayer*)p.layers + l + 1, s_x);
      if (kTlbWarm && wave == kCW - 1 && lane == 0) {
        // one load per 2 MiB page of the next layer's weights, spread over the
        // workgroups, so their address translations are warm when the layer starts
        CLayer* Ln = (CLayer*)p.layers + l + 1;
        const size_t bw1 = (size_t)h * rb1, bw2 = (size_t)f * rb2, brow = (size_t)f * rb1;
        const size_t n1 = (bw1 + (1u << 21) - 1) >> 21, n2 = (bw2 + (1u << 21) - 1) >> 21;
        const size_t n3 = (brow + (1u << 21) - 1) >> 21;
        for (size_t pg = w; pg < n1 + n2 + 2 * n3; pg += P) {
          const uint8_t* base;
          size_t off;
          if (pg < n1) { base = (const uint8_t*)Ln->W1; off = pg << 21; }
          else if (pg < n1 + n2) { base = (const uint8_t*)Ln->W2; off = (pg - n1) << 21; }
          else if (pg < n1 + n2 + n3) { base = (const uint8_t*)Ln->Wa; off = (pg - n1 - n2) << 21; }
          else { base = (const uint8_t*)Ln->Wd; off = (pg - n1 - n2 - n3) << 21; }
          const uint32_t v = __builtin_nontemporal_load((const uint32_t*)(base + off));
          if (v == 0x7fc00001u && f < 0) Ld->y[0] = 0.f;   // keeps the load
        }
      }
      if (wave == kCW) wait_flags(p.fbar, P, tag, p.err, 1u);
      lds_barrier();
    }
  }
  // Every workgroup ends with all its flags at e0 + L, so all flags agree at the next call.
  if (threadIdx.x == 0) store_through(p.fbar + (size_t)blockIdx.x * kFS, e0 + (uint32_t)p.L);
}

template <class T, int NB, int DL>
hipError_t run_step(hipStream_t s, const StepParams& p, int act, int P) {
  if (act == 1) k_step<T, NB, true, DL><<<dim3(P), dim3(kNT), 0, s>>>(p);
  else k_step<T, NB, false, DL><<<dim3(P), dim3(kNT), 0, s>>>(p);
  return hipGetLastError();
}

// Workgroups of this instantiation that fit on one compute unit at once (registers,
// LDS): the grid of one workgroup per compute unit is resident only when this is >= 1.
template <class T, int NB, int DL>
int blocks_per_cu(int act) {
  int n = 0;
  hipError_t e = act == 1 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_step<T, NB, true, DL>, kNT, 0)
                          : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_step<T, NB, false, DL>, kNT, 0);
  return e == hipSuccess ? n : 0;
}
template <class T>
int step_blocks_per_cu(int act, int B) {
  switch (nb_class(B)) {
    case 1: return blocks_per_cu<T, 1, 1>(act);
    case 2: return blocks_per_cu<T, 2, 1>(act);
    default: return blocks_per_cu<T, 4, 1>(act);
  }
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
