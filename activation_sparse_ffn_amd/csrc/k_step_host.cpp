// Host side of the fused multi-layer step: which shapes it is built for, its
// workspace and its launch.
#include <hip/hip_runtime.h>

#include <atomic>

#include "sfx_common.hpp"
#include "sfx_launch.hpp"
#include "sfx_step.hpp"

namespace sfx {

hipError_t launch_step_f16(hipStream_t s, const StepParams& p, int act, int P, int DL);
hipError_t launch_step_bf16(hipStream_t s, const StepParams& p, int act, int P, int DL);
int step_blocks_per_cu_f16(int act, int B);
int step_blocks_per_cu_bf16(int act, int B);
hipError_t launch_pipe_f16(hipStream_t s, const StepParams& p, int act, int P);
hipError_t launch_pipe_bf16(hipStream_t s, const StepParams& p, int act, int P);
int pipe_blocks_per_cu_f16(int act, int B);
int pipe_blocks_per_cu_bf16(int act, int B);

namespace {
constexpr int kNT = 512, kW2Bytes = 131072, kRedFloats = 1024;
constexpr int kXBytes = 163840 - kW2Bytes - kRedFloats * 4 - 768;
constexpr int kMaxWords = 1024;
constexpr int kPrefBytes = (kMaxWords + 8) * 4, kUwBytes = kMaxWords * 4;
}  // namespace

StepGeom step_geometry(int wdt, int act, int B, int d, int h, int f, int P) {
  StepGeom g{};
  g.ok = false;
  g.P = P;
  // P = 64, 128 or 256: the fused step rebuilds union words from the owners' masks
  // with one ballot per 64 owners, the 8 waves split evenly over the owner groups
  if (P != 64 && P != 128 && P != 256) return g;
  if ((wdt != DT_F16 && wdt != DT_BF16) || B < 1 || B > 4 || (act != 0 && act != 1)) return g;
  if (d < 8 || h < 8 || d % 8 != 0 || h % 8 != 0 || f < 1) return g;
  const int W = (f + 31) / 32;
  if (W > kMaxWords) return g;
  const int nch1 = d / 8, nch2 = h / 8;
  g.dl = nch1 <= 512 ? 1 : 0;
  if (g.dl == 0) return g;
  g.nr1 = (h + P - 1) / P;
  if (g.nr1 > 4) return g;                  // one W1 row per wave of waves 0..3
  const int NB = nb_class(B);
  const int nw2max = (W + P - 1) / P;
  if (32 * nw2max * NB > kRedFloats) return g;
  const long long items = 32LL * nw2max * nch2;
  g.w2_lds = ((items + 63) / 64) * 64 * 16 <= kW2Bytes ? 1 : 0;
  const int TB = NB < 4 ? NB : 4;
  const long long hid_bytes = 4LL * TB * h;
  if (hid_bytes > (g.w2_lds ? kXBytes : kW2Bytes)) return g;
  int nct = (d + 8 * P - 1) / (8 * P);
  int n = 1;
  while (n < nct) n <<= 1;
  if (n > 2) return g;                       // down: at most 2 lane groups of 8 columns
  g.cw = 8 * n;
  // fused step's down phase: 64-column tiles, each split over dsplit workgroups
  g.dtiles = (d + 63) / 64;
  g.dsplit = P / g.dtiles < 8 ? P / g.dtiles : 8;
  g.ok = true;
  (void)kNT;
  return g;
}

// The Live Pipeline kernel: the fused step's shapes, with the scores of the owned
// rows in half of the reduction scratch (the down sums use the other half) and the
// hidden staged behind the list area of s_x, which stays live while it is read.
StepGeom pipe_geometry(int wdt, int act, int B, int d, int h, int f, int P) {
  StepGeom g = step_geometry(wdt, act, B, d, h, f, P);
  if (!g.ok) return g;
  const int W = (f + 31) / 32;
  const int nw2max = (W + P - 1) / P;
  const int NB = nb_class(B);
  const int TB = NB < 4 ? NB : 4;
  if (32 * nw2max * NB > kRedFloats / 2) g.ok = false;
  if (kPrefBytes + kUwBytes + 4LL * TB * h > kXBytes) g.ok = false;
  return g;
}

namespace {
size_t up256(size_t n) { return (n + 255) & ~(size_t)255; }
}  // namespace

// Tagged words per workgroup block of the union exchange: the fused step's own
// mask words (rows w + P j) and, for the per-token masks, B more of them; the Live
// Pipeline kernel's union words (words w + P m).
int step_union_block(int f, int P, int B) {
  const int W = (f + 31) / 32;
  const int nw2max = (W + P - 1) / P;
  const int nwm = ((f + P - 1) / P + 31) / 32;
  const int n = nw2max > nwm * (1 + B) ? nw2max : nwm * (1 + B);
  return (n + 7) & ~7;
}

// control line | barrier flags [P][kFlagStride] | hidden [P][16] | union [P][us] |
// hact [f][B] | tile shares of y [2][P][64 NB]  (tagged words: 8 bytes)
size_t step_ws_bytes(int B, int h, int f, int P) {
  (void)h;
  const size_t fl = up256((size_t)P * kFlagStride * 4);
  return 256 + fl + up256((size_t)P * 16 * 8) + up256((size_t)P * step_union_block(f, P, B) * 8) +
         up256((size_t)f * B * 8) + up256((size_t)2 * P * 64 * nb_class(B) * 8);
}

StepParams step_params(int B, int d, int h, int f, int L, const LayerDesc* layers, void* ws, const StepGeom& g) {
  StepParams p{};
  p.layers = layers;
  p.L = L;
  p.B = B;
  p.d = d;
  p.h = h;
  p.f = f;
  p.W = (f + 31) / 32;
  p.nr1 = g.nr1;
  p.w2_lds = g.w2_lds;
  p.cw = g.cw;
  uint8_t* base = (uint8_t*)ws;
  p.err = (uint32_t*)base;
  p.us = step_union_block(f, g.P, B);
  const size_t fl = up256((size_t)g.P * kFlagStride * 4);
  p.fbar = (uint32_t*)(base + 256);
  size_t off = 256 + fl;
  p.hid = (unsigned long long*)(base + off);
  off += up256((size_t)g.P * 16 * 8);
  p.uni = (unsigned long long*)(base + off);
  off += up256((size_t)g.P * p.us * 8);
  p.hact = (unsigned long long*)(base + off);
  off += up256((size_t)f * B * 8);
  p.ypart = (unsigned long long*)(base + off);
  p.dsplit = g.dsplit;
  p.dtiles = g.dtiles;
  return p;
}

// The persistent grid (one workgroup per compute unit) is only resident when one
// workgroup of the instantiation fits on a compute unit.  Host-side occupancy query,
// cached per device and instantiation.
bool step_resident(int wdt, int act, int B) {
  static std::atomic<int> cache[8][2][2][3];   // device, dtype, act, token class: 0 unknown, 1 yes, 2 no
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return false;
  const int nb = nb_class(B), ci = nb == 1 ? 0 : nb == 2 ? 1 : 2;
  const int di = wdt == DT_BF16 ? 1 : 0;
  std::atomic<int>* c = dev < 8 ? &cache[dev][di][act & 1][ci] : nullptr;
  if (c != nullptr) {
    const int v = c->load(std::memory_order_relaxed);
    if (v != 0) return v == 1;
  }
  const int n = wdt == DT_BF16 ? step_blocks_per_cu_bf16(act, B) : step_blocks_per_cu_f16(act, B);
  if (c != nullptr) c->store(n >= 1 ? 1 : 2, std::memory_order_relaxed);
  return n >= 1;
}

bool pipe_resident(int wdt, int act, int B) {
  static std::atomic<int> cache[8][2][2][3];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return false;
  const int nb = nb_class(B), ci = nb == 1 ? 0 : nb == 2 ? 1 : 2;
  const int di = wdt == DT_BF16 ? 1 : 0;
  std::atomic<int>* c = dev < 8 ? &cache[dev][di][act & 1][ci] : nullptr;
  if (c != nullptr) {
    const int v = c->load(std::memory_order_relaxed);
    if (v != 0) return v == 1;
  }
  const int n = wdt == DT_BF16 ? pipe_blocks_per_cu_bf16(act, B) : pipe_blocks_per_cu_f16(act, B);
  if (c != nullptr) c->store(n >= 1 ? 1 : 2, std::memory_order_relaxed);
  return n >= 1;
}

hipError_t launch_pipe(hipStream_t s, int wdt, int act, int B, int d, int h, int f, int L, const LayerDesc* layers,
                       void* ws, const StepGeom& g) {
  const StepParams p = step_params(B, d, h, f, L, layers, ws, g);
  if (wdt == DT_F16) return launch_pipe_f16(s, p, act, g.P);
  return launch_pipe_bf16(s, p, act, g.P);
}

hipError_t launch_step(hipStream_t s, int wdt, int act, int B, int d, int h, int f, int L, const LayerDesc* layers,
                       void* ws, const StepGeom& g) {
  const StepParams p = step_params(B, d, h, f, L, layers, ws, g);
  if (wdt == DT_F16) return launch_step_f16(s, p, act, g.P, g.dl);
  return launch_step_bf16(s, p, act, g.P, g.dl);
}

}  // namespace sfx
