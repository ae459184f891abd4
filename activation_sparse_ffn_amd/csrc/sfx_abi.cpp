// C ABI of libsfx: host-side argument checks, workspace queries, status strings.
// Every check runs before anything is enqueued, and no check touches the GPU
// except the CU-count query that sizes persistent grids.
#include <hip/hip_runtime.h>

#include <atomic>

#include "../../include/sfx.h"
#include "sfx_launch.hpp"
#include "sfx_step.hpp"

namespace sfx {

int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

}  // namespace sfx

namespace {

int elem_bytes(int wdt) {
  switch (wdt) {
    case SFX_F32: return 4;
    case SFX_F16: return 2;
    case SFX_BF16: return 2;
    default: return 0;
  }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }
bool aligned256(const void* p) { return ((uintptr_t)p & 255u) == 0; }

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return SFX_OK;
  if (ws == nullptr || !aligned256(ws) || ws_bytes < need) return SFX_E_WORKSPACE;
  return SFX_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? SFX_OK : SFX_E_LAUNCH; }

// Row of `n` stored elements of `wdt` (Q4: n codes) spans a multiple of 16 bytes.
bool row_ok(int wdt, long long n) {
  if (wdt == SFX_Q4G32) return n % 32 == 0;
  return (n * elem_bytes(wdt)) % 16 == 0;
}

}  // namespace

extern "C" {

const char* sfx_status_str(int status) {
  switch (status) {
    case SFX_OK: return "ok";
    case SFX_E_NULL: return "required pointer is NULL";
    case SFX_E_SHAPE: return "size out of range or inconsistent";
    case SFX_E_DTYPE: return "unknown or unsupported dtype / activation for this call";
    case SFX_E_ALIGN: return "pointer or row not 16-byte aligned";
    case SFX_E_WORKSPACE: return "workspace NULL, misaligned or too small";
    case SFX_E_LAUNCH: return "HIP reported a launch error";
    case SFX_E_UNSUPPORTED: return "combination not built";
    case SFX_E_DEVICE: return "no current HIP device";
    case SFX_E_SCRATCH: return "needs more scratch than the static maximum (SFX_DOWN_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int sfx_abi_version(void) { return SFX_ABI_VERSION; }

// ------------------------------------------------------------------------------ predict

size_t sfx_predict_ws(int wdt, int B, int d, int h, int f) {
  if (B < 1 || B > SFX_MAX_B || h < 1) return 0;
  if (wdt < SFX_F32 || wdt > SFX_Q4G32) return 0;
  return sfx::predict_ws_bytes(wdt, B, d, h, f);
}

int sfx_predict(void* stream, int wdt, int B, int d, int h, int f, const void* x, const void* W1,
                const void* W2, float* scores, void* ws, size_t ws_bytes) {
  if (wdt != SFX_F32 && wdt != SFX_F16 && wdt != SFX_BF16) return SFX_E_DTYPE;
  if (B < 1 || B > SFX_MAX_B || d < 1 || h < 1 || f < 1) return SFX_E_SHAPE;
  if (!x || !W1 || !W2 || !scores) return SFX_E_NULL;
  if (!row_ok(wdt, d) || !row_ok(wdt, h)) return SFX_E_ALIGN;
  if (!aligned16(x) || !aligned16(W1) || !aligned16(W2) || !aligned16(scores)) return SFX_E_ALIGN;
  const int w = check_ws(ws, ws_bytes, sfx::predict_ws_bytes(wdt, B, d, h, f));
  if (w != SFX_OK) return w;
  return launch_status(
      sfx::launch_predict((hipStream_t)stream, wdt, B, d, h, f, x, W1, W2, scores, ws));
}

int sfx_predict_q4(void* stream, int B, int d, int h, int f, const void* x, const void* W1, const void* W1_scales,
                   const void* W2, const void* W2_scales, float* scores, void* ws, size_t ws_bytes) {
  if (B < 1 || B > SFX_MAX_B || d < 1 || h < 1 || f < 1) return SFX_E_SHAPE;
  if (d % 32 != 0 || h % 32 != 0) return SFX_E_SHAPE;
  if (!x || !W1 || !W1_scales || !W2 || !W2_scales || !scores) return SFX_E_NULL;
  if (!aligned16(x) || !aligned16(W1) || !aligned16(W2) || !aligned16(scores)) return SFX_E_ALIGN;
  if (((uintptr_t)W1_scales & 1u) != 0 || ((uintptr_t)W2_scales & 1u) != 0) return SFX_E_ALIGN;
  const int w = check_ws(ws, ws_bytes, sfx::predict_ws_bytes(SFX_Q4G32, B, d, h, f));
  if (w != SFX_OK) return w;
  return launch_status(
      sfx::launch_predict_q4((hipStream_t)stream, B, d, h, f, x, W1, W1_scales, W2, W2_scales, scores, ws));
}

// ------------------------------------------------------------------------------ compact

size_t sfx_compact_ws(int B, int f) {
  if (B < 1 || f < 1) return 0;
  return sfx::compact_ws_bytes(B, f);
}

int sfx_compact(void* stream, int B, int f, const float* scores, float threshold, uint32_t* tok_bits,
                uint32_t* union_bits, int32_t* idx, int kmax, int32_t* count, void* ws, size_t ws_bytes) {
  if (B < 1 || B > SFX_MAX_B || f < 1) return SFX_E_SHAPE;
  if (kmax < f) return SFX_E_SHAPE;
  if (!scores || !union_bits || !idx || !count) return SFX_E_NULL;
  if (!aligned16(scores) || !aligned4(union_bits) || !aligned4(idx) || (tok_bits && !aligned4(tok_bits)))
    return SFX_E_ALIGN;
  const int w = check_ws(ws, ws_bytes, sfx::compact_ws_bytes(B, f));
  if (w != SFX_OK) return w;
  return launch_status(sfx::launch_compact((hipStream_t)stream, B, f, scores, threshold, tok_bits, union_bits,
                                           idx, kmax, count, ws));
}

// ------------------------------------------------------------------------------ up

int sfx_sparse_up(void* stream, int wdt, int act, int B, int d, int f, const void* x, const void* Wa,
                  const void* Wa_scales, const float* ba, const void* Wl, const void* Wl_scales,
                  const int32_t* idx, const int32_t* count, int kmax, float* hact) {
  if (wdt < SFX_F32 || wdt > SFX_Q4G32) return SFX_E_DTYPE;
  if (act != SFX_RELU && act != SFX_REGLU && act != SFX_RELU2) return SFX_E_DTYPE;
  if (B < 1 || B > SFX_MAX_B || d < 1 || f < 1 || kmax < 1) return SFX_E_SHAPE;
  if (!x || !Wa || !idx || !count || !hact) return SFX_E_NULL;
  if (act == SFX_REGLU && !Wl) return SFX_E_NULL;
  if (wdt == SFX_Q4G32 && (!Wa_scales || (act == SFX_REGLU && !Wl_scales))) return SFX_E_NULL;
  if (!row_ok(wdt, d)) return wdt == SFX_Q4G32 ? SFX_E_SHAPE : SFX_E_ALIGN;
  if (!aligned16(x) || !aligned16(Wa) || !aligned16(hact) || (Wl && !aligned16(Wl))) return SFX_E_ALIGN;
  if (!sfx::up_supported(wdt, act, B)) return SFX_E_UNSUPPORTED;
  return launch_status(sfx::launch_up((hipStream_t)stream, wdt, act, B, d, f, x, Wa, Wa_scales, ba,
                                      act == SFX_REGLU ? Wl : nullptr, Wl_scales, idx, count, kmax, hact));
}

// ------------------------------------------------------------------------------ down

size_t sfx_sparse_down_ws(int wdt, int B, int d, int kmax) {
  if (wdt < SFX_F32 || wdt > SFX_Q4G32 || B < 1 || B > SFX_MAX_B || d < 1 || kmax < 1) return 0;
  return sfx::down_ws_bytes(wdt, B, d, kmax);
}

int sfx_sparse_down(void* stream, int wdt, int B, int d, int f, const void* Wd, const void* Wd_scales,
                    const int32_t* idx, const int32_t* count, int kmax, const float* hact, float* y, void* ws,
                    size_t ws_bytes) {
  if (wdt < SFX_F32 || wdt > SFX_Q4G32) return SFX_E_DTYPE;
  if (B < 1 || B > SFX_MAX_B || d < 1 || f < 1 || kmax < 1) return SFX_E_SHAPE;
  if (!Wd || !idx || !count || !hact || !y) return SFX_E_NULL;
  if (wdt == SFX_Q4G32 && !Wd_scales) return SFX_E_NULL;
  if (!row_ok(wdt, d)) return wdt == SFX_Q4G32 ? SFX_E_SHAPE : SFX_E_ALIGN;
  if (!aligned16(Wd) || !aligned16(hact) || !aligned16(y)) return SFX_E_ALIGN;
  if (!sfx::down_supported(wdt, B)) return SFX_E_UNSUPPORTED;
  const int w = check_ws(ws, ws_bytes, sfx::down_ws_bytes(wdt, B, d, kmax));
  if (w != SFX_OK) return w;
  return launch_status(sfx::launch_down((hipStream_t)stream, wdt, B, d, f, Wd, Wd_scales, idx, count, kmax,
                                        hact, y, ws));
}

int sfx_sparse_down_noalloc(void* stream, int wdt, int B, int d, int f, const void* Wd, const void* Wd_scales,
                            const int32_t* idx, const int32_t* count, int kmax, const float* hact, float* y) {
  if (wdt < SFX_F32 || wdt > SFX_Q4G32) return SFX_E_DTYPE;
  if (B < 1 || B > SFX_MAX_B || d < 1 || f < 1 || kmax < 1) return SFX_E_SHAPE;
  if (!Wd || !idx || !count || !hact || !y) return SFX_E_NULL;
  if (wdt == SFX_Q4G32 && !Wd_scales) return SFX_E_NULL;
  if (!row_ok(wdt, d)) return wdt == SFX_Q4G32 ? SFX_E_SHAPE : SFX_E_ALIGN;
  if (!aligned16(Wd) || !aligned16(hact) || !aligned16(y)) return SFX_E_ALIGN;
  if (!sfx::down_supported(wdt, B)) return SFX_E_UNSUPPORTED;
  const size_t need = sfx::down_ws_bytes(wdt, B, d, kmax);
  if (need > sfx::kDownScratchBytes) return SFX_E_SCRATCH;
  void* scratch = nullptr;
  if (sfx::down_scratch(&scratch) != hipSuccess) return SFX_E_DEVICE;
  return launch_status(sfx::launch_down((hipStream_t)stream, wdt, B, d, f, Wd, Wd_scales, idx, count, kmax,
                                        hact, y, scratch));
}

// ------------------------------------------------------------------------------ dense step

size_t sfx_dense_ffn_ws(int wdt, int B, int d, int f) {
  if (wdt < SFX_F32 || wdt > SFX_Q4G32 || B < 1 || B > SFX_MAX_B || d < 1 || f < 1) return 0;
  return sfx::dense_ws_bytes(wdt, B, d, f);
}

int sfx_dense_ffn(void* stream, int wdt, int act, int B, int d, int f, const void* x, const void* Wa,
                  const void* Wa_scales, const float* ba, const void* Wl, const void* Wl_scales, const void* Wd,
                  const void* Wd_scales, float* hact, float* y, void* ws, size_t ws_bytes) {
  if (wdt < SFX_F32 || wdt > SFX_Q4G32) return SFX_E_DTYPE;
  if (act != SFX_RELU && act != SFX_REGLU && act != SFX_RELU2) return SFX_E_DTYPE;
  if (B < 1 || B > SFX_MAX_B || d < 1 || f < 1) return SFX_E_SHAPE;
  if (!x || !Wa || !Wd || !hact || !y) return SFX_E_NULL;
  if (act == SFX_REGLU && !Wl) return SFX_E_NULL;
  if (wdt == SFX_Q4G32 && (!Wa_scales || !Wd_scales || (act == SFX_REGLU && !Wl_scales))) return SFX_E_NULL;
  if (!row_ok(wdt, d)) return wdt == SFX_Q4G32 ? SFX_E_SHAPE : SFX_E_ALIGN;
  if (!aligned16(x) || !aligned16(Wa) || !aligned16(Wd) || !aligned16(hact) || !aligned16(y) ||
      (Wl && !aligned16(Wl)))
    return SFX_E_ALIGN;
  if (!sfx::up_supported(wdt, act, B) || !sfx::down_supported(wdt, B)) return SFX_E_UNSUPPORTED;
  const int w = check_ws(ws, ws_bytes, sfx::dense_ws_bytes(wdt, B, d, f));
  if (w != SFX_OK) return w;
  return launch_status(sfx::launch_dense((hipStream_t)stream, wdt, act, B, d, f, x, Wa, Wa_scales, ba,
                                         act == SFX_REGLU ? Wl : nullptr, Wl_scales, Wd, Wd_scales, hact, y, ws));
}

// ------------------------------------------------------------------------------ TAM

size_t sfx_tam_ws(int G, int K) { return sfx::tam_ws_bytes(G, K); }

int sfx_tam_update(void* stream, int L, int G, const uint32_t* union_bits, float lambda, float eps, int K,
                   float* score, uint32_t* hot_bits, uint32_t* entered_bits, uint32_t* left_bits,
                   int32_t* topk, int32_t* topk_count, void* ws, size_t ws_bytes) {
  (void)ws;
  (void)ws_bytes;
  if (L < 1 || G < 1 || G > SFX_MAX_GROUPS || K < 0 || K > G) return SFX_E_SHAPE;
  if (!(lambda > 0.0f && lambda < 1.0f) || !(eps >= 0.0f)) return SFX_E_SHAPE;
  if (!union_bits || !score || !hot_bits || !entered_bits || !left_bits || !topk_count) return SFX_E_NULL;
  if (K > 0 && !topk) return SFX_E_NULL;
  return launch_status(sfx::launch_tam((hipStream_t)stream, L, G, union_bits, lambda, eps, K, score, hot_bits,
                                       entered_bits, left_bits, topk, topk_count));
}

int sfx_topk_now_update(void* stream, int L, int G, const uint32_t* union_bits, int K, uint32_t* hot_bits,
                        uint32_t* entered_bits, uint32_t* left_bits, int32_t* topk, int32_t* topk_count) {
  if (L < 1 || G < 1 || G > SFX_MAX_GROUPS || K < 0 || K > G) return SFX_E_SHAPE;
  if (!union_bits || !hot_bits || !entered_bits || !left_bits || !topk_count) return SFX_E_NULL;
  if (K > 0 && !topk) return SFX_E_NULL;
  return launch_status(sfx::launch_topk_now((hipStream_t)stream, L, G, union_bits, K, hot_bits, entered_bits,
                                            left_bits, topk, topk_count));
}

// ------------------------------------------------------------------------------ hot region

int sfx_hot_update(void* stream, int L, int G, int K, const uint32_t* entered_bits, const uint32_t* left_bits,
                   int32_t* slot_of, int32_t* group_of, int32_t* copies, int32_t* ncopies, int nmat,
                   const size_t* group_bytes, const void* const* src, void* const* dst) {
  if (L < 1 || G < 1 || G > SFX_MAX_GROUPS || K < 1 || K > G) return SFX_E_SHAPE;
  if (L > sfx::kHotMaxLayers) return SFX_E_SHAPE;
  if (nmat < 0 || nmat > sfx::kHotMaxMats) return SFX_E_SHAPE;
  if (!entered_bits || !left_bits || !slot_of || !group_of || !copies || !ncopies) return SFX_E_NULL;
  if (!aligned4(entered_bits) || !aligned4(left_bits) || !aligned4(slot_of) || !aligned4(group_of) ||
      !aligned4(copies) || !aligned4(ncopies))
    return SFX_E_ALIGN;
  sfx::HotMats mats{};
  mats.n = nmat;
  if (nmat > 0) {
    if (!group_bytes || !src || !dst) return SFX_E_NULL;
    if (((uintptr_t)src & 7u) || ((uintptr_t)dst & 7u)) return SFX_E_ALIGN;
    int64_t chunks = 0;
    for (int m = 0; m < nmat; ++m) {
      if (group_bytes[m] == 0 || (group_bytes[m] & 15u)) return SFX_E_SHAPE;
      mats.group_bytes[m] = group_bytes[m];
      mats.chunk_off[m] = (int)chunks;
      chunks += (int64_t)((group_bytes[m] + sfx::kHotChunk - 1) / sfx::kHotChunk);
      if (chunks > (int64_t)(1 << 20)) return SFX_E_SHAPE;      // 16 GiB per group
    }
    mats.chunk_off[nmat] = (int)chunks;
  }
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = sfx::launch_hot_assign(st, L, G, K, entered_bits, left_bits, slot_of, group_of, copies, ncopies);
  if (e == hipSuccess && nmat > 0) e = sfx::launch_hot_copy(st, L, K, mats, src, dst, copies, ncopies);
  return launch_status(e);
}

// ------------------------------------------------------------------------------ calibration

int sfx_count_active(void* stream, int B, int f, const uint32_t* tok_bits, int32_t* counts) {
  if (B < 1 || B > SFX_MAX_B || f < 1) return SFX_E_SHAPE;
  if (!tok_bits || !counts) return SFX_E_NULL;
  if (!aligned4(tok_bits) || !aligned4(counts)) return SFX_E_ALIGN;
  return launch_status(sfx::launch_count_active((hipStream_t)stream, B, f, tok_bits, counts));
}

size_t sfx_select_kth_ws(void) { return sfx::select_ws_bytes(); }

int sfx_select_kth(void* stream, size_t n, const float* values, size_t k, float* out, void* ws, size_t ws_bytes) {
  if (n < 1 || n > (size_t)0xFFFFFFFFu || k >= n) return SFX_E_SHAPE;
  if (!values || !out) return SFX_E_NULL;
  if (!aligned4(values) || !aligned4(out)) return SFX_E_ALIGN;
  if (!ws || ((uintptr_t)ws & 255u) || ws_bytes < sfx::select_ws_bytes()) return SFX_E_WORKSPACE;
  return launch_status(sfx::launch_select_kth((hipStream_t)stream, n, values, k, out, ws));
}

size_t sfx_hot_first_order_ws(int f) { return f < 1 ? 0 : sfx::order_ws_bytes(f); }

int sfx_hot_first_order(void* stream, int f, const int32_t* counts, const int32_t* group, int32_t* perm, void* ws,
                        size_t ws_bytes) {
  if (f < 1 || f > (1 << 24)) return SFX_E_SHAPE;
  if (!counts || !perm) return SFX_E_NULL;
  if (!aligned4(counts) || !aligned4(perm) || (group && !aligned4(group))) return SFX_E_ALIGN;
  if (group && (!ws || ((uintptr_t)ws & 255u) || ws_bytes < sfx::order_ws_bytes(f))) return SFX_E_WORKSPACE;
  return launch_status(sfx::launch_hot_first_order((hipStream_t)stream, f, counts, group, perm, ws));
}

int sfx_gather_rows(void* stream, int n_dst, int n_src, size_t row_bytes, const void* src, const int32_t* idx,
                    void* dst) {
  if (n_dst < 1 || n_src < 1 || row_bytes == 0 || (row_bytes & 3u)) return SFX_E_SHAPE;
  if (!src || !idx || !dst) return SFX_E_NULL;
  if (!aligned4(src) || !aligned4(idx) || !aligned4(dst)) return SFX_E_ALIGN;
  return launch_status(sfx::launch_gather_rows((hipStream_t)stream, n_dst, n_src, row_bytes, src, idx, dst));
}

// ------------------------------------------------------------------------------ fused step

size_t sfx_ffn_step_ws(int wdt, int act, int B, int d, int h, int f) {
  const int P = sfx::device_cu_count();
  if (P <= 0) return 0;
  if (!sfx::step_geometry(wdt, act, B, d, h, f, P).ok) return 0;
  if (!sfx::step_resident(wdt, act, B)) return 0;
  return sfx::step_ws_bytes(B, h, f, P);
}

int sfx_ffn_step(void* stream, int wdt, int act, int B, int d, int h, int f, int L, const sfx_layer* layers,
                 void* ws, size_t ws_bytes) {
  if (wdt < SFX_F32 || wdt > SFX_Q4G32) return SFX_E_DTYPE;
  if (act == SFX_RELU2) return SFX_E_UNSUPPORTED;   // squared ReLU: the separate calls
  if (act != SFX_RELU && act != SFX_REGLU) return SFX_E_DTYPE;
  if (B < 1 || B > SFX_MAX_B || d < 1 || h < 1 || f < 1 || L < 1) return SFX_E_SHAPE;
  if (!layers) return SFX_E_NULL;
  if (!ws) return SFX_E_WORKSPACE;
  const int P = sfx::device_cu_count();
  if (P <= 0) return SFX_E_DEVICE;
  const sfx::StepGeom g = sfx::step_geometry(wdt, act, B, d, h, f, P);
  if (!g.ok) return SFX_E_UNSUPPORTED;
  if (!sfx::step_resident(wdt, act, B)) return SFX_E_UNSUPPORTED;
  const int w = check_ws(ws, ws_bytes, sfx::step_ws_bytes(B, h, f, P));
  if (w != SFX_OK) return w;
  return launch_status(sfx::launch_step((hipStream_t)stream, wdt, act, B, d, h, f, L, layers, ws, g));
}

// ------------------------------------------------------------------------------ Live Pipeline

size_t sfx_ffn_pipeline_ws(int wdt, int act, int B, int d, int h, int f) {
  const int P = sfx::device_cu_count();
  if (P <= 0) return 0;
  if (!sfx::pipe_geometry(wdt, act, B, d, h, f, P).ok) return 0;
  if (!sfx::pipe_resident(wdt, act, B)) return 0;
  return sfx::step_ws_bytes(B, h, f, P);
}

int sfx_ffn_pipeline(void* stream, int wdt, int act, int B, int d, int h, int f, int L, const sfx_layer* layers,
                     void* ws, size_t ws_bytes) {
  if (wdt < SFX_F32 || wdt > SFX_Q4G32) return SFX_E_DTYPE;
  if (act == SFX_RELU2) return SFX_E_UNSUPPORTED;   // squared ReLU: the separate calls
  if (act != SFX_RELU && act != SFX_REGLU) return SFX_E_DTYPE;
  if (B < 1 || B > SFX_MAX_B || d < 1 || h < 1 || f < 1 || L < 1) return SFX_E_SHAPE;
  if (!layers) return SFX_E_NULL;
  if (!ws) return SFX_E_WORKSPACE;
  const int P = sfx::device_cu_count();
  if (P <= 0) return SFX_E_DEVICE;
  const sfx::StepGeom g = sfx::pipe_geometry(wdt, act, B, d, h, f, P);
  if (!g.ok) return SFX_E_UNSUPPORTED;
  if (!sfx::pipe_resident(wdt, act, B)) return SFX_E_UNSUPPORTED;
  const int w = check_ws(ws, ws_bytes, sfx::step_ws_bytes(B, h, f, P));
  if (w != SFX_OK) return w;
  return launch_status(sfx::launch_pipe((hipStream_t)stream, wdt, act, B, d, h, f, L, layers, ws, g));
}

// ------------------------------------------------------------------------------ measurement helper

int sfx_stream_read(void* stream, const void* buf, size_t nbytes, uint32_t* out) {
  if (nbytes < 16 || nbytes % 16 != 0) return SFX_E_SHAPE;
  if (!buf || !out) return SFX_E_NULL;
  if (!aligned16(buf) || !aligned4(out)) return SFX_E_ALIGN;
  return launch_status(sfx::launch_stream_read((hipStream_t)stream, buf, nbytes, out));
}

}  // extern "C"
