// Internal launchers, one per kernel family.  Arguments are already validated by
// the C ABI layer; each launcher only picks an instantiation and enqueues it.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/sfx.h"

namespace sfx {

int device_cu_count();  // cached per device; 0 if no device

size_t predict_ws_bytes(int wdt, int B, int d, int h, int f);
hipError_t launch_predict(hipStream_t s, int wdt, int B, int d, int h, int f, const void* x,
                          const void* W1, const void* W2, float* scores, void* ws);

hipError_t launch_predict_q4(hipStream_t s, int B, int d, int h, int f, const void* x, const void* W1,
                             const void* W1_s, const void* W2, const void* W2_s, float* scores, void* ws);

size_t compact_ws_bytes(int B, int f);
hipError_t launch_compact(hipStream_t s, int B, int f, const float* scores, float t,
                          uint32_t* tok_bits, uint32_t* union_bits, int32_t* idx, int kmax,
                          int32_t* count, void* ws);

hipError_t launch_up(hipStream_t s, int wdt, int act, int B, int d, int f, const void* x,
                     const void* Wa, const void* Wa_s, const float* ba, const void* Wl,
                     const void* Wl_s, const int32_t* idx, const int32_t* count, int kmax,
                     float* hact);
bool up_supported(int wdt, int act, int B);

size_t down_ws_bytes(int wdt, int B, int d, int kmax);
hipError_t launch_down(hipStream_t s, int wdt, int B, int d, int f, const void* Wd,
                       const void* Wd_s, const int32_t* idx, const int32_t* count, int kmax,
                       const float* hact, float* y, void* ws);
bool down_supported(int wdt, int B);
size_t dense_ws_bytes(int wdt, int B, int d, int f);
hipError_t launch_dense(hipStream_t s, int wdt, int act, int B, int d, int f, const void* x, const void* Wa,
                        const void* Wa_s, const float* ba, const void* Wl, const void* Wl_s, const void* Wd,
                        const void* Wd_s, float* hact, float* y, void* ws);
// Static scratch of the down kernel for callers that cannot allocate: its size, and
// its device address on the current device (looked up on the first call per device).
constexpr size_t kDownScratchBytes = SFX_DOWN_SCRATCH_BYTES;
hipError_t down_scratch(void** ptr);

size_t stream_read_out_words();
hipError_t launch_stream_read(hipStream_t s, const void* buf, size_t nbytes, uint32_t* out);

size_t tam_ws_bytes(int G, int K);
hipError_t launch_tam(hipStream_t s, int L, int G, const uint32_t* union_bits, float lambda,
                      float eps, int K, float* score, uint32_t* hot_bits, uint32_t* entered,
                      uint32_t* left, int32_t* topk, int32_t* topk_count);
hipError_t launch_topk_now(hipStream_t s, int L, int G, const uint32_t* union_bits, int K, uint32_t* hot_bits,
                           uint32_t* entered, uint32_t* left, int32_t* topk, int32_t* topk_count);

hipError_t launch_count_active(hipStream_t s, int B, int f, const uint32_t* tok_bits, int32_t* counts);
size_t select_ws_bytes();
hipError_t launch_select_kth(hipStream_t s, size_t n, const float* v, size_t k, float* out, void* ws);
size_t order_ws_bytes(int f);
hipError_t launch_hot_first_order(hipStream_t s, int f, const int32_t* counts, const int32_t* group, int32_t* perm,
                                  void* ws);
hipError_t launch_gather_rows(hipStream_t s, int n_dst, int n_src, size_t row_bytes, const void* src,
                              const int32_t* idx, void* dst);

constexpr int kHotMaxMats = 8;
constexpr int kHotMaxLayers = 1024;
constexpr int kHotChunk = 16384;         // bytes per work item of the copy kernel
struct HotMats {
  int n;                                 // matrices per layer, 0..kHotMaxMats
  size_t group_bytes[kHotMaxMats];       // bytes of one group's rows in matrix m
  int chunk_off[kHotMaxMats + 1];        // first chunk of matrix m; chunk_off[n] = chunks per group
};
hipError_t launch_hot_assign(hipStream_t s, int L, int G, int K, const uint32_t* entered, const uint32_t* left,
                             int32_t* slot_of, int32_t* group_of, int32_t* copies, int32_t* ncopies);
hipError_t launch_hot_copy(hipStream_t s, int L, int K, const HotMats& mats, const void* const* src,
                           void* const* dst, const int32_t* copies, const int32_t* ncopies);

}  // namespace sfx
