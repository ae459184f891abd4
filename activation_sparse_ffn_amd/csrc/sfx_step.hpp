// Parameters of the fused multi-layer step kernel (k_step.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/sfx.h"

namespace sfx {

typedef sfx_layer LayerDesc;

struct StepParams {
  const LayerDesc* layers;
  int L, B, d, h, f, W;
  int nr1;        // hidden rows per workgroup (ceil(h / P))
  int w2_lds;     // 1: the workgroup's W2 rows are staged in LDS
  int cw;         // columns of y per workgroup in the down phase (8, 16, 32 or 64)
  int us;         // tagged union words per workgroup block (multiple of 8)
  int dsplit;     // fused step, down phase: workgroups per 64-column tile (<= 8)
  int dtiles;     // fused step, down phase: 64-column tiles, ceil(d / 64)
  uint32_t* err;               // nonzero after a wait timed out
  uint32_t* fbar;              // [P] x kFlagStride: layer done (grid barrier); holds layer tags
  unsigned long long* hid;     // [P][16]  {tag, hidden}: rows w + P s, s < nr1, all tokens
  unsigned long long* uni;     // P us words {tag, union word}: word-major: word m of workgroup o at m P + o
  unsigned long long* hact;    // [f][B]   {tag, activation} by active rank
  unsigned long long* ypart;   // [2][P][64 NB] {tag, share of y}: fused step's tile shares
};

struct StepGeom {
  bool ok;
  int P, nr1, w2_lds, cw, dl, dsplit, dtiles;
};

StepGeom step_geometry(int wdt, int act, int B, int d, int h, int f, int P);
#ifndef SFX_FLAG_STRIDE
#define SFX_FLAG_STRIDE 16
#endif
constexpr int kFlagStride = SFX_FLAG_STRIDE;   // words between two workgroups' flags
size_t step_ws_bytes(int B, int h, int f, int P);
StepParams step_params(int B, int d, int h, int f, int L, const LayerDesc* layers, void* ws, const StepGeom& g);
bool step_resident(int wdt, int act, int B);
StepGeom pipe_geometry(int wdt, int act, int B, int d, int h, int f, int P);
bool pipe_resident(int wdt, int act, int B);
hipError_t launch_pipe(hipStream_t s, int wdt, int act, int B, int d, int h, int f, int L,
                       const LayerDesc* layers, void* ws, const StepGeom& g);
hipError_t launch_step(hipStream_t s, int wdt, int act, int B, int d, int h, int f, int L,
                       const LayerDesc* layers, void* ws, const StepGeom& g);

}  // namespace sfx
