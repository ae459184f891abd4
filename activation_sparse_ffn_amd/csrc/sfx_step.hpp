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
  uint32_t* err;               // nonzero after a wait timed out
  uint32_t* go;
  uint32_t* flags;             // one arrival counter per workgroup
  unsigned long long* hid;     // [B][h]  {tag, hidden}
  unsigned long long* uni;     // [W]     {tag, union word}
  unsigned long long* hact;    // [f][B]  {tag, activation}
};

struct StepGeom {
  bool ok;
  int P, nr1, w2_lds, cw, dl;
};

StepGeom step_geometry(int wdt, int act, int B, int d, int h, int f, int P);
size_t step_ws_bytes(int B, int h, int f, int P);
hipError_t launch_step(hipStream_t s, int wdt, int act, int B, int d, int h, int f, int L,
                       const LayerDesc* layers, void* ws, const StepGeom& g);

}  // namespace sfx
