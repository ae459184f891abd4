// Fused multi-layer step kernel, fp16 instantiations (see k_step.hpp).
#include "k_step.hpp"

namespace sfx {
hipError_t launch_step_f16(hipStream_t s, const StepParams& p, int act, int P, int DL) {
  (void)DL;
  return step::dispatch_step<TF16>(s, p, act, P);
}
int step_blocks_per_cu_f16(int act, int B) { return step::step_blocks_per_cu<TF16>(act, B); }
}  // namespace sfx
