// Live Pipeline fused step kernel, fp16 instantiations (see k_pipe.hpp).
#include "k_pipe.hpp"

namespace sfx {
hipError_t launch_pipe_f16(hipStream_t s, const StepParams& p, int act, int P) {
  return step::dispatch_pipe<TF16>(s, p, act, P);
}
int pipe_blocks_per_cu_f16(int act, int B) { return step::pipe_blocks_per_cu<TF16>(act, B); }
}  // namespace sfx
