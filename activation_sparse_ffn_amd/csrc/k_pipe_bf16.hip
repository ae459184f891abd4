// Live Pipeline fused step kernel, bf16 instantiations (see k_pipe.hpp).
#include "k_pipe.hpp"

namespace sfx {
hipError_t launch_pipe_bf16(hipStream_t s, const StepParams& p, int act, int P) {
  return step::dispatch_pipe<TBF16>(s, p, act, P);
}
int pipe_blocks_per_cu_bf16(int act, int B) { return step::pipe_blocks_per_cu<TBF16>(act, B); }
}  // namespace sfx
