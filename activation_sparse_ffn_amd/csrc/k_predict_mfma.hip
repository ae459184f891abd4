// Predictor layer 2 on the matrix cores for B >= 16 (filled in with the MFMA path).
#include "sfx_common.hpp"
#include "sfx_launch.hpp"

namespace sfx {

bool pred_mfma_eligible(int wdt, int B, int h, int f) {
  (void)wdt; (void)B; (void)h; (void)f;
  return false;
}

hipError_t launch_pred_scores_mfma(hipStream_t s, int wdt, int B, int h, int f, const void* W2,
                                   const float* hid, float* scores) {
  (void)s; (void)wdt; (void)B; (void)h; (void)f; (void)W2; (void)hid; (void)scores;
  return hipErrorInvalidValue;
}

}  // namespace sfx
