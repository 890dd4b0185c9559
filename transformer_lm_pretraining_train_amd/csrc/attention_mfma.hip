// Matrix-core (MFMA) flash attention for bf16, head size 64.
#include "common.h"
#include "kernels.h"

namespace gk {

bool attention_mfma_supported(int dt, int hd) { return false; }

hipError_t attention_forward_mfma(void*, float*, const void*, int, int, int, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t attention_backward_mfma(void*, const void*, const void*, const void*, const float*,
                                   float*, int, int, int, hipStream_t) {
  return hipErrorInvalidValue;
}

}  // namespace gk
