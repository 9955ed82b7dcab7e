// Sparse attention backward: placeholder until the dK/dV and dQ kernels land.
#include "bsa_internal.h"

hipError_t launch_attn_bwd(const bsa_plan&, const void*, const void*, const void*, const void*,
                           const void*, const float*, const int32_t*, const int32_t*, void*,
                           void*, void*, void*, hipStream_t) {
  return hipErrorNotSupported;
}
