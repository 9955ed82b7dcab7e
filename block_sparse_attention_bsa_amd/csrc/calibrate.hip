// Exact block masses (LoSA abstract): placeholder until the dense two-pass kernels land.
#include "bsa_internal.h"

hipError_t launch_calibrate(const bsa_plan&, const void*, const void*, float*, void*,
                            hipStream_t) {
  return hipErrorNotSupported;
}
