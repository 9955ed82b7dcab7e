// Host stand-ins for a CPU-only build of the library's host code (plan construction, partition
// building, argument validation, workspace layouts) under AddressSanitizer: the HIP runtime calls
// it makes are backed by malloc/memcpy, and every kernel launcher only counts its call. Nothing
// here computes any part of the method.
#include <hip/hip_runtime_api.h>

#include <cstdlib>
#include <cstring>

#include "../../block_sparse_attention_bsa_amd/csrc/bsa_internal.h"

int g_launches = 0;

extern "C" {
hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}
hipError_t hipMalloc(void** ptr, size_t size) {
  *ptr = std::malloc(size ? size : 1);
  return *ptr ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipFree(void* ptr) {
  std::free(ptr);
  return hipSuccess;
}
hipError_t hipMemcpy(void* dst, const void* src, size_t n, hipMemcpyKind) {
  std::memcpy(dst, src, n);
  return hipSuccess;
}
const char* hipGetErrorString(hipError_t) { return "stub"; }
}

#define COUNT \
  {               \
    ++g_launches; \
    return hipSuccess; \
  }
hipError_t launch_pool(const bsa_plan&, int, const void*, float*, hipStream_t) COUNT;
hipError_t launch_pool_qk(const bsa_plan&, const void*, float*, const void*, float*,
                          hipStream_t) COUNT;
hipError_t launch_score(const bsa_plan&, const float*, const float*, int, float*,
                        hipStream_t) COUNT;
hipError_t launch_select(const bsa_plan&, const float*, const bsa_select_params&, int32_t*,
                         int32_t*, int32_t*, int32_t*, void*, hipStream_t) COUNT;
hipError_t launch_select_eg(const bsa_plan&, const float*, const bsa_eg_params&, int32_t*,
                            int32_t*, int32_t*, float*, int32_t*, void*, hipStream_t) COUNT;
hipError_t launch_attn_fwd(const bsa_plan&, const void*, const void*, const void*,
                           const int32_t*, const int32_t*, void*, float*, void*,
                           hipStream_t) COUNT;
hipError_t launch_attn_fwd_tokens(const bsa_plan&, const void*, const void*, const void*,
                                  const int32_t*, const int32_t*, const int32_t*, int, void*,
                                  float*, void*, hipStream_t) COUNT;
hipError_t launch_select_tokens(const bsa_plan&, const void*, const float*, int, int32_t*,
                                int32_t*, int32_t*, void*, hipStream_t) COUNT;
hipError_t launch_calibrate(const bsa_plan&, const void*, const void*, const void*, float*,
                            void*, float*, void*, hipStream_t) COUNT;
hipError_t launch_attn_bwd(const bsa_plan&, const void*, const void*, const void*, const void*,
                           const void*, const float*, const int32_t*, const int32_t*, void*,
                           void*, void*, void*, hipStream_t) COUNT;

// The allocation-free selection's device scratch: a host buffer of the same size here.
static unsigned char g_scratch[kSelectScratchBytes];
hipError_t select_scratch(void** ptr) {
  *ptr = g_scratch;
  return hipSuccess;
}
hipError_t launch_score_select_csr(const bsa_plan&, const float*, const float*,
                                   const bsa_select_params&, float*, int32_t*, int32_t*, int32_t*,
                                   int32_t*, void*, hipStream_t) COUNT;
hipError_t launch_select_tokens_global(const bsa_plan&, const void*, const float*, double,
                                       uint32_t*, int32_t*, int32_t*, void*, hipStream_t) COUNT;
hipError_t launch_attn_fwd_token_bits(const bsa_plan&, const void*, const void*, const void*,
                                      const int32_t*, const int32_t*, const uint32_t*, void*,
                                      float*, void*, hipStream_t) COUNT;
