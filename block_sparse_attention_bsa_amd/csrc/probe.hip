// Measurement helpers, not part of the attention path: the ceilings the kernels' rates are
// compared with, measured on the GPU they run on.
//
//   mfma_peak_kernel  back-to-back v_mfma_f32_32x32x16_bf16 (the forward's instruction), or
//                     v_mfma_f32_16x16x32_bf16, on register operands, independent accumulators,
//                     two wavefronts per SIMD: the sustained dense bf16 matrix rate.
//   mix_kernel        the forward's mix at its occupancy (three wavefronts per SIMD): per round
//                     16 independent v_mfma_f32_16x16x32_bf16 and/or 32 independent v_exp_f32
//                     or v_fma_f32, so that the time of a mix against its parts shows how much
//                     of the vector work the matrix pipe hides.
//   copy_kernel       a grid-stride 16-byte copy: the sustained HBM read + write rate.
#include "bsa_internal.h"
#include "device_common.h"

namespace {

template <int SHAPE>
__global__ __launch_bounds__(256, 2) void mfma_peak_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(lane + i));
    b[i] = (__bf16)(0.002f * (float)(lane - i));
  }
  float s = 0.f;
  if constexpr (SHAPE == 0) {  // 32x32x16: eight independent 16-register accumulators
    f32x16_t acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[k][e] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int k = 0; k < 8; ++k)
        acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += acc[k][e];
  } else {  // 16x16x32: sixteen independent 4-register accumulators, the same FLOPs per round
    f32x4_t acc[16];
#pragma unroll
    for (int k = 0; k < 16; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[k][e] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int k = 0; k < 16; ++k)
        acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[k], 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < 16; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) s += acc[k][e];
  }
  if (s == 12345.678f) sink[blockIdx.x * 256 + threadIdx.x] = s;  // keeps the work alive
}

// NM MFMAs, then NE exponentials (0 or 32), then NF FMAs (0 or 32) per round, each on its own
// register chain, so that nothing waits for anything within a round.
template <int NM, int NE, int NF>
__global__ __launch_bounds__(256, 3) void mix_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(lane + i));
    b[i] = (__bf16)(0.002f * (float)(lane - i));
  }
  f32x4_t acc[16];
  float x[32], y[32];
#pragma unroll
  for (int k = 0; k < 16; ++k)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[k][e] = 0.f;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    x[j] = 0.01f * (float)(lane + j);
    y[j] = 0.02f * (float)(lane + j);
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < NM; ++k)
      acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[k], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < NE; ++j) x[j] = __builtin_amdgcn_exp2f(-x[j]);
#pragma unroll
    for (int j = 0; j < NF; ++j) y[j] = fmaf(y[j], 0.999f, 0.0001f);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k)
#pragma unroll
    for (int e = 0; e < 4; ++e) s += acc[k][e];
#pragma unroll
  for (int j = 0; j < 32; ++j) s += x[j] + y[j];
  if (s == 12345.678f) sink[blockIdx.x * 256 + threadIdx.x] = s;  // keeps the work alive
}

__global__ __launch_bounds__(256) void copy_kernel(const uint4* __restrict__ src,
                                                   uint4* __restrict__ dst, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    dst[i] = src[i];
}

}  // namespace

extern "C" {

int bsa_probe_mfma(int32_t shape, int32_t workgroups, int32_t iters, float* sink, double* flops,
                   void* stream) {
  if (shape < 0 || shape > 6 || workgroups < 1 || iters < 1 || !sink) return BSA_EINVAL;
  const hipStream_t s = (hipStream_t)stream;
  switch (shape) {
    case 0: mfma_peak_kernel<0><<<workgroups, 256, 0, s>>>(iters, sink); break;
    case 1: mfma_peak_kernel<1><<<workgroups, 256, 0, s>>>(iters, sink); break;
    case 2: mix_kernel<16, 0, 0><<<workgroups, 256, 0, s>>>(iters, sink); break;
    case 3: mix_kernel<16, 32, 0><<<workgroups, 256, 0, s>>>(iters, sink); break;
    case 4: mix_kernel<0, 32, 0><<<workgroups, 256, 0, s>>>(iters, sink); break;
    case 5: mix_kernel<16, 0, 32><<<workgroups, 256, 0, s>>>(iters, sink); break;
    default: mix_kernel<0, 0, 32><<<workgroups, 256, 0, s>>>(iters, sink); break;
  }
  // per wavefront and round: 8 x 32x32x16 or 16 x 16x16x32, 2 * 32 * 32 * 16 * 8 FLOPs either way
  // (shapes 4 and 6 issue no MFMA)
  if (flops)
    *flops = (shape == 4 || shape == 6)
                 ? 0.0
                 : (double)workgroups * 4 * iters * 8 * (2.0 * 32 * 32 * 16);
  return hipGetLastError() == hipSuccess ? BSA_OK : BSA_EHIP;
}

int bsa_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst || bytes % 16) return BSA_EINVAL;
  const int64_t n = (int64_t)(bytes / 16);
  copy_kernel<<<8192, 256, 0, (hipStream_t)stream>>>(static_cast<const uint4*>(src),
                                                     static_cast<uint4*>(dst), n);
  return hipGetLastError() == hipSuccess ? BSA_OK : BSA_EHIP;
}

}  // extern "C"
