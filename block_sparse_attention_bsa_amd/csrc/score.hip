// Query-block x key-block similarity of block means (pith.science review of VMoBA, "What
// carries the argument": queries score the block means; referee report major comment 1:
// Eq. 3 ranks entries of the whole query-by-block matrix of a head).
//
//   logits_kernel   L[bh, I, J] = sigma_h * <Qbar_I, Kbar_J> in fp32 on the matrix cores
//                   (v_mfma_f32_32x32x2_f32), one wavefront per 32 x 32 tile, four per
//                   workgroup sharing their operand rows through LDS.
//   row_softmax     one wavefront per row: S = exp(L - max) / sum, fp32, fixed reduction order.
//   head_softmax    one 1024-thread workgroup per head: W = |I| exp(L - M) / Z with the head max
//                   M and Z = sum |I| exp(L - M) accumulated in fp64 (fixed order).
#include "bsa_internal.h"
#include "device_common.h"

namespace {

constexpr int kWI = 64, kWJ = 64;  // one workgroup: a 64 x 64 region of L, four 32 x 32 tiles

// A workgroup stages the region's 64 rows of Qbar and of Kbar in LDS with coalesced 16-byte
// loads (rows padded by 16 bytes, so that the 16 lanes of a read start in different banks), and
// wavefront w forms tile (w / 2, w % 2) of the region. In each k-step of the MFMA the two 32-lane
// halves supply the two k-indices; half h takes d = (D/2) h + s at step s, reading one
// contiguous half row of Qbar (A operand, row I0 + lane % 32) and of Kbar (B operand, column
// J0 + lane % 32). The products and sums are fp32; the summation order over d is the matrix
// core's.
template <int D>
__global__ __launch_bounds__(256) void logits_kernel(const float* __restrict__ Qbar,
                                                     const float* __restrict__ Kbar,
                                                     const float* __restrict__ scale, int H,
                                                     int nq, int nkv, float* __restrict__ S) {
  constexpr int kHalf = D / 2, kVec = kHalf / 4, R = D + 4;
  __shared__ __attribute__((aligned(16))) float qs[kWI * R];
  __shared__ __attribute__((aligned(16))) float ks[kWJ * R];
  const int bh = blockIdx.z;
  const int IW = blockIdx.y * kWI, JW = blockIdx.x * kWJ;
  const int t = threadIdx.x;
  // rows past the matrix edge load the last row (in bounds); their results are not stored
  constexpr int kUnits = D / 4;  // 16-byte units per row
  for (int u = t; u < kWI * kUnits; u += 256) {
    const int row = u / kUnits, c = u % kUnits;
    const float4 qv = reinterpret_cast<const float4*>(
        Qbar + ((size_t)bh * nq + min(IW + row, nq - 1)) * D)[c];
    const float4 kv = reinterpret_cast<const float4*>(
        Kbar + ((size_t)bh * nkv + min(JW + row, nkv - 1)) * D)[c];
    *reinterpret_cast<float4*>(&qs[row * R + 4 * c]) = qv;
    *reinterpret_cast<float4*>(&ks[row * R + 4 * c]) = kv;
  }
  __syncthreads();
  const int lane = t & 63, wave = t >> 6, l32 = lane & 31, h = lane >> 5;
  const int ti = 32 * (wave >> 1), tj = 32 * (wave & 1);
  const float4* qp = reinterpret_cast<const float4*>(&qs[(ti + l32) * R + kHalf * h]);
  const float4* kp = reinterpret_cast<const float4*>(&ks[(tj + l32) * R + kHalf * h]);
  f32x16_t acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
  for (int i = 0; i < kVec; ++i) {
    const float4 qa = qp[i], kb = kp[i];
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qa.x, kb.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qa.y, kb.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qa.z, kb.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qa.w, kb.w, acc, 0, 0, 0);
  }
  // lane holds column J0 + lane % 32 and rows I0 + 8 (e / 4) + 4 h + e % 4
  const float sig = scale[bh % H];
  const int I0 = IW + ti, J = JW + tj + l32;
  if (J >= nkv) return;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int I = I0 + 8 * (e >> 2) + 4 * h + (e & 3);
    if (I < nq) S[((size_t)bh * nq + I) * nkv + J] = sig * acc[e];
  }
}

// 4 rows per 256-thread workgroup, one wavefront each.
__global__ __launch_bounds__(256) void row_softmax_kernel(float* __restrict__ S, int64_t rows,
                                                          int nkv) {
  const int64_t r = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;
  if (r >= rows) return;
  const int lane = threadIdx.x & 63;
  float* row = S + r * nkv;
  float m = -INFINITY;
  for (int j = lane; j < nkv; j += 64) m = fmaxf(m, row[j]);
  m = wave_max_f32(m);
  float s = 0.f;
  for (int j = lane; j < nkv; j += 64) s += expf(row[j] - m);
  s = wave_sum_f32(s);
  const float inv = 1.f / s;
  for (int j = lane; j < nkv; j += 64) row[j] = expf(row[j] - m) * inv;
}

__global__ __launch_bounds__(1024) void head_softmax_kernel(float* __restrict__ S,
                                                            const int32_t* __restrict__ qstart,
                                                            int nq, int nkv) {
  __shared__ float smax[16];
  __shared__ double ssum[16];
  const int bh = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t n = (int64_t)nq * nkv;
  float* W = S + (size_t)bh * n;
  float m = -INFINITY;
  for (int64_t j = t; j < n; j += 1024) m = fmaxf(m, W[j]);
  m = wave_max_f32(m);
  if (lane == 0) smax[wave] = m;
  __syncthreads();
  m = smax[0];
  for (int w = 1; w < 16; ++w) m = fmaxf(m, smax[w]);
  const double M = (double)m;
  double z = 0.0;
  for (int64_t j = t; j < n; j += 1024) {
    const int I = (int)(j / nkv);
    z += (double)(qstart[I + 1] - qstart[I]) * exp((double)W[j] - M);
  }
  z = wave_sum_f64(z);
  if (lane == 0) ssum[wave] = z;
  __syncthreads();
  double Z = 0.0;
  for (int w = 0; w < 16; ++w) Z += ssum[w];
  const double invZ = 1.0 / Z;
  __syncthreads();
  for (int64_t j = t; j < n; j += 1024) {
    const int I = (int)(j / nkv);
    W[j] = (float)((double)(qstart[I + 1] - qstart[I]) * exp((double)W[j] - M) * invZ);
  }
}

}  // namespace

hipError_t launch_score(const bsa_plan& p, const float* Qbar, const float* Kbar, int norm,
                        float* S, hipStream_t s) {
  const int BH = p.prob.B * p.prob.H;
  dim3 grid((p.nkv + kWJ - 1) / kWJ, (p.nq + kWI - 1) / kWI, BH);
  if (p.prob.d == 128)
    logits_kernel<128><<<grid, 256, 0, s>>>(Qbar, Kbar, p.scale, p.prob.H, p.nq, p.nkv, S);
  else
    logits_kernel<64><<<grid, 256, 0, s>>>(Qbar, Kbar, p.scale, p.prob.H, p.nq, p.nkv, S);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (norm == BSA_NORM_ROW) {
    const int64_t rows = (int64_t)BH * p.nq;
    row_softmax_kernel<<<(unsigned)((rows + 3) / 4), 256, 0, s>>>(S, rows, p.nkv);
  } else {
    head_softmax_kernel<<<BH, 1024, 0, s>>>(S, p.qstart, p.nq, p.nkv);
  }
  return hipGetLastError();
}
