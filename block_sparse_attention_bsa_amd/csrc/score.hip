// Query-block x key-block similarity of block means (pith.science review of VMoBA, "What
// carries the argument": queries score the block means; referee report major comment 1:
// Eq. 3 ranks entries of the whole query-by-block matrix of a head).
//
//   logits_kernel   L[bh, I, J] = sigma_h * <Qbar_I, Kbar_J> in fp32, 32 x 64 output tiles,
//                   each thread a 2 x 4 micro-tile, operands staged in padded LDS.
//   row_softmax     one wavefront per row: S = exp(L - max) / sum, fp32, fixed reduction order.
//   head_softmax    one 1024-thread workgroup per head: W = |I| exp(L - M) / Z with the head max
//                   M and Z = sum |I| exp(L - M) accumulated in fp64 (fixed order).
#include "bsa_internal.h"
#include "device_common.h"

namespace {

constexpr int kTI = 32, kTJ = 64;

template <int D>
__global__ __launch_bounds__(256) void logits_kernel(const float* __restrict__ Qbar,
                                                     const float* __restrict__ Kbar,
                                                     const float* __restrict__ scale, int H,
                                                     int nq, int nkv, float* __restrict__ S) {
  __shared__ float qs[kTI][D + 1];
  __shared__ float ks[kTJ][D + 1];
  const int bh = blockIdx.z;
  const int I0 = blockIdx.y * kTI, J0 = blockIdx.x * kTJ;
  const int t = threadIdx.x;
  const float* Qh = Qbar + (size_t)bh * nq * D;
  const float* Kh = Kbar + (size_t)bh * nkv * D;
  for (int e = t; e < kTI * D; e += 256) {
    const int r = e / D, c = e % D;
    qs[r][c] = (I0 + r < nq) ? Qh[(size_t)(I0 + r) * D + c] : 0.f;
  }
  for (int e = t; e < kTJ * D; e += 256) {
    const int r = e / D, c = e % D;
    ks[r][c] = (J0 + r < nkv) ? Kh[(size_t)(J0 + r) * D + c] : 0.f;
  }
  __syncthreads();
  const int ty = t / 16, tx = t % 16;
  float acc[2][4] = {};
#pragma unroll 8
  for (int k = 0; k < D; ++k) {
    const float a0 = qs[2 * ty][k], a1 = qs[2 * ty + 1][k];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float b = ks[tx + 16 * c][k];
      acc[0][c] = fmaf(a0, b, acc[0][c]);
      acc[1][c] = fmaf(a1, b, acc[1][c]);
    }
  }
  const float sig = scale[bh % H];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int I = I0 + 2 * ty + r;
    if (I >= nq) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int J = J0 + tx + 16 * c;
      if (J < nkv) S[((size_t)bh * nq + I) * nkv + J] = sig * acc[r][c];
    }
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
  dim3 grid((p.nkv + kTJ - 1) / kTJ, (p.nq + kTI - 1) / kTI, BH);
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
