// Query-block x key-block similarity of block means (pith.science review of VMoBA, "What
// carries the argument": queries score the block means; referee report major comment 1:
// Eq. 3 ranks entries of the whole query-by-block matrix of a head).
//
//   score_rows      (rows of at most 2048 blocks) a workgroup owns 16 query blocks of a head and
//                   all their kv blocks: L = sigma_h * <Qbar_I, Kbar_J> in fp32 on the matrix
//                   cores (v_mfma_f32_16x16x4_f32, one 16 x 16 tile per wavefront and step),
//                   passed through LDS so that each wavefront then holds four whole rows in
//                   registers; it writes L (the head pool normalises afterwards), or the row
//                   softmax S, or selects from S in the same kernel (the fused score-and-select
//                   of bsa_score_select: S never has to go through memory).
//   logits_kernel   (longer rows) the same L, one wavefront per 32 x 32 tile
//                   (v_mfma_f32_32x32x2_f32), four per workgroup sharing operand rows in LDS.
//   row_softmax     (longer rows) one wavefront per row: S = exp(L - max) / sum, fp32, the same
//                   reduction order as score_rows.
//   head_softmax    one 1024-thread workgroup per head: W = |I| exp(L - M) / Z with the head max
//                   M and Z = sum |I| exp(L - M) accumulated in fp64 (fixed order).
#include <algorithm>

#include "bsa_internal.h"
#include "device_common.h"
#include "row_select.h"

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

// score_rows: 16 query blocks x every kv block per workgroup of four wavefronts.
constexpr int kRowsWg = 16;
enum ScoreMode { kLogitsOut = 0, kSoftmaxOut = 1, kSelectRows = 2 };

// Row softmax of one score row held by a wavefront (value i of the lane is column lane + 64 i):
// S = exp(L - max) / sum, with the max, the lane's sum in ascending i and the butterfly sum of
// row_softmax_kernel, so both give the same bits.
template <int kVpl>
__device__ __forceinline__ void row_softmax_regs(float (&x)[kVpl], int n) {
  const int lane = threadIdx.x & 63;
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kVpl; ++i)
    if (lane + 64 * i < n) m = fmaxf(m, x[i]);
  m = wave_max_f32(m);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kVpl; ++i)
    if (lane + 64 * i < n) s += expf(x[i] - m);
  s = wave_sum_f32(s);
  const float inv = 1.f / s;
#pragma unroll
  for (int i = 0; i < kVpl; ++i) x[i] = expf(x[i] - m) * inv;
}

// The logits of 16 query blocks (I0 ..) against every kv block of head bh, kept whole in LDS
// (16 x 64 kVpl floats). Wavefront w forms the 64-column groups w, w + 4, ..., each as four
// 16 x 16 tiles with independent accumulators (v_mfma_f32_16x16x4_f32, so consecutive MFMAs do
// not wait on each other): lane (i = lane % 16, g = lane / 16) supplies Qbar[I0 + i][(D/4) g + m]
// and Kbar[J + i][(D/4) g + m] at step m, the four lane groups being the k dimension and each
// lane reading one contiguous quarter row of each operand. After one barrier wavefront w takes
// rows I0 + 4 w .. + 4, value i of a lane being column lane + 64 i. MODE: kLogitsOut writes L;
// kSoftmaxOut writes the row softmax S; kSelectRows selects each row (top-p with the exact sums
// of row_select.h) into the bitmap and counts, and writes S too when S is given (the per-head
// minimum count needs it afterwards).
template <int D, int kVpl, int MODE>
__global__ __launch_bounds__(256) void score_rows_kernel(
    const float* __restrict__ Qbar, const float* __restrict__ Kbar,
    const float* __restrict__ scale, int H, int nq, int nkv, float* __restrict__ S,
    unsigned long long target, bool select_all, int nwords, uint32_t* __restrict__ bitmap,
    int32_t* __restrict__ base_counts) {
  constexpr int kQ = D / 4;  // floats of a row each lane group covers
  // The 16 score rows (row stride 64 * ngroups + 4 floats), sized at launch; once every
  // wavefront holds its rows in registers the same LDS holds the selection histograms.
  extern __shared__ float sb[];
  WaveHist* hist = reinterpret_cast<WaveHist*>(sb);
  const int ngroups = (nkv + 63) / 64, kStride = 64 * ngroups + 4;
  const int bh = blockIdx.y, I0 = blockIdx.x * kRowsWg;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, li = lane & 15, g = lane >> 4;
  const float sig = scale[bh % H];
  float qa[kQ];
  {
    const float4* qp = reinterpret_cast<const float4*>(
        Qbar + ((size_t)bh * nq + min(I0 + li, nq - 1)) * D + kQ * g);
#pragma unroll
    for (int c = 0; c < kQ / 4; ++c) {
      const float4 v = qp[c];
      qa[4 * c] = v.x;
      qa[4 * c + 1] = v.y;
      qa[4 * c + 2] = v.z;
      qa[4 * c + 3] = v.w;
    }
  }
  const float* kb_head = Kbar + (size_t)bh * nkv * D;
  for (int grp = w; grp < ngroups; grp += 4) {
    const float4* kp[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
      kp[tt] = reinterpret_cast<const float4*>(
          kb_head + (size_t)min(64 * grp + 16 * tt + li, nkv - 1) * D + kQ * g);
    f32x4_t acc[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) acc[tt] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kQ / 4; ++c) {
      float4 kv[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) kv[tt] = kp[tt][c];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[4 * c], kv[tt].x, acc[tt], 0, 0, 0);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[4 * c + 1], kv[tt].y, acc[tt], 0, 0, 0);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[4 * c + 2], kv[tt].z, acc[tt], 0, 0, 0);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[4 * c + 3], kv[tt].w, acc[tt], 0, 0, 0);
    }
    // tile tt: lane holds L[I0 + 4 g + e][64 grp + 16 tt + li]
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sb[(4 * g + e) * kStride + 64 * grp + 16 * tt + li] = sig * acc[tt][e];
  }
  __syncthreads();
  float x[4][kVpl];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int i = 0; i < kVpl; ++i)
      x[r][i] = lane + 64 * i < 64 * ngroups ? sb[(4 * w + r) * kStride + lane + 64 * i] : 0.f;
  if constexpr (MODE == kSelectRows) __syncthreads();  // the rows are read: LDS holds histograms
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int I = I0 + 4 * w + r;
    if (I >= nq) break;  // wave-uniform
    float* srow = S ? S + ((size_t)bh * nq + I) * nkv : nullptr;
    if constexpr (MODE != kLogitsOut) row_softmax_regs(x[r], nkv);
    if (MODE != kSelectRows || srow) {
#pragma unroll
      for (int i = 0; i < kVpl; ++i)
        if (lane + 64 * i < nkv) srow[lane + 64 * i] = x[r][i];
    }
    if constexpr (MODE == kSelectRows) {
      const int64_t row = (int64_t)bh * nq + I;
      bool sel[kVpl];
      const uint32_t count = wave_select(x[r], nkv, target, false, select_all, hist[w], sel);
      write_row_bits(sel, nwords, bitmap + row * nwords);
      if (lane == 0) base_counts[row] = (int32_t)count;
    }
  }
}

template <int D, int MODE>
hipError_t launch_score_rows(const bsa_plan& p, const float* Qbar, const float* Kbar, float* S,
                             unsigned long long target, bool all, int nwords, uint32_t* bitmap,
                             int32_t* base_counts, hipStream_t s) {
  const dim3 grid((p.nq + kRowsWg - 1) / kRowsWg, p.prob.B * p.prob.H);
  const size_t rows_bytes = (size_t)kRowsWg * (64 * ((p.nkv + 63) / 64) + 4) * sizeof(float);
  const size_t lds = MODE == kSelectRows ? std::max(rows_bytes, 4 * sizeof(WaveHist)) : rows_bytes;
  hipError_t e = hipSuccess;
  with_vpl(p.nkv, [&](auto vpl) {
    auto* kern = &score_rows_kernel<D, decltype(vpl)::value, MODE>;
    // the score rows of long rows need more than the default dynamic LDS limit
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e == hipSuccess)
      kern<<<grid, 256, lds, s>>>(Qbar, Kbar, p.scale, p.prob.H, p.nq, p.nkv, S, target, all,
                                  nwords, bitmap, base_counts);
  });
  return e;
}

}  // namespace

hipError_t launch_score_select(const bsa_plan& p, const float* Qbar, const float* Kbar, float* S,
                               unsigned long long target, bool all, int nwords,
                               uint32_t* bitmap, int32_t* base_counts, hipStream_t s) {
  const hipError_t e =
      p.prob.d == 128 ? launch_score_rows<128, kSelectRows>(p, Qbar, Kbar, S, target, all,
                                                            nwords, bitmap, base_counts, s)
                      : launch_score_rows<64, kSelectRows>(p, Qbar, Kbar, S, target, all, nwords,
                                                           bitmap, base_counts, s);
  return e != hipSuccess ? e : hipGetLastError();
}

hipError_t launch_score(const bsa_plan& p, const float* Qbar, const float* Kbar, int norm,
                        float* S, hipStream_t s) {
  const int BH = p.prob.B * p.prob.H;
  if (p.nkv <= kWaveRowMax) {  // logits (and the row softmax) from the 16-row tiles
    const bool row = norm == BSA_NORM_ROW;
    hipError_t e;
    if (p.prob.d == 128)
      e = row ? launch_score_rows<128, kSoftmaxOut>(p, Qbar, Kbar, S, 0, false, 0, nullptr,
                                                    nullptr, s)
              : launch_score_rows<128, kLogitsOut>(p, Qbar, Kbar, S, 0, false, 0, nullptr,
                                                   nullptr, s);
    else
      e = row ? launch_score_rows<64, kSoftmaxOut>(p, Qbar, Kbar, S, 0, false, 0, nullptr,
                                                   nullptr, s)
              : launch_score_rows<64, kLogitsOut>(p, Qbar, Kbar, S, 0, false, 0, nullptr,
                                                  nullptr, s);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess || row) return e;
    head_softmax_kernel<<<BH, 1024, 0, s>>>(S, p.qstart, p.nq, p.nkv);
    return hipGetLastError();
  }
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
