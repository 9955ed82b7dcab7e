// Block means of Q or K (pith.science review of VMoBA, "What carries the argument" and the
// Figure 2 caption: each block is represented by the mean of its token vectors).
//
// One workgroup of 256 threads per (block J, head bh, d slice). A token row of d elements is read
// as 16-byte segments: the SEGS / slices segments of the workgroup's d slice are covered by as
// many threads, and 256 / (SEGS / slices) rows are in flight per pass, so a wavefront reads whole
// rows or whole slices of rows (a 4x4x8 tile is 16 runs of 8 contiguous tokens, 2 KiB each for
// bf16, d = 128). Blocks of a few hundred tokens take one slice (the whole row); a side whose
// blocks reach thousands of tokens (1D and 2D partitions) is split into 2 or 4 d slices, so
// that its few long blocks spread over more workgroups. Each thread accumulates its segment over
// the rows it visits in fp32; the partial sums are combined across row groups in LDS in a fixed
// order (deterministic).
#include "bsa_internal.h"
#include "device_common.h"

namespace {

template <typename T>
struct Seg;

template <>
struct Seg<uint16_t> {  // bf16 words: 8 per 16 bytes
  static constexpr int kVec = 8;
  __device__ static void add(float* acc, uint4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += bf16_lo(w[i]);
      acc[2 * i + 1] += bf16_hi(w[i]);
    }
  }
};

template <>
struct Seg<float> {  // fp32: 4 per 16 bytes
  static constexpr int kVec = 4;
  __device__ static void add(float* acc, uint4 v) {
    acc[0] += __uint_as_float(v.x);
    acc[1] += __uint_as_float(v.y);
    acc[2] += __uint_as_float(v.z);
    acc[3] += __uint_as_float(v.w);
  }
};

// One pooling pass: X over the blocks of a partition (perm, start) into Xbar.
template <typename T>
struct PoolSide {
  const T* X;
  float* Xbar;
  const int32_t* perm;
  const int32_t* start;
  int nblk;
  int slices;  // d slices per block (1, 2 or 4): one workgroup each
};

// One workgroup's block and d slice (SL slices per block, a compile-time constant so that the
// thread mapping needs no division).
template <typename T, int D, int SL>
__device__ __forceinline__ void pool_block(const PoolSide<T>& sd, int w, int N,
                                           float (*red)[Seg<T>::kVec + 1]) {
  constexpr int VEC = Seg<T>::kVec;
  constexpr int SEGS = D / VEC;
  constexpr int SSEG = SEGS / SL;       // segments of this workgroup's d slice
  constexpr int GROUPS = 256 / SSEG;    // rows in flight per pass
  constexpr int UNROLL = 8;             // one pass covers a 128-token block: all its rows in flight
  const int J = w / SL, slice = w - J * SL;
  const int bh = blockIdx.y;
  const int seg = slice * SSEG + (int)threadIdx.x % SSEG;
  const int grp = (int)threadIdx.x / SSEG;
  const int s0 = sd.start[J];
  const int cnt = sd.start[J + 1] - s0;
  const T* __restrict__ Xh = sd.X + (size_t)bh * N * D + seg * VEC;

  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;

  for (int k = grp; k < cnt; k += UNROLL * GROUPS) {
    uint4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int kk = k + u * GROUPS;
      if (kk < cnt) {
        const int n = sd.perm[s0 + kk];
        v[u] = *reinterpret_cast<const uint4*>(Xh + (size_t)n * D);
      } else {
        v[u] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
      if (k + u * GROUPS < cnt) Seg<T>::add(acc, v[u]);
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) red[threadIdx.x][e] = acc[e];
  __syncthreads();
  constexpr int DW = D / SL;  // d values of the slice
  if ((int)threadIdx.x < DW) {
    const int c = threadIdx.x, cs = c / VEC, ce = c % VEC;
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < GROUPS; ++g) s += red[g * SSEG + cs][ce];
    sd.Xbar[((size_t)bh * sd.nblk + J) * D + slice * DW + c] = s / (float)cnt;
  }
}

// blockIdx.x < a.nblk * a.slices pools side a, the rest side b (both in one launch: more
// workgroups in flight than either alone, for the short 480p passes).
template <typename T, int D>
__global__ __launch_bounds__(256) void pool_kernel(const PoolSide<T> a, const PoolSide<T> b,
                                                   int N) {
  __shared__ float red[256][Seg<T>::kVec + 1];
  const int na = a.nblk * a.slices;
  const bool first = (int)blockIdx.x < na;
  const PoolSide<T>& sd = first ? a : b;
  const int w = first ? (int)blockIdx.x : (int)blockIdx.x - na;
  if (sd.slices == 1)
    pool_block<T, D, 1>(sd, w, N, red);
  else if (sd.slices == 2)
    pool_block<T, D, 2>(sd, w, N, red);
  else
    pool_block<T, D, 4>(sd, w, N, red);
}

template <typename T>
PoolSide<T> side(const bsa_plan& p, int which, const void* X, float* Xbar) {
  PoolSide<T> sd;
  sd.X = static_cast<const T*>(X);
  sd.Xbar = Xbar;
  sd.perm = which == 0 ? p.qperm : p.kvperm;
  sd.start = which == 0 ? p.qstart : p.kvstart;
  sd.nblk = X ? (which == 0 ? p.nq : p.nkv) : 0;
  const int mx = which == 0 ? p.max_qblk : p.max_kvblk;
  sd.slices = mx > 1024 ? 4 : (mx > 512 ? 2 : 1);
  return sd;
}

// Q (which 0) and/or K (which 1); a NULL X skips that side.
template <typename T, int D>
hipError_t launch(const bsa_plan& p, const void* Q, float* Qbar, const void* K, float* Kbar,
                  hipStream_t s) {
  const PoolSide<T> a = side<T>(p, 0, Q, Qbar), b = side<T>(p, 1, K, Kbar);
  const dim3 grid(a.nblk * a.slices + b.nblk * b.slices, p.prob.B * p.prob.H);
  pool_kernel<T, D><<<grid, 256, 0, s>>>(a, b, p.prob.N);
  return hipGetLastError();
}

hipError_t launch_any(const bsa_plan& p, const void* Q, float* Qbar, const void* K, float* Kbar,
                      hipStream_t s) {
  if (p.prob.dtype == BSA_BF16)
    return p.prob.d == 128 ? launch<uint16_t, 128>(p, Q, Qbar, K, Kbar, s)
                           : launch<uint16_t, 64>(p, Q, Qbar, K, Kbar, s);
  return p.prob.d == 128 ? launch<float, 128>(p, Q, Qbar, K, Kbar, s)
                         : launch<float, 64>(p, Q, Qbar, K, Kbar, s);
}

}  // namespace

hipError_t launch_pool(const bsa_plan& p, int which, const void* X, float* Xbar, hipStream_t s) {
  return which == 0 ? launch_any(p, X, Xbar, nullptr, nullptr, s)
                    : launch_any(p, nullptr, nullptr, X, Xbar, s);
}

hipError_t launch_pool_qk(const bsa_plan& p, const void* Q, float* Qbar, const void* K,
                          float* Kbar, hipStream_t s) {
  return launch_any(p, Q, Qbar, K, Kbar, s);
}
