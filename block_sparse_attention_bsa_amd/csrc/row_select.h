// Exact selection of one score row held in the registers of one wavefront (value j of the row is
// value i = j / 64 of lane j % 64): the shortest prefix of the (score descending, index ascending)
// order whose sum reaches a target, or the top k. Shared by the row selection kernels (scores
// from memory) and the fused score-and-select kernel (scores formed in the same workgroup).
//
// Rule (pith.science review of VMoBA, referee report major comment 1: Sec. 3.4 Eq. 4 keeps the
// smallest k' whose cumulative normalised similarity reaches the threshold; LoSA abstract: the
// smallest block set meeting the retained-mass threshold). Sums are exact: every score is a
// 2^-56 fixed-point integer, so the result does not depend on the order of additions.
#pragma once

#include <type_traits>

#include "device_common.h"

namespace {

constexpr double kFix = 72057594037927936.0;  // 2^56

__device__ __forceinline__ uint32_t sel_key(float s) {
  const uint32_t k = __float_as_uint(s);
  return (k & 0x80000000u) ? 0u : k;  // negative values rank below every non-negative one
}

__device__ __forceinline__ unsigned long long sel_fix(float s) {
  double x = (double)s * kFix;
  if (!(x > 0.0)) return 0ull;  // also NaN
  if (x > kFix) x = kFix;
  return (unsigned long long)rint(x);
}

// Rows of at most kWaveRowMax candidates are selected by one wavefront each (the row in
// registers, kVpl values per lane, a wave-private LDS histogram per radix pass, no workgroup
// barrier). Same rule, exact sums and tie order as the block-wide radix select of longer rows:
// results are identical.
constexpr int kWaveRowMax = 2048;

struct WaveHist {
  unsigned int cnt[256];
  unsigned long long sum[256];
};

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, d, 64));
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, d, 64));
  return v;
}

// by_count: target is a count (top-k); else a 2^-56 fixed-point sum. Returns the chosen flags in
// `sel` (value i of this lane) and the selected count.
//
// The radix runs on u = key - kmin (an order-preserving map of the row's keys onto
// [0, kmax - kmin]) and its first digit is the top 8 of the bits u can have: that digit spreads a
// row over up to 256 bins in proportion to its spread of keys (about log2 of the scores), where
// the fixed top byte of the key put a softmax row into two or three bins and serialised the LDS
// atomics on them. Later digits take the next 8 bits (the last one fewer). The result is the same
// set as with any other digit split of the same total order.
template <int kVpl>
__device__ uint32_t wave_select(const float (&v)[kVpl], int n, unsigned long long target,
                                bool by_count, bool all, WaveHist& h, bool (&sel)[kVpl]) {
  const int lane = threadIdx.x & 63;
  uint32_t u[kVpl];
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int i = 0; i < kVpl; ++i) {
    const bool valid = lane + 64 * i < n;
    u[i] = valid ? sel_key(v[i]) : 0u;
    if (valid) {
      kmin = min(kmin, u[i]);
      kmax = max(kmax, u[i]);
    }
  }
  if (all) {
#pragma unroll
    for (int i = 0; i < kVpl; ++i) sel[i] = lane + 64 * i < n;
    return (uint32_t)n;
  }
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
#pragma unroll
  for (int i = 0; i < kVpl; ++i) u[i] -= kmin;  // invalid slots are never candidates
  // fixed-point value of every score, formed once (the passes below add them)
  unsigned long long fx[kVpl];
#pragma unroll
  for (int i = 0; i < kVpl; ++i) fx[i] = by_count ? 0ull : sel_fix(v[i]);
  const uint32_t spread = kmax - kmin;           // < 2^31: keys of non-negative floats
  int rem = spread ? 32 - __clz(spread) : 0;     // bits of u that can be set
  uint32_t hi = 0;                               // candidates: (u >> rem) == hi
  uint32_t eq_cnt = (uint32_t)n;                 // candidates left (spread 0: all are equal)
  unsigned long long above_sum = 0;
  uint32_t above_cnt = 0;
  bool every = false;
  while (rem > 0) {
    const int db = rem < 8 ? rem : 8, sh = rem - db;
    const uint32_t dmask = (1u << db) - 1u;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      h.cnt[4 * lane + k] = 0u;
      h.sum[4 * lane + k] = 0ull;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < kVpl; ++i) {
      if (lane + 64 * i < n && (u[i] >> rem) == hi) {
        const uint32_t b = (u[i] >> sh) & dmask;
        atomicAdd(&h.cnt[b], 1u);
        if (!by_count) atomicAdd(&h.sum[b], fx[i]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // Bins in descending order: lane l holds bins 255 - 4l - k (k = 0..3).
    unsigned long long lsum = 0;
    int lcnt = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (!by_count) lsum += h.sum[255 - 4 * lane - k];
      lcnt += (int)h.cnt[255 - 4 * lane - k];
    }
    const unsigned long long isum = by_count ? 0ull : wave_incl_scan_u64(lsum);
    const int icnt = wave_incl_scan_i32(lcnt);
    unsigned long long asum = above_sum + (isum - lsum);
    unsigned long long acnt = above_cnt + (unsigned long long)(icnt - lcnt);
    int my_bin = -1;
    unsigned long long my_asum = 0, my_acnt = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int b = 255 - 4 * lane - k;
      const unsigned long long cur = by_count ? acnt : asum;
      const unsigned long long sb = by_count ? 0ull : h.sum[b];
      const unsigned long long mb = by_count ? (unsigned long long)h.cnt[b] : sb;
      if (my_bin < 0 && cur < target && cur + mb >= target) {
        my_bin = b;
        my_asum = asum;
        my_acnt = acnt;
      }
      asum += sb;
      acnt += h.cnt[b];
    }
    const unsigned long long found = __ballot(my_bin >= 0);
    if (found == 0) {  // the target is never reached: keep every candidate
      every = true;
      break;
    }
    const int src = __ffsll((long long)found) - 1;
    const int b = __shfl(my_bin, src, 64);
    above_sum = ((unsigned long long)(uint32_t)__shfl((int)(my_asum >> 32), src, 64) << 32) |
                (uint32_t)__shfl((int)(uint32_t)my_asum, src, 64);
    above_cnt = (uint32_t)__shfl((int)my_acnt, src, 64);
    hi = (hi << db) | (uint32_t)b;
    rem = sh;
    eq_cnt = h.cnt[b];
    __builtin_amdgcn_wave_barrier();
    if (eq_cnt == 1) break;
  }
  if (spread == 0) {  // every value equal: no pass ran; the whole row is the boundary class
    if (by_count) {
      every = target >= (unsigned long long)n;
    } else {
      const unsigned long long vfix = sel_fix(__uint_as_float(kmin));
      every = vfix == 0 || (target + vfix - 1) / vfix >= (unsigned long long)n;
    }
  }
  if (every) {
#pragma unroll
    for (int i = 0; i < kVpl; ++i) sel[i] = lane + 64 * i < n;
    return (uint32_t)n;
  }
  uint32_t m;
  if (by_count) {
    m = (uint32_t)(target - above_cnt);
  } else if (eq_cnt == 1) {
    m = 1;
  } else {  // rem == 0: the boundary class is one key, hi + kmin
    const unsigned long long vfix = sel_fix(__uint_as_float(hi + kmin));
    m = (uint32_t)((target - above_sum + vfix - 1) / vfix);
  }
  if (m > eq_cnt) m = eq_cnt;
  // Everything strictly above the boundary class, plus its m lowest-index members.
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < kVpl; ++i) {
    const bool valid = lane + 64 * i < n;
    const uint32_t k = u[i] >> rem;
    const bool eq = valid && k == hi;
    const unsigned long long bal = __ballot(eq);
    const uint32_t rank = taken + __popcll(bal & ((1ull << lane) - 1ull));
    sel[i] = valid && (k > hi || (eq && rank < m));
    taken += __popcll(bal);
  }
  return above_cnt + m;
}

// Bitmap words of one row from per-value flags (value j = lane + 64 i): words 2i and 2i + 1.
template <int kVpl>
__device__ __forceinline__ void write_row_bits(const bool (&sel)[kVpl], int nwords,
                                               uint32_t* __restrict__ words) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < kVpl; ++i) {
    const unsigned long long bal = __ballot(sel[i]);
    const int w = 2 * i + lane;
    if (lane < 2 && w < nwords) words[w] = (uint32_t)(bal >> (32 * lane));
  }
}


// Calls f with std::integral_constant<int, V> for the smallest instantiated V with 64 V >= n
// (n <= kWaveRowMax): values per lane of the one-wavefront-per-row kernels.
template <typename F>
void with_vpl(int n, F&& f) {
  const int v = (n + 63) / 64;
  if (v <= 1) f(std::integral_constant<int, 1>());
  else if (v <= 2) f(std::integral_constant<int, 2>());
  else if (v <= 4) f(std::integral_constant<int, 4>());
  else if (v <= 6) f(std::integral_constant<int, 6>());
  else if (v <= 8) f(std::integral_constant<int, 8>());
  else if (v <= 12) f(std::integral_constant<int, 12>());
  else if (v <= 16) f(std::integral_constant<int, 16>());
  else if (v <= 20) f(std::integral_constant<int, 20>());
  else if (v <= 24) f(std::integral_constant<int, 24>());
  else f(std::integral_constant<int, 32>());
}

// with_vpl for the selection kernels, plus an exact fit for rows of 1025..1088 blocks (17 values
// per lane, e.g. 1080-block rows): the 20-value form spends its per-value work on three empty
// slots there (720p select stage 0.150 -> 0.138 ms, same selections). The score kernel keeps
// with_vpl: its 17-value form measured slower (0.18 -> 0.28 ms).
template <typename F>
void with_sel_vpl(int n, F&& f) {
  if ((n + 63) / 64 == 17) f(std::integral_constant<int, 17>());
  else with_vpl(n, static_cast<F&&>(f));
}

}  // namespace
