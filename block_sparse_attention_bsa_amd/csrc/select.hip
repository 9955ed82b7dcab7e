// Block selection (step 3).
//
// Rule: rank the candidates by (score descending, index ascending) and keep the shortest prefix
// whose cumulative score reaches p (pith.science review of VMoBA, referee report major comment 1:
// Sec. 3.4 Eq. 4 takes the smallest k' whose cumulative normalised similarity reaches tau; LoSA
// abstract: the smallest block set meeting the retained-mass threshold). Candidates are the kv
// blocks of one query block (ROW pool) or every (I, J) pair of a head (HEAD pool, VMoBA Eq. 3).
// SCOPE abstract (mlsift listing): rows whose retained count is below the head's count-weighted
// mean get the next blocks of the same ranking up to that count.
//
// Instead of sorting, each pool runs a most-significant-digit radix select on the fp32 bit
// pattern (monotone for non-negative scores): 8-bit digits, per-bin counts and per-bin sums.
// Sums are exact: every score is converted to a 2^-56 fixed-point integer, so sums of fp32 scores
// carry no rounding and integer LDS atomics make the result independent of thread order. Pass
// by pass it narrows to the digit bin where the cumulative sum (or count) first reaches the
// target; when that bin holds a single candidate it stops early. Ties on the final bit pattern are
// resolved by index with a wavefront ballot scan.
//
// The chosen set is written as a bitmap (one bit per (row, kv block)); a scan over the final row
// counts gives row_ptr, and a per-row pass expands the bitmap into ascending column indices.
#include "bsa_internal.h"
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

struct RadixShared {
  unsigned int cnt[256];
  unsigned long long sum[256];
  unsigned int prefix, mask;
  unsigned long long above_sum;
  unsigned int above_cnt;
  unsigned int eq_cnt;
  int bin;
  unsigned long long new_above_sum;
  unsigned int new_above_cnt;
};

struct RadixResult {
  bool all;            // every candidate is selected
  uint32_t prefix, mask;
  uint32_t m;          // how many of the boundary class (lowest indices first) are selected
  bool eq_all;         // m == size of the boundary class
  uint32_t count;      // selected count
};

// Block-wide radix select over vals[0, n). by_count: target is a count; else a 2^-56 sum.
template <int NT>
__device__ RadixResult radix_select(const float* __restrict__ vals, int64_t n,
                                    unsigned long long target, bool by_count, RadixShared& sh) {
  const int t = threadIdx.x;
  RadixResult res;
  res.all = false;
  if (t == 0) {
    sh.prefix = 0;
    sh.mask = 0;
    sh.above_sum = 0;
    sh.above_cnt = 0;
    sh.eq_cnt = 0;
  }
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int b = t; b < 256; b += NT) {
      sh.cnt[b] = 0;
      sh.sum[b] = 0;
    }
    __syncthreads();
    const uint32_t prefix = sh.prefix, mask = sh.mask;
    for (int64_t j = t; j < n; j += NT) {
      const float v = vals[j];
      const uint32_t key = sel_key(v);
      if ((key & mask) == prefix) {
        const uint32_t b = (key >> shift) & 255u;
        atomicAdd(&sh.cnt[b], 1u);
        if (!by_count) atomicAdd(&sh.sum[b], sel_fix(v));
      }
    }
    __syncthreads();
    if (t < 64) {
      const int lane = t;
      unsigned long long lsum = 0;
      unsigned int lcnt = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int b = 255 - 4 * lane - i;
        lsum += sh.sum[b];
        lcnt += sh.cnt[b];
      }
      const unsigned long long isum = wave_incl_scan_u64(lsum);
      const unsigned long long icnt = wave_incl_scan_u64(lcnt);
      unsigned long long asum = sh.above_sum + (isum - lsum);
      unsigned long long acnt = sh.above_cnt + (icnt - lcnt);
      bool found = false;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int b = 255 - 4 * lane - i;
        const unsigned long long cur = by_count ? acnt : asum;
        const unsigned long long mb = by_count ? (unsigned long long)sh.cnt[b] : sh.sum[b];
        if (!found && cur < target && cur + mb >= target) {
          found = true;
          sh.bin = b;
          sh.new_above_sum = asum;
          sh.new_above_cnt = (unsigned int)acnt;
        }
        asum += sh.sum[b];
        acnt += sh.cnt[b];
      }
      const unsigned long long any = __ballot(found);
      if (any == 0 && lane == 0) sh.bin = -1;
    }
    __syncthreads();
    if (sh.bin < 0) {  // the target is never reached: keep every candidate
      res.all = true;
      res.count = (uint32_t)n;
      return res;
    }
    __syncthreads();
    if (t == 0) {
      const uint32_t b = (uint32_t)sh.bin;
      sh.prefix |= b << shift;
      sh.mask |= 255u << shift;
      sh.above_sum = sh.new_above_sum;
      sh.above_cnt = sh.new_above_cnt;
      sh.eq_cnt = sh.cnt[b];
    }
    __syncthreads();
    if (sh.eq_cnt == 1) break;
  }
  res.prefix = sh.prefix;
  res.mask = sh.mask;
  const uint32_t eq = sh.eq_cnt;
  uint32_t m;
  if (by_count) {
    m = (uint32_t)(target - sh.above_cnt);
  } else if (eq == 1) {
    m = 1;
  } else {
    const unsigned long long v = sel_fix(__uint_as_float(sh.prefix));
    m = (uint32_t)((target - sh.above_sum + v - 1) / v);
  }
  if (m > eq) m = eq;
  res.m = m;
  res.eq_all = (m == eq);
  res.count = sh.above_cnt + m;
  __syncthreads();
  return res;
}

__device__ __forceinline__ bool sel_fast(const RadixResult& r, uint32_t key) {
  if (r.all) return true;
  const uint32_t k = key & r.mask;
  return k > r.prefix || (k == r.prefix && r.eq_all);
}

// Write the bitmap words of `nrows` consecutive rows (nkv candidates each, flattened index
// j = I * nkv + J) and, for the boundary class when only part of it is kept, set the bits of its
// m lowest-index members. Optionally accumulates per-row counts with integer atomics.
template <int NT>
__device__ void mark_pool(const float* __restrict__ vals, int nrows, int nkv, int nwords,
                          uint32_t* __restrict__ bitmap, const RadixResult& r,
                          int32_t* __restrict__ row_counts) {
  const int t = threadIdx.x;
  const int64_t nw_total = (int64_t)nrows * nwords;
  for (int64_t wi = t; wi < nw_total; wi += NT) {
    const int I = (int)(wi / nwords), w = (int)(wi % nwords);
    uint32_t word = 0;
    const float* rowv = vals + (int64_t)I * nkv;
    for (int b = 0; b < 32; ++b) {
      const int J = 32 * w + b;
      if (J >= nkv) break;
      if (sel_fast(r, sel_key(rowv[J]))) word |= 1u << b;
    }
    bitmap[wi] = word;
    if (row_counts && word) atomicAdd(&row_counts[I], __popc(word));
  }
  if (r.all || r.eq_all) return;
  __threadfence();
  __syncthreads();
  if (t < 64) {
    const int lane = t;
    const int64_t n = (int64_t)nrows * nkv;
    uint32_t taken = 0;
    for (int64_t base = 0; base < n && taken < r.m; base += 64) {
      const int64_t j = base + lane;
      bool eq = false;
      if (j < n) eq = (sel_key(vals[j]) & r.mask) == r.prefix;
      const unsigned long long bal = __ballot(eq);
      const uint32_t rank = taken + __popcll(bal & ((1ull << lane) - 1ull));
      if (eq && rank < r.m) {
        const int I = (int)(j / nkv), J = (int)(j % nkv);
        atomicOr(&bitmap[(int64_t)I * nwords + J / 32], 1u << (J % 32));
        if (row_counts) atomicAdd(&row_counts[I], 1);
      }
      taken += __popcll(bal);
    }
  }
}

// ROW pool: one workgroup per row (b, h, I).
__global__ __launch_bounds__(256) void mark_row_kernel(const float* __restrict__ S, int nkv,
                                                       int nwords, unsigned long long target,
                                                       bool select_all,
                                                       uint32_t* __restrict__ bitmap,
                                                       int32_t* __restrict__ base_counts) {
  __shared__ RadixShared sh;
  const int64_t r = blockIdx.x;
  const float* row = S + r * nkv;
  RadixResult res;
  if (select_all) {
    res.all = true;
    res.count = nkv;
  } else {
    res = radix_select<256>(row, nkv, target, false, sh);
  }
  mark_pool<256>(row, 1, nkv, nwords, bitmap + r * nwords, res, nullptr);
  if (threadIdx.x == 0) base_counts[r] = (int32_t)res.count;
}

// HEAD pool: one 1024-thread workgroup per head (b, h); candidates are its nq * nkv pairs.
__global__ __launch_bounds__(1024) void mark_head_kernel(const float* __restrict__ S, int nq,
                                                         int nkv, int nwords,
                                                         unsigned long long target,
                                                         bool select_all,
                                                         uint32_t* __restrict__ bitmap,
                                                         int32_t* __restrict__ base_counts) {
  __shared__ RadixShared sh;
  const int64_t bh = blockIdx.x;
  const float* W = S + bh * (int64_t)nq * nkv;
  int32_t* counts = base_counts + bh * nq;
  for (int I = threadIdx.x; I < nq; I += 1024) counts[I] = 0;
  __threadfence();
  __syncthreads();
  RadixResult res;
  if (select_all) {
    res.all = true;
    res.count = (uint32_t)((int64_t)nq * nkv);
  } else {
    res = radix_select<1024>(W, (int64_t)nq * nkv, target, false, sh);
  }
  mark_pool<1024>(W, nq, nkv, nwords, bitmap + bh * (int64_t)nq * nwords, res, counts);
}

// Per-head minimum count: mode 1 fixed_k, mode 2 ceil(sum |I| c_I / sum |I|) (SCOPE abstract),
// capped at nkv; mode 0 writes 0.
__global__ __launch_bounds__(256) void head_k_kernel(const int32_t* __restrict__ base_counts,
                                                     const int32_t* __restrict__ qstart, int nq,
                                                     int nkv, int mode, int fixed_k,
                                                     int32_t* __restrict__ head_k_ws,
                                                     int32_t* __restrict__ head_k_out) {
  __shared__ unsigned long long snum[4], sden[4];
  const int bh = blockIdx.x, t = threadIdx.x;
  unsigned long long num = 0, den = 0;
  if (mode == BSA_MINK_WEIGHTED_MEAN) {
    for (int I = t; I < nq; I += 256) {
      const unsigned long long w = (unsigned long long)(qstart[I + 1] - qstart[I]);
      num += w * (unsigned long long)base_counts[(int64_t)bh * nq + I];
      den += w;
    }
  }
  num = wave_incl_scan_u64(num);
  den = wave_incl_scan_u64(den);
  if ((t & 63) == 63) {
    snum[t >> 6] = num;
    sden[t >> 6] = den;
  }
  __syncthreads();
  if (t == 0) {
    long long k = 0;
    if (mode == BSA_MINK_WEIGHTED_MEAN) {
      const unsigned long long N = snum[0] + snum[1] + snum[2] + snum[3];
      const unsigned long long Dn = sden[0] + sden[1] + sden[2] + sden[3];
      k = (long long)((N + Dn - 1) / Dn);
    } else if (mode == BSA_MINK_FIXED) {
      k = fixed_k;
    }
    if (k > nkv) k = nkv;
    head_k_ws[bh] = (int32_t)k;
    if (head_k_out) head_k_out[bh] = (int32_t)k;
  }
}

// Rows below their head's minimum take the top-k of the same ranking (by count).
__global__ __launch_bounds__(256) void topup_kernel(const float* __restrict__ S, int nq, int nkv,
                                                    int nwords,
                                                    const int32_t* __restrict__ base_counts,
                                                    const int32_t* __restrict__ head_k,
                                                    uint32_t* __restrict__ bitmap) {
  __shared__ RadixShared sh;
  const int64_t r = blockIdx.x;
  const int k = head_k[r / nq];
  if (base_counts[r] >= k) return;
  const float* row = S + r * nkv;
  const RadixResult res = radix_select<256>(row, nkv, (unsigned long long)k, true, sh);
  mark_pool<256>(row, 1, nkv, nwords, bitmap + r * nwords, res, nullptr);
}

// row_ptr = exclusive scan of the final counts (one workgroup, any number of rows).
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* __restrict__ base_counts,
                                                    const int32_t* __restrict__ head_k,
                                                    bool use_min_k, int64_t rows, int nq,
                                                    int32_t* __restrict__ row_ptr,
                                                    int32_t* __restrict__ counts_out) {
  __shared__ int wtot[16];
  __shared__ int carry_s;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  if (t == 0) {
    carry_s = 0;
    row_ptr[0] = 0;
  }
  __syncthreads();
  for (int64_t base = 0; base < rows; base += 1024) {
    const int64_t r = base + t;
    int f = 0;
    if (r < rows) {
      f = base_counts[r];
      if (use_min_k) f = max(f, head_k[r / nq]);
      if (counts_out) counts_out[r] = f;
    }
    const int incl = wave_incl_scan_i32(f);
    if (lane == 63) wtot[wave] = incl;
    __syncthreads();
    int before = carry_s;
    for (int w = 0; w < wave; ++w) before += wtot[w];
    if (r < rows) row_ptr[r + 1] = before + incl;
    __syncthreads();
    if (t == 0) {
      int tot = 0;
      for (int w = 0; w < 16; ++w) tot += wtot[w];
      carry_s += tot;
    }
    __syncthreads();
  }
}

// Expand each row's bitmap into ascending kv-block indices at row_ptr[r].
__global__ __launch_bounds__(256) void emit_kernel(const uint32_t* __restrict__ bitmap,
                                                   int nwords,
                                                   const int32_t* __restrict__ row_ptr,
                                                   int32_t* __restrict__ col_idx) {
  __shared__ int wtot[4];
  const int64_t r = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const uint32_t word = t < nwords ? bitmap[r * nwords + t] : 0u;
  const int c = __popc(word);
  const int incl = wave_incl_scan_i32(c);
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  int pos = row_ptr[r] + incl - c;
  const int end = row_ptr[r + 1];
  for (int w = 0; w < wave; ++w) pos += wtot[w];
  uint32_t bits = word;
  while (bits && pos < end) {
    const int b = __ffs(bits) - 1;
    col_idx[pos++] = 32 * t + b;
    bits &= bits - 1;
  }
}


// ------------------------------------------------------------------ one wavefront per row

// ROW-pool selection for rows of at most 64 * VPL candidates (VPL = 16 or 32): one wavefront per
// row (four rows per workgroup), the row held in registers (value j = lane + 64 i), a wave-private
// LDS histogram per radix pass, and no workgroup barrier at all. Same rule, same exact 2^-56 sums
// and the same tie order as radix_select: results are identical.
constexpr int kWaveRowMax = 2048;

struct WaveHist {
  unsigned int cnt[256];
  unsigned long long sum[256];
};

// by_count: target is a count (top-k); else a 2^-56 fixed-point sum. Returns the chosen flags in
// `sel` (value i of this lane) and the selected count.
template <int kVpl>
__device__ uint32_t wave_select(const float (&v)[kVpl], int n, unsigned long long target,
                                bool by_count, bool all, WaveHist& h, bool (&sel)[kVpl]) {
  const int lane = threadIdx.x & 63;
  uint32_t key[kVpl];
#pragma unroll
  for (int i = 0; i < kVpl; ++i) key[i] = (lane + 64 * i < n) ? sel_key(v[i]) : 0u;
  if (all) {
#pragma unroll
    for (int i = 0; i < kVpl; ++i) sel[i] = lane + 64 * i < n;
    return (uint32_t)n;
  }
  uint32_t prefix = 0, mask = 0, eq_cnt = 0;
  unsigned long long above_sum = 0;
  uint32_t above_cnt = 0;
  bool every = false;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      h.cnt[4 * lane + k] = 0u;
      h.sum[4 * lane + k] = 0ull;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < kVpl; ++i) {
      if (lane + 64 * i < n && (key[i] & mask) == prefix) {
        const uint32_t b = (key[i] >> shift) & 255u;
        atomicAdd(&h.cnt[b], 1u);
        if (!by_count) atomicAdd(&h.sum[b], sel_fix(v[i]));
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // Bins in descending order: lane l holds bins 255 - 4l - k (k = 0..3).
    unsigned long long lsum = 0, lcnt = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      lsum += h.sum[255 - 4 * lane - k];
      lcnt += h.cnt[255 - 4 * lane - k];
    }
    const unsigned long long isum = wave_incl_scan_u64(lsum);
    const unsigned long long icnt = wave_incl_scan_u64(lcnt);
    unsigned long long asum = above_sum + (isum - lsum);
    unsigned long long acnt = above_cnt + (icnt - lcnt);
    int my_bin = -1;
    unsigned long long my_asum = 0, my_acnt = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int b = 255 - 4 * lane - k;
      const unsigned long long cur = by_count ? acnt : asum;
      const unsigned long long mb = by_count ? (unsigned long long)h.cnt[b] : h.sum[b];
      if (my_bin < 0 && cur < target && cur + mb >= target) {
        my_bin = b;
        my_asum = asum;
        my_acnt = acnt;
      }
      asum += h.sum[b];
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
    prefix |= (uint32_t)b << shift;
    mask |= 255u << shift;
    eq_cnt = h.cnt[b];
    __builtin_amdgcn_wave_barrier();
    if (eq_cnt == 1) break;
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
  } else {
    const unsigned long long vfix = sel_fix(__uint_as_float(prefix));
    m = (uint32_t)((target - above_sum + vfix - 1) / vfix);
  }
  if (m > eq_cnt) m = eq_cnt;
  // Everything strictly above the boundary class, plus its m lowest-index members.
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < kVpl; ++i) {
    const bool valid = lane + 64 * i < n;
    const uint32_t k = key[i] & mask;
    const bool eq = valid && k == prefix;
    const unsigned long long bal = __ballot(eq);
    const uint32_t rank = taken + __popcll(bal & ((1ull << lane) - 1ull));
    sel[i] = valid && (k > prefix || (eq && rank < m));
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

template <int kVpl>
__global__ __launch_bounds__(256) void mark_row_wave_kernel(const float* __restrict__ S,
                                                            int64_t rows, int nkv, int nwords,
                                                            unsigned long long target,
                                                            bool select_all,
                                                            uint32_t* __restrict__ bitmap,
                                                            int32_t* __restrict__ base_counts) {
  __shared__ WaveHist hist[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r = (int64_t)blockIdx.x * 4 + wave;
  if (r >= rows) return;  // whole wavefronts
  const float* row = S + r * nkv;
  float v[kVpl];
#pragma unroll
  for (int i = 0; i < kVpl; ++i) v[i] = lane + 64 * i < nkv ? row[lane + 64 * i] : 0.f;
  bool sel[kVpl];
  const uint32_t count = wave_select(v, nkv, target, false, select_all, hist[wave], sel);
  write_row_bits(sel, nwords, bitmap + r * nwords);
  if (lane == 0) base_counts[r] = (int32_t)count;
}

template <int kVpl>
__global__ __launch_bounds__(256) void topup_wave_kernel(const float* __restrict__ S, int64_t rows,
                                                         int nq, int nkv, int nwords,
                                                         const int32_t* __restrict__ base_counts,
                                                         const int32_t* __restrict__ head_k,
                                                         uint32_t* __restrict__ bitmap) {
  __shared__ WaveHist hist[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r = (int64_t)blockIdx.x * 4 + wave;
  if (r >= rows) return;
  const int k = head_k[r / nq];
  if (base_counts[r] >= k) return;
  const float* row = S + r * nkv;
  float v[kVpl];
#pragma unroll
  for (int i = 0; i < kVpl; ++i) v[i] = lane + 64 * i < nkv ? row[lane + 64 * i] : 0.f;
  bool sel[kVpl];
  wave_select(v, nkv, (unsigned long long)k, true, false, hist[wave], sel);
  write_row_bits(sel, nwords, bitmap + r * nwords);
}

// CSR columns of one row from its bitmap (at most 64 words), one wavefront per row: each 64-bit
// word pair is a mask over 64 consecutive candidates; every set lane writes its column at the
// running position plus its rank, so the stores of a wavefront are consecutive.
__global__ __launch_bounds__(256) void emit_wave_kernel(const uint32_t* __restrict__ bitmap,
                                                        int nwords, int64_t rows,
                                                        const int32_t* __restrict__ row_ptr,
                                                        int32_t* __restrict__ col_idx) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const uint32_t word = lane < nwords ? bitmap[r * nwords + lane] : 0u;
  int pos = row_ptr[r];
  const int end = row_ptr[r + 1];
  for (int g = 0; 2 * g < nwords; ++g) {
    const uint32_t lo = (uint32_t)__shfl((int)word, 2 * g, 64);
    const uint32_t hi = (uint32_t)__shfl((int)word, 2 * g + 1, 64);  // 0 past nwords
    const unsigned long long m = ((unsigned long long)hi << 32) | lo;
    const int at = pos + __popcll(m & ((1ull << lane) - 1ull));
    if ((m >> lane) & 1ull && at < end) col_idx[at] = 64 * g + lane;
    pos += __popcll(m);
  }
}

}  // namespace

hipError_t launch_select(const bsa_plan& p, const float* S, const bsa_select_params& prm,
                         int32_t* row_ptr, int32_t* col_idx, int32_t* counts, int32_t* head_k,
                         void* ws, hipStream_t s) {
  const SelectWs L = select_ws_layout(p);
  char* base = static_cast<char*>(ws);
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(base + L.bitmap);
  int32_t* base_counts = reinterpret_cast<int32_t*>(base + L.base_counts);
  int32_t* head_k_ws = reinterpret_cast<int32_t*>(base + L.head_k);
  const int BH = p.prob.B * p.prob.H;
  const int64_t rows = (int64_t)BH * p.nq;
  const bool all = prm.p >= 1.0;
  const unsigned long long target = all ? 0ull : (unsigned long long)ceil(prm.p * kFix);
  if (rows == 0) return hipSuccess;

  const bool wave_rows = p.nkv <= kWaveRowMax;
  const unsigned wgrid = (unsigned)((rows + 3) / 4);
  if (prm.pool == BSA_POOL_ROW && p.nkv <= 1024)
    mark_row_wave_kernel<16><<<wgrid, 256, 0, s>>>(S, rows, p.nkv, L.nwords, target, all, bitmap,
                                                   base_counts);
  else if (prm.pool == BSA_POOL_ROW && wave_rows)
    mark_row_wave_kernel<32><<<wgrid, 256, 0, s>>>(S, rows, p.nkv, L.nwords, target, all, bitmap,
                                                   base_counts);
  else if (prm.pool == BSA_POOL_ROW)
    mark_row_kernel<<<(unsigned)rows, 256, 0, s>>>(S, p.nkv, L.nwords, target, all, bitmap,
                                                   base_counts);
  else
    mark_head_kernel<<<BH, 1024, 0, s>>>(S, p.nq, p.nkv, L.nwords, target, all, bitmap,
                                         base_counts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool use_min_k = prm.min_k_mode != BSA_MINK_NONE;
  if (use_min_k || head_k) {
    head_k_kernel<<<BH, 256, 0, s>>>(base_counts, p.qstart, p.nq, p.nkv, prm.min_k_mode,
                                     prm.fixed_k, head_k_ws, head_k);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (use_min_k && wave_rows) {
    if (p.nkv <= 1024)
      topup_wave_kernel<16><<<wgrid, 256, 0, s>>>(S, rows, p.nq, p.nkv, L.nwords, base_counts,
                                                  head_k_ws, bitmap);
    else
      topup_wave_kernel<32><<<wgrid, 256, 0, s>>>(S, rows, p.nq, p.nkv, L.nwords, base_counts,
                                                  head_k_ws, bitmap);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  } else if (use_min_k) {
    topup_kernel<<<(unsigned)rows, 256, 0, s>>>(S, p.nq, p.nkv, L.nwords, base_counts,
                                                head_k_ws, bitmap);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  scan_kernel<<<1, 1024, 0, s>>>(base_counts, head_k_ws, use_min_k, rows, p.nq, row_ptr, counts);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (L.nwords <= 64)
    emit_wave_kernel<<<(unsigned)((rows + 3) / 4), 256, 0, s>>>(bitmap, L.nwords, rows, row_ptr,
                                                                col_idx);
  else
    emit_kernel<<<(unsigned)rows, 256, 0, s>>>(bitmap, L.nwords, row_ptr, col_idx);
  return hipGetLastError();
}
