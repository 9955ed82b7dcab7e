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
#include <climits>
#include <mutex>
#include <unordered_map>

#include <array>
#include <type_traits>
#include <utility>

#include "bsa_internal.h"
#include "device_common.h"
#include "row_select.h"

namespace {

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

// ROW pool: one workgroup per row (b, h, I). Rows of heads flagged in skip_head (nullable; the
// pooled heads of bsa_select_eg, whose rows are written later) are left alone.
__global__ __launch_bounds__(256) void mark_row_kernel(const float* __restrict__ S, int nkv,
                                                       int nwords, unsigned long long target,
                                                       bool select_all,
                                                       uint32_t* __restrict__ bitmap,
                                                       int32_t* __restrict__ base_counts,
                                                       int nq,
                                                       const int32_t* __restrict__ skip_head) {
  __shared__ RadixShared sh;
  const int64_t r = blockIdx.x;
  if (skip_head && skip_head[r / nq]) return;
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

// row_ptr = exclusive scan of the final counts, in two passes over 1024-row chunks: the first
// scans each chunk locally and records its total, the second adds the totals of the chunks
// before it (summed by each workgroup from the totals array).
__device__ __forceinline__ int final_count(const int32_t* __restrict__ base_counts,
                                           const int32_t* __restrict__ head_k, bool use_min_k,
                                           int64_t r, int nq) {
  const int f = base_counts[r];
  return use_min_k ? max(f, head_k[r / nq]) : f;
}

__global__ __launch_bounds__(1024) void scan_local_kernel(const int32_t* __restrict__ base_counts,
                                                          const int32_t* __restrict__ head_k,
                                                          bool use_min_k, int64_t rows, int nq,
                                                          int32_t* __restrict__ row_ptr,
                                                          int32_t* __restrict__ counts_out,
                                                          int32_t* __restrict__ partial) {
  __shared__ int wtot[16];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t r = (int64_t)blockIdx.x * 1024 + t;
  const int f = r < rows ? final_count(base_counts, head_k, use_min_k, r, nq) : 0;
  const int incl = wave_incl_scan_i32(f);
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  int pos = incl;
  for (int w = 0; w < wave; ++w) pos += wtot[w];
  if (r < rows) {
    row_ptr[r + 1] = pos;
    if (counts_out) counts_out[r] = f;
  }
  if (t == 1023) partial[blockIdx.x] = pos;
}

__global__ __launch_bounds__(1024) void scan_add_kernel(int64_t rows,
                                                        const int32_t* __restrict__ partial,
                                                        int32_t* __restrict__ row_ptr) {
  __shared__ int wtot[16];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int off = 0;
  for (int b = t; b < (int)blockIdx.x; b += 1024) off += partial[b];
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) off += __shfl_xor(off, d, 64);
  if (lane == 0) wtot[wave] = off;
  __syncthreads();
  off = 0;
  for (int w = 0; w < 16; ++w) off += wtot[w];
  const int64_t r = (int64_t)blockIdx.x * 1024 + t;
  if (r < rows) row_ptr[r + 1] += off;
  if (blockIdx.x == 0 && t == 0) row_ptr[0] = 0;
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

template <int kVpl>
__global__ __launch_bounds__(256) void mark_row_wave_kernel(const float* __restrict__ S,
                                                            int64_t rows, int nkv, int nwords,
                                                            unsigned long long target,
                                                            bool select_all,
                                                            uint32_t* __restrict__ bitmap,
                                                            int32_t* __restrict__ base_counts,
                                                            int nq,
                                                            const int32_t* __restrict__ skip_head) {
  __shared__ WaveHist hist[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r = (int64_t)blockIdx.x * 4 + wave;
  if (r >= rows) return;  // whole wavefronts
  if (skip_head && skip_head[r / nq]) return;  // as mark_row_kernel
  const float* row = S + r * nkv;
  float v[kVpl];
#pragma unroll
  for (int i = 0; i < kVpl; ++i) v[i] = lane + 64 * i < nkv ? row[lane + 64 * i] : 0.f;
  bool sel[kVpl];
  const uint32_t count = wave_select(v, nkv, target, false, select_all, hist[wave], sel);
  write_row_bits(sel, nwords, bitmap + r * nwords);
  if (lane == 0) base_counts[r] = (int32_t)count;
}

// The per-head minimum's top-up and the emission in one pass (row_ptr already holds the scan of
// the final counts max(base count, k)): a row below its head's k re-reads its scores, takes the
// top k of the same ranking (by count) and writes its columns from the flags in registers; any
// other row writes its columns from the marking pass's bitmap. Columns ascend in both cases
// (value i of lane l is column l + 64 i). Rows of at most 64 * kVpl blocks (nwords <= 64).
template <int kVpl>
__global__ __launch_bounds__(256) void topup_emit_wave_kernel(
    const float* __restrict__ S, int64_t rows, int nq, int nkv, int nwords,
    const int32_t* __restrict__ base_counts, const int32_t* __restrict__ head_k,
    const uint32_t* __restrict__ bitmap, const int32_t* __restrict__ row_ptr,
    int32_t* __restrict__ col_idx) {
  __shared__ WaveHist hist[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r = (int64_t)blockIdx.x * 4 + wave;
  if (r >= rows) return;  // whole wavefronts
  const int k = head_k[r / nq];
  int pos = row_ptr[r];
  const int end = row_ptr[r + 1];
  if (base_counts[r] < k) {
    const float* row = S + r * nkv;
    float v[kVpl];
#pragma unroll
    for (int i = 0; i < kVpl; ++i) v[i] = lane + 64 * i < nkv ? row[lane + 64 * i] : 0.f;
    bool sel[kVpl];
    wave_select(v, nkv, (unsigned long long)k, true, false, hist[wave], sel);
#pragma unroll
    for (int i = 0; i < kVpl; ++i) {
      const unsigned long long m = __ballot(sel[i]);
      const int at = pos + __popcll(m & ((1ull << lane) - 1ull));
      if (sel[i] && at < end) col_idx[at] = lane + 64 * i;
      pos += __popcll(m);
    }
    return;
  }
  const uint32_t word = lane < nwords ? bitmap[r * nwords + lane] : 0u;
  for (int g = 0; 2 * g < nwords; ++g) {
    const uint32_t lo = (uint32_t)__shfl((int)word, 2 * g, 64);
    const uint32_t hi = (uint32_t)__shfl((int)word, 2 * g + 1, 64);  // 0 past nwords
    const unsigned long long m = ((unsigned long long)hi << 32) | lo;
    const int at = pos + __popcll(m & ((1ull << lane) - 1ull));
    if ((m >> lane) & 1ull && at < end) col_idx[at] = 64 * g + lane;
    pos += __popcll(m);
  }
}

// Local + TopK (VMoBA review: the training-free selection, referee report major comment 2): row
// (b, h, I) keeps the local kv blocks of I (those holding one of its tokens, from the plan) and
// then, k times, the best remaining block by (score desc, index asc): one wavefront per row, a
// 64-bit wavefront max of (score bits, ~index) per round. Rows of at most 64 * kVpl blocks.
template <int kVpl>
__global__ __launch_bounds__(256) void mark_local_topk_kernel(
    const float* __restrict__ S, int64_t rows, int nq, int nkv, int nwords, int k,
    const int32_t* __restrict__ local_ptr, const int32_t* __restrict__ local_idx,
    uint32_t* __restrict__ bitmap, int32_t* __restrict__ base_counts) {
  static_assert(kVpl <= 32, "one mask bit per value");
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int I = (int)(r % nq);
  const float* row = S + r * nkv;
  uint32_t key[kVpl];
#pragma unroll
  for (int i = 0; i < kVpl; ++i) key[i] = lane + 64 * i < nkv ? sel_key(row[lane + 64 * i]) : 0u;
  uint32_t lmask = 0u, pmask = 0u;  // bit i: value i of this lane is local / picked
  for (int e = local_ptr[I]; e < local_ptr[I + 1]; ++e) {
    const int J = local_idx[e];
    if ((J & 63) == lane) lmask |= 1u << (J >> 6);
  }
  for (int round = 0; round < k; ++round) {
    unsigned long long best = 0ull;  // (key << 32) | ~J; 0 = nothing left in this lane
#pragma unroll
    for (int i = 0; i < kVpl; ++i) {
      const int J = lane + 64 * i;
      if (J < nkv && !(((lmask | pmask) >> i) & 1u)) {
        const unsigned long long c = ((unsigned long long)key[i] << 32) | (uint32_t)~J;
        best = c > best ? c : best;
      }
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      const unsigned long long o = shfl_xor_u64(best, d);
      best = o > best ? o : best;
    }
    if (best == 0ull) break;  // every block is taken
    const int J = (int)~(uint32_t)best;
    if ((J & 63) == lane) pmask |= 1u << (J >> 6);
  }
  bool sel[kVpl];
  int count = 0;
#pragma unroll
  for (int i = 0; i < kVpl; ++i) {
    sel[i] = lane + 64 * i < nkv && (((lmask | pmask) >> i) & 1u);
    count += __popcll(__ballot(sel[i]));
  }
  write_row_bits(sel, nwords, bitmap + r * nwords);
  if (lane == 0) base_counts[r] = count;
}

// Order-preserving key of a float (for every sign): larger gates give larger keys.
__device__ __forceinline__ uint32_t gate_key(float g) {
  const uint32_t b = __float_as_uint(g);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Kbar split into two bf16 terms, hi = bf16(Kbar) and lo = bf16(Kbar - hi), so that the gates
// can run on the bf16 matrix cores: hi + lo carries Kbar to 2^-17 relative (Q is bf16 already).
__global__ __launch_bounds__(256) void kbar_split_kernel(const float* __restrict__ Kbar,
                                                         int64_t n, uint16_t* __restrict__ hi,
                                                         uint16_t* __restrict__ lo) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float x = Kbar[i];
  const uint32_t h2 = pack_bf16x2(x, 0.f);
  const float xh = bf16_lo(h2);
  hi[i] = (uint16_t)(h2 & 0xffffu);
  lo[i] = (uint16_t)(pack_bf16x2(x - xh, 0.f) & 0xffffu);
}

// Per-token gates and their top-k in one pass (no gate matrix in memory). A workgroup owns 128
// tokens of one head (frame-major n0 .. n0 + 128), a wavefront 32 of them. Per 32-block tile the
// workgroup stages the blocks' hi and lo rows in LDS; each wavefront forms G^T = Kbar Q^T for its
// tokens with 16 bf16 MFMAs (Kbar's two terms as A, Q as B), so each lane holds 16 gates of one
// token (lanes l and l + 32 different blocks of the same token) and keeps that token's best k
// (key, ~J) pairs in registers, sorted: a candidate enters only above the current k-th. One
// instantiation per k, so the list has exactly k slots. The two halves' lists are merged at the
// end; the own block is never a candidate.
constexpr int kGateTile = 32;
constexpr int kGateQueueK = 4;  // from this k on, candidates go through a per-lane queue
template <int K>
__global__ __launch_bounds__(256) void tok_gate_topk_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ Khi,
    const uint16_t* __restrict__ Klo, const float* __restrict__ scale, int H, int N, int nkv,
    int nslots, const int32_t* __restrict__ kv_of, int32_t* __restrict__ sel) {
  constexpr int D = 128;
  // [stage][hi/lo]; rows padded by 16 bytes so that the 32 rows an operand read touches start
  // in different banks
  constexpr int R = D + 8;
  __shared__ __attribute__((aligned(16))) uint16_t kt[2][2][kGateTile * R];
  // per-lane candidate queue of the current tile: [wave][tile position][lane]
  __shared__ uint32_t gq[K >= kGateQueueK ? 4 * 16 * 64 : 1];
  const int bh = blockIdx.y, n0 = blockIdx.x * 128;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, l32 = lane & 31, hl = lane >> 5;
  const float sig = scale[bh % H];
  const int n = n0 + 32 * wave + l32;
  const bool valid = n < N;
  const int own = valid ? kv_of[n] : -1;
  bf16x8_t qf[8];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(Q + ((size_t)bh * N + min(n, N - 1)) * D +
                                                     8 * hl);
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) qf[kc] = __builtin_bit_cast(bf16x8_t, qp[2 * kc]);
  }
  const uint16_t* kh = Khi + (size_t)bh * nkv * D;
  const uint16_t* kl = Klo + (size_t)bh * nkv * D;
  // tile `tile` (rows J0 .. J0 + 32, clamped at nkv - 1) is 2 x 8 KB: 64 B per thread, loaded
  // into registers one tile ahead and written to LDS after the current tile's work
  // thread t moves 16-byte units t and t + 256: rows t / 16 and t / 16 + 16, unit t % 16
  uint4 ph0, pl0, ph1, pl1;
  const int off0 = (t >> 4) * R + 8 * (t & 15), off1 = off0 + 16 * R;
  auto load = [&](int tile) {
    const int r0 = tile * kGateTile + (t >> 4);
    const size_t s0 = (size_t)min(r0, nkv - 1) * D + 8 * (t & 15);
    const size_t s1 = (size_t)min(r0 + 16, nkv - 1) * D + 8 * (t & 15);
    ph0 = *reinterpret_cast<const uint4*>(kh + s0);
    pl0 = *reinterpret_cast<const uint4*>(kl + s0);
    ph1 = *reinterpret_cast<const uint4*>(kh + s1);
    pl1 = *reinterpret_cast<const uint4*>(kl + s1);
  };
  auto store = [&](int st) {
    *reinterpret_cast<uint4*>(&kt[st][0][off0]) = ph0;
    *reinterpret_cast<uint4*>(&kt[st][1][off0]) = pl0;
    *reinterpret_cast<uint4*>(&kt[st][0][off1]) = ph1;
    *reinterpret_cast<uint4*>(&kt[st][1][off1]) = pl1;
  };
  unsigned long long top[K];  // best first; 0 = empty; top[K - 1] is the k-th best so far
#pragma unroll
  for (int s = 0; s < K; ++s) top[s] = 0ull;
  // sorted insertion (the last entry falls off); every index static
  auto insert = [&](unsigned long long c) {
#pragma unroll
    for (int s = 0; s < K; ++s) {
      const bool in = c > top[s];
      const unsigned long long x = top[s];
      top[s] = in ? c : x;
      c = in ? x : c;
    }
  };
  // The walk over the block tiles starts at the tile holding the own block of the workgroup's
  // middle token and wraps around: blocks near a token tend to score high, so the threshold
  // rises early and later candidates mostly skip the insertion. The top k by key (score, then
  // lower index) do not depend on the order the candidates arrive in.
  const int ntiles = (nkv + kGateTile - 1) / kGateTile;
  const int tile0 = kv_of[min(n0 + 64, N - 1)] / kGateTile;
  auto tile_at = [&](int it) { return tile0 + it < ntiles ? tile0 + it : tile0 + it - ntiles; };
  load(tile_at(0));
  store(0);
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int st = it & 1, tile = tile_at(it);
    if (it + 1 < ntiles) load(tile_at(it + 1));
    f32x16_t acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
    // A operand: block row l32 of the tile, d = 16 kc + 8 hl .. + 8
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      const bf16x8_t ah =
          *reinterpret_cast<const bf16x8_t*>(&kt[st][0][l32 * R + 16 * kc + 8 * hl]);
      const bf16x8_t al =
          *reinterpret_cast<const bf16x8_t*>(&kt[st][1][l32 * R + 16 * kc + 8 * hl]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, qf[kc], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, qf[kc], acc, 0, 0, 0);
    }
    // lane holds token column l32 and block rows 8 (e / 4) + 4 hl + e % 4 of the tile
    const int J0 = tile * kGateTile;
    if constexpr (K < kGateQueueK) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int J = J0 + 8 * (e >> 2) + 4 * hl + (e & 3);
        const unsigned long long c0 =
            ((unsigned long long)gate_key(sig * acc[e]) << 32) | (uint32_t)~J;
        const bool in = J < nkv && J != own && c0 > top[K - 1];
        if (__ballot(in) != 0ull) {  // skipped by the whole wavefront when no lane inserts
          if (in) insert(c0);
        }
      }
    } else {
      // Candidates above the k-th best as the tile starts are queued (their gate bits, in
      // LDS) and inserted one per lane per round: the wavefront runs as many insertion rounds
      // as its longest queue, not one per tile position some lane inserts at.
      uint32_t pend = 0;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int J = J0 + 8 * (e >> 2) + 4 * hl + (e & 3);
        const uint32_t g = gate_key(sig * acc[e]);
        const unsigned long long c0 = ((unsigned long long)g << 32) | (uint32_t)~J;
        if (J < nkv && J != own && c0 > top[K - 1]) {
          gq[(wave * 16 + e) * 64 + lane] = g;
          pend |= 1u << e;
        }
      }
      while (__ballot(pend != 0u) != 0ull) {
        if (pend != 0u) {
          const int e = __builtin_ctz(pend);
          pend &= pend - 1u;
          const int J = J0 + 8 * (e >> 2) + 4 * hl + (e & 3);
          const unsigned long long c =
              ((unsigned long long)gq[(wave * 16 + e) * 64 + lane] << 32) | (uint32_t)~J;
          if (c > top[K - 1]) insert(c);  // the k-th best may have risen since it was queued
        }
      }
    }
    if (it + 1 < ntiles) store(st ^ 1);  // the stage step it - 1 used, free since its barrier
    __syncthreads();  // the next tile staged; every wavefront done with this one
  }
  // merge the other half's list (lanes l and l ^ 32 hold the same token)
  unsigned long long other[K];
#pragma unroll
  for (int s = 0; s < K; ++s) other[s] = shfl_xor_u64(top[s], 32);
#pragma unroll
  for (int s = 0; s < K; ++s)
    if (other[s] > top[K - 1]) insert(other[s]);
  if (!valid || hl) return;
  // own block plus the k picks, ascending: each value's rank is the count of smaller ones
  int32_t* out = sel + ((size_t)bh * N + n) * nslots;
  int jv[K];
#pragma unroll
  for (int s = 0; s < K; ++s) jv[s] = (int)~(uint32_t)top[s];
  int r_own = 0;
#pragma unroll
  for (int s = 0; s < K; ++s) r_own += jv[s] < own;
  out[r_own] = own;
#pragma unroll
  for (int s = 0; s < K; ++s) {
    int r = jv[s] > own;
#pragma unroll
    for (int u = 0; u < K; ++u) r += jv[u] < jv[s];
    out[r] = jv[s];
  }
}

// k = 0: each token's list is its own block alone.
__global__ __launch_bounds__(256) void tok_own_kernel(const int32_t* __restrict__ kv_of, int N,
                                                      int64_t n_tokens,
                                                      int32_t* __restrict__ sel) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n_tokens) sel[i] = kv_of[i % N];
}

using GateLaunch = void (*)(dim3, hipStream_t, const uint16_t*, const uint16_t*, const uint16_t*,
                            const float*, int, int, int, int, const int32_t*, int32_t*);
template <int K>
void gate_launch(dim3 grid, hipStream_t s, const uint16_t* Q, const uint16_t* khi,
                 const uint16_t* klo, const float* scale, int H, int N, int nkv, int nslots,
                 const int32_t* kv_of, int32_t* sel) {
  tok_gate_topk_kernel<K><<<grid, 256, 0, s>>>(Q, khi, klo, scale, H, N, nkv, nslots, kv_of, sel);
}
// entry k - 1 launches the instantiation for k
template <int... Ks>
constexpr std::array<GateLaunch, sizeof...(Ks)> gate_table(std::integer_sequence<int, Ks...>) {
  return {{&gate_launch<Ks + 1>...}};
}

// Union of the token lists of each query block (b, h, I), one wavefront per row: an LDS bitmap
// of nkv bits per wavefront (at most 2048 blocks), then the row's bitmap words and count.
__global__ __launch_bounds__(256) void tok_union_kernel(const int32_t* __restrict__ sel,
                                                        int nslots, int H, int N, int nq,
                                                        int nwords,
                                                        const int32_t* __restrict__ qstart,
                                                        const int32_t* __restrict__ qperm,
                                                        int64_t rows,
                                                        uint32_t* __restrict__ bitmap,
                                                        int32_t* __restrict__ counts) {
  __shared__ uint32_t words[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r = (int64_t)blockIdx.x * 4 + wave;
  if (r >= rows) return;
  const int I = (int)(r % nq);
  const int64_t bh = r / nq;
  words[wave][lane] = 0u;
  __builtin_amdgcn_wave_barrier();
  const int t0 = qstart[I], n_entries = (qstart[I + 1] - t0) * nslots;
  for (int e = lane; e < n_entries; e += 64) {
    const int tok = qperm[t0 + e / nslots];
    const int J = sel[((size_t)bh * N + tok) * nslots + e % nslots];
    atomicOr(&words[wave][J >> 5], 1u << (J & 31));
  }
  __builtin_amdgcn_wave_barrier();
  const uint32_t w = lane < nwords ? words[wave][lane] : 0u;
  if (lane < nwords) bitmap[r * nwords + lane] = w;
  int c = __popc(w);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) c += __shfl_xor(c, d, 64);
  if (lane == 0) counts[r] = c;
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


// ---------------------------------------------------- entropy-routed competition domains
//
// EG-Sparse abstract (readsearch page "Competition Domains Matter: Selective Head Globalization
// for Training-Free Sparse Attention in Video Diffusion Transformers"): heads whose block scores
// have low entropy compete in a pool shared by their group of heads, the others keep per-row
// selection, and only the scores already computed are used. Here a head's entropy is the
// |I|-weighted mean of its rows' Shannon entropies over ln nkv; a group is a run of group_size
// consecutive heads; a group's pool holds every (h, I, J) of its pooled heads, weighted
// S * |I| / (N m) so that it sums to 1, with the prefix rule, tie order and exact sums of the
// other pools. A pool can hold millions of candidates, so its radix select is spread over many
// workgroups: per 8-bit digit, workgroup histograms in LDS are added into one global histogram
// per group, and one wavefront per group picks the digit bin from it.

constexpr int kEgHistChunk = 4096;  // pool candidates per histogram workgroup (16 per thread)

struct EgGroup {
  uint32_t prefix, mask;
  unsigned long long above_sum;
  uint32_t above_cnt, eq_cnt;
  int32_t m;       // pooled heads of the group
  int32_t done;    // no further digit pass
  int32_t all;     // every candidate is kept
  uint32_t keep;   // members of the boundary class kept, lowest pool indices first
  int32_t eq_all;  // keep == eq_cnt
  int32_t pad[5];
};
struct EgHist {
  unsigned int cnt[256];
  unsigned long long sum[256];
};
static_assert(sizeof(EgGroup) == kEgGroupBytes, "group state size");
static_assert(sizeof(EgHist) == kEgHistBytes, "group histogram size");

// Pool weight of one score: S * |I| / (N m), the same float on every pass.
__device__ __forceinline__ float eg_weight(float s, int qsize, int N, int m) {
  return s * (float)((double)qsize / ((double)N * (double)m));
}

__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

// Shannon entropy of every score row in fp64, one wavefront per row (a fixed butterfly sum).
__global__ __launch_bounds__(256) void eg_row_entropy_kernel(const float* __restrict__ S,
                                                             int64_t rows, int nkv,
                                                             double* __restrict__ row_ent) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const float* row = S + r * nkv;
  double h = 0.0;
  for (int J = lane; J < nkv; J += 64) {
    const double x = (double)row[J];
    if (x > 0.0) h -= x * log(x);
  }
  h = wave_sum_f64(h);
  if (lane == 0) row_ent[r] = h;
}

// One wavefront per head (b, h): the |I|-weighted mean of its rows' entropies over ln nkv (lane
// l sums rows l, l + 64, ... in order, then a fixed butterfly), and the routing flag.
__global__ __launch_bounds__(64) void eg_head_entropy_kernel(const double* __restrict__ row_ent,
                                                             const int32_t* __restrict__ qstart,
                                                             int nq, int nkv, int N,
                                                             double theta,
                                                             int32_t* __restrict__ route,
                                                             float* __restrict__ ent_out,
                                                             int32_t* __restrict__ pooled_out) {
  const int bh = blockIdx.x, lane = threadIdx.x;
  double acc = 0.0;
  for (int I = lane; I < nq; I += 64)
    acc += (double)(qstart[I + 1] - qstart[I]) * row_ent[(int64_t)bh * nq + I];
  acc = wave_sum_f64(acc);
  if (lane == 0) {
    const double e = nkv > 1 ? acc / ((double)N * log((double)nkv)) : 0.0;
    const int pooled = e < theta ? 1 : 0;
    route[bh] = pooled;
    if (ent_out) ent_out[bh] = (float)e;
    if (pooled_out) pooled_out[bh] = pooled;
  }
}

// One wavefront per group (b, g): its pooled heads in head order, the radix state, a cleared
// histogram.
__global__ __launch_bounds__(64) void eg_setup_kernel(const int32_t* __restrict__ route, int H,
                                                      int G, int ngh, int keep_all,
                                                      int32_t* __restrict__ members,
                                                      EgGroup* __restrict__ groups,
                                                      EgHist* __restrict__ hist) {
  const int gi = blockIdx.x, b = gi / ngh, g = gi % ngh, lane = threadIdx.x;
  if (lane == 0) {
    int m = 0;
    const int h1 = min(H, (g + 1) * G);
    for (int h = g * G; h < h1; ++h)
      if (route[b * H + h]) members[b * H + g * G + m++] = h;
    EgGroup st{};
    st.m = m;
    st.done = (m == 0 || keep_all) ? 1 : 0;
    st.all = keep_all;
    groups[gi] = st;
  }
  for (int i = lane; i < 256; i += 64) {
    hist[gi].cnt[i] = 0u;
    hist[gi].sum[i] = 0ull;
  }
}

// Candidate j of group gi's pool: pooled head k = j / (nq nkv), then (I, J). Returns its weight
// and its score row (b * H + h) * nq + I.
__device__ __forceinline__ float eg_candidate(const float* __restrict__ S,
                                              const int32_t* __restrict__ qstart,
                                              const int32_t* __restrict__ members, int b, int g,
                                              int H, int G, int nq, int nkv, int N, int m, int j,
                                              int64_t& row, int& J) {
  const int per = nq * nkv;
  const int k = j / per, rem = j - k * per;
  const int I = rem / nkv;
  J = rem - I * nkv;
  const int h = members[b * H + g * G + k];
  row = ((int64_t)b * H + h) * nq + I;
  return eg_weight(S[row * nkv + J], qstart[I + 1] - qstart[I], N, m);
}

// Digit pass: the candidates still matching the radix prefix add their count and 2^-56 sum to
// their digit's bin, through an LDS histogram per workgroup.
__global__ __launch_bounds__(256) void eg_hist_kernel(const float* __restrict__ S,
                                                      const int32_t* __restrict__ qstart, int H,
                                                      int G, int ngh, int nq, int nkv, int N,
                                                      int pass,
                                                      const int32_t* __restrict__ members,
                                                      const EgGroup* __restrict__ groups,
                                                      EgHist* __restrict__ hist) {
  __shared__ unsigned int scnt[256];
  __shared__ unsigned long long ssum[256];
  const int gi = blockIdx.y;
  const EgGroup st = groups[gi];
  if (st.done) return;
  const int pool_n = st.m * nq * nkv;
  const int base = blockIdx.x * kEgHistChunk;
  if (base >= pool_n) return;
  const int t = threadIdx.x;
  scnt[t] = 0u;
  ssum[t] = 0ull;
  __syncthreads();
  const int b = gi / ngh, g = gi % ngh, shift = 24 - 8 * pass;
  // Candidate j = base + t + 256 u (neighbouring lanes read neighbouring scores: coalesced),
  // its (pooled head k, query block I, kv block J) advanced from one u to the next without a
  // division per candidate. The early passes put most candidates into one or two bins, so runs
  // of equal bins are summed in registers and added to the LDS histogram once per run.
  constexpr int kPer = kEgHistChunk / 256;
  const int per = nq * nkv, dq = 256 / nkv, dJ = 256 - dq * nkv;
  int j = base + t;
  int k = j / per, I = (j - k * per) / nkv, J = j - k * per - I * nkv;
  uint32_t run_bin = 256u, run_cnt = 0u;
  unsigned long long run_sum = 0ull;
  for (int u = 0; u < kPer; ++u, j += 256) {
    if (j >= pool_n) break;
    if (u) {
      J += dJ;
      I += dq;
      if (J >= nkv) {
        J -= nkv;
        ++I;
      }
      if (I >= nq) {
        k += I / nq;
        I %= nq;
      }
    }
    const int64_t row = ((int64_t)b * H + members[b * H + g * G + k]) * nq + I;
    const float v = eg_weight(S[row * nkv + J], qstart[I + 1] - qstart[I], N, st.m);
    const uint32_t key = sel_key(v);
    if ((key & st.mask) == st.prefix) {
      const uint32_t bin = (key >> shift) & 255u;
      if (bin != run_bin) {
        if (run_cnt) {
          atomicAdd(&scnt[run_bin], run_cnt);
          atomicAdd(&ssum[run_bin], run_sum);
        }
        run_bin = bin;
        run_cnt = 0u;
        run_sum = 0ull;
      }
      ++run_cnt;
      run_sum += sel_fix(v);
    }
  }
  if (run_cnt) {
    atomicAdd(&scnt[run_bin], run_cnt);
    atomicAdd(&ssum[run_bin], run_sum);
  }
  __syncthreads();
  if (scnt[t]) {
    atomicAdd(&hist[gi].cnt[t], scnt[t]);
    atomicAdd(&hist[gi].sum[t], ssum[t]);
  }
}

// One wavefront per group: the bin (in descending digit order) where the cumulative sum first
// reaches the target narrows the prefix; none means the pool never reaches it (keep all). The
// histogram is cleared for the next digit.
__global__ __launch_bounds__(64) void eg_pick_kernel(int pass, unsigned long long target,
                                                     EgGroup* __restrict__ groups,
                                                     EgHist* __restrict__ hist) {
  const int gi = blockIdx.x, lane = threadIdx.x;
  EgGroup st = groups[gi];
  if (st.done) return;
  EgHist& hs = hist[gi];
  unsigned long long bsum[4];
  unsigned int bcnt[4];
  unsigned long long lsum = 0;
  unsigned int lcnt = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int bin = 255 - 4 * lane - i;
    bsum[i] = hs.sum[bin];
    bcnt[i] = hs.cnt[bin];
    lsum += bsum[i];
    lcnt += bcnt[i];
  }
  const unsigned long long isum = wave_incl_scan_u64(lsum);
  const unsigned long long icnt = wave_incl_scan_u64(lcnt);
  unsigned long long asum = st.above_sum + (isum - lsum);
  unsigned long long acnt = st.above_cnt + (icnt - lcnt);
  int found = -1;
  unsigned long long fsum = 0, fcnt = 0;
  unsigned int feq = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (found < 0 && asum < target && asum + bsum[i] >= target) {
      found = 255 - 4 * lane - i;
      fsum = asum;
      fcnt = acnt;
      feq = bcnt[i];
    }
    asum += bsum[i];
    acnt += bcnt[i];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int bin = 255 - 4 * lane - i;
    hs.sum[bin] = 0ull;
    hs.cnt[bin] = 0u;
  }
  const bool any = __ballot(found >= 0) != 0ull;
  if (!any) {
    if (lane == 0) {
      st.all = 1;
      st.done = 1;
      groups[gi] = st;
    }
    return;
  }
  if (found >= 0) {  // exactly one lane: the cumulative sums are monotone
    const int shift = 24 - 8 * pass;
    st.prefix |= (uint32_t)found << shift;
    st.mask |= 255u << shift;
    st.above_sum = fsum;
    st.above_cnt = (uint32_t)fcnt;
    st.eq_cnt = feq;
    if (feq == 1u || pass == 3) {
      st.done = 1;
      uint32_t keep;
      if (feq == 1u) {
        keep = 1u;
      } else {
        const unsigned long long v = sel_fix(__uint_as_float(st.prefix));
        keep = (uint32_t)((target - st.above_sum + v - 1) / v);
      }
      if (keep > feq) keep = feq;
      st.keep = keep;
      st.eq_all = keep == feq ? 1 : 0;
    }
    groups[gi] = st;
  }
}

__device__ __forceinline__ bool eg_selected(const EgGroup& st, uint32_t key) {
  if (st.all) return true;
  const uint32_t k = key & st.mask;
  return k > st.prefix || (k == st.prefix && st.eq_all);
}

// Bitmap words and counts of the pooled heads' rows (overwriting their per-row selection), and
// the number of boundary-class candidates in each chunk of kEgRowChunk pool rows.
__global__ __launch_bounds__(256) void eg_mark_kernel(const float* __restrict__ S,
                                                      const int32_t* __restrict__ qstart, int H,
                                                      int G, int ngh, int nq, int nkv, int N,
                                                      int nwords, int nrchunk,
                                                      const int32_t* __restrict__ members,
                                                      const EgGroup* __restrict__ groups,
                                                      uint32_t* __restrict__ bitmap,
                                                      int32_t* __restrict__ base_counts,
                                                      int32_t* __restrict__ bnd) {
  __shared__ int sbnd[4];
  const int gi = blockIdx.y;
  const EgGroup st = groups[gi];
  if (st.m == 0) return;
  const int prow = st.m * nq, R0 = blockIdx.x * kEgRowChunk;
  if (R0 >= prow) return;
  const int nr = min(kEgRowChunk, prow - R0), t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int b = gi / ngh, g = gi % ngh;
  // wavefront w takes pool rows w, w + 4, ...: lane l tests blocks 64 i + l (coalesced), a
  // ballot gives two bitmap words per 64 blocks and the row's count
  int my_bnd = 0;
  for (int rr = wave; rr < nr; rr += 4) {
    const int R = R0 + rr, k = R / nq, I = R - k * nq;
    const int64_t row = ((int64_t)b * H + members[b * H + g * G + k]) * nq + I;
    const float* srow = S + row * nkv;
    const int qsize = qstart[I + 1] - qstart[I];
    int cnt = 0;
    for (int J0 = 0; J0 < nkv; J0 += 64) {
      const int J = J0 + lane;
      bool sel = false, bd = false;
      if (J < nkv) {
        const uint32_t key = sel_key(eg_weight(srow[J], qsize, N, st.m));
        sel = eg_selected(st, key);
        bd = !sel && !st.all && (key & st.mask) == st.prefix;
      }
      const unsigned long long bal = __ballot(sel);
      cnt += __popcll(bal);
      my_bnd += __popcll(__ballot(bd));
      const int w = (J0 >> 5) + lane;
      if (lane < 2 && w < nwords) bitmap[row * nwords + w] = (uint32_t)(bal >> (32 * lane));
    }
    if (lane == 0) base_counts[row] = cnt;
  }
  if (lane == 0) sbnd[wave] = my_bnd;
  __syncthreads();
  if (t == 0) bnd[(int64_t)gi * nrchunk + blockIdx.x] = (sbnd[0] + sbnd[1]) + (sbnd[2] + sbnd[3]);
}

// When only part of the boundary class is kept: its members in pool index order, chunk by chunk
// (the counts of the earlier chunks give each chunk's starting rank), the first `keep` of them.
__global__ __launch_bounds__(64) void eg_boundary_kernel(const float* __restrict__ S,
                                                         const int32_t* __restrict__ qstart,
                                                         int H, int G, int ngh, int nq, int nkv,
                                                         int N, int nwords, int nrchunk,
                                                         const int32_t* __restrict__ members,
                                                         const EgGroup* __restrict__ groups,
                                                         const int32_t* __restrict__ bnd,
                                                         uint32_t* __restrict__ bitmap,
                                                         int32_t* __restrict__ base_counts) {
  const int gi = blockIdx.y, c = blockIdx.x, lane = threadIdx.x;
  const EgGroup st = groups[gi];
  if (st.m == 0 || st.all || st.eq_all) return;
  const int prow = st.m * nq, R0 = c * kEgRowChunk;
  if (R0 >= prow) return;
  const int32_t* gb = bnd + (int64_t)gi * nrchunk;
  if (gb[c] == 0) return;
  int before = 0;
  for (int i = lane; i < c; i += 64) before += gb[i];
  before = wave_sum_i32(before);
  if ((uint32_t)before >= st.keep) return;
  const int b = gi / ngh, g = gi % ngh;
  const int j0 = R0 * nkv, n = min(kEgRowChunk, prow - R0) * nkv;
  uint32_t taken = (uint32_t)before;
  for (int base = 0; base < n && taken < st.keep; base += 64) {
    const int jj = base + lane;
    bool eq = false;
    int64_t row = 0;
    int J = 0;
    if (jj < n) {
      const float v =
          eg_candidate(S, qstart, members, b, g, H, G, nq, nkv, N, st.m, j0 + jj, row, J);
      eq = (sel_key(v) & st.mask) == st.prefix;
    }
    const unsigned long long bal = __ballot(eq);
    const uint32_t rank = taken + __popcll(bal & ((1ull << lane) - 1ull));
    if (eq && rank < st.keep) {
      atomicOr(&bitmap[row * nwords + J / 32], 1u << (J % 32));
      atomicAdd(&base_counts[row], 1);
    }
    taken += __popcll(bal);
  }
}

}  // namespace

hipError_t launch_scan(const int32_t* base_counts, const int32_t* head_k, bool use_min_k,
                       int64_t rows, int nq, int32_t* row_ptr, int32_t* counts_out,
                       int32_t* partial, hipStream_t s) {
  const unsigned nb = (unsigned)((rows + 1023) / 1024);
  scan_local_kernel<<<nb, 1024, 0, s>>>(base_counts, head_k, use_min_k, rows, nq, row_ptr,
                                        counts_out, partial);
  scan_add_kernel<<<nb, 1024, 0, s>>>(rows, partial, row_ptr);
  return hipGetLastError();
}

hipError_t launch_kbar_split(const float* Kbar, int64_t n, uint16_t* hi, uint16_t* lo,
                             hipStream_t s) {
  kbar_split_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(Kbar, n, hi, lo);
  return hipGetLastError();
}

hipError_t launch_emit(const uint32_t* bitmap, int nwords, int64_t rows, const int32_t* row_ptr,
                       int32_t* col_idx, hipStream_t s) {
  if (nwords <= 64)
    emit_wave_kernel<<<(unsigned)((rows + 3) / 4), 256, 0, s>>>(bitmap, nwords, rows, row_ptr,
                                                                col_idx);
  else
    emit_kernel<<<(unsigned)rows, 256, 0, s>>>(bitmap, nwords, row_ptr, col_idx);
  return hipGetLastError();
}

// ROW-pool marks of every row (bitmap and counts), except the rows of heads flagged in
// skip_head (nullable).
static hipError_t mark_rows(const bsa_plan& p, const float* S, unsigned long long target,
                            bool all, const SelectWs& L, uint32_t* bitmap, int32_t* base_counts,
                            const int32_t* skip_head, hipStream_t s) {
  const int64_t rows = (int64_t)p.prob.B * p.prob.H * p.nq;
  const unsigned wgrid = (unsigned)((rows + 3) / 4);
  if (p.nkv <= kWaveRowMax)
    with_sel_vpl(p.nkv, [&](auto vpl) {
      mark_row_wave_kernel<decltype(vpl)::value><<<wgrid, 256, 0, s>>>(
          S, rows, p.nkv, L.nwords, target, all, bitmap, base_counts, p.nq, skip_head);
    });
  else
    mark_row_kernel<<<(unsigned)rows, 256, 0, s>>>(S, p.nkv, L.nwords, target, all, bitmap,
                                                   base_counts, p.nq, skip_head);
  return hipGetLastError();
}

// row_ptr from the final counts, then the column lists from the bitmap.
static hipError_t scan_emit(const bsa_plan& p, const SelectWs& L, const uint32_t* bitmap,
                            const int32_t* base_counts, const int32_t* head_k_ws, bool use_min_k,
                            int32_t* row_ptr, int32_t* col_idx, int32_t* counts,
                            int32_t* partial, hipStream_t s) {
  const int64_t rows = (int64_t)p.prob.B * p.prob.H * p.nq;
  hipError_t e = launch_scan(base_counts, head_k_ws, use_min_k, rows, p.nq, row_ptr, counts,
                             partial, s);
  if (e != hipSuccess) return e;
  if (L.nwords <= 64)
    emit_wave_kernel<<<(unsigned)((rows + 3) / 4), 256, 0, s>>>(bitmap, L.nwords, rows, row_ptr,
                                                                col_idx);
  else
    emit_kernel<<<(unsigned)rows, 256, 0, s>>>(bitmap, L.nwords, row_ptr, col_idx);
  return hipGetLastError();
}

static hipError_t select_finish(const bsa_plan& p, const float* S, const bsa_select_params& prm,
                                void* ws, int32_t* row_ptr, int32_t* col_idx, int32_t* counts,
                                int32_t* head_k, hipStream_t s);

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
  hipError_t e;
  if (prm.pool == BSA_POOL_ROW) {
    e = mark_rows(p, S, target, all, L, bitmap, base_counts, nullptr, s);
  } else if (prm.pool == BSA_POOL_LOCAL_TOPK) {
    if (p.nkv <= 1024)
      mark_local_topk_kernel<16><<<wgrid, 256, 0, s>>>(S, rows, p.nq, p.nkv, L.nwords,
                                                       prm.fixed_k, p.local_ptr, p.local_idx,
                                                       bitmap, base_counts);
    else
      mark_local_topk_kernel<32><<<wgrid, 256, 0, s>>>(S, rows, p.nq, p.nkv, L.nwords,
                                                       prm.fixed_k, p.local_ptr, p.local_idx,
                                                       bitmap, base_counts);
    e = hipGetLastError();
  } else {
    mark_head_kernel<<<BH, 1024, 0, s>>>(S, p.nq, p.nkv, L.nwords, target, all, bitmap,
                                         base_counts);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  return select_finish(p, S, prm, ws, row_ptr, col_idx, counts, head_k, s);
}

// After the marking pass: the per-head minimum and the top-up of the rows below it (ROW pool),
// then row_ptr and the column lists.
static hipError_t select_finish(const bsa_plan& p, const float* S, const bsa_select_params& prm,
                                void* ws, int32_t* row_ptr, int32_t* col_idx, int32_t* counts,
                                int32_t* head_k, hipStream_t s) {
  const SelectWs L = select_ws_layout(p);
  char* base = static_cast<char*>(ws);
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(base + L.bitmap);
  int32_t* base_counts = reinterpret_cast<int32_t*>(base + L.base_counts);
  int32_t* head_k_ws = reinterpret_cast<int32_t*>(base + L.head_k);
  const int BH = p.prob.B * p.prob.H;
  const int64_t rows = (int64_t)BH * p.nq;
  const bool wave_rows = p.nkv <= kWaveRowMax;
  const unsigned wgrid = (unsigned)((rows + 3) / 4);
  hipError_t e;
  const bool use_min_k = prm.min_k_mode != BSA_MINK_NONE;
  if (use_min_k || head_k) {
    head_k_kernel<<<BH, 256, 0, s>>>(base_counts, p.qstart, p.nq, p.nkv, prm.min_k_mode,
                                     prm.fixed_k, head_k_ws, head_k);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (use_min_k && wave_rows) {  // row_ptr from the final counts, then top-up and emission
    e = launch_scan(base_counts, head_k_ws, true, rows, p.nq, row_ptr, counts,
                    reinterpret_cast<int32_t*>(base + L.partial), s);
    if (e != hipSuccess) return e;
    with_sel_vpl(p.nkv, [&](auto vpl) {
      topup_emit_wave_kernel<decltype(vpl)::value><<<wgrid, 256, 0, s>>>(
          S, rows, p.nq, p.nkv, L.nwords, base_counts, head_k_ws, bitmap, row_ptr, col_idx);
    });
    return hipGetLastError();
  } else if (use_min_k) {
    topup_kernel<<<(unsigned)rows, 256, 0, s>>>(S, p.nq, p.nkv, L.nwords, base_counts,
                                                head_k_ws, bitmap);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return scan_emit(p, L, bitmap, base_counts, head_k_ws, use_min_k, row_ptr, col_idx, counts,
                   reinterpret_cast<int32_t*>(base + L.partial), s);
}

hipError_t launch_score_select_csr(const bsa_plan& p, const float* Qbar, const float* Kbar,
                                   const bsa_select_params& prm, float* S, int32_t* row_ptr,
                                   int32_t* col_idx, int32_t* counts, int32_t* head_k, void* ws,
                                   hipStream_t s) {
  const SelectWs L = select_ws_layout(p);
  char* base = static_cast<char*>(ws);
  const int64_t rows = (int64_t)p.prob.B * p.prob.H * p.nq;
  if (rows == 0) return hipSuccess;
  const bool all = prm.p >= 1.0;
  const unsigned long long target = all ? 0ull : (unsigned long long)ceil(prm.p * kFix);
  hipError_t e = launch_score_select(p, Qbar, Kbar, S, target, all, L.nwords,
                                     reinterpret_cast<uint32_t*>(base + L.bitmap),
                                     reinterpret_cast<int32_t*>(base + L.base_counts), s);
  if (e != hipSuccess) return e;
  return select_finish(p, S, prm, ws, row_ptr, col_idx, counts, head_k, s);
}

hipError_t launch_select_eg(const bsa_plan& p, const float* S, const bsa_eg_params& prm,
                            int32_t* row_ptr, int32_t* col_idx, int32_t* counts,
                            float* head_entropy, int32_t* head_pooled, void* ws, hipStream_t s) {
  const SelectWs L = select_ws_layout(p);
  char* base = static_cast<char*>(ws);
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(base + L.bitmap);
  int32_t* base_counts = reinterpret_cast<int32_t*>(base + L.base_counts);
  int32_t* route = reinterpret_cast<int32_t*>(base + L.eg_route);
  int32_t* members = reinterpret_cast<int32_t*>(base + L.eg_members);
  EgGroup* groups = reinterpret_cast<EgGroup*>(base + L.eg_groups);
  EgHist* hist = reinterpret_cast<EgHist*>(base + L.eg_hist);
  int32_t* bnd = reinterpret_cast<int32_t*>(base + L.eg_bnd);
  const int B = p.prob.B, H = p.prob.H, N = p.prob.N, nq = p.nq, nkv = p.nkv;
  const int G = std::min(std::max(prm.group_size, 1), H), ngh = (H + G - 1) / G;
  const int ngroups = B * ngh;
  const int64_t rows = (int64_t)B * H * nq;
  if (rows == 0) return hipSuccess;
  const bool all = prm.p >= 1.0;
  const unsigned long long target = all ? 0ull : (unsigned long long)ceil(prm.p * kFix);

  eg_row_entropy_kernel<<<(unsigned)((rows + 3) / 4), 256, 0, s>>>(
      S, rows, nkv, reinterpret_cast<double*>(base + L.eg_rowent));
  eg_head_entropy_kernel<<<B * H, 64, 0, s>>>(reinterpret_cast<const double*>(base + L.eg_rowent),
                                              p.qstart, nq, nkv, N, prm.theta, route,
                                              head_entropy, head_pooled);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = mark_rows(p, S, target, all, L, bitmap, base_counts, route, s);
  if (e != hipSuccess) return e;
  eg_setup_kernel<<<ngroups, 64, 0, s>>>(route, H, G, ngh, all ? 1 : 0, members, groups, hist);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // grids sized for a pool of all G heads; workgroups past a group's pool return at once
  const unsigned nchunk = (unsigned)(((int64_t)G * nq * nkv + kEgHistChunk - 1) / kEgHistChunk);
  for (int pass = 0; pass < 4; ++pass) {
    eg_hist_kernel<<<dim3(nchunk, ngroups), 256, 0, s>>>(S, p.qstart, H, G, ngh, nq, nkv, N, pass,
                                                         members, groups, hist);
    eg_pick_kernel<<<ngroups, 64, 0, s>>>(pass, target, groups, hist);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const unsigned nrc = (unsigned)(((int64_t)G * nq + kEgRowChunk - 1) / kEgRowChunk);
  eg_mark_kernel<<<dim3(nrc, ngroups), 256, 0, s>>>(S, p.qstart, H, G, ngh, nq, nkv, N, L.nwords,
                                                    L.eg_nrchunk, members, groups, bitmap,
                                                    base_counts, bnd);
  eg_boundary_kernel<<<dim3(nrc, ngroups), 64, 0, s>>>(S, p.qstart, H, G, ngh, nq, nkv, N,
                                                       L.nwords, L.eg_nrchunk, members, groups,
                                                       bnd, bitmap, base_counts);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return scan_emit(p, L, bitmap, base_counts, nullptr, false, row_ptr, col_idx, counts,
                   reinterpret_cast<int32_t*>(base + L.partial), s);
}

hipError_t launch_select_tokens(const bsa_plan& p, const void* Q, const float* Kbar, int k,
                                int32_t* sel, int32_t* row_ptr, int32_t* col_idx, void* ws,
                                hipStream_t s) {
  const TokWs L = tok_ws_layout(p);
  char* base = static_cast<char*>(ws);
  uint16_t* khi = reinterpret_cast<uint16_t*>(base + L.khi);
  uint16_t* klo = reinterpret_cast<uint16_t*>(base + L.klo);
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(base + L.bitmap);
  int32_t* counts = reinterpret_cast<int32_t*>(base + L.counts);
  const int BH = p.prob.B * p.prob.H, N = p.prob.N, nkv = p.nkv;
  const int kk = std::min(k, nkv - 1), nslots = 1 + kk;
  const int64_t rows = (int64_t)BH * p.nq;
  const int64_t nk = (int64_t)BH * nkv * 128;
  kbar_split_kernel<<<(unsigned)((nk + 255) / 256), 256, 0, s>>>(Kbar, nk, khi, klo);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((N + 127) / 128, BH);
  const uint16_t* q16 = static_cast<const uint16_t*>(Q);
  if (kk == 0) {
    const int64_t nt = (int64_t)BH * N;
    tok_own_kernel<<<(unsigned)((nt + 255) / 256), 256, 0, s>>>(p.kv_of, N, nt, sel);
  } else {
    static constexpr auto table = gate_table(std::make_integer_sequence<int, kMaxTokenK>());
    table[kk - 1](grid, s, q16, khi, klo, p.scale, p.prob.H, N, nkv, nslots, p.kv_of, sel);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  tok_union_kernel<<<(unsigned)((rows + 3) / 4), 256, 0, s>>>(
      sel, nslots, p.prob.H, N, p.nq, L.nwords, p.qstart, p.qperm, rows, bitmap, counts);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  e = launch_scan(counts, nullptr, false, rows, p.nq, row_ptr, nullptr,
                  reinterpret_cast<int32_t*>(base + L.partial), s);
  if (e != hipSuccess) return e;
  emit_wave_kernel<<<(unsigned)((rows + 3) / 4), 256, 0, s>>>(bitmap, L.nwords, rows, row_ptr,
                                                              col_idx);
  return hipGetLastError();
}

// Workspace of the allocation-free selection entry point: a file-scope device array (each GPU
// holds its own copy for the life of the process). Host code never uses the array's name as an
// address; it asks the runtime for the device address once per device and keeps it.
static __device__ __align__(256) unsigned char scratch[kSelectScratchBytes];

hipError_t select_scratch(void** ptr) {
  static std::mutex mu;
  static std::unordered_map<int, void*> addr;  // device -> address of its copy of `scratch`
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  auto it = addr.find(dev);
  if (it == addr.end()) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    it = addr.emplace(dev, p).first;
  }
  *ptr = it->second;
  return hipSuccess;
}
