// Per-token global threshold selection (pith.science review of VMoBA: "What carries the argument"
// -- global selection pools the scores of all queries of a head; referee report major comment 1
// -- Eq. 3 keeps the top entries of the whole query-by-block matrix and Eq. 4 the smallest count
// whose cumulative normalised similarity reaches tau, so a query may keep no block at all).
//
// Per head, the gate of every (query token i, kv block J), g = sigma_h q_i . kbar_J, is formed
// once on the bf16 matrix cores (kbar split into two bf16 terms, 2^-17 relative, fp32 sums) and
// kept in the workspace with the head's smallest and largest gate; every pass that reads a gate
// forms e = exp(g - max g) from it (the same expression everywhere, so the same bits), so no pass
// writes the exponentials back. The head's weights are e / Z with
// Z = sum e, so "the shortest prefix of the (weight desc, pair index i * nkv + J asc) order whose
// weights reach tau" is the same set as the prefix of e reaching tau * Z. The head pool (N * nkv
// candidates) runs the radix select of the other pools on e's bit pattern over many workgroups:
// exact fixed-point sums (e * 2^s, s chosen so that a head's total fits 64 bits), the first digit
// taken relative to the pool's range of keys, global per-head histograms, one wavefront per head
// picking each digit's bin. Each token's kept blocks are written as a bitmap; a query block's
// union of its tokens' bitmaps is the CSR row the attention walks.
#include <algorithm>
#include <climits>

#include "bsa_internal.h"
#include "device_common.h"
#include "row_select.h"

namespace {

// pool candidates per histogram workgroup (256 per thread): large enough that the workgroups'
// additions into a head's global histogram stay few
constexpr int kTgChunk = 65536;
constexpr int kTgRows = 32;      // token rows per marking workgroup
constexpr int kTgTile = 32;      // kv blocks per gate tile

struct TgHead {
  uint32_t gmax;        // order-preserving key of the head's largest gate
  uint32_t kmin, kmax;  // keys of the smallest and largest e
  int32_t rem;          // bits of u = key(e) - kmin still undecided
  uint32_t hi;          // candidates: (u >> rem) == hi
  int32_t done, all, eq_all;
  uint32_t keep, eq_cnt, above_cnt, shift;  // shift: the fixed-point scale 2^shift of e
  unsigned long long above_sum, target, total;
  uint32_t gmin;  // order-preserving key of the head's smallest gate
  int32_t pad;
};
static_assert(sizeof(TgHead) == kTgHeadBytes, "head state size");
struct TgHist {
  unsigned int cnt[kTgBins];
  unsigned long long sum[kTgBins];
};

__device__ __forceinline__ uint32_t tg_gate_key(float g) {
  const uint32_t b = __float_as_uint(g);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float tg_gate_from_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// e = exp(g - max g), as exp2 of the log2 e-scaled difference (v_exp_f32), ml = max g * log2 e;
// at most 1 (the max gate's rounding could give exp2 of a tiny positive number).
__device__ __forceinline__ float tg_e(float g, float ml) {
  return fminf(__builtin_amdgcn_exp2f(fmaf(g, kLog2e, -ml)), 1.f);
}
__device__ __forceinline__ float tg_ml(const TgHead& h) {
  return tg_gate_from_key(h.gmax) * kLog2e;
}
// key(e) - kmin, with key(e) held to [kmin, kmax]: the range comes from e of the head's smallest
// and largest gates, which bound every e as long as exp2 does not decrease anywhere; the clamp
// keeps every candidate in the pool's first digit even if it did.
__device__ __forceinline__ uint32_t tg_ukey(const TgHead& h, float e) {
  return min(max(sel_key(e), h.kmin), h.kmax) - h.kmin;
}

// e * 2^shift, rounded to nearest (e in [0, 1]).
__device__ __forceinline__ unsigned long long tg_fix(float e, uint32_t shift) {
  const double x = (double)e * ldexp(1.0, (int)shift);
  if (!(x > 0.0)) return 0ull;
  return (unsigned long long)rint(x);
}

__global__ __launch_bounds__(256) void tg_init_kernel(TgHead* __restrict__ heads,
                                                      TgHist* __restrict__ hist, uint32_t shift) {
  const int bh = blockIdx.x, t = threadIdx.x;
  if (t == 0) {
    TgHead h{};
    h.gmax = 0u;
    h.gmin = 0xffffffffu;
    h.kmin = 0xffffffffu;
    h.kmax = 0u;
    h.shift = shift;
    heads[bh] = h;
  }
  for (int b = t; b < kTgBins; b += 256) {
    hist[bh].cnt[b] = 0u;
    hist[bh].sum[b] = 0ull;
  }
}

// Gates of 128 tokens (one workgroup, a wavefront per 32) against every kv block of the head:
// per 32-block tile, G^T = Kbar Q^T with Kbar's two bf16 terms as A and Q as B, so each lane
// holds 16 gates of one token; written as sigma_h * gate (fp32) to g[bh][n][J], and the head's
// largest and smallest gates are updated with integer atomics on their order-preserving keys.
__global__ __launch_bounds__(256) void tg_gates_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ Khi,
    const uint16_t* __restrict__ Klo, const float* __restrict__ scale, int H, int N, int nkv,
    float* __restrict__ g, TgHead* __restrict__ heads) {
  constexpr int D = 128, R = D + 8;
  __shared__ __attribute__((aligned(16))) uint16_t kt[2][2][kTgTile * R];
  const int bh = blockIdx.y, n0 = blockIdx.x * 128;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, l32 = lane & 31, hl = lane >> 5;
  const float sig = scale[bh % H];
  const int n = n0 + 32 * wave + l32;
  const bool valid = n < N;
  bf16x8_t qf[8];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(Q + ((size_t)bh * N + min(n, N - 1)) * D +
                                                     8 * hl);
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) qf[kc] = __builtin_bit_cast(bf16x8_t, qp[2 * kc]);
  }
  const uint16_t* kh = Khi + (size_t)bh * nkv * D;
  const uint16_t* kl = Klo + (size_t)bh * nkv * D;
  uint4 ph0, pl0, ph1, pl1;
  const int off0 = (t >> 4) * R + 8 * (t & 15), off1 = off0 + 16 * R;
  auto load = [&](int tile) {
    const int r0 = tile * kTgTile + (t >> 4);
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
  const int ntiles = (nkv + kTgTile - 1) / kTgTile;
  float* grow = g + ((size_t)bh * N + (valid ? n : 0)) * nkv;
  float gmax = -INFINITY, gmin = INFINITY;
  load(0);
  store(0);
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int st = it & 1;
    if (it + 1 < ntiles) load(it + 1);
    f32x16_t acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      const bf16x8_t ah =
          *reinterpret_cast<const bf16x8_t*>(&kt[st][0][l32 * R + 16 * kc + 8 * hl]);
      const bf16x8_t al =
          *reinterpret_cast<const bf16x8_t*>(&kt[st][1][l32 * R + 16 * kc + 8 * hl]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, qf[kc], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, qf[kc], acc, 0, 0, 0);
    }
    // lane holds token column l32 and block rows 8 (e / 4) + 4 hl + e % 4 of the tile: four
    // runs of four consecutive blocks, stored 16 bytes at a time when rows are 16-byte aligned
    const int J0 = it * kTgTile;
    if (valid) {
      if ((nkv & 3) == 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int J = J0 + 8 * q + 4 * hl;
          if (J < nkv) {
            const float4 v = make_float4(sig * acc[4 * q], sig * acc[4 * q + 1],
                                         sig * acc[4 * q + 2], sig * acc[4 * q + 3]);
            *reinterpret_cast<float4*>(grow + J) = v;
            gmax = fmaxf(gmax, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
            gmin = fminf(gmin, fminf(fminf(v.x, v.y), fminf(v.z, v.w)));
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int J = J0 + 8 * (e >> 2) + 4 * hl + (e & 3);
          if (J < nkv) {
            const float v = sig * acc[e];
            grow[J] = v;
            gmax = fmaxf(gmax, v);
            gmin = fminf(gmin, v);
          }
        }
      }
    }
    if (it + 1 < ntiles) store(st ^ 1);
    __syncthreads();
  }
  // one integer atomic per workgroup on each of the head's order-preserving max and min keys
  __shared__ float wmax[4], wmin[4];
  gmax = wave_max_f32(gmax);
  gmin = -wave_max_f32(-gmin);
  if (lane == 0) {
    wmax[wave] = gmax;
    wmin[wave] = gmin;
  }
  __syncthreads();
  if (t == 0) {
    const float m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const float mn = fminf(fminf(wmin[0], wmin[1]), fminf(wmin[2], wmin[3]));
    if (mn < INFINITY) atomicMin(&heads[bh].gmin, tg_gate_key(mn));
    if (m > -INFINITY) atomicMax(&heads[bh].gmax, tg_gate_key(m));
  }
}

// Per head: the range of e's keys, from e of the smallest and largest gate, and the first digit's
// width from it (u = key - kmin has rem bits).
__global__ __launch_bounds__(64) void tg_setup_kernel(TgHead* __restrict__ heads) {
  const int bh = blockIdx.x;
  if (threadIdx.x != 0) return;
  TgHead h = heads[bh];
  const float ml = tg_ml(h);
  h.kmin = sel_key(tg_e(tg_gate_from_key(h.gmin), ml));
  h.kmax = sel_key(tg_e(tg_gate_from_key(h.gmax), ml));
  const uint32_t spread = h.kmax - h.kmin;
  h.rem = spread ? 32 - __clz(spread) : 0;
  h.hi = 0u;
  heads[bh] = h;
}

__device__ __forceinline__ void tg_digit(const TgHead& h, int& db, int& sh, uint32_t& dmask) {
  db = h.rem < kTgDigitBits ? h.rem : kTgDigitBits;
  sh = h.rem - db;
  dmask = (1u << db) - 1u;
}

// One digit pass over a chunk of the head pool (gates, each turned into e as it is read): the
// candidates still matching the prefix add their count and fixed-point sum to their digit's bin
// (LDS histogram, runs of equal bins summed in registers first), then to the head's global
// histogram.
__global__ __launch_bounds__(256) void tg_hist_kernel(const float* __restrict__ g,
                                                      int64_t per_head,
                                                      const TgHead* __restrict__ heads,
                                                      TgHist* __restrict__ hist) {
  __shared__ unsigned int scnt[kTgBins];
  __shared__ unsigned long long ssum[kTgBins];
  const int bh = blockIdx.y;
  const TgHead h = heads[bh];
  if (h.done) return;
  const int64_t base = (int64_t)blockIdx.x * kTgChunk;
  if (base >= per_head) return;
  const int t = threadIdx.x;
  for (int b = t; b < kTgBins; b += 256) {
    scnt[b] = 0u;
    ssum[b] = 0ull;
  }
  __syncthreads();
  int db, sh;
  uint32_t dmask;
  tg_digit(h, db, sh, dmask);
  const float* p = g + (size_t)bh * per_head;
  const float ml = tg_ml(h);
  constexpr int kPer = kTgChunk / 256;
  uint32_t run_bin = (uint32_t)kTgBins, run_cnt = 0u;
  unsigned long long run_sum = 0ull;
  auto add = [&](float gv) {
    const float v = tg_e(gv, ml);
    const uint32_t uk = tg_ukey(h, v);
    if ((uk >> h.rem) == h.hi) {
      const uint32_t bin = (uk >> sh) & dmask;
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
      run_sum += tg_fix(v, h.shift);
    }
  };
  // kPer / 4 rounds of 16-byte loads, each round 4 KB of consecutive pool entries (the pool of
  // a head starts 16-byte aligned when nkv * N is a multiple of 4; else one value at a time)
  if ((per_head & 3) == 0) {
    for (int q0 = 0; q0 < kPer / 4; q0 += 4) {  // four 16-byte loads in flight per thread
      float4 v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t j = base + 4 * (t + 256 * (q0 + q));
        v[q] = j < per_head ? *reinterpret_cast<const float4*>(p + j)
                            : make_float4(0.f, 0.f, 0.f, 0.f);  // not added (the test below)
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (base + 4 * (t + 256 * (q0 + q)) < per_head) {
          add(v[q].x);
          add(v[q].y);
          add(v[q].z);
          add(v[q].w);
        }
      }
    }
  } else {
    for (int q = 0; q < kPer; ++q) {
      const int64_t j = base + t + 256 * q;
      if (j < per_head) add(p[j]);
    }
  }
  if (run_cnt) {
    atomicAdd(&scnt[run_bin], run_cnt);
    atomicAdd(&ssum[run_bin], run_sum);
  }
  __syncthreads();
  for (int b = t; b < kTgBins; b += 256) {
    if (scnt[b]) {
      atomicAdd(&hist[bh].cnt[b], scnt[b]);
      atomicAdd(&hist[bh].sum[b], ssum[b]);
    }
  }
}

// One wavefront per head: on the first pass the pool total Z (every candidate is in the
// histogram) gives the target ceil(tau * Z); then the bin, in descending order, where the
// cumulative sum first reaches it narrows the prefix. The histogram is cleared for the next pass.
__global__ __launch_bounds__(64) void tg_pick_kernel(int pass, double tau,
                                                     TgHead* __restrict__ heads,
                                                     TgHist* __restrict__ hist) {
  const int bh = blockIdx.x, lane = threadIdx.x;
  TgHead h = heads[bh];
  if (h.done) return;
  TgHist& hs = hist[bh];
  // bins in descending order: lane l holds bins kTgBins - 1 - kPerLane l - i
  constexpr int kPerLane = kTgBins / 64;
  unsigned long long bsum[kPerLane];
  unsigned int bcnt[kPerLane];
  unsigned long long lsum = 0;
  int lcnt = 0;
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const int bin = kTgBins - 1 - kPerLane * lane - i;
    bsum[i] = hs.sum[bin];
    bcnt[i] = hs.cnt[bin];
    lsum += bsum[i];
    lcnt += (int)bcnt[i];
  }
  const unsigned long long isum = wave_incl_scan_u64(lsum);
  const int icnt = wave_incl_scan_i32(lcnt);
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const int bin = kTgBins - 1 - kPerLane * lane - i;
    hs.sum[bin] = 0ull;
    hs.cnt[bin] = 0u;
  }
  if (pass == 0) {
    const unsigned long long tot = __shfl(isum, 63, 64);  // lane 63 holds the pool total
    h.total = tot;
    h.target = (unsigned long long)ceil(tau * (double)tot);
    if (tau >= 1.0 || h.target == 0ull || h.target > tot) {
      if (lane == 0) {
        h.all = 1;
        h.done = 1;
        heads[bh] = h;
      }
      return;
    }
  }
  unsigned long long asum = h.above_sum + (isum - lsum);
  unsigned long long acnt = h.above_cnt + (unsigned long long)(icnt - lcnt);
  int found = -1;
  unsigned long long fsum = 0, fcnt = 0;
  unsigned int feq = 0;
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    if (found < 0 && asum < h.target && asum + bsum[i] >= h.target) {
      found = kTgBins - 1 - kPerLane * lane - i;
      fsum = asum;
      fcnt = acnt;
      feq = bcnt[i];
    }
    asum += bsum[i];
    acnt += bcnt[i];
  }
  if (__ballot(found >= 0) == 0ull) {  // not reached: keep every pair
    if (lane == 0) {
      h.all = 1;
      h.done = 1;
      heads[bh] = h;
    }
    return;
  }
  if (found < 0) return;  // exactly one lane found the bin: it writes the new state
  int db, sh;
  uint32_t dmask;
  tg_digit(h, db, sh, dmask);
  h.hi = (h.hi << db) | (uint32_t)found;
  h.rem = sh;
  h.above_sum = fsum;
  h.above_cnt = (uint32_t)fcnt;
  h.eq_cnt = feq;
  if (feq == 1u || h.rem == 0) {
    h.done = 1;
    uint32_t keep;
    if (feq == 1u) {
      keep = 1u;
    } else {
      const unsigned long long v = tg_fix(__uint_as_float(h.kmin + h.hi), h.shift);
      keep = v ? (uint32_t)((h.target - h.above_sum + v - 1) / v) : feq;
    }
    if (keep > feq) keep = feq;
    h.keep = keep;
    h.eq_all = keep == feq ? 1 : 0;
  }
  heads[bh] = h;
}

__device__ __forceinline__ bool tg_selected(const TgHead& h, float e, bool& boundary) {
  boundary = false;
  if (h.all) return true;
  const uint32_t k = tg_ukey(h, e) >> h.rem;
  if (k > h.hi) return true;
  if (k == h.hi) {
    boundary = !h.eq_all;
    return h.eq_all;
  }
  return false;
}

// Per token row: the bitmap of its kept blocks (every pair above the boundary class, and the
// whole class when all of it is kept), and per chunk of kTgRows rows the count of boundary-class
// pairs not yet kept.
__global__ __launch_bounds__(256) void tg_mark_kernel(const float* __restrict__ g, int N,
                                                      int nkv, int nwords,
                                                      const TgHead* __restrict__ heads,
                                                      uint32_t* __restrict__ tbits,
                                                      int32_t* __restrict__ bnd, int nchunk) {
  __shared__ int sbnd[4];
  const int bh = blockIdx.y, c = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const TgHead h = heads[bh];
  const float ml = tg_ml(h);
  const int r0 = c * kTgRows, nr = min(kTgRows, N - r0);
  // wavefront w takes rows w, w + 4, ..., two at a time (rows rr and rr + 4) with up to eight
  // loads of each in flight: lane l tests blocks 64 i + l (coalesced reads), a ballot gives two
  // bitmap words per 64 blocks
  int my = 0;
  for (int rr = wave; rr < nr; rr += 8) {
    const int nrow = rr + 4 < nr ? 2 : 1;  // wave-uniform
    const float* row0 = g + ((size_t)bh * N + r0 + rr) * nkv;
    const float* row1 = row0 + (size_t)4 * nkv;
    uint32_t* out0 = tbits + ((size_t)bh * N + r0 + rr) * nwords;
    uint32_t* out1 = out0 + (size_t)4 * nwords;
    for (int J1 = 0; J1 < nkv; J1 += 512) {
      float v[2][8];
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int J = J1 + 64 * i + lane;
          v[q][i] = (q < nrow && J < nkv) ? (q ? row1 : row0)[J] : 0.f;
        }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        if (q >= nrow) break;
        uint32_t* out = q ? out1 : out0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int J0 = J1 + 64 * i;
          if (J0 >= nkv) break;
          bool sel = false, bd = false;
          if (J0 + lane < nkv) sel = tg_selected(h, tg_e(v[q][i], ml), bd);
          const unsigned long long bal = __ballot(sel);
          my += __popcll(__ballot(bd));
          const int w = (J0 >> 5) + lane;
          if (lane < 2 && w < nwords) out[w] = (uint32_t)(bal >> (32 * lane));
        }
      }
    }
  }
  if (lane == 0) sbnd[wave] = my;
  __syncthreads();
  if (t == 0) bnd[(size_t)bh * nchunk + c] = (sbnd[0] + sbnd[1]) + (sbnd[2] + sbnd[3]);
}

// When only part of the boundary class is kept: its members in pool index order (token, then
// block), chunk by chunk, the counts of the earlier chunks giving each chunk's first rank.
__global__ __launch_bounds__(64) void tg_boundary_kernel(const float* __restrict__ g, int N,
                                                         int nkv, int nwords,
                                                         const TgHead* __restrict__ heads,
                                                         const int32_t* __restrict__ bnd,
                                                         int nchunk,
                                                         uint32_t* __restrict__ tbits) {
  const int bh = blockIdx.y, c = blockIdx.x, lane = threadIdx.x;
  const TgHead h = heads[bh];
  if (h.all || h.eq_all || !h.done) return;
  const int32_t* hb = bnd + (size_t)bh * nchunk;
  if (hb[c] == 0) return;
  int before = 0;
  for (int i = lane; i < c; i += 64) before += hb[i];
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) before += __shfl_xor(before, d, 64);
  if ((uint32_t)before >= h.keep) return;
  const int r0 = c * kTgRows;
  const int64_t n = (int64_t)min(kTgRows, N - r0) * nkv;
  const float* p = g + ((size_t)bh * N + r0) * nkv;
  const float ml = tg_ml(h);
  uint32_t taken = (uint32_t)before;
  for (int64_t base = 0; base < n && taken < h.keep; base += 64) {
    const int64_t j = base + lane;
    bool eq = false;
    if (j < n) {
      bool bd;
      tg_selected(h, tg_e(p[j], ml), bd);
      eq = bd;
    }
    const unsigned long long bal = __ballot(eq);
    const uint32_t rank = taken + __popcll(bal & ((1ull << lane) - 1ull));
    if (eq && rank < h.keep) {
      const int rr = (int)(j / nkv), J = (int)(j - (int64_t)rr * nkv);
      atomicOr(&tbits[((size_t)bh * N + r0 + rr) * nwords + J / 32], 1u << (J % 32));
    }
    taken += __popcll(bal);
  }
}

// Union of the token bitmaps of each query block (b, h, I), one wavefront per row: lane w ORs
// word w over the block's tokens.
__global__ __launch_bounds__(256) void tg_union_kernel(const uint32_t* __restrict__ tbits,
                                                       int N, int nq, int nwords,
                                                       const int32_t* __restrict__ qstart,
                                                       const int32_t* __restrict__ qperm,
                                                       int64_t rows,
                                                       uint32_t* __restrict__ bitmap,
                                                       int32_t* __restrict__ counts) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int I = (int)(r % nq);
  const int64_t bh = r / nq;
  uint32_t w = 0u;
  if (lane < nwords)
    for (int s = qstart[I]; s < qstart[I + 1]; ++s)
      w |= tbits[((size_t)bh * N + qperm[s]) * nwords + lane];
  if (lane < nwords) bitmap[r * nwords + lane] = w;
  int c = __popc(w);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) c += __shfl_xor(c, d, 64);
  if (lane == 0) counts[r] = c;
}

}  // namespace

hipError_t launch_select_tokens_global(const bsa_plan& p, const void* Q, const float* Kbar,
                                       double tau, uint32_t* tbits, int32_t* row_ptr,
                                       int32_t* col_idx, void* ws, hipStream_t s) {
  const TgWs L = tg_ws_layout(p);
  char* base = static_cast<char*>(ws);
  uint16_t* khi = reinterpret_cast<uint16_t*>(base + L.khi);
  uint16_t* klo = reinterpret_cast<uint16_t*>(base + L.klo);
  float* g = reinterpret_cast<float*>(base + L.e);  // the gates
  TgHead* heads = reinterpret_cast<TgHead*>(base + L.heads);
  TgHist* hist = reinterpret_cast<TgHist*>(base + L.hist);
  int32_t* bnd = reinterpret_cast<int32_t*>(base + L.bnd);
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(base + L.bitmap);
  int32_t* counts = reinterpret_cast<int32_t*>(base + L.counts);
  int32_t* partial = reinterpret_cast<int32_t*>(base + L.partial);
  const int BH = p.prob.B * p.prob.H, N = p.prob.N, nkv = p.nkv;
  const int64_t per_head = (int64_t)N * nkv, rows = (int64_t)BH * p.nq;
  // the fixed-point scale: a head's total (at most per_head * 2^shift) stays below 2^63
  int lg = 0;
  while ((1ll << lg) < per_head) ++lg;
  const uint32_t shift = (uint32_t)std::min(56, 63 - lg);
  hipError_t err = launch_kbar_split(Kbar, (int64_t)BH * nkv * 128, khi, klo, s);
  if (err != hipSuccess) return err;
  tg_init_kernel<<<BH, 256, 0, s>>>(heads, hist, shift);
  tg_gates_kernel<<<dim3((N + 127) / 128, BH), 256, 0, s>>>(
      static_cast<const uint16_t*>(Q), khi, klo, p.scale, p.prob.H, N, nkv, g, heads);
  tg_setup_kernel<<<BH, 64, 0, s>>>(heads);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const unsigned nch = (unsigned)((per_head + kTgChunk - 1) / kTgChunk);
  // at most 31 key bits in digits of kTgDigitBits (a head stops once its class is decided)
  for (int pass = 0; pass < (31 + kTgDigitBits - 1) / kTgDigitBits; ++pass) {
    tg_hist_kernel<<<dim3(nch, BH), 256, 0, s>>>(g, per_head, heads, hist);
    tg_pick_kernel<<<BH, 64, 0, s>>>(pass, tau, heads, hist);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const int nchunk = (N + kTgRows - 1) / kTgRows;
  tg_mark_kernel<<<dim3(nchunk, BH), 256, 0, s>>>(g, N, nkv, L.nwords, heads, tbits, bnd,
                                                  nchunk);
  tg_boundary_kernel<<<dim3(nchunk, BH), 64, 0, s>>>(g, N, nkv, L.nwords, heads, bnd, nchunk,
                                                     tbits);
  tg_union_kernel<<<(unsigned)((rows + 3) / 4), 256, 0, s>>>(tbits, N, p.nq, L.nwords, p.qstart,
                                                             p.qperm, rows, bitmap, counts);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  err = launch_scan(counts, nullptr, false, rows, p.nq, row_ptr, nullptr, partial, s);
  if (err != hipSuccess) return err;
  return launch_emit(bitmap, L.nwords, rows, row_ptr, col_idx, s);
}
