// Backward of the block-sparse attention (training through the sparse attention: pith.science
// review of VMoBA, "The reading"), with the selection held fixed as a hard gate. For every
// selected pair (i, j): P = exp(sigma q_i.k_j - lse_i), dV_j += P dO_i, dP = dO_i.v_j,
// dS = P (dP - D_i) with D_i = dO_i.O_i, dQ_i += sigma dS k_j, dK_j += sigma dS q_i.
//
// Passes, all deterministic (no atomics on floating point):
//   1. bwd_prep_kernel D = rowsum(dO * O) (token order, for the dQ pass), and Q, dO, LSE and D
//                      copied into query block order for the dK/dV pass (one read of Q, O, dO).
//   2. CSR -> CSC      a per-row bitmap of the selection, then for every (head, kv block) the
//                      ascending list of query blocks that selected it (column counts, a scan,
//                      and a fill that walks the bitmap in query-block order).
//   3. dkdv_kernel     kv-stationary: a workgroup owns 128 tokens of one kv block (4 wavefronts x
//                      32 tokens, K and V held in registers as MFMA B operands) and streams the
//                      64-query chunks of every query block in its CSC column through LDS (Q, dO,
//                      lse, D; double-buffered direct copies of consecutive block-order rows). Per chunk and wave: S = Q K^T and
//                      dP = dO V^T (lane = kv token), P and dS in registers, then
//                      dV^T += dO^T P and dK^T += Q^T dS with dO^T / Q^T from transposing reads.
//   4. dq16_kernel     query-stationary over the CSR, on the forward's work items (one
//                      workgroup of four wavefronts per 128 queries, or the packed slots of up to
//                      four small query blocks; two workgroups per CU), K and V tiles from
//                      block-ordered copies, S and dP recomputed per tile, 16x16x32 MFMAs.
#include "bsa_internal.h"
#include "device_common.h"
#include "kv_cursor.h"

namespace {

constexpr int kRowBytes = 256;
constexpr int kChunkQ = 64;                     // queries per streamed chunk
constexpr int kTileBytes = kChunkQ * kRowBytes;  // one of Q / dO
constexpr int kStage = 2 * kTileBytes + 2 * kChunkQ * 4;  // Q, dO, lse2, D
constexpr int kKvTileBytes = 2 * 128 * kRowBytes;          // an item's K and V rows

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;



// Per query position pos of the block order (token n = qperm[pos]): D = dO_n . O_n, written in
// token order (for the dQ pass) and in block order; Q_n and dO_n copied to block order; LSE
// (times log2 e) in block order. Rows N <= pos < Npad are zero. 16 lanes per row, 16 rows per
// workgroup.
__global__ __launch_bounds__(256) void bwd_prep_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ O,
    const uint16_t* __restrict__ dO, const float* __restrict__ lse,
    const int32_t* __restrict__ qperm, int N, int Npad, uint16_t* __restrict__ Qp,
    uint16_t* __restrict__ dOp, float* __restrict__ lsep, float* __restrict__ Dp,
    float* __restrict__ Dnat) {
  const int pos = blockIdx.x * 16 + (threadIdx.x >> 4), seg = threadIdx.x & 15;
  const size_t bh = blockIdx.y;
  const bool valid = pos < N;
  const int tok = valid ? qperm[pos] : 0;
  uint4 q = make_uint4(0, 0, 0, 0), g = q;
  float s = 0.f;
  if (valid) {
    const size_t src = (bh * N + (size_t)tok) * 128 + 8 * seg;
    q = *reinterpret_cast<const uint4*>(Q + src);
    g = *reinterpret_cast<const uint4*>(dO + src);
    const uint4 o = *reinterpret_cast<const uint4*>(O + src);
    const uint32_t ow[4] = {o.x, o.y, o.z, o.w}, gw[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      s += bf16_lo(ow[i]) * bf16_lo(gw[i]) + bf16_hi(ow[i]) * bf16_hi(gw[i]);
  }
#pragma unroll
  for (int d = 8; d >= 1; d >>= 1) s += __shfl_xor(s, d, 64);
  if (pos >= Npad) return;
  const size_t dst = (bh * Npad + (size_t)pos) * 128 + 8 * seg;
  *reinterpret_cast<uint4*>(Qp + dst) = q;
  *reinterpret_cast<uint4*>(dOp + dst) = g;
  if (seg == 0) {
    Dp[bh * Npad + pos] = s;
    lsep[bh * Npad + pos] = valid ? lse[bh * N + tok] * kLog2e : 0.f;
    if (valid) Dnat[bh * N + tok] = s;
  }
}

// Selection bitmap of one CSR row (one workgroup per row, nwords <= 256); entries outside
// [0, nkv) are skipped, as the forward's cursor skips them.
__global__ __launch_bounds__(256) void csr_bitmap_kernel(const int32_t* __restrict__ row_ptr,
                                                         const int32_t* __restrict__ col_idx,
                                                         int nkv, int nwords,
                                                         uint32_t* __restrict__ bm) {
  __shared__ uint32_t w[256];
  const int64_t r = blockIdx.x;
  for (int i = threadIdx.x; i < nwords; i += 256) w[i] = 0u;
  __syncthreads();
  for (int s = row_ptr[r] + threadIdx.x; s < row_ptr[r + 1]; s += 256) {
    const int J = col_idx[s];
    if ((uint32_t)J < (uint32_t)nkv) atomicOr(&w[J >> 5], 1u << (J & 31));
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nwords; i += 256) bm[r * nwords + i] = w[i];
}

// One thread per column (bh, J): count (fill == false) or write (fill == true) the query blocks
// that selected J, in ascending order.
__global__ __launch_bounds__(256) void csc_kernel(const uint32_t* __restrict__ bm, int nq,
                                                  int nkv, int nwords, int64_t cols, bool fill,
                                                  int32_t* __restrict__ col_cnt,
                                                  const int32_t* __restrict__ col_ptr,
                                                  int32_t* __restrict__ row_idx) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= cols) return;
  const int64_t bh = c / nkv;
  const int J = (int)(c % nkv);
  const uint32_t* b = bm + bh * nq * (int64_t)nwords + (J >> 5);
  const uint32_t bit = 1u << (J & 31);
  int pos = fill ? col_ptr[c] : 0;
  int n = 0;
  for (int I = 0; I < nq; ++I) {
    if (b[(int64_t)I * nwords] & bit) {
      if (fill) row_idx[pos++] = I;
      ++n;
    }
  }
  if (!fill) col_cnt[c] = n;
}

// Exclusive scan of the column counts (one workgroup).
__global__ __launch_bounds__(1024) void col_scan_kernel(const int32_t* __restrict__ cnt,
                                                        int64_t cols,
                                                        int32_t* __restrict__ col_ptr) {
  __shared__ int wtot[16];
  __shared__ int carry_s;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  if (t == 0) {
    carry_s = 0;
    col_ptr[0] = 0;
  }
  __syncthreads();
  for (int64_t base = 0; base < cols; base += 1024) {
    const int64_t c = base + t;
    const int f = c < cols ? cnt[c] : 0;
    const int incl = wave_incl_scan_i32(f);
    if (lane == 63) wtot[wave] = incl;
    __syncthreads();
    int before = carry_s;
    for (int w = 0; w < wave; ++w) before += wtot[w];
    if (c < cols) col_ptr[c + 1] = before + incl;
    __syncthreads();
    if (t == 0) {
      int tot = 0;
      for (int w = 0; w < 16; ++w) tot += wtot[w];
      carry_s += tot;
    }
    __syncthreads();
  }
}

struct DkdvArgs {
  const uint16_t* Qp;   // Q, dO, LSE * log2 e and D in query block order ([B*H][Npad])
  const uint16_t* Kp;   // K and V in kv block order ([B*H][Npad][d])
  const uint16_t* Vp;
  const uint16_t* dOp;
  const float* lsep;
  const float* Dp;
  const int32_t* col_ptr;
  const int32_t* row_idx;
  const int32_t* qstart;
  const int32_t* kvperm;
  const int32_t* kvstart;
  const int32_t* kvitems;
  const float* scale;
  uint16_t* dK;
  uint16_t* dV;
  int n_kvitems, H, N, nkv, Npad;
};

// Walks the query blocks of a CSC column as 64-query chunks.
struct QCursor {
  int slot, end, sub, base, size;
};

__device__ __forceinline__ void qcur_load(QCursor& c, const int32_t* __restrict__ row_idx,
                                          const int32_t* __restrict__ qstart) {
  if (c.slot < c.end) {
    const int I = ld_ro(row_idx + c.slot);
    c.base = ld_ro(qstart + I);
    c.size = ld_ro(qstart + I + 1) - c.base;
  } else {
    c.base = 0;
    c.size = 0;
  }
}

struct QChunk {
  int pos, nv;
};

__device__ __forceinline__ QChunk qcur_take(QCursor& c, const int32_t* __restrict__ row_idx,
                                            const int32_t* __restrict__ qstart) {
  QChunk k;
  if (c.slot < c.end) {
    k.pos = c.base + kChunkQ * c.sub;
    k.nv = min(kChunkQ, c.size - kChunkQ * c.sub);
    ++c.sub;
    if (kChunkQ * c.sub >= c.size) {
      ++c.slot;
      c.sub = 0;
      qcur_load(c, row_idx, qstart);
    }
  } else {
    k.pos = 0;
    k.nv = 0;
  }
  return k;
}

// Eight wavefronts: wave w owns kv tokens 32 (w % 4) .. +32 of the 128-token item and query half
// w / 4 (32 queries) of every 64-query chunk, so two wavefronts share each SIMD; the two halves'
// partial dK and dV are summed through LDS at the end (a fixed order: deterministic).
__global__ __launch_bounds__(512, 2) void dkdv_kernel(const DkdvArgs a) {
  constexpr int D = 128;
  // Two Q/dO stages, then this item's K and V tiles (128 rows each, swizzled like the stages).
  __shared__ __attribute__((aligned(1024))) char lds[2 * kStage + kKvTileBytes];
  char* const lds_a = lds;
  char* const lds_b = lds + kStage;
  char* const kv_lds = lds + 2 * kStage;

  const int total = a.n_kvitems * (int)gridDim.y;
  const int lin = xcd_remap(blockIdx.x + blockIdx.y * gridDim.x, total);
  const int bh = lin / a.n_kvitems, item = lin % a.n_kvitems;
  const int J = ld_ro(a.kvitems + 2 * item), off = ld_ro(a.kvitems + 2 * item + 1);
  const int k0 = ld_ro(a.kvstart + J) + off;
  const int nkvrows = min(128, ld_ro(a.kvstart + J + 1) - k0);
  const size_t head_off = (size_t)bh * a.N * D;
  const float c2 = ld_ro(a.scale + bh % a.H) * kLog2e;

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int kvg = wave & 3, mb = wave >> 2;  // kv group, query half
  const int l32 = lane & 31, hl = lane >> 5;

  // This lane's kv token. The item's 128 rows of K and V (block order, so consecutive rows from
  // k0; rows past the item's end are other tokens or zero padding, all finite) are copied into
  // LDS once; the S and dP MFMAs read their B operands (K and V fragments) from there, which
  // keeps the register budget within two wavefronts per SIMD.
  const int kvrow = 32 * kvg + l32;
  const bool kvvalid = kvrow < nkvrows;
  const bool active = 32 * kvg < nkvrows;  // wave-uniform
  const int kvtok = kvvalid ? a.kvperm[k0 + kvrow] : 0;
  {
    const uint16_t* kb = a.Kp + ((size_t)bh * a.Npad + k0) * D;
    const uint16_t* vb = a.Vp + ((size_t)bh * a.Npad + k0) * D;
    const uint32_t kv_m0 = lds_addr(kv_lds);
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // wave w: rows 16w + 4i + lane/16
      const int row = 16 * wave + 4 * i + (lane >> 4);
      const uint32_t vo =
          (uint32_t)(row * kRowBytes) + 16u * (uint32_t)((lane & 15) ^ lds_key(row));
      const uint32_t m0v = kv_m0 + (uint32_t)((16 * wave + 4 * i) * kRowBytes);
      lds_dma16_so(kb, vo, m0v);
      lds_dma16_so(vb, vo, m0v + kKvTileBytes / 2);
    }
  }
  f32x16_t dk[4], dv[4];  // dK^T, dV^T: lane = kv token, registers = d
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      dk[i][e] = 0.f;
      dv[i][e] = 0.f;
    }

  const int64_t col = (int64_t)bh * a.nkv + J;
  QCursor cur;
  cur.slot = ld_ro(a.col_ptr + col);
  cur.end = ld_ro(a.col_ptr + col + 1);
  cur.sub = 0;
  qcur_load(cur, a.row_idx, a.qstart);

  // Loader roles: wave w copies rows 8w + 4i + lane/16 (i = 0, 1) of a chunk's Q and dO tiles
  // (direct global->LDS copies into swizzled rows); wave 0 copies the chunk's 64 LSE values and
  // wave 1 its 64 D values. Everything is read in query block order, so a chunk is consecutive rows
  // starting at its position and the copies need no token ids. Rows past a chunk's end (the next
  // block's queries, or zero padding) get LSE = +inf once their copy has landed, so their P and
  // dS are exactly 0.
  const int lgrp = lane >> 4;
  const size_t qoff = (size_t)bh * a.Npad;
  const uint16_t* const qbase = a.Qp + qoff * D;
  const uint16_t* const gbase = a.dOp + qoff * D;
  uint32_t voff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
    voff[i] = (uint32_t)((8 * wave + 4 * i + lgrp) * kRowBytes) +
              16u * (uint32_t)((lane & 15) ^ lds_key(8 * wave + 4 * i + lgrp));
  auto chunk_issue = [&](QChunk c, uint32_t st_m0) {
    const uint16_t* qb = qbase + (size_t)c.pos * D;
    const uint16_t* gb = gbase + (size_t)c.pos * D;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t m0v = st_m0 + (uint32_t)((8 * wave + 4 * i) * kRowBytes);
      lds_dma16_so(qb, voff[i], m0v);
      lds_dma16_so(gb, voff[i], m0v + kTileBytes);
    }
    if (wave == 0) lds_dma4_so(a.lsep + qoff + c.pos, 4u * lane, st_m0 + 2 * kTileBytes);
    if (wave == 1)
      lds_dma4_so(a.Dp + qoff + c.pos, 4u * lane, st_m0 + 2 * kTileBytes + kChunkQ * 4);
  };
  // After this wave's copies have landed: padding rows of a partial chunk get LSE = +inf.
  auto chunk_finish = [&](QChunk c, char* st) {
    if (wave == 0 && lane >= c.nv) reinterpret_cast<float*>(st + 2 * kTileBytes)[lane] = INFINITY;
  };

  // Transposing-read offsets (as for V^T in the forward kernel).
  const int vrow_l = 4 * hl + ((lane & 15) >> 2);
  const int vunit_l = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int vhalf_l = 8 * (lane & 1);

  const uint32_t m0_a = lds_addr(lds_a), m0_b = lds_addr(lds_b);
  QChunk c0 = qcur_take(cur, a.row_idx, a.qstart);
  if (c0.nv > 0) chunk_issue(c0, m0_a);
  QChunk c1 = qcur_take(cur, a.row_idx, a.qstart);
  vmem_wait_all();
  if (c0.nv > 0) chunk_finish(c0, lds_a);
  __syncthreads();

  auto step = [&](const char* st, char* nx, uint32_t nx_m0) {
    if (c1.nv > 0) chunk_issue(c1, nx_m0);
    const QChunk c2n = qcur_take(cur, a.row_idx, a.qstart);

    const float* lse2 = reinterpret_cast<const float*>(st + 2 * kTileBytes);
    const float* dd = reinterpret_cast<const float*>(st + 2 * kTileBytes + kChunkQ * 4);
    // This wave's 32-query half (M block) of the chunk; kv groups past a ragged item's end skip.
    if (active) {
      // S = Q K^T and dP = dO V^T (lane = kv token, registers = query).
      const int row = 32 * mb + l32;
      const char* qp = st + row * kRowBytes;
      const char* gp = st + kTileBytes + row * kRowBytes;
      f32x16_t sacc, dpacc;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        sacc[e] = 0.f;
        dpacc[e] = 0.f;
      }
      const char* kr = kv_lds + kvrow * kRowBytes;
      const char* vr = kr + kKvTileBytes / 2;
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) {
        const bf16x8_t qa = *reinterpret_cast<const bf16x8_t*>(qp + lds_swz(row, 2 * kc + hl));
        const bf16x8_t ga = *reinterpret_cast<const bf16x8_t*>(gp + lds_swz(row, 2 * kc + hl));
        const bf16x8_t kf =
            *reinterpret_cast<const bf16x8_t*>(kr + lds_swz(kvrow, 2 * kc + hl));
        const bf16x8_t vf =
            *reinterpret_cast<const bf16x8_t*>(vr + lds_swz(kvrow, 2 * kc + hl));
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf, sacc, 0, 0, 0);
        dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, vf, dpacc, 0, 0, 0);
      }
      // P = exp(sigma s - lse) and dS = P (dP - D), rounded to bf16 (B operands below).
      uint32_t pw[8], dw[8];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int q = 32 * mb + 8 * g + 4 * hl;
        const float4 l4 = *reinterpret_cast<const float4*>(lse2 + q);
        const float4 d4 = *reinterpret_cast<const float4*>(dd + q);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv4[4] = {d4.x, d4.y, d4.z, d4.w};
        float pr[4], dsr[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int e = 4 * g + rr;
          pr[rr] = kvvalid ? __builtin_amdgcn_exp2f(fmaf(sacc[e], c2, -lv[rr])) : 0.f;
          dsr[rr] = pr[rr] * (dpacc[e] - dv4[rr]);
        }
        pw[2 * g] = pack_bf16x2(pr[0], pr[1]);
        pw[2 * g + 1] = pack_bf16x2(pr[2], pr[3]);
        dw[2 * g] = pack_bf16x2(dsr[0], dsr[1]);
        dw[2 * g + 1] = pack_bf16x2(dsr[2], dsr[3]);
      }
      // dV^T += dO^T P and dK^T += Q^T dS over this half's 32 queries (two 16-query k-steps);
      // A operands from transposing reads of the dO / Q tiles.
#pragma unroll
      for (int dm = 0; dm < 4; ++dm) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int kc = 2 * mb + kk;
          const int row_lo = 16 * kc + vrow_l, row_hi = row_lo + 8;
          const int olo = row_lo * kRowBytes + lds_swz(row_lo, 4 * dm + vunit_l) + vhalf_l;
          const int ohi = row_hi * kRowBytes + lds_swz(row_hi, 4 * dm + vunit_l) + vhalf_l;
          const v4i16_t glo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4i16_t*)((lds_char_t*)st + kTileBytes + olo));
          const v4i16_t ghi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4i16_t*)((lds_char_t*)st + kTileBytes + ohi));
          const v4i16_t qlo =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)((lds_char_t*)st + olo));
          const v4i16_t qhi =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)((lds_char_t*)st + ohi));
          const uint2 g0 = __builtin_bit_cast(uint2, glo), g1 = __builtin_bit_cast(uint2, ghi);
          const uint2 q0 = __builtin_bit_cast(uint2, qlo), q1 = __builtin_bit_cast(uint2, qhi);
          const bf16x8_t gt = __builtin_bit_cast(bf16x8_t, make_uint4(g0.x, g0.y, g1.x, g1.y));
          const bf16x8_t qt = __builtin_bit_cast(bf16x8_t, make_uint4(q0.x, q0.y, q1.x, q1.y));
          const bf16x8_t pb = __builtin_bit_cast(
              bf16x8_t, make_uint4(pw[4 * kk], pw[4 * kk + 1], pw[4 * kk + 2], pw[4 * kk + 3]));
          const bf16x8_t db = __builtin_bit_cast(
              bf16x8_t, make_uint4(dw[4 * kk], dw[4 * kk + 1], dw[4 * kk + 2], dw[4 * kk + 3]));
          dv[dm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(gt, pb, dv[dm], 0, 0, 0);
          dk[dm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qt, db, dk[dm], 0, 0, 0);
        }
      }
    }
    vmem_wait_all();
    if (c1.nv > 0) chunk_finish(c1, nx);
    __syncthreads();
    c0 = c1;
    c1 = c2n;
  };
  while (true) {
    if (c0.nv <= 0) break;
    step(lds_a, lds_b, m0_b);
    if (c0.nv <= 0) break;
    step(lds_b, lds_a, m0_a);
  }

  // Sum the two query halves' partial dK^T and dV^T in a fixed order: the half-1 waves store
  // theirs ([kv group][register][lane] floats, 64 KB, in the now idle stages), the half-0 waves
  // add them; dK first, then dV.
  static_assert(4 * 64 * 64 * 4 <= 2 * kStage, "reduction buffer");
  float* red = reinterpret_cast<float*>(lds) + kvg * 64 * 64 + lane;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    f32x16_t* acc = pass == 0 ? dk : dv;
    if (mb == 1) {
#pragma unroll
      for (int dm = 0; dm < 4; ++dm)
#pragma unroll
        for (int e = 0; e < 16; ++e) red[(16 * dm + e) * 64] = acc[dm][e];
    }
    __syncthreads();
    if (mb == 0) {
#pragma unroll
      for (int dm = 0; dm < 4; ++dm)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[dm][e] += red[(16 * dm + e) * 64];
    }
    __syncthreads();
  }
  if (mb != 0 || !kvvalid) return;
  const float sig = a.scale[bh % a.H];
  uint16_t* kop = a.dK + head_off + (size_t)kvtok * D;
  uint16_t* vop = a.dV + head_off + (size_t)kvtok * D;
#pragma unroll
  for (int dm = 0; dm < 4; ++dm)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint2 pk, pv;
      pk.x = pack_bf16x2(dk[dm][4 * g] * sig, dk[dm][4 * g + 1] * sig);
      pk.y = pack_bf16x2(dk[dm][4 * g + 2] * sig, dk[dm][4 * g + 3] * sig);
      pv.x = pack_bf16x2(dv[dm][4 * g], dv[dm][4 * g + 1]);
      pv.y = pack_bf16x2(dv[dm][4 * g + 2], dv[dm][4 * g + 3]);
      *reinterpret_cast<uint2*>(kop + 32 * dm + 8 * g + 4 * hl) = pk;
      *reinterpret_cast<uint2*>(vop + 32 * dm + 8 * g + 4 * hl) = pv;
    }
}

// ------------------------------------------------------------------------------- dQ pass

struct DqArgs {
  const uint16_t* Q;
  const uint16_t* dO;
  const uint16_t* Kp;  // K and V in kv block order ([B*H][Npad][d])
  const uint16_t* Vp;
  const float* lse;    // forward LSE per token
  const float* delta;  // D per token
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const int32_t* qperm;
  const int32_t* qstart;
  const int32_t* kvstart;
  const int32_t* items;
  const float* scale;
  uint16_t* dQ;
  int n_items, H, N, nq, nkv, Npad;
  // the forward's work items (kFItemInts ints each): a query block's 128-row chunk, or the
  // 32-row slots of up to four small query blocks packed into one workgroup
  const int32_t* fitems;
  int n_fitems;
};

// dQ_i = sigma sum_j dS_ij k_j over the CSR row of i's query block, dS = P (dP - D) with
// P = exp(sigma q.k - lse) and dP = dO.v recomputed per tile. Query-stationary, as the forward
// pass: a workgroup of four wavefronts (two workgroups per CU) streams the selected K/V as
// 64-token tiles (two 32-token chunks) through two LDS stages; each wavefront owns 32 queries.
//
// dQ on v_mfma_f32_16x16x32_bf16, over the forward's work items (small query blocks packed four
// 32-row slots to a workgroup, the tile stream the merged walk of their CSR rows, a wavefront
// computing only the chunks its own block selected). The lane layouts are the sparse forward's
// (lane = 16 g + t; wavefront w owns 32 query rows in two 16-row tiles qt):
//   S^T and dP^T per 16 kv rows (mt) x 16 queries: A = K (or V) rows from LDS, row 16 mt + t,
//     d 32 kc + 8 g .. +8; B = Q^T (dO^T) from registers; lane holds [16 mt + 4 g + e][16 qt + t];
//   dQ^T per 16 d (dt) x 16 queries, K = the chunk's 32 kv rows in the order the score tiles
//     left them (k = 8 g + i: row 4 g + i, or 16 + 4 g + i - 4): A = K^T from two transposing
//     reads, B = the lane's own dS^T values; lane holds dQ^T[16 dt + 4 g + e][16 qt + t].
// Per 32-row chunk: 16 + 16 MFMAs for S^T and dP^T, dS^T = P^T (dP^T - D) in bf16, 16 MFMAs for
// dQ^T. No running max: P = exp(sigma s - lse) with the forward's LSE.
template <bool PACK>
__device__ __forceinline__ void dq16_body(const DqArgs& a, char* lds) {
  constexpr int D = 128;
  constexpr int kTile = 64 * kRowBytes;  // one of K / V
  constexpr int kDqStage = 2 * kTile;
  char* const lds_a = lds;
  char* const lds_b = lds + kDqStage;

  const int n_items = a.n_fitems;
  const int total = n_items * (int)gridDim.y;
  const int lin = xcd_remap(blockIdx.x + blockIdx.y * gridDim.x, total);
  const int bh = lin / n_items, item = lin % n_items;
  const int32_t* const desc = a.fitems + kFItemInts * item;
  const int I = ld_ro(desc + 1);
  const int q0 = ld_ro(a.qstart + I) + ld_ro(desc + 6);
  const int nrows = min(128, ld_ro(a.qstart + I + 1) - q0);
  const int64_t r = (int64_t)bh * a.nq + I;
  const size_t head_off = (size_t)bh * a.N * D;
  const float c2 = ld_ro(a.scale + bh % a.H) * kLog2e;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t = lane & 15, g = lane >> 4;
  int q0w = q0 + 32 * wave, nroww = nrows - 32 * wave, lw = 0;
  if constexpr (PACK) {
    lw = ld_ro(desc + 5 + 2 * wave);
    const int Iw = ld_ro(desc + 1 + (lw < 0 ? 0 : lw));
    q0w = ld_ro(a.qstart + Iw) + ld_ro(desc + 6 + 2 * wave);
    nroww = lw < 0 ? 0 : min(32, ld_ro(a.qstart + Iw + 1) - q0w);
  }
  const bool active = nroww > 0;  // wave-uniform

  // Q and dO fragments, -lse (log2 domain; -inf for padding queries, so their P is 0) and D of
  // queries 16 qt + t of the wavefront's rows.
  bool qvalid[2];
  int qtok[2];
  float nlse2[2], dq_d[2];
  bf16x8_t qf[2][4], dof[2][4];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    qvalid[qt] = 16 * qt + t < nroww;
    qtok[qt] = qvalid[qt] ? a.qperm[q0w + 16 * qt + t] : 0;
    const uint4* qp = reinterpret_cast<const uint4*>(a.Q + head_off + (size_t)qtok[qt] * D);
    const uint4* gp = reinterpret_cast<const uint4*>(a.dO + head_off + (size_t)qtok[qt] * D);
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      qf[qt][kc] = __builtin_bit_cast(bf16x8_t, qvalid[qt] ? qp[4 * kc + g] : make_uint4(0, 0, 0, 0));
      dof[qt][kc] =
          __builtin_bit_cast(bf16x8_t, qvalid[qt] ? gp[4 * kc + g] : make_uint4(0, 0, 0, 0));
    }
    nlse2[qt] = qvalid[qt] ? -a.lse[(size_t)bh * a.N + qtok[qt]] * kLog2e : -INFINITY;
    dq_d[qt] = qvalid[qt] ? a.delta[(size_t)bh * a.N + qtok[qt]] : 0.f;
  }
  f32x4_t acc[2][8];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[qt][dt][e] = 0.f;

  Cursor cur;
  MultiCursor mc;
  if constexpr (PACK) {
    mc.nl = ld_ro(desc);
#pragma unroll
    for (int l = 0; l < 4; ++l) {
      const int64_t rl = (int64_t)bh * a.nq + ld_ro(desc + 1 + l);
      mc.slot[l] = l < mc.nl ? ld_ro(a.row_ptr + rl) : 0;
      mc.end[l] = l < mc.nl ? ld_ro(a.row_ptr + rl + 1) : 0;
    }
    mcursor_load(mc, a.col_idx, a.kvstart, a.nkv);
  } else {
    cur.slot = ld_ro(a.row_ptr + r);
    cur.end = ld_ro(a.row_ptr + r + 1);
    cur.sub = 0;
    cursor_load<false>(cur, a.col_idx, a.kvstart, a.nkv);
  }
  auto take = [&]() {
    if constexpr (PACK)
      return mtake_chunk(mc, a.col_idx, a.kvstart, a.nkv);
    else
      return take_chunk<false>(cur, a.col_idx, a.kvstart, a.nkv);
  };

  // Loader: wave w copies rows 16 w + 4 i + lane / 16 of the 64-row K and V tiles.
  const int lchunk = wave >> 1, loff = 16 * (wave & 1), lgrp = lane >> 4;
  const size_t kv_off = (size_t)bh * a.Npad * D;
  uint32_t voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    voff[i] = (uint32_t)((loff + 4 * i + lgrp) * kRowBytes) +
              16u * (uint32_t)((lane & 15) ^ lds_key16(16 * wave + 4 * i + lgrp));
  auto tile_issue = [&](Chunk ca, Chunk cb, uint32_t st_m0) {
    const int pos = (lchunk && cb.nv > 0) ? cb.pos : ca.pos;
    const uint16_t* kb = a.Kp + kv_off + (size_t)pos * D;
    const uint16_t* vb = a.Vp + kv_off + (size_t)pos * D;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t m0v = st_m0 + (uint32_t)((16 * wave + 4 * i) * kRowBytes);
      lds_dma16_so(kb, voff[i], m0v);
      lds_dma16_so(vb, voff[i], m0v + kTile);
    }
  };
  // Byte offsets within a stage: K (V) fragment (mt, kc) of chunk s at kofs[kc] + 4096 (2 s + mt)
  // (+ kTile for V); K^T fragment dt of chunk s at tofs[dt] + 8192 s, its second read 4096 on.
  int kofs[4], tofs[8];
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) kofs[kc] = t * kRowBytes + lds_swz16(t, 4 * kc + g);
  {
    const int trow = 4 * g + (t >> 2);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      tofs[dt] = trow * kRowBytes + lds_swz16(trow, 2 * dt + ((t & 3) >> 1)) + 8 * (t & 1);
  }

  const uint32_t m0_a = lds_addr(lds_a), m0_b = lds_addr(lds_b);
  Chunk a0 = take();
  Chunk b0 = take();
  if (a0.nv > 0) tile_issue(a0, b0, m0_a);
  Chunk a1 = take();
  Chunk b1 = take();
  vmem_wait_all();
  __syncthreads();

  // One 32-row chunk s of the tile at st.
  auto chunk = [&](const char* st, int s, int nv) {
    f32x4_t sacc[2][2], dpacc[2][2];  // [qt][mt]
    __builtin_amdgcn_s_setprio(2);
    {
      bf16x8_t kf[4][2], vf[4][2];  // [kc][mt]
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          kf[kc][mt] = *reinterpret_cast<const bf16x8_t*>(st + kofs[kc] + 4096 * (2 * s + mt));
          vf[kc][mt] =
              *reinterpret_cast<const bf16x8_t*>(st + kTile + kofs[kc] + 4096 * (2 * s + mt));
        }
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sacc[qt][mt][e] = 0.f;
            dpacc[qt][mt][e] = 0.f;
          }
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) {
            sacc[qt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kc][mt], qf[qt][kc],
                                                                    sacc[qt][mt], 0, 0, 0);
            dpacc[qt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[kc][mt], dof[qt][kc],
                                                                     dpacc[qt][mt], 0, 0, 0);
          }
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    }
    __builtin_amdgcn_s_setprio(0);
    if (nv < 32) {  // partial chunk: padded kv rows get P = 0
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (16 * mt + 4 * g + e >= nv) {
            sacc[0][mt][e] = -INFINITY;
            sacc[1][mt][e] = -INFINITY;
          }
    }
    // K^T fragments of the chunk, read ahead of the vector work.
    auto tfrag = [&](int dt) {
      const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_v4i16_t*)((lds_char_t*)st + tofs[dt] + 8192 * s));
      const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_v4i16_t*)((lds_char_t*)st + tofs[dt] + 8192 * s + 4096));
      const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
      return __builtin_bit_cast(bf16x8_t, make_uint4(l2.x, l2.y, h2.x, h2.y));
    };
    const bf16x8_t kt0 = tfrag(0);
    __builtin_amdgcn_sched_barrier(0);
    // dS^T = P^T (dP^T - D), rounded to bf16: the B operand of dQ^T += K^T dS^T.
    bf16x8_t dsb[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      uint32_t w[4];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[qt][mt][e], c2, nlse2[qt]));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[qt][mt][e + 1], c2, nlse2[qt]));
          w[2 * mt + (e >> 1)] = pack_bf16x2(p0 * (dpacc[qt][mt][e] - dq_d[qt]),
                                             p1 * (dpacc[qt][mt][e + 1] - dq_d[qt]));
        }
      dsb[qt] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
    }
    __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const bf16x8_t kt = dt == 0 ? kt0 : tfrag(dt);
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
        acc[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt, dsb[qt], acc[qt][dt], 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x002, 100, 0);
#pragma unroll
    for (int i = 0; i < 7; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_s_setprio(0);
  };

  auto step = [&](const char* st, uint32_t nx_m0) {
    bool pa = true, pb = b0.nv > 0;
    if constexpr (PACK) {  // chunks of blocks this wavefront's query block selected
      pa = (a0.lmask >> lw) & 1;
      pb = pb && ((b0.lmask >> lw) & 1);
    }
    if (active) {
      if (pa) chunk(st, 0, a0.nv);
      if (pb) chunk(st, 1, b0.nv);
    }
    const Chunk an = take();
    const Chunk bn = take();
    if (a1.nv > 0) tile_issue(a1, b1, nx_m0);
    vmem_wait_all();
    __syncthreads();
    a0 = a1;
    b0 = b1;
    a1 = an;
    b1 = bn;
  };
  while (true) {
    if (a0.nv <= 0) break;
    step(lds_a, m0_b);
    if (a0.nv <= 0) break;
    step(lds_b, m0_a);
  }

  const float sig = a.scale[bh % a.H];  // dQ = sigma_h dS K
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    if (!qvalid[qt]) continue;
    uint16_t* op = a.dQ + head_off + (size_t)qtok[qt] * D + 4 * g;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      uint2 pk;
      pk.x = pack_bf16x2(acc[qt][dt][0] * sig, acc[qt][dt][1] * sig);
      pk.y = pack_bf16x2(acc[qt][dt][2] * sig, acc[qt][dt][3] * sig);
      *reinterpret_cast<uint2*>(op + 16 * dt) = pk;
    }
  }
}

__global__ __launch_bounds__(256, 2) void dq16_kernel(const DqArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[4 * 64 * kRowBytes];
  const int total = a.n_fitems * (int)gridDim.y;
  const int lin = xcd_remap(blockIdx.x + blockIdx.y * gridDim.x, total);
  if (ld_ro(a.fitems + kFItemInts * (lin % a.n_fitems)) > 1)
    dq16_body<true>(a, lds);
  else
    dq16_body<false>(a, lds);
}

}  // namespace

hipError_t launch_attn_bwd(const bsa_plan& p, const void* Q, const void* K, const void* V,
                           const void* O, const void* dO, const float* lse,
                           const int32_t* row_ptr, const int32_t* col_idx, void* dQ, void* dK,
                           void* dV, void* ws, hipStream_t s) {
  const BwdWs L = bwd_ws_layout(p);
  char* base = static_cast<char*>(ws);
  float* delta = reinterpret_cast<float*>(base + L.delta);
  uint16_t* Qp = reinterpret_cast<uint16_t*>(base + L.qp);
  uint16_t* dOp = reinterpret_cast<uint16_t*>(base + L.gp);
  float* lsep = reinterpret_cast<float*>(base + L.lsep);
  float* Dp = reinterpret_cast<float*>(base + L.dp);
  const int Npad = p.prob.N + kPermPad;
  uint32_t* bm = reinterpret_cast<uint32_t*>(base + L.bitmap);
  int32_t* col_cnt = reinterpret_cast<int32_t*>(base + L.col_cnt);
  int32_t* col_ptr = reinterpret_cast<int32_t*>(base + L.col_ptr);
  int32_t* row_idx = reinterpret_cast<int32_t*>(base + L.row_idx);
  const int BH = p.prob.B * p.prob.H;
  const int64_t rows = (int64_t)BH * p.nq, cols = (int64_t)BH * p.nkv;
  hipError_t e;
  bwd_prep_kernel<<<dim3((Npad + 15) / 16, BH), 256, 0, s>>>(
      static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(O),
      static_cast<const uint16_t*>(dO), lse, p.qperm, p.prob.N, Npad, Qp, dOp, lsep, Dp, delta);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = launch_permute_rows(p, K, base + L.kp, s)) != hipSuccess) return e;
  if ((e = launch_permute_rows(p, V, base + L.vp, s)) != hipSuccess) return e;
  csr_bitmap_kernel<<<(unsigned)rows, 256, 0, s>>>(row_ptr, col_idx, p.nkv, L.nwords, bm);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const unsigned cblocks = (unsigned)((cols + 255) / 256);
  csc_kernel<<<cblocks, 256, 0, s>>>(bm, p.nq, p.nkv, L.nwords, cols, false, col_cnt, nullptr,
                                     nullptr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  col_scan_kernel<<<1, 1024, 0, s>>>(col_cnt, cols, col_ptr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  csc_kernel<<<cblocks, 256, 0, s>>>(bm, p.nq, p.nkv, L.nwords, cols, true, nullptr, col_ptr,
                                     row_idx);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  DkdvArgs a{};
  a.Qp = Qp;
  a.Kp = reinterpret_cast<const uint16_t*>(base + L.kp);
  a.Vp = reinterpret_cast<const uint16_t*>(base + L.vp);
  a.dOp = dOp;
  a.lsep = lsep;
  a.Dp = Dp;
  a.Npad = Npad;
  a.col_ptr = col_ptr;
  a.row_idx = row_idx;
  a.qstart = p.qstart;
  a.kvperm = p.kvperm;
  a.kvstart = p.kvstart;
  a.kvitems = p.kvitems;
  a.scale = p.scale;
  a.dK = static_cast<uint16_t*>(dK);
  a.dV = static_cast<uint16_t*>(dV);
  a.n_kvitems = p.n_kvitems;
  a.H = p.prob.H;
  a.N = p.prob.N;
  a.nkv = p.nkv;
  dkdv_kernel<<<dim3(p.n_kvitems, BH), 512, 0, s>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  DqArgs q{};
  q.Q = static_cast<const uint16_t*>(Q);
  q.dO = static_cast<const uint16_t*>(dO);
  q.Kp = a.Kp;
  q.Vp = a.Vp;
  q.lse = lse;
  q.delta = delta;
  q.row_ptr = row_ptr;
  q.col_idx = col_idx;
  q.qperm = p.qperm;
  q.qstart = p.qstart;
  q.kvstart = p.kvstart;
  q.items = p.items;
  q.scale = p.scale;
  q.dQ = static_cast<uint16_t*>(dQ);
  q.n_items = p.n_items;
  q.H = p.prob.H;
  q.N = p.prob.N;
  q.nq = p.nq;
  q.nkv = p.nkv;
  q.Npad = Npad;
  q.fitems = p.fitems;
  q.n_fitems = p.n_fitems;
  dq16_kernel<<<dim3(p.n_fitems, BH), 256, 0, s>>>(q);
  return hipGetLastError();
}
