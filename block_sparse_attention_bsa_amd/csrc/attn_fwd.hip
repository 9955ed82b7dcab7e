// Sparse attention forward (step 4) and the two dense passes of the exact block-mass calibration
// (step 2'), on bf16 matrix cores for d = 128, plus a plain VALU path for fp32 and d = 64.
//
// Forward: every query of block I attends only to the tokens of the kv blocks listed in CSR row I
// (pith.science review of VMoBA, Figure 2 caption: attention over the selected blocks only; "What
// carries the argument": only the highest-scoring blocks contribute their key-value pairs), with
// a FlashAttention-style online softmax. Calibration (LoSA abstract, scholarbro author page):
// exact block attention masses from one dense step, computed as a dense log-sum-exp pass over all
// N keys followed by a dense pass that sums exp(sigma q.k - lse) per (query block, kv block).
//
// KV stream. The kv blocks of a row (the CSR list, or all blocks for the dense passes) are walked
// as a sequence of 32-token chunks: block J contributes ceil(|J| / 32) chunks, the last one
// possibly partial. Chunks are padded per block, not concatenated; K and V are first copied into
// block order (permute_rows_kernel), so a chunk is rows kvstart[J] + 32 * sub .. +32 of that copy
// and no search is needed; 3D tiles clipped at the grid edge (8..128 tokens) waste at most a few
// percent.
//
// MFMA path. One workgroup = 4 wavefronts = 128 query rows of one query block. Per iteration a
// 64-token tile (two chunks) of K (and V for the forward pass) is copied global -> LDS with direct
// 16-byte loads (no staging registers) into one stage while another stage is computed; rows are
// 256 bytes with the 16-byte units XOR-swizzled by a per-row key, so that the MFMA operand reads
// (straight 16-byte and transposing 8-byte) are conflict free. Each wavefront computes
// S^T = K Q^T for its 32 queries with
// v_mfma_f32_32x32x16_bf16 (Q stays in registers as the B operand), so each lane holds 16 scores
// of a single query: the row max needs one cross-half exchange and the row sum none. P^T is
// converted to bf16 in registers and is directly the B operand of O^T += V^T P^T, whose A operand
// comes from two transposing 8-byte LDS reads (ds_read_b64_tr_b16) of the row-major V tile. The
// running max is raised lazily: only when a tile's weights against the current max would sum past
// 2^32, which is detected from the row sum the softmax needs anyway, so no per-tile max is formed
// and the O rescale is rare. When no LSE is requested (an inference call) the fp32 row sum is not
// formed: the sum of the bf16-rounded weights, which O is normalised by, serves as the bound.
#include <climits>

#include "bsa_internal.h"
#include "device_common.h"
#include "kv_cursor.h"

namespace {

// ------------------------------------------------------------------------------- MFMA path

// kFwd: sparse attention with its LSE; kFwdO: sparse attention, output only; kLse / kMass: the
// two dense calibration passes; kMassO: the second calibration pass that also forms the dense
// attention output from the same exact weights.
enum Mode { kFwd = 0, kLse = 1, kMass = 2, kMassO = 3, kFwdO = 4 };


constexpr int kTileKV = 64;                    // kv tokens per iteration (two chunks)
constexpr int kRowBytes = 256;                 // one token row of d = 128 bf16
constexpr int kTileBytes = kTileKV * kRowBytes;
// Lazy rescaling: the running max used for exp2 is only raised when a lane's sum of one tile's
// weights exceeds this, so every weight stays <= 2^32 (bf16 and fp32 hold it, and the fp32 sums
// over any row stay far from overflow) and the O rescale is rare.
constexpr float kSumMax = 4294967296.f;

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

// K and V tiles are row-major in LDS (one 256-byte row per kv token); the 16-byte units of a row
// are XOR-swizzled with lds_key(row) so that the MFMA operand reads hit distinct banks.

struct MfmaArgs {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* V;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const int32_t* qperm;
  const int32_t* qstart;
  const int32_t* kvperm;
  const int32_t* kvstart;
  const int32_t* items;
  const float* scale;
  const float* lse_in;  // kMass, kMassO: per-token log-sum-exp (from the kLse pass)
  uint16_t* O;          // kFwd, kFwdO, kMassO
  float* lse;           // kFwd (required), kMassO (nullable), kLse
  float* part;          // kMass: [bh][item][wave][nkv] per-wave block sums
  int n_items, H, N, nq, nkv;
  int Npad;  // K and V are permuted into block order: [B*H][Npad][d], Npad = N + kPermPad
  // per-token block lists (the TOK variant): [B*H][N][tslots], ascending
  const int32_t* tsel;
  int tslots;
};

// LDS row stride of the per-token lists in the TOK variant (at most 1 + kMaxTokenK blocks).
constexpr int kTokSlots = kMaxTokenK + 1;

// Two LDS stages: tile t is computed while tile t+1 streams in.
// TOK: each query token attends only to the blocks of its own list (VMoBA review: each query
// token scores the block means and keeps its best blocks); the workgroup walks the union of its
// tokens' lists (the CSR row) and masks, per lane, the chunks of blocks its token did not pick.
template <int MODE, bool TOK = false>
__device__ __forceinline__ void attn_mfma_body(const MfmaArgs& a) {
  constexpr int D = 128;
  constexpr bool kDense = MODE == kLse || MODE == kMass || MODE == kMassO;  // all kv blocks
  constexpr bool kPV = MODE == kFwd || MODE == kFwdO || MODE == kMassO;  // O = P V is formed
  constexpr bool kNeedV = kPV;
  constexpr int kStage = kNeedV ? 2 * kTileBytes : kTileBytes;
  __shared__ __attribute__((aligned(1024))) char lds[2 * kStage];
  __shared__ int32_t tlist[TOK ? kAttnRows * kTokSlots : 1];
  char* const lds_a = lds;
  char* const lds_b = lds + kStage;

  const int n_items = a.n_items;
  const int total = n_items * (int)gridDim.y;
  const int lin = xcd_remap(blockIdx.x + blockIdx.y * gridDim.x, total);
  const int bh = lin / n_items, item = lin % n_items;
  const int I = ld_ro(a.items + 2 * item), off = ld_ro(a.items + 2 * item + 1);
  const int q0 = ld_ro(a.qstart + I) + off;
  const int nrows = min(128, ld_ro(a.qstart + I + 1) - q0);
  const int64_t r = (int64_t)bh * a.nq + I;
  const size_t head_off = (size_t)bh * a.N * D;
  const float c2 = ld_ro(a.scale + bh % a.H) * kLog2e;  // sigma_h > 0 (checked at plan creation)

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const bool active = 32 * wave < nrows;  // wave-uniform
  const int l32 = lane & 31, hl = lane >> 5;

  // Q fragments (B operand of S^T = K Q^T): query row 32*wave + l32, d = 16*kc + 8*hl .. +8.
  const int qrow = 32 * wave + l32;
  const bool qvalid = qrow < nrows;
  const int qtok = qvalid ? a.qperm[q0 + qrow] : 0;
  bf16x8_t qf[8];
  {
    const uint4* qp =
        reinterpret_cast<const uint4*>(a.Q + head_off + (size_t)qtok * D + 8 * hl);
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      uint4 v = qvalid ? qp[2 * kc] : make_uint4(0, 0, 0, 0);
      qf[kc] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  f32x16_t oacc[4];  // kFwd: O^T (lane = query, registers = d)
  if constexpr (kPV) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[i][e] = 0.f;
  }
  // l_run: fp32 sum of the weights (for the LSE); lb_run: sum of the same weights rounded to bf16
  // as the PV product uses them (O is normalised by it, an exactly normalised combination)
  // TOK: a finite floor instead of -inf, so that a tile whose chunks this lane's token did not
  // pick (all scores -inf) gives weights 0, not exp2(-inf + inf)
  float m_run = TOK ? -1e30f : -INFINITY, l_run = 0.f, lb_run = 0.f;
  // kMass: log2-domain lse of this lane's query (+inf for padding rows, so they add nothing)
  float nlse2 = 0.f, blk_acc = 0.f;
  if constexpr (MODE == kMass || MODE == kMassO)
    nlse2 = qvalid ? -a.lse_in[(size_t)bh * a.N + qtok] * kLog2e : -INFINITY;

  // Loader role: wave w fills tile rows 16w + 4i + lane/16 (i = 0..3), 16-byte unit lane%16 of
  // the swizzled row, for K (and V), with direct global->LDS copies (no staging registers). K and
  // V arrive permuted into block order ([B*H][Npad][d], see permute_rows_kernel), so a chunk is
  // 32 consecutive rows starting at its position: the per-lane byte offset of each copy is fixed
  // and the chunk's position goes into the scalar base address. Rows past a chunk's end are the
  // next rows of the permuted array (other tokens, or the zero padding after the last block):
  // their scores are masked and their weights are exactly 0.
  const int lchunk = wave >> 1, loff = 16 * (wave & 1), lgrp = lane >> 4;

  Cursor cur;
  cur.slot = kDense ? 0 : ld_ro(a.row_ptr + r);
  cur.end = kDense ? a.nkv : ld_ro(a.row_ptr + r + 1);
  cur.sub = 0;
  cursor_load<kDense>(cur, a.col_idx, a.kvstart);

  const size_t kv_off = (size_t)bh * a.Npad * D;
  const uint16_t* const kbase = a.K + kv_off;
  const uint16_t* const vbase = kNeedV ? a.V + kv_off : a.K;
  uint32_t voff[4];  // byte offset of this lane's copy i within its chunk
#pragma unroll
  for (int i = 0; i < 4; ++i)
    voff[i] = (uint32_t)((loff + 4 * i + lgrp) * kRowBytes) +
              16u * (uint32_t)((lane & 15) ^ lds_key(16 * wave + 4 * i + lgrp));
  // Copies of this wave's 16 rows of the tile (chunks ca, cb) into the stage at LDS address st_m0.
  auto tile_issue = [&](Chunk ca, Chunk cb, uint32_t st_m0) {
    const int pos = (lchunk && cb.nv > 0) ? cb.pos : ca.pos;
    const uint16_t* kb = kbase + (size_t)pos * D;
    const uint16_t* vb = vbase + (size_t)pos * D;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t m0v = st_m0 + (uint32_t)((16 * wave + 4 * i) * kRowBytes);
      lds_dma16_so(kb, voff[i], m0v);
      if constexpr (kNeedV) lds_dma16_so(vb, voff[i], m0v + kTileBytes);
    }
  };

  // Pipeline: tile t (chunks a0, b0) is in LDS and tile t+1 (a1, b1) is copied into the other
  // stage while tile t is computed.
  const uint32_t m0_a = lds_addr(lds_a), m0_b = lds_addr(lds_b);
  Chunk a0 = take_chunk<kDense>(cur, a.col_idx, a.kvstart);
  Chunk b0 = take_chunk<kDense>(cur, a.col_idx, a.kvstart);
  if (a0.nv > 0) tile_issue(a0, b0, m0_a);
  Chunk a1 = take_chunk<kDense>(cur, a.col_idx, a.kvstart);
  Chunk b1 = take_chunk<kDense>(cur, a.col_idx, a.kvstart);
  if constexpr (TOK) {  // the block lists of this item's query rows (INT_MAX past the rows)
    for (int idx = t; idx < kAttnRows * a.tslots; idx += 256) {
      const int row = idx / a.tslots, slot = idx - row * a.tslots;
      int v = INT_MAX;
      if (row < nrows)
        v = a.tsel[((size_t)bh * a.N + a.qperm[q0 + row]) * a.tslots + slot];
      tlist[row * kTokSlots + slot] = v;
    }
  }
  vmem_wait_all();
  __syncthreads();
  // TOK: position in this lane's list and the block there (lists and the CSR row ascend)
  int tptr = 0;
  int tcur = TOK && qvalid ? tlist[qrow * kTokSlots] : INT_MAX;

  // V transposed reads: row 16*kc + 8*sh + 4*hl + (lane%16)/4, column 32*dm + 16*((lane/16)&1)
  // + 4*(lane&3): 16-byte unit 4*dm + 2*((lane/16)&1) + ((lane&3)>>1), 8-byte half (lane&1).
  const int vrow_l = 4 * hl + ((lane & 15) >> 2);
  const int vunit_l = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int vhalf_l = 8 * (lane & 1);

  // One tile: compute tile t from stage `st` while tile t+1 is copied into the other stage (LDS
  // address nx_m0), which tile t-1 used.
  auto step = [&](const char* st, uint32_t nx_m0) {
    // A wavefront whose 32 query rows all lie past the end of the query block (ragged blocks at
    // the grid edge) only takes part in the copies and barriers, leaving its SIMD to the other
    // resident workgroup.
    // S^T for this wave's 32 queries: two 32-kv M blocks (raw, unscaled scores).
    f32x16_t sacc[2];
    // TOK: whether this lane's token picked each chunk's block. A wavefront none of whose tokens
    // picked either skips the tile's matrix and vector work: all its weights would be exactly 0,
    // adding nothing to O or the sums.
    bool pa = true, pb = true, act = active;
    if constexpr (TOK) {
      if (active) {
        auto picked = [&](int J) {
          while (tcur < J) {
            ++tptr;
            tcur = tptr < a.tslots ? tlist[qrow * kTokSlots + tptr] : INT_MAX;
          }
          return tcur == J;
        };
        pa = picked(a0.J);
        pb = b0.nv > 0 && picked(b0.J);
        act = __ballot(pa || pb) != 0ull;
      }
    }
    if (act) {
      // Raised wave priority while the matrix phases issue: the co-resident wavefront (the other
      // workgroup) then fills the gaps with its VALU work instead of competing for issue.
      __builtin_amdgcn_s_setprio(2);
      {
        bf16x8_t kf[2][8];
#pragma unroll
        for (int kc = 0; kc < 8; ++kc)
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) {
            const int row = 32 * mb + l32;
            kf[mb][kc] = *reinterpret_cast<const bf16x8_t*>(st + row * kRowBytes +
                                                            lds_swz(row, 2 * kc + hl));
          }
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int e = 0; e < 16; ++e) sacc[mb][e] = 0.f;
#pragma unroll
        for (int kc = 0; kc < 8; ++kc)
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
            sacc[mb] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[mb][kc], qf[kc], sacc[mb], 0, 0, 0);
        // Keep eight K reads in flight ahead of the MFMAs that consume them (LDS latency exceeds
        // an MFMA's duration): 8 reads, then alternate one MFMA and one read, then the last 8.
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
      }
      __builtin_amdgcn_s_setprio(0);
    }
    // The next tile's copies are issued while the score MFMAs execute.
    const Chunk an = take_chunk<kDense>(cur, a.col_idx, a.kvstart);
    const Chunk bn = take_chunk<kDense>(cur, a.col_idx, a.kvstart);
    if (a1.nv > 0) tile_issue(a1, b1, nx_m0);

    if (act) {
      if (a0.nv < 32 || b0.nv < 32) {  // partial chunk(s): mask padded kv rows
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const int nv = mb ? b0.nv : a0.nv;
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (8 * (e >> 2) + 4 * hl + (e & 3) >= nv) sacc[mb][e] = -INFINITY;
        }
      }
      if constexpr (TOK) {  // chunks of blocks this lane's token did not pick
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          if (!pa) sacc[0][e] = -INFINITY;
          if (!pb) sacc[1][e] = -INFINITY;
        }
      }

      // V^T fragment (d block dm, kv rows 16 kc .. +16) of this tile: two transposing 8-byte LDS
      // reads. The first d block's fragments are read before the weights are formed, so their
      // latency hides behind that VALU work.
      const char* vt = st + kTileBytes;
      auto vfrag = [&](int dm, int kc) {
        const int row_lo = 16 * kc + vrow_l, row_hi = row_lo + 8;
        const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16_t*)((lds_char_t*)vt + row_lo * kRowBytes +
                           lds_swz(row_lo, 4 * dm + vunit_l) + vhalf_l));
        const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16_t*)((lds_char_t*)vt + row_hi * kRowBytes +
                           lds_swz(row_hi, 4 * dm + vunit_l) + vhalf_l));
        const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
        return __builtin_bit_cast(bf16x8_t, make_uint4(l2.x, l2.y, h2.x, h2.y));
      };
      bf16x8_t vf0[4];
      if constexpr (kPV) {
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) vf0[kc] = vfrag(0, kc);
        __builtin_amdgcn_sched_barrier(0);  // keep these reads ahead of the VALU work below
      }
      // P rounded to bf16 (the B operand of the PV product); returns the sum of the rounded
      // weights (one bf16 dot product with (1, 1) per packed word).
      auto pack_weights = [&](const float (&pv)[2][16], bf16x8_t (&pb)[4]) -> float {
        uint32_t pw[2][8];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int e = 0; e < 16; e += 2) pw[mb][e >> 1] = pack_bf16x2(pv[mb][e], pv[mb][e + 1]);
        const bf16x2_t one2 = {(__bf16)1.f, (__bf16)1.f};
        float lb[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 16; ++i)
          lb[i & 3] = __builtin_amdgcn_fdot2_f32_bf16(
              __builtin_bit_cast(bf16x2_t, pw[i >> 3][i & 7]), one2, lb[i & 3], false);
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          const uint32_t* src = &pw[kc >> 1][4 * (kc & 1)];
          pb[kc] = __builtin_bit_cast(bf16x8_t, make_uint4(src[0], src[1], src[2], src[3]));
        }
        return (lb[0] + lb[1]) + (lb[2] + lb[3]);
      };
      // O^T += V^T P^T.
      auto pv_product = [&](const bf16x8_t (&pb)[4]) {
        __builtin_amdgcn_s_setprio(2);
#pragma unroll
        for (int dm = 0; dm < 4; ++dm) {
          bf16x8_t vf[4];
#pragma unroll
          for (int kc = 0; kc < 4; ++kc) vf[kc] = dm == 0 ? vf0[kc] : vfrag(dm, kc);
#pragma unroll
          for (int kc = 0; kc < 4; ++kc)
            oacc[dm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[kc], pb[kc], oacc[dm], 0, 0, 0);
        }
        // Weights first (their VALU work covers the first reads' latency), then the MFMAs with
        // the remaining V reads interleaved, two per MFMA.
        __builtin_amdgcn_sched_group_barrier(0x002, 100, 0);
#pragma unroll
        for (int i = 0; i < 12; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        __builtin_amdgcn_s_setprio(0);
      };

      if constexpr (MODE == kMass || MODE == kMassO) {
        // Exact weights exp(sigma q.k - lse) (the LSE over all N keys is known from the kLse
        // pass). Block sums: one chunk per M block, flushed at block ends; kMassO also forms
        // the dense output O from the same weights.
        float pv[2][16];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int e = 0; e < 16; ++e) pv[mb][e] = __builtin_amdgcn_exp2f(fmaf(sacc[mb][e], c2, nlse2));
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const Chunk& c = mb ? b0 : a0;
          if (c.nv > 0) {
            float cs0 = 0.f, cs1 = 0.f;
#pragma unroll
            for (int e = 0; e < 16; e += 2) {
              cs0 += pv[mb][e];
              cs1 += pv[mb][e + 1];
            }
            blk_acc += cs0 + cs1;
            if (c.last) {
              const float tot = wave_sum_f32(blk_acc);
              if (lane == 0)
                a.part[(((size_t)bh * n_items + item) * 4 + wave) * a.nkv + c.J] = tot;
              blk_acc = 0.f;
            }
          }
        }
        if constexpr (MODE == kMassO) {
          bf16x8_t pb[4];
          lb_run += pack_weights(pv, pb);
          pv_product(pb);
        }
      } else if constexpr (MODE == kFwdO) {
        // As the path below, with the bf16-rounded weights' sum (which O is normalised by) as
        // the only sum: it bounds every weight as well, and no LSE is formed.
        float pv[2][16];
        bf16x8_t pb[4];
        auto weights = [&]() {
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int e = 0; e < 16; ++e)
              pv[mb][e] = __builtin_amdgcn_exp2f(fmaf(sacc[mb][e], c2, -m_run));
          return pack_weights(pv, pb);
        };
        float lsum = weights();
        if (__ballot(!(lsum <= kSumMax)) != 0) {
          asm volatile("");  // keep this a branch
          float sm = fmaxf(sacc[0][0], sacc[1][0]);
#pragma unroll
          for (int e = 1; e < 16; ++e) sm = fmaxf(sm, fmaxf(sacc[0][e], sacc[1][e]));
          const float m_new = fmaxf(m_run, pair_max(sm) * c2);
          const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
          lb_run *= alpha;
#pragma unroll
          for (int dm = 0; dm < 4; ++dm)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[dm][e] *= alpha;
          m_run = m_new;
          lsum = weights();
        }
        lb_run += lsum;
        pv_product(pb);
      } else {
        // Weights p = exp2(c2 * s - m_run) against the running max as it stands, and this
        // lane's partial sum. No tile max is formed on this path: the sum bounds every weight,
        // and while it stays <= kSumMax the weights (bf16 for the PV product) and the fp32 sums
        // cannot overflow. Otherwise (the first tile, where m_run = -inf gives +inf weights, or
        // a tile far above the running max) the running max is raised to the exact max of
        // c2 * s so far and the tile's weights are formed again.
        float pv[2][16];
        auto weights = [&]() {
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int e = 0; e < 16; ++e)
              pv[mb][e] = __builtin_amdgcn_exp2f(fmaf(sacc[mb][e], c2, -m_run));
          float ls[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) ls[i] = pv[0][i];
#pragma unroll
          for (int i = 4; i < 32; ++i) ls[i & 3] += pv[i >> 4][i & 15];
          return (ls[0] + ls[1]) + (ls[2] + ls[3]);
        };
        float lsum = weights();
        if (__ballot(!(lsum <= kSumMax)) != 0) {
          asm volatile("");  // keep this a branch: the compiler would otherwise form both paths
          // exact tile max of c2 * s (every tile has an unmasked kv row in one of the halves)
          float sm = fmaxf(sacc[0][0], sacc[1][0]);
#pragma unroll
          for (int e = 1; e < 16; ++e) sm = fmaxf(sm, fmaxf(sacc[0][e], sacc[1][e]));
          const float m_new = fmaxf(m_run, pair_max(sm) * c2);
          const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the first tile
          l_run *= alpha;
          lb_run *= alpha;
          if constexpr (MODE == kFwd) {
#pragma unroll
            for (int dm = 0; dm < 4; ++dm)
#pragma unroll
              for (int e = 0; e < 16; ++e) oacc[dm][e] *= alpha;
          }
          m_run = m_new;
          lsum = weights();
        }
        l_run += lsum;
        if constexpr (MODE == kFwd) {
          bf16x8_t pb[4];
          lb_run += pack_weights(pv, pb);
          pv_product(pb);
        }
      }
    }
    // Tile t+1 must be in LDS before the barrier that opens step t+1.
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

  if constexpr (MODE == kMass) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (!qvalid) return;
  if constexpr (kPV) {
    const float lb_tot = lb_run + __shfl_xor(lb_run, 32, 64);  // both halves of the wave
    const float inv = lb_tot > 0.f ? 1.f / lb_tot : 0.f;
    uint16_t* op = a.O + head_off + (size_t)qtok * D;
#pragma unroll
    for (int dm = 0; dm < 4; ++dm)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 pk;
        pk.x = pack_bf16x2(oacc[dm][4 * g] * inv, oacc[dm][4 * g + 1] * inv);
        pk.y = pack_bf16x2(oacc[dm][4 * g + 2] * inv, oacc[dm][4 * g + 3] * inv);
        *reinterpret_cast<uint2*>(op + 32 * dm + 8 * g + 4 * hl) = pk;
      }
  }
  if constexpr (MODE == kMassO) {
    // the dense step's LSE is the kLse pass's (the weights above are normalised by it)
    if (a.lse && hl == 0) a.lse[(size_t)bh * a.N + qtok] = a.lse_in[(size_t)bh * a.N + qtok];
    return;
  }
  if constexpr (MODE == kFwdO) return;
  if (hl == 0)
    a.lse[(size_t)bh * a.N + qtok] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
}

// Two waves per SIMD: two workgroups share a CU.
template <int MODE>
__global__ __launch_bounds__(256, 2) void attn_mfma_d128(const MfmaArgs a) {
  attn_mfma_body<MODE>(a);
}

template <int MODE>
__global__ __launch_bounds__(256, 2) void attn_mfma_d128_tok(const MfmaArgs a) {
  attn_mfma_body<MODE, true>(a);
}

// M[bh, I, J] = (sum over I's work items and their active waves of the block sums) / |I|, in fp64
// and in a fixed order. Wave w of an item is active iff it holds a valid query row (32 w < rows).
__global__ __launch_bounds__(256) void mass_combine_kernel(const float* __restrict__ part,
                                                           const int32_t* __restrict__ qstart,
                                                           const int32_t* __restrict__ qitem0,
                                                           const int32_t* __restrict__ items,
                                                           int n_items, int nq, int nkv,
                                                           float* __restrict__ M) {
  const int I = blockIdx.x, bh = blockIdx.y;
  const int i0 = qitem0[I], i1 = qitem0[I + 1];
  const int size = qstart[I + 1] - qstart[I];
  const double inv = 1.0 / (double)size;
  for (int J = threadIdx.x; J < nkv; J += 256) {
    double s = 0.0;
    for (int it = i0; it < i1; ++it) {
      const int rows = min(128, size - items[2 * it + 1]);
      for (int w = 0; 32 * w < rows; ++w)
        s += part[(((size_t)bh * n_items + it) * 4 + w) * nkv + J];
    }
    M[((size_t)bh * nq + I) * nkv + J] = (float)(s * inv);
  }
}

// dst[bh][pos] = src[bh][perm[pos]] for pos < N (256-byte rows of d = 128 bf16) and zero rows for
// N <= pos < Npad: K or V in block order, so that the 32 rows of a chunk are contiguous and the
// rows past any chunk's end exist. One 16-byte unit per thread, 16 rows per workgroup.
__global__ __launch_bounds__(256) void permute_rows_kernel(const uint16_t* __restrict__ src,
                                                           const int32_t* __restrict__ perm,
                                                           int N, int Npad,
                                                           uint16_t* __restrict__ dst) {
  const int row = blockIdx.x * 16 + (threadIdx.x >> 4), unit = threadIdx.x & 15;
  if (row >= Npad) return;
  const size_t bh = blockIdx.y;
  uint4 v = make_uint4(0, 0, 0, 0);
  if (row < N)
    v = *reinterpret_cast<const uint4*>(src + (bh * N + (size_t)perm[row]) * 128 + 8 * unit);
  *reinterpret_cast<uint4*>(dst + (bh * Npad + (size_t)row) * 128 + 8 * unit) = v;
}

MfmaArgs mfma_args(const bsa_plan& p) {
  MfmaArgs a{};
  a.qperm = p.qperm;
  a.qstart = p.qstart;
  a.kvperm = p.kvperm;
  a.kvstart = p.kvstart;
  a.items = p.items;
  a.scale = p.scale;
  a.n_items = p.n_items;
  a.H = p.prob.H;
  a.N = p.prob.N;
  a.nq = p.nq;
  a.nkv = p.nkv;
  a.Npad = p.prob.N + kPermPad;
  return a;
}

// ------------------------------------------------------------------------------- VALU path

template <typename T>
__device__ __forceinline__ float ld_elem(const T* p);
template <>
__device__ __forceinline__ float ld_elem<float>(const float* p) {
  return *p;
}
template <>
__device__ __forceinline__ float ld_elem<uint16_t>(const uint16_t* p) {
  return __uint_as_float((uint32_t)*p << 16);
}
template <typename T>
__device__ __forceinline__ void st_elem(T* p, float v);
template <>
__device__ __forceinline__ void st_elem<float>(float* p, float v) {
  *p = v;
}
template <>
__device__ __forceinline__ void st_elem<uint16_t>(uint16_t* p, float v) {
  *p = (uint16_t)(pack_bf16x2(v, 0.f) & 0xffffu);
}

// One thread per query row (128 rows per workgroup); KV staged chunk by chunk in LDS as fp32;
// exact expf. Used for fp32 inputs and for bf16 with d = 64.
template <typename T, int D>
__global__ __launch_bounds__(128) void attn_fwd_valu(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    const int32_t* __restrict__ qperm, const int32_t* __restrict__ qstart,
    const int32_t* __restrict__ kvperm, const int32_t* __restrict__ kvstart,
    const int32_t* __restrict__ items, int n_items, const float* __restrict__ scale, int H,
    int N, int nq, T* __restrict__ O, float* __restrict__ lse) {
  __shared__ float ks[32][D + 1];
  __shared__ float vs[32][D + 1];
  const int bh = blockIdx.y, item = blockIdx.x;
  const int I = items[2 * item], off = items[2 * item + 1];
  const int q0 = qstart[I] + off;
  const int nrows = min(128, qstart[I + 1] - q0);
  const int64_t r = (int64_t)bh * nq + I;
  const size_t head_off = (size_t)bh * N * D;
  const float sig = scale[bh % H];
  const int t = threadIdx.x;
  const bool qvalid = t < nrows;
  const int qtok = qvalid ? qperm[q0 + t] : 0;
  float q[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = qvalid ? ld_elem(Q + head_off + (size_t)qtok * D + d) : 0.f;
    acc[d] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  Cursor cur;
  cur.slot = row_ptr[r];
  cur.end = row_ptr[r + 1];
  cur.sub = 0;
  cursor_load<false>(cur, col_idx, kvstart);
  while (true) {
    const Chunk c = take_chunk<false>(cur, col_idx, kvstart);
    if (c.nv == 0) break;
    __syncthreads();
    for (int e = t; e < 32 * D; e += 128) {
      const int row = e / D, d = e % D;
      float kv = 0.f, vv = 0.f;
      if (row < c.nv) {
        const size_t o = head_off + (size_t)kvperm[c.pos + row] * D + d;
        kv = ld_elem(K + o);
        vv = ld_elem(V + o);
      }
      ks[row][d] = kv;
      vs[row][d] = vv;
    }
    __syncthreads();
    float s[32];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) dot = fmaf(q[d], ks[j][d], dot);
      s[j] = j < c.nv ? dot * sig : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float alpha = expf(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] *= alpha;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const float p = expf(s[j] - m_new);
      l_run += p;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(p, vs[j][d], acc[d]);
    }
    m_run = m_new;
  }
  if (!qvalid) return;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  T* op = O + head_off + (size_t)qtok * D;
#pragma unroll
  for (int d = 0; d < D; ++d) st_elem(op + d, acc[d] * inv);
  if (lse) lse[(size_t)bh * N + qtok] = l_run > 0.f ? m_run + logf(l_run) : -INFINITY;
}

template <typename T, int D>
hipError_t launch_valu(const bsa_plan& p, const void* Q, const void* K, const void* V,
                       const int32_t* row_ptr, const int32_t* col_idx, void* O, float* lse,
                       hipStream_t s) {
  dim3 grid(p.n_items, p.prob.B * p.prob.H);
  attn_fwd_valu<T, D><<<grid, 128, 0, s>>>(
      static_cast<const T*>(Q), static_cast<const T*>(K), static_cast<const T*>(V), row_ptr,
      col_idx, p.qperm, p.qstart, p.kvperm, p.kvstart, p.items, p.n_items, p.scale, p.prob.H,
      p.prob.N, p.nq, static_cast<T*>(O), lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_permute_rows(const bsa_plan& p, const void* src, void* dst, hipStream_t s) {
  const int N = p.prob.N, Npad = N + kPermPad;
  permute_rows_kernel<<<dim3((Npad + 15) / 16, p.prob.B * p.prob.H), 256, 0, s>>>(
      static_cast<const uint16_t*>(src), p.kvperm, N, Npad, static_cast<uint16_t*>(dst));
  return hipGetLastError();
}

hipError_t launch_attn_fwd(const bsa_plan& p, const void* Q, const void* K, const void* V,
                           const int32_t* row_ptr, const int32_t* col_idx, void* O, float* lse,
                           void* ws, hipStream_t s) {
  if (p.prob.dtype == BSA_BF16 && p.prob.d == 128) {
    const FwdWs L = fwd_ws_layout(p);
    char* base = static_cast<char*>(ws);
    hipError_t e = launch_permute_rows(p, K, base + L.kp, s);
    if (e == hipSuccess) e = launch_permute_rows(p, V, base + L.vp, s);
    if (e != hipSuccess) return e;
    MfmaArgs a = mfma_args(p);
    a.Q = static_cast<const uint16_t*>(Q);
    a.K = reinterpret_cast<const uint16_t*>(base + L.kp);
    a.V = reinterpret_cast<const uint16_t*>(base + L.vp);
    a.row_ptr = row_ptr;
    a.col_idx = col_idx;
    a.O = static_cast<uint16_t*>(O);
    a.lse = lse;
    // gridDim.x * gridDim.y is exactly n_items * B * H (the XCD remap is a bijection on it).
    const dim3 grid(p.n_items, p.prob.B * p.prob.H);
    if (lse)
      attn_mfma_d128<kFwd><<<grid, 256, 0, s>>>(a);
    else
      attn_mfma_d128<kFwdO><<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
  }
  if (p.prob.dtype == BSA_BF16)
    return launch_valu<uint16_t, 64>(p, Q, K, V, row_ptr, col_idx, O, lse, s);
  if (p.prob.d == 128) return launch_valu<float, 128>(p, Q, K, V, row_ptr, col_idx, O, lse, s);
  return launch_valu<float, 64>(p, Q, K, V, row_ptr, col_idx, O, lse, s);
}

hipError_t launch_attn_fwd_tokens(const bsa_plan& p, const void* Q, const void* K, const void* V,
                                  const int32_t* row_ptr, const int32_t* col_idx,
                                  const int32_t* sel, int nslots, void* O, float* lse, void* ws,
                                  hipStream_t s) {
  const FwdWs L = fwd_ws_layout(p);
  char* base = static_cast<char*>(ws);
  hipError_t e = launch_permute_rows(p, K, base + L.kp, s);
  if (e == hipSuccess) e = launch_permute_rows(p, V, base + L.vp, s);
  if (e != hipSuccess) return e;
  MfmaArgs a = mfma_args(p);
  a.Q = static_cast<const uint16_t*>(Q);
  a.K = reinterpret_cast<const uint16_t*>(base + L.kp);
  a.V = reinterpret_cast<const uint16_t*>(base + L.vp);
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.O = static_cast<uint16_t*>(O);
  a.lse = lse;
  a.tsel = sel;
  a.tslots = nslots;
  const dim3 grid(p.n_items, p.prob.B * p.prob.H);
  if (lse)
    attn_mfma_d128_tok<kFwd><<<grid, 256, 0, s>>>(a);
  else
    attn_mfma_d128_tok<kFwdO><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_calibrate(const bsa_plan& p, const void* Q, const void* K, const void* V,
                            float* M, void* O, float* lse_out, void* ws, hipStream_t s) {
  const CalibWs L = calib_ws_layout(p);
  char* base = static_cast<char*>(ws);
  float* lse = reinterpret_cast<float*>(base + L.lse);
  float* part = reinterpret_cast<float*>(base + L.part);
  hipError_t e = launch_permute_rows(p, K, base + L.kp, s);
  if (e == hipSuccess && V) e = launch_permute_rows(p, V, base + L.vp, s);
  if (e != hipSuccess) return e;
  const dim3 grid(p.n_items, p.prob.B * p.prob.H);
  MfmaArgs a = mfma_args(p);
  a.Q = static_cast<const uint16_t*>(Q);
  a.K = reinterpret_cast<const uint16_t*>(base + L.kp);
  a.lse = lse;
  attn_mfma_d128<kLse><<<grid, 256, 0, s>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  a.lse = nullptr;
  a.lse_in = lse;
  a.part = part;
  if (V) {  // the masses and the dense output from the same weights
    a.V = reinterpret_cast<const uint16_t*>(base + L.vp);
    a.O = static_cast<uint16_t*>(O);
    a.lse = lse_out;
    attn_mfma_d128<kMassO><<<grid, 256, 0, s>>>(a);
  } else {
    attn_mfma_d128<kMass><<<grid, 256, 0, s>>>(a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  mass_combine_kernel<<<dim3(p.nq, p.prob.B * p.prob.H), 256, 0, s>>>(
      part, p.qstart, p.qitem0, p.items, p.n_items, p.nq, p.nkv, M);
  return hipGetLastError();
}

