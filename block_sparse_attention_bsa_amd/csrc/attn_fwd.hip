// Sparse attention forward (step 4): every query of block I attends only to the tokens of the kv
// blocks listed in CSR row I (pith.science review of VMoBA, Figure 2 caption: attention over the
// selected blocks only; "What carries the argument": only the highest-scoring blocks contribute
// their key-value pairs). Online softmax in the FlashAttention style.
//
// KV stream. The selected blocks of a row are walked as a sequence of 32-token chunks: block J
// contributes ceil(|J| / 32) chunks, the last one possibly partial. Chunks are padded per block,
// not concatenated, so each chunk's token ids are perm[kvstart[J] + 32 * sub + r] and no search is
// needed; 3D tiles clipped at the grid edge (8..128 tokens) waste at most a few percent.
//
// bf16, d = 128 (MFMA path). One workgroup = 4 wavefronts = 128 query rows of one query block.
// Per iteration it gathers a 64-token KV tile (two chunks) into one of two LDS stages: K
// row-major with a 16-byte row pad, V transposed (d-major, kv permuted within groups of 16,
// 16-byte units XOR-swizzled by row) so that each MFMA operand is one conflict-free 16-byte read. Each wavefront computes S^T = K Q^T for its 32 queries with
// v_mfma_f32_32x32x16_bf16 (Q stays in registers as the B operand), so that each lane holds 16
// scores of a single query: the row max needs one cross-half exchange, the row sum none. P^T is
// converted to bf16 in registers and used directly as the B operand of O^T += V^T P^T. While tile t
// is computed from one LDS stage, tile t+1 is written to the other from registers, the K/V data
// of tile t+2 and the token ids of tile t+3 are in flight; one barrier per tile. The running max
// is raised lazily (only when it grows by more than 2^8), so the O rescale is rare.
#include "bsa_internal.h"
#include "device_common.h"

namespace {

// ------------------------------------------------------------------------------- KV cursor

struct Cursor {
  int slot, end, sub, base, size;  // position in col_idx, block token base and size
};

__device__ __forceinline__ void cursor_load(Cursor& c, const int32_t* __restrict__ col_idx,
                                            const int32_t* __restrict__ kvstart) {
  if (c.slot < c.end) {
    const int J = col_idx[c.slot];
    c.base = kvstart[J];
    c.size = kvstart[J + 1] - c.base;
  } else {
    c.base = 0;
    c.size = 0;
  }
}

__device__ __forceinline__ void cursor_next(Cursor& c, const int32_t* __restrict__ col_idx,
                                            const int32_t* __restrict__ kvstart) {
  if (c.slot >= c.end) return;
  ++c.sub;
  if (32 * c.sub >= c.size) {
    ++c.slot;
    c.sub = 0;
    cursor_load(c, col_idx, kvstart);
  }
}

// One chunk: first token position in perm and number of valid rows (0 = past the end).
struct Chunk {
  int pos, nv;
};

__device__ __forceinline__ Chunk take_chunk(Cursor& c, const int32_t* __restrict__ col_idx,
                                            const int32_t* __restrict__ kvstart) {
  Chunk k;
  if (c.slot < c.end) {
    k.pos = c.base + 32 * c.sub;
    k.nv = min(32, c.size - 32 * c.sub);
  } else {
    k.pos = 0;
    k.nv = 0;
  }
  cursor_next(c, col_idx, kvstart);
  return k;
}

// ------------------------------------------------------------------------------- MFMA path

constexpr int kTileKV = 64;                    // kv tokens per iteration (two chunks)
constexpr int kRowBytes = 256;                 // one token row of d = 128 bf16
constexpr int kTileBytes = kTileKV * kRowBytes;
constexpr int kStage = 2 * kTileBytes;         // K tile then V tile
// Lazy rescaling: the running max used for exp2 is only raised when a tile's max exceeds it by
// more than this (log2 units), so P stays <= 2^8 and the O rescale is rare.
constexpr float kRescaleSlack = 8.f;

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
typedef __attribute__((address_space(3))) char lds_char_t;

// K and V tiles are row-major in LDS (one 256-byte row per kv token); the 16-byte units of a row
// are XOR-swizzled by the row index so that the MFMA operand reads hit distinct banks.
__device__ __forceinline__ int swz(int row, int unit) { return (unit ^ (row & 15)) << 4; }

__device__ __forceinline__ void wait_vmem_all() {
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0); expcnt and lgkmcnt left unconstrained
}

__global__ __launch_bounds__(256, 2) void attn_fwd_mfma_d128(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col_idx, const int32_t* __restrict__ qperm,
    const int32_t* __restrict__ qstart, const int32_t* __restrict__ kvperm,
    const int32_t* __restrict__ kvstart, const int32_t* __restrict__ items, int n_items,
    const float* __restrict__ scale, int H, int N, int nq, uint16_t* __restrict__ O,
    float* __restrict__ lse) {
  constexpr int D = 128;
  __shared__ __attribute__((aligned(1024))) char lds_a[kStage];
  __shared__ __attribute__((aligned(1024))) char lds_b[kStage];

  const int total = n_items * (int)gridDim.y;
  const int lin = xcd_remap(blockIdx.x + blockIdx.y * gridDim.x, total);
  const int bh = lin / n_items, item = lin % n_items;
  const int I = items[2 * item], off = items[2 * item + 1];
  const int q0 = qstart[I] + off;
  const int nrows = min(128, qstart[I + 1] - q0);
  const int64_t r = (int64_t)bh * nq + I;
  const size_t head_off = (size_t)bh * N * D;
  const float c2 = scale[bh % H] * kLog2e;  // sigma_h > 0 (checked at plan creation)

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int l32 = lane & 31, hl = lane >> 5;

  // Q fragments (B operand of S^T = K Q^T): query row 32*wave + l32, d = 16*kc + 8*hl .. +8.
  const int qrow = 32 * wave + l32;
  const bool qvalid = qrow < nrows;
  const int qtok = qvalid ? qperm[q0 + qrow] : 0;
  bf16x8_t qf[8];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(Q + head_off + (size_t)qtok * D + 8 * hl);
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      uint4 v = qvalid ? qp[2 * kc] : make_uint4(0, 0, 0, 0);
      qf[kc] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  f32x16_t oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[i][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // Loader role: wave w fills tile rows 16w + 4i + lane/16 (i = 0..3), 16-byte unit lane%16 of
  // the swizzled row, for K and for V, with direct global->LDS loads (no staging registers).
  // Rows past a chunk's end repeat the chunk's first token: their scores are masked and their
  // probabilities are exactly 0, so any finite row will do.
  const int lrow0 = 16 * wave + (lane >> 4);
  const int lchunk = wave >> 1;

  Cursor cur;
  cur.slot = row_ptr[r];
  cur.end = row_ptr[r + 1];
  cur.sub = 0;
  cursor_load(cur, col_idx, kvstart);

  auto tile_ids = [&](Chunk a, Chunk b, int* ids) {
    const Chunk c = lchunk ? b : a;
    const Chunk c0 = a;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = (lrow0 + 4 * i) & 31;
      const int pos = c.nv > 0 ? c.pos + (rr < c.nv ? rr : 0) : c0.pos;
      ids[i] = kvperm[pos];
    }
  };
  auto tile_issue = [&](const int* ids, char* st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int lunit = (lane & 15) ^ ((lrow0 + 4 * i) & 15);  // logical unit at this position
      const size_t o = head_off + (size_t)ids[i] * D + 8 * lunit;
      char* dst = st + (16 * wave + 4 * i) * kRowBytes;
      __builtin_amdgcn_global_load_lds(K + o, dst, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(V + o, dst + kTileBytes, 16, 0, 0);
    }
  };

  // Pipeline: LDS stage buf holds tile t; tile t+1 is being loaded into the other stage; ids
  // hold the token ids of tile t+2.
  Chunk a0 = take_chunk(cur, col_idx, kvstart), b0 = take_chunk(cur, col_idx, kvstart);
  int ids[4];
  if (a0.nv > 0) {
    tile_ids(a0, b0, ids);
    tile_issue(ids, lds_a);
  }
  Chunk a1 = take_chunk(cur, col_idx, kvstart), b1 = take_chunk(cur, col_idx, kvstart);
  if (a1.nv > 0) tile_ids(a1, b1, ids);
  wait_vmem_all();
  __syncthreads();

  // Per-lane read offsets (bytes within a stage).
  const int krow0 = l32;                       // K row for M block mb: 32*mb + l32
  // V transposed reads: row 16*kc + 8*sh + 4*hl + (lane%16)/4, column 32*dm + 16*((lane/16)&1)
  // + 4*(lane&3): 16-byte unit 4*dm + 2*((lane/16)&1) + ((lane&3)>>1), 8-byte half (lane&1).
  const int vrow_l = 4 * hl + ((lane & 15) >> 2);
  const int vunit_l = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int vhalf_l = 8 * (lane & 1);

  // One tile: compute from stage `st` while the next tile streams into `nx`. The two stages
  // are distinct arrays so that the compiler can tell the streamed writes never alias the reads.
  auto step = [&](const char* st, char* nx) {
    if (a1.nv > 0) tile_issue(ids, nx);
    const Chunk a2 = take_chunk(cur, col_idx, kvstart), b2 = take_chunk(cur, col_idx, kvstart);
    if (a2.nv > 0) tile_ids(a2, b2, ids);

    // S^T for this wave's 32 queries: two 32-kv M blocks (raw, unscaled scores).
    f32x16_t sacc[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int row = 32 * mb + krow0;
      const char* kp = st + row * kRowBytes;
      bf16x8_t kf[8];
#pragma unroll
      for (int kc = 0; kc < 8; ++kc)
        kf[kc] = *reinterpret_cast<const bf16x8_t*>(kp + swz(row, 2 * kc + hl));
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[mb][e] = 0.f;
#pragma unroll
      for (int kc = 0; kc < 8; ++kc)
        sacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kc], qf[kc], sacc[mb], 0, 0, 0);
    }
    if (a0.nv < 32 || b0.nv < 32) {  // partial chunk(s): mask padded kv rows
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int nv = mb ? b0.nv : a0.nv;
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (8 * (e >> 2) + 4 * hl + (e & 3) >= nv) sacc[mb][e] = -INFINITY;
      }
    }
    float mx0 = fmaxf(sacc[0][0], sacc[0][1]), mx1 = fmaxf(sacc[1][0], sacc[1][1]);
#pragma unroll
    for (int e = 2; e < 16; e += 2) {
      mx0 = fmaxf(mx0, fmaxf(sacc[0][e], sacc[0][e + 1]));
      mx1 = fmaxf(mx1, fmaxf(sacc[1][e], sacc[1][e + 1]));
    }
    float mx = fmaxf(mx0, mx1);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * c2;
    const bool grow = mx > m_run + kRescaleSlack;
    if (__ballot(grow) != 0) {
      const float m_new = grow ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dm = 0; dm < 4; ++dm)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[dm][e] *= alpha;
      m_run = m_new;
    }
    const float nm = -m_run;
    float ls[4] = {0.f, 0.f, 0.f, 0.f};
    bf16x8_t pb[4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[mb][e], c2, nm));
        ls[e & 3] += p;
        pb[2 * mb + (e >> 3)][e & 7] = (__bf16)p;
      }
    l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
    // O^T += V^T P^T; each V^T fragment is two transposing 8-byte LDS reads.
    const char* vt = st + kTileBytes;
#pragma unroll
    for (int dm = 0; dm < 4; ++dm) {
      bf16x8_t vf[4];
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        v4i16_t lo, hi;
        {
          const int row = 16 * kc + vrow_l;
          lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4i16_t*)((lds_char_t*)vt + row * kRowBytes + swz(row, 4 * dm + vunit_l) +
                             vhalf_l));
        }
        {
          const int row = 16 * kc + 8 + vrow_l;
          hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4i16_t*)((lds_char_t*)vt + row * kRowBytes + swz(row, 4 * dm + vunit_l) +
                             vhalf_l));
        }
        const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
        vf[kc] = __builtin_bit_cast(bf16x8_t, make_uint4(l2.x, l2.y, h2.x, h2.y));
      }
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
        oacc[dm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[kc], pb[kc], oacc[dm], 0, 0, 0);
    }
    wait_vmem_all();
    __syncthreads();
    a0 = a1;
    b0 = b1;
    a1 = a2;
    b1 = b2;
    };
  while (true) {
    if (a0.nv <= 0) break;
    step(lds_a, lds_b);
    if (a0.nv <= 0) break;
    step(lds_b, lds_a);
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (!qvalid) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  uint16_t* op = O + head_off + (size_t)qtok * D;
#pragma unroll
  for (int dm = 0; dm < 4; ++dm)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint2 pk;
      pk.x = pack_bf16x2(oacc[dm][4 * g] * inv, oacc[dm][4 * g + 1] * inv);
      pk.y = pack_bf16x2(oacc[dm][4 * g + 2] * inv, oacc[dm][4 * g + 3] * inv);
      *reinterpret_cast<uint2*>(op + 32 * dm + 8 * g + 4 * hl) = pk;
    }
  if (lse && hl == 0)
    lse[(size_t)bh * N + qtok] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
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
  cursor_load(cur, col_idx, kvstart);
  while (true) {
    const Chunk c = take_chunk(cur, col_idx, kvstart);
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

hipError_t launch_attn_fwd(const bsa_plan& p, const void* Q, const void* K, const void* V,
                           const int32_t* row_ptr, const int32_t* col_idx, void* O, float* lse,
                           hipStream_t s) {
  if (p.prob.dtype == BSA_BF16 && p.prob.d == 128) {
    const int BH = p.prob.B * p.prob.H;
    // Flattened (item, head) space; gridDim.x * gridDim.y must equal n_items * BH exactly.
    dim3 grid(p.n_items, BH);
    attn_fwd_mfma_d128<<<grid, 256, 0, s>>>(
        static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(K),
        static_cast<const uint16_t*>(V), row_ptr, col_idx, p.qperm, p.qstart, p.kvperm,
        p.kvstart, p.items, p.n_items, p.scale, p.prob.H, p.prob.N, p.nq,
        static_cast<uint16_t*>(O), lse);
    return hipGetLastError();
  }
  if (p.prob.dtype == BSA_BF16) return launch_valu<uint16_t, 64>(p, Q, K, V, row_ptr, col_idx, O, lse, s);
  if (p.prob.d == 128) return launch_valu<float, 128>(p, Q, K, V, row_ptr, col_idx, O, lse, s);
  return launch_valu<float, 64>(p, Q, K, V, row_ptr, col_idx, O, lse, s);
}
