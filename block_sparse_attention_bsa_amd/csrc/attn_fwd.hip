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
// Per iteration it gathers a 64-token KV tile (two chunks) into LDS: K row-major with a 16-byte
// row pad, V transposed (d-major) with an XOR swizzle of 8-byte units so that the MFMA operand
// reads are bank-conflict free. Each wavefront computes S^T = K Q^T for its 32 queries with
// v_mfma_f32_32x32x16_bf16 (Q stays in registers as the B operand), so that each lane holds 16
// scores of a single query: the row max needs one cross-half exchange, the row sum none. P^T is
// converted to bf16 in registers and used directly as the B operand of O^T += V^T P^T. Token ids
// of tile t+2 and the K/V data of tile t+1 are in flight while tile t is computed.
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

constexpr int kKStride = 272;   // bytes per K row in LDS: 256 + 16 pad
constexpr int kTileKV = 64;     // kv tokens per iteration (two chunks)

__device__ __forceinline__ int vt_offset(int d, int unit) {  // byte offset of a 4-kv unit
  return d * 128 + ((unit ^ ((d >> 1) & 15)) << 3);
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
  __shared__ __attribute__((aligned(16))) char k_lds[kTileKV * kKStride];
  __shared__ __attribute__((aligned(16))) char vt_lds[D * kTileKV * 2];

  const int total = n_items * (int)gridDim.y;
  const int lin = xcd_remap(blockIdx.x + blockIdx.y * gridDim.x, total);
  const int bh = lin / n_items, item = lin % n_items;
  const int I = items[2 * item], off = items[2 * item + 1];
  const int q0 = qstart[I] + off;
  const int nrows = min(128, qstart[I + 1] - q0);
  const int64_t r = (int64_t)bh * nq + I;
  const size_t head_off = (size_t)bh * N * D;
  const float c2 = scale[bh % H] * kLog2e;

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

  // Loader role: 4 consecutive kv rows (4*quad ..) x 8 d values (8*dseg ..).
  const int dseg = t & 15, quad = t >> 4, half = quad >> 3, r0 = (4 * quad) & 31;

  Cursor cur;
  cur.slot = row_ptr[r];
  cur.end = row_ptr[r + 1];
  cur.sub = 0;
  cursor_load(cur, col_idx, kvstart);

  auto tile_ids = [&](Chunk a, Chunk b, int* ids) {
    const Chunk c = half ? b : a;
#pragma unroll
    for (int u = 0; u < 4; ++u) ids[u] = (r0 + u < c.nv) ? kvperm[c.pos + r0 + u] : -1;
  };
  uint4 kreg[4], vreg[4];
  auto tile_load = [&](const int* ids) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (ids[u] >= 0) {
        const size_t o = head_off + (size_t)ids[u] * D + 8 * dseg;
        kreg[u] = *reinterpret_cast<const uint4*>(K + o);
        vreg[u] = *reinterpret_cast<const uint4*>(V + o);
      } else {
        kreg[u] = make_uint4(0, 0, 0, 0);
        vreg[u] = make_uint4(0, 0, 0, 0);
      }
    }
  };

  Chunk a0 = take_chunk(cur, col_idx, kvstart), b0 = take_chunk(cur, col_idx, kvstart);
  int ids[4];
  tile_ids(a0, b0, ids);
  tile_load(ids);
  Chunk a1 = take_chunk(cur, col_idx, kvstart), b1 = take_chunk(cur, col_idx, kvstart);
  tile_ids(a1, b1, ids);

  while (a0.nv > 0) {
    __syncthreads();
    // Stage tile t: K row-major, V transposed.
#pragma unroll
    for (int u = 0; u < 4; ++u)
      *reinterpret_cast<uint4*>(k_lds + (4 * quad + u) * kKStride + 16 * dseg) = kreg[u];
    {
      const uint32_t w0[4] = {vreg[0].x, vreg[0].y, vreg[0].z, vreg[0].w};
      const uint32_t w1[4] = {vreg[1].x, vreg[1].y, vreg[1].z, vreg[1].w};
      const uint32_t w2[4] = {vreg[2].x, vreg[2].y, vreg[2].z, vreg[2].w};
      const uint32_t w3[4] = {vreg[3].x, vreg[3].y, vreg[3].z, vreg[3].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int d = 8 * dseg + i;
        uint2 pk;
        if (i & 1) {
          pk.x = (w0[i >> 1] >> 16) | (w1[i >> 1] & 0xffff0000u);
          pk.y = (w2[i >> 1] >> 16) | (w3[i >> 1] & 0xffff0000u);
        } else {
          pk.x = (w0[i >> 1] & 0xffffu) | (w1[i >> 1] << 16);
          pk.y = (w2[i >> 1] & 0xffffu) | (w3[i >> 1] << 16);
        }
        *reinterpret_cast<uint2*>(vt_lds + vt_offset(d, quad)) = pk;
      }
    }
    __syncthreads();

    // Tile t+1 data and tile t+2 ids in flight during the compute of tile t.
    const int nvA = a0.nv, nvB = b0.nv;
    tile_load(ids);
    Chunk a2 = take_chunk(cur, col_idx, kvstart), b2 = take_chunk(cur, col_idx, kvstart);
    tile_ids(a2, b2, ids);

    // S^T for this wave's 32 queries: two 32-kv M blocks.
    f32x16_t sacc[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[mb][e] = 0.f;
      const char* kp = k_lds + (32 * mb + l32) * kKStride + 16 * hl;
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) {
        const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(kp + 32 * kc);
        sacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[kc], sacc[mb], 0, 0, 0);
      }
    }
    // Online softmax (base 2, scale folded in).
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int nv = mb ? nvB : nvA;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int i = 8 * (e >> 2) + 4 * hl + (e & 3);
        const float s = i < nv ? sacc[mb][e] * c2 : -INFINITY;
        sacc[mb][e] = s;
        mx = fmaxf(mx, s);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float lsum = 0.f;
    bf16x8_t pb[4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(sacc[mb][e] - m_new);
        lsum += p;
        pb[2 * mb + (e >> 3)][e & 7] = (__bf16)p;
      }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
#pragma unroll
    for (int dm = 0; dm < 4; ++dm)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[dm][e] *= alpha;
    // O^T += V^T P^T
#pragma unroll
    for (int dm = 0; dm < 4; ++dm) {
      const int d = 32 * dm + l32;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const uint2 lo = *reinterpret_cast<const uint2*>(vt_lds + vt_offset(d, 4 * kc + hl));
        const uint2 hi = *reinterpret_cast<const uint2*>(vt_lds + vt_offset(d, 4 * kc + 2 + hl));
        const uint4 av = make_uint4(lo.x, lo.y, hi.x, hi.y);
        oacc[dm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                           pb[kc], oacc[dm], 0, 0, 0);
      }
    }
    a0 = a1;
    b0 = b1;
    a1 = a2;
    b1 = b2;
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
