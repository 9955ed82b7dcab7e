// Device helpers for gfx950 kernels: vector types, bf16 packing, wave reductions, XCD mapping.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round two floats to bf16 (nearest even, one v_cvt_pk_bf16_f32) and pack them, a in the low half.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// Workgroup ids are dealt round-robin to the 8 XCDs (id % 8). Renumber them so that logical
// ids [x * q + min(x, r), ...) all run on XCD x: consecutive logical work (one head's query
// blocks) then shares one XCD's L2. A bijection on [0, total).
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  const int xcd = bid & 7, idx = bid >> 3;
  const int q = total >> 3, r = total & 7;
  return xcd * q + (xcd < r ? xcd : r) + idx;
}

__device__ __forceinline__ unsigned long long shfl_up_u64(unsigned long long v, int delta) {
  uint32_t lo = __shfl_up((uint32_t)v, delta, 64);
  uint32_t hi = __shfl_up((uint32_t)(v >> 32), delta, 64);
  return ((unsigned long long)hi << 32) | lo;
}

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int mask) {
  uint32_t lo = __shfl_xor((uint32_t)v, mask, 64);
  uint32_t hi = __shfl_xor((uint32_t)(v >> 32), mask, 64);
  return ((unsigned long long)hi << 32) | lo;
}

// Inclusive prefix sum over the 64 lanes of a wavefront.
__device__ __forceinline__ unsigned long long wave_incl_scan_u64(unsigned long long v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    unsigned long long o = shfl_up_u64(v, d);
    if (lane >= d) v += o;
  }
  return v;
}

__device__ __forceinline__ int wave_incl_scan_i32(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

// max / sum of the values held by lanes l and l ^ 32 (gfx950 v_permlane32_swap exchanges the
// two 32-lane halves between two registers; combining both outputs does not depend on which
// output holds which half).
__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

typedef __attribute__((address_space(3))) char lds_char_t;

// LDS tiles of bf16 rows with d = 128 (256 bytes, sixteen 16-byte units): logical unit u of row r
// is stored at unit u ^ lds_key(r). The key (a bijection on units for every row) makes both read
// patterns of the matrix-core kernels bank-conflict free, for 32 or 64 four-byte banks:
//   16-byte reads of one unit from 8 (16) consecutive aligned rows need key mod 8 (16) distinct;
//   transposing 8-byte reads of units {4m, 4m+1} (4m .. 4m+3) from 4 consecutive aligned rows
//   need bits 1-2 (2-3) of the key distinct over those rows.
// Rows 0..3 take keys 0, 10, 6, 12; bit 2 of the row flips key bit 0 and bit 3 flips key bit 3.
__device__ __forceinline__ int lds_key(int row) {
  return ((0xC6A0 >> (4 * (row & 3))) & 15) ^ ((row >> 2) & 1) ^ (row & 8);
}
__device__ __forceinline__ int lds_swz(int row, int unit) { return (unit ^ lds_key(row)) << 4; }

// The key of the kernels on 16x16x32 MFMAs: lds_key16(r) = 2 (r mod 8) + bit 3 of r. Their
// transposing 8-byte reads (a 16-lane group: 4 rows x units {2 m, 2 m + 1}; the wavefront: 16
// consecutive rows) need bits 1-3 of the key distinct over 8 aligned rows, which holds: no bank
// conflicts (SQ_LDS_BANK_CONFLICT = 0 in a probe). Their 16-byte row reads (lane 16 g + t: row
// t, unit 4 c + g) conflict under this key and under the 32x32 kernels' (4 cycles per read):
// the forward stores K in fragment tiles instead, where those reads are contiguous.
__device__ __forceinline__ int lds_key16(int row) { return ((row & 7) << 1) | ((row >> 3) & 1); }
__device__ __forceinline__ int lds_swz16(int row, int unit) {
  return (unit ^ lds_key16(row)) << 4;
}

// Direct global -> LDS copy of 16 bytes per lane (gfx950 global_load_lds_dwordx4): lane i of the
// wavefront writes LDS bytes [lds_base + 16 i, +16). lds_base must be wave-uniform. Issued from
// inline assembly so that the compiler does not order later LDS reads of *other* buffers behind
// it; the caller waits for it explicitly (vmem_wait_all) and then synchronises the workgroup
// before any wavefront reads the destination.
__device__ __forceinline__ void lds_dma16(const void* gsrc, char* lds_base) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(
      (uint32_t)reinterpret_cast<uintptr_t>((lds_char_t*)lds_base));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gsrc), "s"(m0v)
               : "m0", "memory");
}

// The same copy with the global address split into a wave-uniform 64-bit base (held in SGPRs,
// the instruction's saddr form) and a per-lane 32-bit byte offset, and the LDS destination given
// as a precomputed M0 value: no 64-bit address arithmetic per copy.
__device__ __forceinline__ void lds_dma16_so(const void* sbase, uint32_t voff, uint32_t m0v) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(m0v)
               : "m0", "memory");
}

// 4 bytes per lane (global_load_lds_dword): lane i writes LDS bytes [m0v + 4 i, +4).
__device__ __forceinline__ void lds_dma4_so(const void* sbase, uint32_t voff, uint32_t m0v) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(m0v)
               : "m0", "memory");
}

// LDS byte address of a __shared__ location, as a wave-uniform value (for M0).
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>((lds_char_t*)p));
}

// Wait until every vector memory operation of this wavefront has completed (vmcnt(0); the
// other counters unconstrained).
__device__ __forceinline__ void vmem_wait_all() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// Wait until at most N vector memory operations of this wavefront are outstanding (they
// complete in issue order, so everything older than the N most recent has completed).
template <int N>
__device__ __forceinline__ void vmem_wait_keep() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0f70 | (N & 15) | ((N >> 4) << 14));
}

// Load from memory that no kernel writes while it runs (plan descriptors, CSR, scales) through
// the constant address space, so that wave-uniform indices become scalar loads.
template <typename T>
__device__ __forceinline__ T ld_ro(const T* p) {
  return *(const __attribute__((address_space(4))) T*)(p);
}
