// Walk over a row's kv blocks (a CSR row, or every block for the dense passes) as 32-token
// chunks, padded per block: block J contributes ceil(|J| / 32) chunks, the last possibly partial.
// Shared by the attention passes (forward, calibration, dQ).
#pragma once

#include "device_common.h"

struct Cursor {
  int slot, end, sub, base, size, J;  // position in the block list, current block and its tokens
};

// A CSR entry outside [0, nkv) is skipped, so that a bad caller-provided index never addresses
// the plan's block table out of bounds.
template <bool kDense>
__device__ __forceinline__ void cursor_load(Cursor& c, const int32_t* __restrict__ col_idx,
                                            const int32_t* __restrict__ kvstart, int nkv) {
  if constexpr (!kDense) {
    while (c.slot < c.end && (uint32_t)ld_ro(col_idx + c.slot) >= (uint32_t)nkv) ++c.slot;
  }
  if (c.slot < c.end) {
    c.J = kDense ? c.slot : ld_ro(col_idx + c.slot);
    c.base = ld_ro(kvstart + c.J);
    c.size = ld_ro(kvstart + c.J + 1) - c.base;
  } else {
    c.J = 0;
    c.base = 0;
    c.size = 0;
  }
}

// One chunk: first token position in perm, number of valid rows (0 = past the end), its block,
// and whether it is the block's last chunk.
struct Chunk {
  int pos, nv, J, last;
};

template <bool kDense>
__device__ __forceinline__ Chunk take_chunk(Cursor& c, const int32_t* __restrict__ col_idx,
                                            const int32_t* __restrict__ kvstart, int nkv) {
  Chunk k;
  if (c.slot < c.end) {
    k.pos = c.base + 32 * c.sub;
    k.nv = min(32, c.size - 32 * c.sub);
    k.J = c.J;
    k.last = 32 * (c.sub + 1) >= c.size;
    ++c.sub;
    if (k.last) {
      ++c.slot;
      c.sub = 0;
      cursor_load<kDense>(c, col_idx, kvstart, nkv);
    }
  } else {
    k.pos = 0;
    k.nv = 0;
    k.J = 0;
    k.last = 0;
  }
  return k;
}

