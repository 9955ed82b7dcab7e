// Walk over a row's kv blocks (a CSR row, or every block for the dense pass) as 32-token
// chunks, padded per block: block J contributes ceil(|J| / 32) chunks, the last possibly partial.
// Shared by the attention passes (forward, calibration, dQ).
#pragma once

#include <climits>

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
// whether it is the block's last chunk, and (merged walks) which of the lists hold its block.
struct Chunk {
  int pos, nv, J, last, lmask;
};

template <bool kDense>
__device__ __forceinline__ Chunk take_chunk(Cursor& c, const int32_t* __restrict__ col_idx,
                                            const int32_t* __restrict__ kvstart, int nkv) {
  Chunk k;
  if (c.slot < c.end) {
    k.pos = c.base + 32 * c.sub;
    k.nv = min(32, c.size - 32 * c.sub);
    k.J = c.J;
    k.lmask = 1;
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
    k.lmask = 0;
  }
  return k;
}

// Merged walk over up to four ascending CSR rows (the rows of the query blocks that share one
// workgroup): every block listed by any of them, once, in ascending order, as 32-token chunks;
// lmask has bit l set when row l lists the block. The row positions point past the current block.
struct MultiCursor {
  int nl;              // rows merged (1..4)
  int slot[4], end[4];
  int J, base, size, sub, lmask;
};

__device__ __forceinline__ void mcursor_load(MultiCursor& c, const int32_t* __restrict__ col_idx,
                                             const int32_t* __restrict__ kvstart, int nkv) {
  int J = INT_MAX;
#pragma unroll
  for (int l = 0; l < 4; ++l) {
    if (l < c.nl) {
      while (c.slot[l] < c.end[l] && (uint32_t)ld_ro(col_idx + c.slot[l]) >= (uint32_t)nkv)
        ++c.slot[l];
      if (c.slot[l] < c.end[l]) J = min(J, ld_ro(col_idx + c.slot[l]));
    }
  }
  c.lmask = 0;
  c.sub = 0;
  if (J == INT_MAX) {
    c.J = 0;
    c.base = 0;
    c.size = 0;
    return;
  }
#pragma unroll
  for (int l = 0; l < 4; ++l) {
    if (l < c.nl && c.slot[l] < c.end[l] && ld_ro(col_idx + c.slot[l]) == J) {
      c.lmask |= 1 << l;
      ++c.slot[l];
    }
  }
  c.J = J;
  c.base = ld_ro(kvstart + J);
  c.size = ld_ro(kvstart + J + 1) - c.base;
}

__device__ __forceinline__ Chunk mtake_chunk(MultiCursor& c, const int32_t* __restrict__ col_idx,
                                             const int32_t* __restrict__ kvstart, int nkv) {
  Chunk k;
  if (c.size > 0) {
    k.pos = c.base + 32 * c.sub;
    k.nv = min(32, c.size - 32 * c.sub);
    k.J = c.J;
    k.lmask = c.lmask;
    k.last = 32 * (c.sub + 1) >= c.size;
    ++c.sub;
    if (k.last) mcursor_load(c, col_idx, kvstart, nkv);
  } else {
    k.pos = 0;
    k.nv = 0;
    k.J = 0;
    k.last = 0;
    k.lmask = 0;
  }
  return k;
}

