// Internal declarations shared by the C-ABI host code and the HIP kernel launchers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <vector>

#include "../../include/bsa.h"

// Largest kv-block count a row selection supports: one bitmap word per thread of a 256-thread
// workgroup in the CSR emit pass.
constexpr int kMaxSelectBlocks = 8192;
// Largest kv-block count of the one-wavefront-per-row kernels (the row held in registers) and of
// the fused score-and-select kernel.
constexpr int kWaveRowMaxBlocks = 2048;
// Query rows one attention workgroup owns (4 wavefronts x 32 rows).
constexpr int kAttnRows = 128;
// Forward work item: [nl, I_0, I_1, I_2, I_3, (l_w, off_w) for w = 0..3, pad]: wavefront w
// takes rows off_w .. off_w + 32 of query block I_{l_w} (l_w = -1: no rows), and the workgroup
// walks the merged CSR rows of I_0 .. I_{nl-1}. A query block's 128-row chunks are items of
// their own (nl = 1, offsets off + 32 w); the rest of every block is cut into 32-row slots,
// packed four to an item in block order, and these packed items come first (they stream the
// union of their blocks' rows, so they are the longest items; starting them first shortened the
// 480p call by 4 % against placing them last).
constexpr int kFItemInts = 16;

struct bsa_plan {
  bsa_problem prob;
  int device = 0;
  int nq = 0, nkv = 0;
  int max_qblk = 0, max_kvblk = 0;
  std::vector<int32_t> h_qperm, h_qstart, h_kvperm, h_kvstart, h_items, h_qitem0, h_kvitems;
  // Device copies (owned by the plan).
  int32_t* qperm = nullptr;
  int32_t* qstart = nullptr;
  int32_t* kvperm = nullptr;
  int32_t* kvstart = nullptr;
  int32_t* items = nullptr;   // attention work items: pairs (I, first row within block I)
  std::vector<int32_t> h_fitems;
  int32_t* fitems = nullptr;  // sparse forward work items (kFItemInts ints each)
  int n_fitems = 0;
  int32_t* qitem0 = nullptr;  // [nq + 1]: first work item of each query block
  int n_items = 0;
  int32_t* kvitems = nullptr;  // backward work items: pairs (J, first token within block J)
  int n_kvitems = 0;
  float* scale = nullptr;     // sigma_h, [H]
  std::vector<float> h_scale;
  // local kv blocks of each query block (those holding one of its tokens), ascending:
  // local_idx[local_ptr[I] .. local_ptr[I + 1])
  std::vector<int32_t> h_local_ptr, h_local_idx;
  int32_t* local_ptr = nullptr;
  int32_t* local_idx = nullptr;
  // kv block of every token (frame-major), for per-token selection
  std::vector<int32_t> h_kv_of;
  int32_t* kv_of = nullptr;
};

inline size_t align_up(size_t x, size_t a = 256) { return (x + a - 1) / a * a; }

// Entropy-routed selection (bsa_select_eg): pool rows per marking workgroup, and the device
// sizes of a group's radix state and of its 256-bin histogram (counts and 2^-56 sums).
constexpr int kEgRowChunk = 32;
constexpr size_t kEgGroupBytes = 64;
constexpr size_t kEgHistBytes = 256 * 4 + 256 * 8;

// Workspace layouts (byte offsets), derived from the plan.
struct SelectWs {
  size_t bitmap, base_counts, head_k, partial;  // partial: 1024-row chunk totals of the scan
  size_t core;  // bytes bsa_select itself uses (bitmap, counts, per-head minimum, scan totals)
  // bsa_select_eg: per row its entropy (fp64); per head the routing flag and its group's member
  // slot; per group (at most B*H groups) the radix state, the histogram and the boundary-class
  // count of each row chunk
  size_t eg_rowent, eg_route, eg_members, eg_groups, eg_hist, eg_bnd;
  size_t total;
  int nwords;
  int eg_nrchunk;  // row chunks of the largest possible pool (all H heads of a batch)
};
SelectWs select_ws_layout(const bsa_plan& p);

struct BwdWs {
  // D = rowsum(dO * O) per token; CSR row bitmap; CSC (per (head, kv block) ascending q-block
  // lists): per-column counts, column pointers, row ids.
  // K and V in block order for the dQ pass; Q, dO, LSE * log2 e and D in query block order
  // for the dK/dV pass.
  size_t delta, bitmap, col_cnt, col_ptr, row_idx, kp, vp, qp, gp, lsep, dp, total;
  int nwords;
};
BwdWs bwd_ws_layout(const bsa_plan& p);

struct CalibWs {
  // per-token log2-domain log-sum-exp; per (item, kv block, row) log2-sums of the block's
  // weights; K and V in block order (V for the variant that also forms the dense output)
  size_t lse, part, kp, vp, total;
};
CalibWs calib_ws_layout(const bsa_plan& p);

// Zero rows appended to each head of a block-ordered copy (K, V; Q, dO, LSE, D), so that the
// rows read for any chunk exist and are finite: 32 for a forward chunk, 64 for a backward
// query chunk, 128 for the K/V rows of a backward kv item.
constexpr int kPermPad = 128;

// Per-token Local + TopK (bsa_select_tokens): Kbar as two bf16 terms (hi, lo; [B*H][nkv][128]
// each), and the bitmap and counts of the per-query-block unions. At most kMaxTokenK others per
// token.
constexpr int kMaxTokenK = 24;
struct TokWs {
  size_t khi, klo, bitmap, counts, partial, total;
  int nwords;
};
TokWs tok_ws_layout(const bsa_plan& p);

// Per-token global threshold selection (bsa_select_tokens_global): Kbar's two bf16 terms, the
// head pools' gates [B*H][N][nkv] fp32 (field e), per-head radix state and histogram,
// boundary counts per 32-token chunk, and the per-query-block union (bitmap, counts, scan).
constexpr size_t kTgHeadBytes = 80;
// The head pool's radix digits: 11 bits (2048 bins), so that two passes decide 22 of a pool's
// key bits and a third (at most 31 bits in all) is rarely needed.
constexpr int kTgDigitBits = 11;
constexpr int kTgBins = 1 << kTgDigitBits;
struct TgWs {
  size_t khi, klo, e, heads, hist, bnd, bitmap, counts, partial, total;
  int nwords, nchunk;
};
TgWs tg_ws_layout(const bsa_plan& p);
hipError_t launch_select_tokens_global(const bsa_plan& p, const void* Q, const float* Kbar,
                                       double tau, uint32_t* tbits, int32_t* row_ptr,
                                       int32_t* col_idx, void* ws, hipStream_t s);
// Attention of each token over the blocks set in its bitmap tbits[B*H][N][nwords] (the union
// CSR walked per query block).
hipError_t launch_attn_fwd_token_bits(const bsa_plan& p, const void* Q, const void* K,
                                      const void* V, const int32_t* row_ptr,
                                      const int32_t* col_idx, const uint32_t* tbits, void* O,
                                      float* lse, void* ws, hipStream_t s);
// Largest kv-block count of the per-token bitmap attention (one LDS row of words per token).
// The per-token bitmap attention stages a window of this many words of each row's bitmap.
constexpr int kTokBitsWords = 24;
constexpr int kTokBitsMaxBlocks = 2048;

struct FwdWs {
  size_t kp, vp, total;  // K and V in block order, [B*H][N + kPermPad][d] (bf16, d = 128 path)
};
FwdWs fwd_ws_layout(const bsa_plan& p);

// The allocation-free selection (bsa_select_noalloc) keeps its workspace in a static device
// array of this many bytes, one per GPU; select_scratch returns its address on the current
// device (looked up once per device).
constexpr size_t kSelectScratchBytes = size_t(8) << 20;
hipError_t select_scratch(void** ptr);

// Kernel launchers (defined in the .hip files). Each returns the launch status.
// Shared pieces of the selections: row_ptr from per-row counts (exclusive scan in 1024-row
// chunks, partial: one int per chunk); Kbar split into two bf16 terms; CSR columns from bitmaps.
hipError_t launch_scan(const int32_t* base_counts, const int32_t* head_k, bool use_min_k,
                       int64_t rows, int nq, int32_t* row_ptr, int32_t* counts_out,
                       int32_t* partial, hipStream_t s);
hipError_t launch_kbar_split(const float* Kbar, int64_t n, uint16_t* hi, uint16_t* lo,
                             hipStream_t s);
hipError_t launch_emit(const uint32_t* bitmap, int nwords, int64_t rows, const int32_t* row_ptr,
                       int32_t* col_idx, hipStream_t s);
hipError_t launch_pool(const bsa_plan& p, int which, const void* X, float* Xbar, hipStream_t s);
hipError_t launch_pool_qk(const bsa_plan& p, const void* Q, float* Qbar, const void* K,
                          float* Kbar, hipStream_t s);
hipError_t launch_score(const bsa_plan& p, const float* Qbar, const float* Kbar, int norm,
                        float* S, hipStream_t s);
// Fused score and ROW-pool selection (nkv <= 2048): the marking pass of bsa_select computed in
// the scoring kernel (S written only when not NULL), then the rest of bsa_select.
hipError_t launch_score_select(const bsa_plan& p, const float* Qbar, const float* Kbar, float* S,
                               unsigned long long target, bool all, int nwords,
                               uint32_t* bitmap, int32_t* base_counts, hipStream_t s);
hipError_t launch_score_select_csr(const bsa_plan& p, const float* Qbar, const float* Kbar,
                                   const bsa_select_params& prm, float* S, int32_t* row_ptr,
                                   int32_t* col_idx, int32_t* counts, int32_t* head_k, void* ws,
                                   hipStream_t s);
hipError_t launch_select(const bsa_plan& p, const float* S, const bsa_select_params& prm,
                         int32_t* row_ptr, int32_t* col_idx, int32_t* counts, int32_t* head_k,
                         void* ws, hipStream_t s);
hipError_t launch_select_eg(const bsa_plan& p, const float* S, const bsa_eg_params& prm,
                            int32_t* row_ptr, int32_t* col_idx, int32_t* counts,
                            float* head_entropy, int32_t* head_pooled, void* ws, hipStream_t s);
hipError_t launch_attn_fwd(const bsa_plan& p, const void* Q, const void* K, const void* V,
                           const int32_t* row_ptr, const int32_t* col_idx, void* O, float* lse,
                           void* ws, hipStream_t s);
// sel: per-token block lists [B*H][N][nslots] (ascending), walked alongside the union CSR.
hipError_t launch_attn_fwd_tokens(const bsa_plan& p, const void* Q, const void* K, const void* V,
                                  const int32_t* row_ptr, const int32_t* col_idx,
                                  const int32_t* sel, int nslots, void* O, float* lse, void* ws,
                                  hipStream_t s);
hipError_t launch_select_tokens(const bsa_plan& p, const void* Q, const float* Kbar, int k,
                                int32_t* sel, int32_t* row_ptr, int32_t* col_idx, void* ws,
                                hipStream_t s);
// dst = src ([B, H, N, 128] bf16) with rows in block order (plan kvperm) and kPermPad zero rows
// per head.
hipError_t launch_permute_rows(const bsa_plan& p, const void* src, void* dst, hipStream_t s);
// V, O, lse_out: NULL for the masses alone; else the dense output O (and its LSE, nullable) too.
hipError_t launch_calibrate(const bsa_plan& p, const void* Q, const void* K, const void* V,
                            float* M, void* O, float* lse_out, void* ws, hipStream_t s);
hipError_t launch_attn_bwd(const bsa_plan& p, const void* Q, const void* K, const void* V,
                           const void* O, const void* dO, const float* lse,
                           const int32_t* row_ptr, const int32_t* col_idx, void* dQ, void* dK,
                           void* dV, void* ws, hipStream_t s);
