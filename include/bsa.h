/*
 * bsa.h - C ABI of a block-sparse attention library for long 3D (frame x height x width) video
 * token sequences, written for AMD Instinct MI355X (gfx950).
 *
 * The path (each step cites the page that defines it):
 *   1. bsa_pool           mean of Q (or K) over each block of a 1D/2D/3D partition of the token grid
 *                         (pith.science review of VMoBA, "What carries the argument": every key
 *                         block is represented by its mean key; Figure 2 caption).
 *   2. bsa_score          query-block x key-block similarity of the block means, normalised per
 *                         query block (row) or over the whole head (VMoBA review, referee report
 *                         major comment 1: Eq. 3 global selection over the query-by-block matrix).
 *      bsa_calibrate_mass exact per-(head, q-block, kv-block) softmax mass from one dense step
 *                         (LoSA abstract, scholarbro author page); bsa_calibrate_mass_fwd also
 *                         returns that dense step's attention output.
 *   3. bsa_select         per (head, q-block) the smallest kv-block set, in descending score
 *                         order, whose cumulative score or mass reaches p (VMoBA review, major
 *                         comment 1 on Sec. 3.4 Eq. 4; LoSA abstract), optionally raised to a
 *                         per-head minimum count (SCOPE abstract, mlsift sparse-attention listing)
 *                         or ranked over a head-global pool of (q-block, kv-block) pairs (VMoBA
 *                         Eq. 3). The result is an int32 CSR list that callers may freeze and
 *                         reuse across denoising steps (LoSA abstract).
 *      bsa_select_tokens  per query token, its own block plus the k blocks of highest gate (VMoBA
 *                         review), with bsa_attn_fwd_tokens to attend over them.
 *      bsa_select_tokens_global  per head, the (token, block) gates ranked as one pool with the
 *                         threshold tau (VMoBA Eq. 3-4), with bsa_attn_fwd_token_bits.
 *      bsa_select_eg      the same rule with the competition domain chosen per head by the
 *                         entropy of its scores: a pool shared by a group of low-entropy heads,
 *                         per-row selection for the rest (EG-Sparse abstract).
 *   4. bsa_attn_fwd       online-softmax attention of every query over the tokens of its selected
 *                         kv blocks only (VMoBA review, Figure 2 caption), and bsa_attn_bwd, its
 *                         gradient for training through the sparse attention (VMoBA review,
 *                         "The reading").
 *
 * Conventions shared by every entry point
 *   - Tensors Q, K, V, O, dO, dQ, dK, dV are [B, H, N, d], d contiguous, in device memory. Tokens
 *     are in frame-major order n = (t * Hg + h) * Wg + w. dtype BSA_BF16 passes raw bf16 words
 *     (uint16); BSA_FP32 passes float.
 *   - Block-level tensors are fp32: Xbar [B, H, nblk, d]; S and M [B, H, nq, nkv].
 *   - CSR row r = (b * H + h) * nq + I lists the kv blocks J selected for query block I of head
 *     (b, h), ascending; row_ptr has B*H*nq + 1 entries, row_ptr[0] = 0.
 *   - Every pointer argument is a device pointer unless it says "host". The caller owns every
 *     tensor, CSR buffer and workspace; the plan owns only its own small device descriptors.
 *   - Every call validates all arguments on the host before enqueuing anything; on an error it
 *     writes nothing and returns a negative status, and bsa_last_error() (thread-local) describes
 *     it. Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the null stream).
 *     Results are deterministic: the same inputs give the same bits.
 *   - NaN inputs propagate into scores and outputs; the selection made from NaN scores is
 *     unspecified but always a valid CSR. A non-finite value in V can also reach queries whose
 *     selection does not include its token: the bf16 attention streams 32-token chunks padded
 *     past a block's end with the next tokens' rows, whose weights are exactly 0, and 0 times a
 *     non-finite value is NaN. Non-finite K values in padded rows are masked and do not leak.
 */
#ifndef BSA_H
#define BSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define BSA_OK 0
#define BSA_EINVAL (-1)        /* a NULL pointer, a bad shape or parameter                       */
#define BSA_EUNSUPPORTED (-2)  /* a valid request the library does not implement (d, dtype, size) */
#define BSA_ECAPACITY (-3)     /* an output or workspace buffer is smaller than required          */
#define BSA_EHIP (-4)          /* the HIP runtime reported an error (no device, launch failure)   */

/* partitions */
#define BSA_PART_FLAT 0        /* contiguous runs of `flat` tokens in frame-major order           */
#define BSA_PART_TILE 1        /* bt x bh x bw tiles of the grid, clipped at the edge             */

/* dtypes */
#define BSA_BF16 0
#define BSA_FP32 1

/* normalisation (bsa_score) and selection pool (bsa_select) */
#define BSA_NORM_ROW 0         /* softmax over kv blocks of each query block                      */
#define BSA_NORM_HEAD 1        /* |I|-weighted softmax over all (I, J) pairs of a head            */
#define BSA_POOL_ROW 0         /* select per (head, query block)                                  */
#define BSA_POOL_HEAD 1        /* select over all (I, J) pairs of a head                          */
#define BSA_POOL_LOCAL_TOPK 2  /* local blocks of I plus the fixed_k best others (VMoBA review)   */

/* per-head minimum count after top-p (bsa_select) */
#define BSA_MINK_NONE 0
#define BSA_MINK_FIXED 1       /* k = fixed_k for every head                                      */
#define BSA_MINK_WEIGHTED_MEAN 2 /* k_h = ceil(sum_I |I| c_I / sum_I |I|), SCOPE abstract          */

/*
 * Block partition of the (T, Hg, Wg) token grid into non-overlapping blocks (VMoBA review,
 * circularity check: Eq. 1-2 build the partition constructively; 1D temporal blocks are
 * (bt, Hg, Wg) tiles, 2D spatial blocks (T, bh, bw), 3D blocks (bt, bh, bw)). Block (a, b, c) of
 * a TILE partition is numbered (a * nbh + b) * nbw + c and holds its tokens in ascending n.
 */
typedef struct {
  int32_t kind;          /* BSA_PART_FLAT or BSA_PART_TILE        */
  int32_t flat;          /* FLAT: tokens per block (>= 1)         */
  int32_t bt, bh, bw;    /* TILE: tile extents (each >= 1)        */
} bsa_partition;

typedef struct {
  int32_t B, H, N, d;    /* batch, heads, tokens (= T * Hg * Wg), head dim (64 or 128)         */
  int32_t dtype;         /* BSA_BF16 or BSA_FP32                                                */
  int32_t T, Hg, Wg;     /* token grid                                                          */
  bsa_partition qpart;   /* partition of the queries (pooled in step 1, one CSR row per block)  */
  bsa_partition kvpart;  /* partition of the keys/values (the selectable blocks)                */
} bsa_problem;

typedef struct {
  double p;              /* threshold in (0, 1]: top-p / retained mass (ROW) or tau (HEAD).
                            Selection keeps the shortest prefix of the (score descending, index
                            ascending) order whose cumulative sum is >= p; p >= 1, or a sum
                            that never reaches p, keeps every block (pair).                     */
  int32_t pool;          /* BSA_POOL_ROW, BSA_POOL_HEAD or BSA_POOL_LOCAL_TOPK (p unused)       */
  int32_t min_k_mode;    /* BSA_MINK_*; ROW pool only                                           */
  int32_t fixed_k;       /* BSA_MINK_FIXED: the per-head minimum (>= 0); LOCAL_TOPK: k (>= 0)  */
} bsa_select_params;

/* Entropy-routed competition domains (EG-Sparse abstract, readsearch page "Competition Domains
 * Matter: Selective Head Globalization for Training-Free Sparse Attention in Video Diffusion
 * Transformers"): heads whose row-normalised scores have low entropy compete in a pool shared
 * by their group of heads; the others keep per-row selection. */
typedef struct {
  double p;              /* threshold in (0, 1] for the per-row selections and for every pool  */
  double theta;          /* a head is pooled when its normalised entropy is < theta (not NaN)  */
  int32_t group_size;    /* heads per group: runs of consecutive heads (>= 1; >= H is one group) */
} bsa_eg_params;

typedef struct bsa_plan bsa_plan;

/* Host only, no device call: fill perm[N] (block-major token order: block j's tokens are
 * perm[blk_start[j] .. blk_start[j+1]), ascending) and blk_start[nblk + 1]; *nblk receives the
 * block count. blk_start must hold cap_blocks + 1 entries; returns BSA_ECAPACITY (with *nblk set)
 * when the partition has more than cap_blocks blocks. */
int bsa_partition_build(int32_t T, int32_t Hg, int32_t Wg, const bsa_partition* part,
                        int32_t* perm, int32_t* blk_start, int32_t cap_blocks, int32_t* nblk);

/* Validate `prob`, build both partitions and upload them to the current device. head_scale is
 * a host array of H softmax scales sigma_h (copied; each finite and > 0), or NULL for
 * 1/sqrt(d). The plan is
 * immutable afterwards and may be shared by calls on several streams. */
int bsa_plan_create(const bsa_problem* prob, const float* head_scale, bsa_plan** out);
int bsa_plan_destroy(bsa_plan* plan);

/* Block counts and the workspace sizes (bytes) that bsa_select, bsa_calibrate_mass,
 * bsa_attn_bwd and bsa_attn_fwd require for this plan (ws_fwd is 0 for the fp32 and d = 64
 * paths). Any output pointer may be NULL. Workspaces are caller-owned device memory; their
 * contents need no initialisation and are scratch between calls. */
int bsa_plan_info(const bsa_plan* plan, int32_t* nq, int32_t* nkv, size_t* ws_select,
                  size_t* ws_calib, size_t* ws_bwd, size_t* ws_fwd);

/* Host copies of a plan's partition (which = 0 queries, 1 keys/values): perm[N] and
 * blk_start[nblk + 1], both host buffers. */
int bsa_plan_blocks(const bsa_plan* plan, int32_t which, int32_t* perm, int32_t* blk_start);

/* Step 1. Xbar[b, h, J, :] = (1/|J|) sum_{n in J} X[b, h, n, :] over the partition `which`
 * (0 = qpart, 1 = kvpart), accumulated in fp32. X is [B, H, N, d] of the plan's dtype, Xbar fp32
 * [B, H, nblk, d]. */
int bsa_pool(const bsa_plan* plan, int32_t which, const void* X, float* Xbar, void* stream);

/* Step 1 for both sides in one launch: Qbar over qpart and Kbar over kvpart, each identical to
 * its bsa_pool call (the same kernel and summation order); more workgroups in flight than either
 * pass alone, which matters for short passes. */
int bsa_pool_qk(const bsa_plan* plan, const void* Q, const void* K, float* Qbar, float* Kbar,
                void* stream);

/* Step 2. L[b, h, I, J] = sigma_h <Qbar_I, Kbar_J>, then
 *   norm = BSA_NORM_ROW : S = softmax over J of each row;
 *   norm = BSA_NORM_HEAD: S[I, J] = |I| exp(L[I, J]) / sum_{I', J'} |I'| exp(L[I', J']) per head.
 * Qbar [B, H, nq, d], Kbar [B, H, nkv, d], S [B, H, nq, nkv], all fp32. */
int bsa_score(const bsa_plan* plan, const float* Qbar, const float* Kbar, int32_t norm, float* S,
              void* stream);

/* Step 2'. Exact block masses of one dense step (LoSA abstract):
 *   M[b, h, I, J] = (1/|I|) sum_{i in I} sum_{j in J} softmax_j(sigma_h q_i . k_j),
 * the softmax taken over all N keys. Q, K [B, H, N, d] of the plan's dtype (bf16 only, d = 128);
 * M fp32 [B, H, nq, nkv]. ws must hold the ws_calib bytes of bsa_plan_info (mostly the per
 * query and kv block log-sums of one pass over the keys: B*H*items*nkv*128 floats, items the
 * 128-row chunks of the query blocks, e.g. 694 MB for the 480p shape). Rows of M sum to 1. */
int bsa_calibrate_mass(const bsa_plan* plan, const void* Q, const void* K, float* M, void* ws,
                       size_t ws_bytes, void* stream);

/* Step 2' as the dense step itself: the same masses M, plus the dense attention output of that
 * step, O[b, h, i, :] = sum_j softmax_j(sigma_h q_i . k_j) v_j over all N keys, and its LSE
 * (natural log, fp32 [B, H, N]; nullable). The LoSA abstract measures the masses at one early
 * step that runs dense attention; both come from one online-softmax pass over the keys, whose
 * weights also multiply V (the masses are formed afterwards from each query's per-block sums and
 * its LSE, bit-identical to bsa_calibrate_mass). Q, K, V, O [B, H, N, d] bf16 (d = 128),
 * M fp32 [B, H, nq, nkv]; ws as for bsa_calibrate_mass (the ws_calib bytes). O is normalised by
 * the sum of the same bf16-rounded weights that multiply V. Errors as bsa_calibrate_mass. */
int bsa_calibrate_mass_fwd(const bsa_plan* plan, const void* Q, const void* K, const void* V,
                           float* M, void* O, float* lse, void* ws, size_t ws_bytes,
                           void* stream);

/* Step 3. Selection from S (scores from bsa_score, or masses from bsa_calibrate_mass), written
 * as CSR: row_ptr [B*H*nq + 1], col_idx with capacity col_cap >= B*H*nq*nkv entries (the number
 * used is row_ptr[B*H*nq], left on the device; nothing is synchronised). counts (nullable,
 * [B*H*nq]) receives each row's final count; head_k (nullable, [B*H]) receives the per-head
 * minimum used (0 when min_k_mode is NONE). ws must hold the ws_select bytes of bsa_plan_info.
 * BSA_EUNSUPPORTED when nkv > 8192 or B*H*nq*nkv exceeds 2^31 - 1 (row_ptr is 32-bit).
 * With BSA_POOL_HEAD a query block may receive no block at all (an empty row, as the VMoBA
 * referee report points out); attention then returns O = 0 and LSE = -inf for its queries.
 * BSA_POOL_LOCAL_TOPK is VMoBA's training-free "Local + TopK" (VMoBA review, referee report
 * major comment 2; free parameters k = 2, 6, 18): query block I keeps its local kv blocks (those
 * holding at least one of its tokens) plus the fixed_k highest-scoring other blocks (score desc,
 * index asc), fewer when fewer remain; p is not used and min_k_mode must be NONE. */
int bsa_select(const bsa_plan* plan, const float* S, const bsa_select_params* params,
               int32_t* row_ptr, int32_t* col_idx, int64_t col_cap, int32_t* counts,
               int32_t* head_k, void* ws, size_t ws_bytes, void* stream);

/* Steps 2 and 3 in one pass for the ROW pool (ROW normalisation, then top-p with an optional
 * per-head minimum count): the same CSR, counts and head_k as bsa_score(BSA_NORM_ROW) followed
 * by bsa_select, bit for bit, without the scores going through memory: each workgroup forms the
 * block-mean logits of 16 query blocks against every kv block, applies the row softmax and
 * selects every row in registers. The selection overhead of dynamic sparse attention is what
 * the pages flag (mlsift listing: the HyperVAttention abstract's clustering overhead and the
 * ScalingAttention abstract's runtime overhead of dynamic pruning). S [B, H, nq, nkv] (nullable)
 * receives the scores when given; it is required with a minimum count, whose top-up reads it.
 * Qbar, Kbar as bsa_score; the rest as bsa_select (ws: its ws_select bytes). BSA_EUNSUPPORTED
 * for another pool or nkv > 2048. */
int bsa_score_select(const bsa_plan* plan, const float* Qbar, const float* Kbar,
                     const bsa_select_params* params, float* S, int32_t* row_ptr,
                     int32_t* col_idx, int64_t col_cap, int32_t* counts, int32_t* head_k,
                     void* ws, size_t ws_bytes, void* stream);

/* Step 3 without a workspace argument, for callers that cannot allocate device memory (code
 * under stream capture into a graph, tight serving loops, harnesses that forbid allocation):
 * the same selection, bit for bit, as bsa_select with the same arguments, and the same checks
 * and errors. The workspace is a static device array inside the library, 8 MiB on each GPU,
 * held until the process ends; the call allocates and frees nothing. A plan whose selection
 * needs more (bitmap of B*H*nq*ceil(nkv/32) words, plus B*H*nq + B*H counts) returns
 * BSA_ECAPACITY; use bsa_select with a workspace then. Every call on one GPU shares that GPU's
 * array, so calls that overlap in time on one GPU (different streams, or several threads)
 * race and must be serialised by the caller; calls on one stream are ordered. Nothing in the
 * array needs to start at zero: every word a call reads was written earlier by that call. */
int bsa_select_noalloc(const bsa_plan* plan, const float* S, const bsa_select_params* params,
                       int32_t* row_ptr, int32_t* col_idx, int64_t col_cap, int32_t* counts,
                       int32_t* head_k, void* stream);

/* Step 3, entropy-routed (EG-Sparse abstract). S: row-normalised scores from bsa_score
 * (BSA_NORM_ROW). Per head, E_h = sum_I |I| H_I / (N ln nkv) with H_I = -sum_J S ln S over row
 * (h, I) (fp64; 0 when nkv = 1); the head is pooled when E_h < theta. Heads are grouped in runs
 * of group_size; within a group the pooled heads' (h, I, J) candidates, weighted
 * S[h, I, J] * |I| / (N m) for m pooled heads (the pool sums to 1), are ranked by (weight desc,
 * index asc over (pooled head in head order, I, J)) and the shortest prefix reaching p is kept,
 * with the exact 2^-56 fixed-point sums of bsa_select; a pooled query block may keep no block.
 * Heads not pooled select per row as bsa_select with BSA_POOL_ROW. Outputs as bsa_select, plus
 * head_entropy (nullable, fp32 [B*H], E_h) and head_pooled (nullable, int32 [B*H], 0 or 1).
 * ws must hold the ws_select bytes of bsa_plan_info. BSA_EUNSUPPORTED when H * nq * nkv
 * exceeds 2^31 - 1 (the pool index is 32-bit). */
int bsa_select_eg(const bsa_plan* plan, const float* S, const bsa_eg_params* params,
                  int32_t* row_ptr, int32_t* col_idx, int64_t col_cap, int32_t* counts,
                  float* head_entropy, int32_t* head_pooled, void* ws, size_t ws_bytes,
                  void* stream);

/* Step 3, per token (VMoBA review, "What carries the argument": each query token scores the
 * block means; the training-free experiments keep "Local + TopK" blocks, k = 2, 6 or 18). Q
 * [B, H, N, 128] bf16; Kbar fp32 [B, H, nkv, 128] from bsa_pool(which = 1). For every token i:
 * sel[b, h, i, 0 .. ns) with ns = 1 + min(k, nkv - 1) holds, ascending, the kv block holding i
 * and the min(k, nkv - 1) others with the highest gate sigma_h q_i . kbar_J (gate desc, index
 * asc), the gates formed on the bf16 matrix cores with kbar split into two bf16 terms (2^-17
 * relative) and fp32 accumulation, and never written to memory. row_ptr / col_idx (as
 * bsa_select) receive, per query block, the union of its tokens' lists, which
 * bsa_attn_fwd_tokens walks. ws >= the bytes bsa_tokens_ws reports (kbar's two bf16 terms plus
 * the union's bitmap and counts). k in [0, 24]; bf16, d = 128, nkv <= 2048 and
 * B*H*nq*nkv <= 2^31 - 1 only (BSA_EUNSUPPORTED otherwise). */
int bsa_tokens_ws(const bsa_plan* plan, size_t* ws_bytes);
int bsa_select_tokens(const bsa_plan* plan, const void* Q, const float* Kbar, int32_t k,
                      int32_t* sel, int32_t* row_ptr, int32_t* col_idx, int64_t col_cap,
                      void* ws, size_t ws_bytes, void* stream);

/* Step 4 over per-token block sets: O_i = sum_j softmax_j(sigma_h q_i . k_j) v_j over the tokens
 * j of the blocks in sel[b, h, i] (and lse_i, nullable), with sel, row_ptr and col_idx from
 * bsa_select_tokens with the same k. Each query block's workgroup streams the union of its
 * tokens' blocks and masks, per token, the blocks that token did not pick. Numerics as
 * bsa_attn_fwd; ws as bsa_attn_fwd (ws_fwd bytes). */
int bsa_attn_fwd_tokens(const bsa_plan* plan, const void* Q, const void* K, const void* V,
                        const int32_t* row_ptr, const int32_t* col_idx, const int32_t* sel,
                        int32_t k, void* O, float* lse, void* ws, size_t ws_bytes,
                        void* stream);

/* Step 3, per token and head-global (VMoBA review: "What carries the argument" -- global
 * selection pools the scores of all queries of a head; referee report major comment 1 -- Eq. 3
 * keeps the top entries of the whole query-by-block matrix and Eq. 4 the smallest count k'
 * whose cumulative normalised similarity reaches tau, so a query may keep no block; tau = 0.25
 * under "Assumptions & free parameters"). Per head, the gates g[i, J] = sigma_h q_i . kbar_J of
 * every query token i and kv block J (bf16 matrix cores, kbar split into two bf16 terms, fp32
 * sums) are normalised by one softmax over the head's whole N x nkv matrix; the pairs are ranked
 * by (weight desc, pair index i * nkv + J asc) and the shortest prefix reaching tau is kept, with
 * exact fixed-point sums of exp(g - max g) (the prefix of e reaching tau * sum e). tbits
 * [B, H, N, ceil(nkv / 32)] (uint32 words, bit J % 32 of word J / 32) receives each token's kept
 * blocks; a token may keep none (an empty row: its attention gives O = 0, LSE = -inf).
 * row_ptr / col_idx (as bsa_select) receive each query block's union of its tokens' blocks, which
 * bsa_attn_fwd_token_bits walks. Q [B, H, N, 128] bf16; Kbar fp32 [B, H, nkv, 128] from
 * bsa_pool(which = 1). ws >= the bytes bsa_tokens_global_ws reports (it holds the B*H*N*nkv fp32
 * gates). BSA_EUNSUPPORTED unless bf16, d = 128, nkv <= 2048 and B*H*nq*nkv <= 2^31 - 1. */
int bsa_tokens_global_ws(const bsa_plan* plan, size_t* ws_bytes);
int bsa_select_tokens_global(const bsa_plan* plan, const void* Q, const float* Kbar, double tau,
                             uint32_t* tbits, int32_t* row_ptr, int32_t* col_idx,
                             int64_t col_cap, void* ws, size_t ws_bytes, void* stream);

/* Step 4 over per-token block bitmaps (from bsa_select_tokens_global): O_i and lse_i (nullable)
 * over the tokens of the blocks set in tbits[b, h, i]; a token with no block gets O = 0 and
 * lse = -inf. Each query block's workgroup walks its union CSR row and masks, per token, the
 * blocks that token did not keep. Numerics and ws as bsa_attn_fwd (ws_fwd bytes). bf16,
 * d = 128 and nkv <= 2048 only (BSA_EUNSUPPORTED otherwise). */
int bsa_attn_fwd_token_bits(const bsa_plan* plan, const void* Q, const void* K, const void* V,
                            const int32_t* row_ptr, const int32_t* col_idx,
                            const uint32_t* tbits, void* O, float* lse, void* ws,
                            size_t ws_bytes, void* stream);

/* Step 4. For every query i of block I: O_i = sum_j softmax_j(sigma_h q_i . k_j) v_j over the
 * tokens j of the kv blocks listed in CSR row I, and lse_i = log sum_j exp(sigma_h q_i . k_j).
 * Q, K, V, O [B, H, N, d] of the plan's dtype; lse fp32 [B, H, N] (nullable). bf16: products on
 * bf16 matrix cores with fp32 accumulation and fp32 online softmax; P is rounded to bf16 before
 * the PV product, and O is normalised by the sum of those rounded weights. With lse NULL the
 * fp32 row sums that only the LSE needs are not formed (the same O; a faster kernel for bf16,
 * d = 128).
 * The CSR should come from bsa_select for this plan (or be equivalent: indices in [0, nkv),
 * ascending or not, no duplicates within a row). The device cannot report an error, so an entry
 * outside [0, nkv) is skipped (as if absent) rather than read; a duplicate counts its block's
 * tokens twice. ws (device, ws_bytes >= ws_fwd of bsa_plan_info;
 * may be NULL when ws_fwd is 0) receives K and V copied into block order; BSA_ECAPACITY if it
 * is too small. */
int bsa_attn_fwd(const bsa_plan* plan, const void* Q, const void* K, const void* V,
                 const int32_t* row_ptr, const int32_t* col_idx, void* O, float* lse, void* ws,
                 size_t ws_bytes, void* stream);

/* Gradient of step 4 with the selection held fixed (a hard gate): given O and lse from
 * bsa_attn_fwd and the upstream gradient dO, writes dQ, dK, dV ([B, H, N, d], plan dtype):
 *   D_i = dO_i . O_i; P_ij = exp(sigma_h q_i . k_j - lse_i) on selected pairs;
 *   dV = P^T dO; dS = P * (dO V^T - D); dQ = sigma_h dS K; dK = sigma_h dS^T Q.
 * Tokens no selected pair touches get zero gradient. bf16, d = 128 only; BSA_EUNSUPPORTED when
 * nkv > 8192 or B*H*nq*nkv exceeds 2^31 - 1 (32-bit column lists). The CSR as for bsa_attn_fwd
 * (entries outside [0, nkv) are skipped). ws must hold the ws_bwd bytes of bsa_plan_info. No
 * atomics: results are deterministic. */
int bsa_attn_bwd(const bsa_plan* plan, const void* Q, const void* K, const void* V,
                 const void* O, const void* dO, const float* lse, const int32_t* row_ptr,
                 const int32_t* col_idx, void* dQ, void* dK, void* dV, void* ws,
                 size_t ws_bytes, void* stream);

/* Measurement helpers, outside the attention path: the ceilings that benches compare the
 * kernels with, measured on the current GPU. bsa_probe_mfma runs `workgroups` x 256 threads of
 * back-to-back bf16 MFMAs on register operands -- shape 0: v_mfma_f32_32x32x16_bf16 (iters x 8
 * per wavefront), shape 1: v_mfma_f32_16x16x32_bf16 (iters x 16) -- or, at three workgroups
 * per CU, rounds of 16 independent v_mfma_f32_16x16x32_bf16 alone (shape 2), with 32
 * independent v_exp_f32 (3), the 32 exponentials alone (4), the MFMAs with 32 v_fma_f32 (5) or
 * the FMAs alone (6), and stores the FLOPs of its MFMAs in *flops (host, nullable; 0 for
 * shapes 4 and 6); sink is device memory of workgroups x 256 floats (not written in practice). bsa_probe_copy copies `bytes` (a multiple of 16) from src to dst with a
 * grid-stride 16-byte kernel. Both enqueue on `stream` and return BSA_EINVAL on bad arguments. */
int bsa_probe_mfma(int32_t shape, int32_t workgroups, int32_t iters, float* sink, double* flops,
                   void* stream);
int bsa_probe_copy(const void* src, void* dst, size_t bytes, void* stream);

/* Thread-local description of the last error on this thread ("" if none). */
const char* bsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BSA_H */
