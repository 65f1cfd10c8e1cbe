/*
 * bsa.h -- block-sparse attention forward for AMD Instinct MI355X (gfx950).
 *
 * A small C ABI over hand-written HIP kernels.  Four calls make up the path:
 *
 *   bsa_pool_scores         block scores for content-driven selection
 *   bsa_select_topk         per query block, keep the top-k key blocks
 *   bsa_build_arrow_layout  arrow / full / skip block layout per head
 *   (bsa_select_meanpool    the first two fused for mean-pool scoring)
 *   bsa_forward             online-softmax attention over the kept blocks
 *
 * Conventions shared by every call
 * --------------------------------
 * Memory.  Every tensor, score matrix, block list and workspace pointer is
 * DEVICE memory allocated and owned by the caller.  Arrays documented as
 * "host" (head modes, windows, groups) are read during the call only.  The
 * library allocates and frees nothing and keeps no mutable global state, so
 * calls are reentrant; calls that share output buffers must be ordered by
 * the caller.  The one exception is bsa_pool_scores_noalloc, whose
 * workspace is a static per-device scratch array shared by its calls.
 *
 * Streams.  `stream` is a hipStream_t (NULL = the default stream).  Every
 * call only enqueues work on it and never synchronises.  Device-side faults
 * surface at the caller's next synchronisation.
 *
 * Errors.  All arguments are validated before anything is enqueued, so a
 * call that returns an error did no work.  bsa_status_string() names a code;
 * bsa_last_error() returns a thread-local message describing the most
 * recent failure on the calling thread.
 *
 * Tensors.  Q, K, V, O and the output cache are bfloat16 [B][H][N][D] with
 * D contiguous and arbitrary element strides for B, H and N (each a
 * multiple of 8, data 16-byte aligned).  Supported: D in {64, 128}, block
 * size in {64, 128}, any N >= 1 (a last partial block is allowed).
 *
 * Block lists (CSR).  Row r = (b*H + h)*nB + i lists the key blocks kept for
 * query block i of head (b, h), nB = ceil(N / block): row_ptr int32
 * [B*H*nB + 1] (row_ptr[0] = 0, non-decreasing) and col_idx int32 [nnz],
 * strictly ascending within a row.  A block list can be reused by any
 * number of bsa_forward calls.
 *
 * Sources (page title and section the operations are defined in):
 *  [W]  "Block-sparse attention in multimodal DiT" write-up (lmnt.cn):
 *       2.2 content-driven block selection, 2.3 cross-modal handling,
 *       3.1 FlashAttention-style kernel over block indices, 3.2 block size.
 *  [D]  DiTFastAttnV2 notes (ICCV 2025): head-wise arrow attention,
 *       head-wise caching, fused kernel with full / skip / arrow(w) modes.
 *  [S]  SparseD notes (ICLR 2026): isolated selection on avgpool of the
 *       attention map, computed once and reused.
 */
#ifndef BSA_H
#define BSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t bsa_status;
enum {
    BSA_OK = 0,
    BSA_ERR_INVALID_ARG = 1,  /* null pointer, bad shape, stride or range   */
    BSA_ERR_UNSUPPORTED = 2,  /* D, block size or a limit not supported    */
    BSA_ERR_CAPACITY = 3,     /* col_idx capacity below the required bound */
    BSA_ERR_WORKSPACE = 4,    /* workspace missing or too small            */
    BSA_ERR_HIP = 5           /* a HIP runtime call failed                 */
};

/* Per-head modes [D]: FULL keeps every block pair, ARROW keeps the arrow
 * pattern with window w, SKIP computes nothing and returns the cached
 * output of the head. */
enum { BSA_HEAD_FULL = 0, BSA_HEAD_ARROW = 1, BSA_HEAD_SKIP = 2 };

/* Block scoring modes. */
enum { BSA_SCORE_MEANPOOL_PROJ = 0, BSA_SCORE_EXACT_AVGPOOL = 1 };

/* A bfloat16 tensor [B][H][N][D] in device memory, D contiguous. */
typedef struct bsa_tensor {
    void *data;
    int64_t B, H, N, D;
    int64_t stride_b, stride_h, stride_n; /* in elements */
} bsa_tensor;

/* One top-k budget: keep the k best columns of [col_begin, col_end). */
typedef struct bsa_group {
    int32_t col_begin, col_end, k;
} bsa_group;

/* ------------------------------------------------------------------------
 * bsa_pool_scores -- block score matrix S [B][H][nB][nB] (fp32, row-major,
 * device), S[b][h][i][j] scoring query block i against key block j.
 *
 * BSA_SCORE_MEANPOOL_PROJ  ([W] 2.2): every block of Q and of K is mean-
 *   pooled over the tokens it holds, projected by one small linear map
 *   w [D][r] (fp32, row-major, device; shared by queries, keys and heads,
 *   no bias) and scored by a dot product:
 *       S_ij = (W^T qbar_i) . (W^T kbar_j).
 *   `scale` is ignored.
 * BSA_SCORE_EXACT_AVGPOOL  ([S] isolated selection): the average over the
 *   block pair of the post-softmax attention map over all N keys,
 *       A = softmax_row(scale * Q K^T),  S_ij = mean_{t in i, s in j} A_ts,
 *   computed per query block without materialising A.  `w` and `r` are
 *   ignored; scale <= 0 selects 1/sqrt(D).
 *
 * workspace: device memory of at least bsa_pool_scores_workspace_size()
 * bytes (scratch; contents on return are unspecified).
 * Errors: INVALID_ARG (null pointers, q/k shapes differ, r outside 1..64,
 * misaligned data or strides), UNSUPPORTED (D or block), WORKSPACE.
 * ---------------------------------------------------------------------- */
size_t bsa_pool_scores_workspace_size(int64_t B, int64_t H, int64_t N, int64_t D,
                                      int32_t block, int32_t mode, int32_t r);
bsa_status bsa_pool_scores(const bsa_tensor *q, const bsa_tensor *k, int32_t block,
                           int32_t mode, const float *w, int32_t r, float scale,
                           float *scores, void *workspace, size_t workspace_bytes,
                           void *stream);

/* ------------------------------------------------------------------------
 * bsa_pool_scores_noalloc -- bsa_pool_scores for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same arguments and results as
 * bsa_pool_scores, without the workspace: the library's own static scratch
 * array of BSA_SCRATCH_BYTES (32 MiB) per device serves instead.  It is
 * resolved once per device, on that device's first call, and held until
 * the process ends; nothing is allocated or freed.  MEANPOOL_PROJ needs
 * 8*B*H*nB*r bytes of it; EXACT_AVGPOOL needs one slot of 4*nB*block bytes
 * and runs with as many slots as fit (the same scores, possibly fewer
 * persistent workgroups than bsa_pool_scores with a large workspace).
 * Larger requests fail with BSA_ERR_WORKSPACE before anything is enqueued.
 * Every call on one device shares that device's scratch and leaves it
 * holding its own intermediate values: calls that overlap in time on one
 * device (different streams or host threads) race and must be ordered by
 * the caller.  No part of the scratch needs to start at zero: every byte a
 * call reads it has written first.
 * ---------------------------------------------------------------------- */
#define BSA_SCRATCH_BYTES (32u << 20)
bsa_status bsa_pool_scores_noalloc(const bsa_tensor *q, const bsa_tensor *k, int32_t block, int32_t mode,
                                   const float *w, int32_t r, float scale, float *scores, void *stream);

/* ------------------------------------------------------------------------
 * bsa_score_grad -- gradient of the BSA_SCORE_MEANPOOL_PROJ score ([W] 2.2:
 * the projection is trained jointly with the model).  The pages state no
 * loss, so this is the vector-Jacobian product of the score map for the
 * caller's upstream gradient dscores = dL/dS:
 *   p_i = W^T qbar_i,  p'_j = W^T kbar_j,  S_ij = p_i . p'_j
 *   g_i = sum_j dS_ij p'_j,   g'_j = sum_i dS_ij p_i
 *   dw      = sum over b, h and blocks of  qbar_i g_i^T + kbar_j g'_j^T
 *   dq_pool = W g_i (dL/dqbar_i),  dk_pool = W g'_j (dL/dkbar_j)
 *
 * q, k, block, w [D][r], r: as for bsa_pool_scores (device; r in 1..64).
 * dscores: fp32 [B][H][nB][nB], row-major, device.
 * dw: fp32 [D][r], device, overwritten (summed over batch and heads).
 * dq_pool, dk_pool: fp32 [B][H][nB][D], device, overwritten, or NULL when
 *   not wanted.  A token t of block i has dL/dQ_t = dq_pool_i / n_i (n_i =
 *   the tokens of block i), and likewise for K.
 * workspace: at least bsa_score_grad_workspace_size() bytes of device
 *   memory, 16-byte aligned (scratch; contents on return are unspecified).
 * Deterministic: fixed summation orders, no atomics.
 * Errors: INVALID_ARG (null pointers, q/k shapes differ, r outside 1..64,
 * misaligned data or strides), UNSUPPORTED (D, block, more than 2^31 - 1
 * blocks), WORKSPACE.
 * ---------------------------------------------------------------------- */
size_t bsa_score_grad_workspace_size(int64_t B, int64_t H, int64_t N, int64_t D,
                                     int32_t block, int32_t r);
bsa_status bsa_score_grad(const bsa_tensor *q, const bsa_tensor *k, int32_t block,
                          const float *w, int32_t r, const float *dscores, float *dw,
                          float *dq_pool, float *dk_pool, void *workspace,
                          size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * bsa_select_topk -- CSR block list from a score matrix ([W] 2.2, 2.3;
 * [S] isolated selection).  For row (b, h, i):
 *   - a text query block (i < text_blocks) keeps every key block;
 *   - otherwise it keeps the text key blocks {j < text_blocks} united with,
 *     for every group g, the k_g columns of [col_begin, col_end) with the
 *     largest scores; equal scores keep the lower column (-0.0 equals +0.0),
 * and a NaN score ranks below every number (NaNs by lower column).
 * Columns are written ascending.
 *
 * scores  : fp32 [B][H][nB][nB] device.   groups: host [n_groups].
 * row_ptr : int32 [B*H*nB + 1] device (written).
 * col_idx : int32 [capacity] device (written); capacity must be at least
 *           bsa_select_capacity(); the actual nnz is row_ptr[B*H*nB].
 * workspace: at least bsa_select_workspace_size() bytes.
 * Errors: INVALID_ARG (null pointers, group range outside [0, nB), k larger
 * than its range, text_blocks outside [0, nB]), UNSUPPORTED (nB > 1024),
 * CAPACITY, WORKSPACE.
 * ---------------------------------------------------------------------- */
int64_t bsa_select_capacity(int64_t B, int64_t H, int32_t n_blocks, int32_t text_blocks,
                            const bsa_group *groups, int32_t n_groups);
size_t bsa_select_workspace_size(int64_t B, int64_t H, int32_t n_blocks);
bsa_status bsa_select_topk(const float *scores, int64_t B, int64_t H, int32_t n_blocks,
                           int32_t text_blocks, const bsa_group *groups, int32_t n_groups,
                           int32_t *row_ptr, int32_t *col_idx, int64_t capacity,
                           void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * bsa_select_meanpool -- content-driven selection in one call ([W] 2.2:
 * mean-pool, one small projection, dot-product score, top-k; [W] 2.3: text
 * rows and columns dense).  Computes the MEANPOOL_PROJ scores of
 * bsa_pool_scores and the selection of bsa_select_topk in two short
 * kernels: every block of Q and K is pooled and projected once (the
 * pooling kernel of bsa_pool_scores), then one wavefront per row scores
 * and selects it without the score matrix leaving the chip.
 * The scores equal bsa_pool_scores' bit for bit (same pooling, same
 * summation order); the CSR is the one bsa_select_topk gives for them.
 *
 * q, k, block, w [D][r] and r as in bsa_pool_scores; text_blocks, groups,
 * row_ptr, col_idx and capacity as in bsa_select_topk.  scores: device fp32
 * [B][H][nB][nB] or NULL (not written).
 * Limits: nB <= 256 and nB * r4 <= 4096 (r4 = r rounded up to a multiple
 * of 4); the groups with k > 0 pairwise disjoint and clear of the text
 * columns (every row's length is then known in advance).  Outside them the call fails with BSA_ERR_UNSUPPORTED; use
 * bsa_pool_scores and bsa_select_topk.
 * workspace: bsa_select_meanpool_workspace_size() bytes, 16-byte aligned
 * (the projected blocks; contents on return are unspecified).
 * Errors: INVALID_ARG, UNSUPPORTED, CAPACITY, WORKSPACE, HIP.
 * ---------------------------------------------------------------------- */
size_t bsa_select_meanpool_workspace_size(int64_t B, int64_t H, int64_t N, int32_t block, int32_t r);
bsa_status bsa_select_meanpool(const bsa_tensor *q, const bsa_tensor *k, int32_t block, const float *w,
                               int32_t r, int32_t text_blocks, const bsa_group *groups, int32_t n_groups,
                               float *scores, int32_t *row_ptr, int32_t *col_idx, int64_t capacity,
                               void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * bsa_build_arrow_layout -- CSR block list of the arrow layout ([D] head-
 * wise arrow attention).  Text occupies tokens [0, text_len); every block
 * holding a text token is a text block, T_b = ceil(text_len / block).
 *   ARROW head (window w >= 0, in blocks):
 *       keep(i, j) = i < T_b  or  j < T_b  or  |i - j| <= w
 *   FULL head : every (i, j);   SKIP head: every row empty.
 * head_modes int8 [H] and head_windows int32 [H] are host arrays shared by
 * every batch entry.  capacity must be at least bsa_arrow_capacity().
 * Errors: INVALID_ARG (unknown mode, negative window, text_len outside
 * [0, N]), UNSUPPORTED (H > 256 or nB > 65536), CAPACITY.
 * ---------------------------------------------------------------------- */
int64_t bsa_arrow_capacity(int64_t B, int64_t H, int64_t N, int32_t block, int64_t text_len,
                           const int8_t *head_modes, const int32_t *head_windows);
bsa_status bsa_build_arrow_layout(int64_t B, int64_t H, int64_t N, int32_t block,
                                  int64_t text_len, const int8_t *head_modes,
                                  const int32_t *head_windows, int32_t *row_ptr,
                                  int32_t *col_idx, int64_t capacity, void *stream);

/* ------------------------------------------------------------------------
 * Long-row splitting for bsa_forward (optional).  Rows with more than
 * chunk_blocks kept blocks are cut into at most max_chunks contiguous chunks
 * of their block list; each chunk runs in its own workgroup and the partial
 * results (unnormalised output, running max and sum per query) are merged
 * afterwards, which is exact up to rounding order.  At most max_split_rows
 * rows are split (in the order text-like long rows are met: query-block
 * major, then batch and head); further long rows run unsplit.  This is a
 * scheduling device only: it balances rows of very different lengths (text
 * rows and full heads next to short windowed rows, [W] 4.3 on the cost of
 * irregular block sets); it does not change the result beyond rounding.
 * ---------------------------------------------------------------------- */
typedef struct bsa_split {
    int32_t chunk_blocks;   /* split rows longer than this (>= 1)            */
    int32_t max_chunks;     /* chunks per split row, 2..64                    */
    int64_t max_split_rows; /* capacity of the partial-result pool, >= 1      */
    void *workspace;        /* device, >= bsa_forward_split_workspace_size()  */
    size_t workspace_bytes;
} bsa_split;

size_t bsa_forward_split_workspace_size(int64_t B, int64_t H, int64_t N, int64_t D, int32_t block,
                                        int32_t max_chunks, int64_t max_split_rows);

/* Split recommendation for the layouts whose row lengths are known in
 * closed form (computed on the host from the layout's parameters; no device
 * data is read and nothing is enqueued).  Each returns 1 and fills
 * chunk_blocks, max_chunks and max_split_rows of *out (workspace set to
 * NULL, workspace_bytes to 0) when cutting the long rows is predicted to
 * shorten the forward, 0 when every row should run whole, and -1 on invalid
 * arguments.  The prediction is a greedy list schedule of the rows, in the
 * forward's dispatch order, over the workgroups that run at once, with the
 * plan and combine cost added; rows longer than max(typical row,
 * ceil(nB / 4)) are the candidates.  Arguments as for the matching layout
 * builder (bsa_build_arrow_layout, bsa_select_topk, and
 * bsa_build_neighborhood_layout with its block). */
int32_t bsa_split_policy_arrow(int64_t B, int64_t H, int64_t N, int32_t block, int64_t text_len,
                               const int8_t *head_modes, const int32_t *head_windows, bsa_split *out);
int32_t bsa_split_policy_select(int64_t B, int64_t H, int32_t n_blocks, int32_t text_blocks,
                                const bsa_group *groups, int32_t n_groups, int32_t block, bsa_split *out);

/* ------------------------------------------------------------------------
 * bsa_forward -- block-sparse attention forward ([W] 3.1, [D] fused
 * kernel, [S] sparse attention with a precomputed mask).  For every token
 * t of a computed head, with i = t / block:
 *     z_s = scale * Q_t . K_s  for keys s in the blocks of row (b, h, i),
 *     O_t = sum_s softmax(z)_s V_s   (bfloat16, fp32 accumulation),
 *     LSE_t = ln sum_s exp(z_s)      (fp32, natural log).
 * Blocks are visited in CSR order with an online softmax; key blocks are
 * all-in or all-out (no masking inside a block except past N).  A row with
 * no kept block gives O = 0 and LSE = -inf.  Column indices outside
 * [0, nB) are ignored; columns of one row must be distinct.
 *
 * head_modes: host int8 [H] or NULL (every head computed).  A SKIP head is
 * not computed: O[b][h] is copied from o_cache[b][h] bit-exactly (nothing is
 * copied when o_cache aliases o with the same strides) and LSE from
 * lse_cache (device fp32 [B][H][N]) when lse_cache is not NULL, else left
 * untouched ([D] head-wise caching).  o_cache is required iff some head is
 * SKIP.
 * scale <= 0 selects 1/sqrt(D).  lse: device fp32 [B][H][N] or NULL.
 * split: NULL (every row in one workgroup) or the long-row splitting above.
 * Errors: INVALID_ARG (null pointers, shape mismatch, misalignment, SKIP
 * without o_cache, bad split parameters), UNSUPPORTED (D or block size),
 * WORKSPACE (split workspace too small).
 * ---------------------------------------------------------------------- */
bsa_status bsa_forward(const bsa_tensor *q, const bsa_tensor *k, const bsa_tensor *v,
                       int32_t block, const int32_t *row_ptr, const int32_t *col_idx,
                       const int8_t *head_modes, const bsa_tensor *o_cache,
                       const float *lse_cache, float scale, const bsa_tensor *o, float *lse,
                       const bsa_split *split, void *stream);

/* ------------------------------------------------------------------------
 * Backward of bsa_forward (the gradient a training step needs; the
 * multimodal-DiT write-up trains its selection projection jointly with the
 * model, section 2.2).  For the softmax restricted to the kept blocks,
 *   dV = P^T dO,  dK = scale * dS^T Q,  dQ = scale * dS K,
 *   dS = P * (dO V^T - rowsum(dO * O)),
 * with P recomputed from Q, K and the forward's LSE.  q, k, v, o, dO, dq, dk,
 * dv are bf16 tensors as in bsa_forward (same shape, any strides); lse is
 * the forward's fp32 [B][H][N] (natural log).  The block list is the
 * forward's; its columns must ascend within each row (as every layout
 * builder here writes them).  Every head is computed (rows of a head with
 * no kept block give zero gradients).  The workspace
 * (bsa_backward_workspace_size bytes, 16-byte aligned) holds two fp32
 * [B][H][N] arrays.  Results are deterministic.  Errors: INVALID_ARG,
 * UNSUPPORTED (D, block, more than 7680 blocks per head), WORKSPACE.
 * ---------------------------------------------------------------------- */
size_t bsa_backward_workspace_size(int64_t B, int64_t H, int64_t N);
bsa_status bsa_backward(const bsa_tensor *q, const bsa_tensor *k, const bsa_tensor *v, const bsa_tensor *o,
                        const bsa_tensor *dO, int32_t block, const int32_t *row_ptr, const int32_t *col_idx,
                        const float *lse, float scale, const bsa_tensor *dq, const bsa_tensor *dk,
                        const bsa_tensor *dv, void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * 2-D neighbourhood attention (GNA notes, 1.1: a window around each query
 * on the latent grid with a stride by which groups of queries share one
 * window; 2.1: fine-grained masking only where a key tile is partially
 * inside the windows; 2.2: token permutation into tiles).
 *
 * The sequence is text_len text tokens, then an rows x cols image grid in
 * row-major ("natural") order.  Text queries see every key and every query
 * sees the text keys.  On an axis of length L with window k and stride s,
 * the image query at position i sees positions
 *     start(i) .. start(i) + k - 1,
 *     start(i) = clamp(s * floor(i / s) + floor(s / 2) - floor(k / 2), 0, L - k),
 * on both axes (s = 1: a sliding window; s = k: blocked attention).
 *
 * Kernels work in tile-major order: text tokens first, then the image cut
 * into tile_rows x tile_cols tiles (tile_rows * tile_cols = block,
 * tile_cols a power of two), tiles row-major, tokens row-major within a
 * tile, so each block is one tile.  text_len must be a whole number of
 * blocks and the grid a whole number of tiles; N = text_len + rows * cols.
 *
 * bsa_permute_tokens moves a bf16 [B][H][N][D] tensor (and optionally an
 * fp32 [B][H][N] LSE) from natural to tile-major order, or back when
 * inverse != 0 (for O and LSE); not in place.
 *
 * bsa_build_neighborhood_layout writes the CSR block list of every
 * (b, h) (all heads alike) in tile-major order plus a flag per entry:
 * 0 = every query of the query tile sees every key of the key tile,
 * 1 = partially covered, masked per token by the forward.  Columns ascend.
 * capacity >= bsa_neighborhood_capacity() entries (-1 on a bad geometry).
 *
 * bsa_forward_neighborhood: bsa_forward (every head computed, no head
 * modes) on tile-major Q, K, V with that block list and its flags; O and
 * LSE come out in tile-major order.  The row max of a partial tile is taken
 * over all its keys (an upper bound of the kept ones): the result is exact
 * unless masked logits exceed every kept one by more than ~87 (natural
 * units), where the kept probabilities would underflow.
 * Errors: INVALID_ARG (geometry, shapes, nulls), UNSUPPORTED, CAPACITY.
 * ---------------------------------------------------------------------- */
typedef struct bsa_neighborhood {
    int64_t text_len;
    int32_t rows, cols;
    int32_t tile_rows, tile_cols;
    int32_t window_rows, window_cols;
    int32_t stride_rows, stride_cols;
} bsa_neighborhood;

bsa_status bsa_permute_tokens(const bsa_tensor *in, const bsa_tensor *out, const float *lse_in, float *lse_out,
                              int32_t block, const bsa_neighborhood *nb, int32_t inverse, void *stream);
/* Split recommendation for a neighbourhood layout (see bsa_split_policy_arrow). */
int32_t bsa_split_policy_neighborhood(int64_t B, int64_t H, int32_t block, const bsa_neighborhood *nb,
                                      bsa_split *out);
int64_t bsa_neighborhood_capacity(int64_t B, int64_t H, int32_t block, const bsa_neighborhood *nb);
bsa_status bsa_build_neighborhood_layout(int64_t B, int64_t H, int32_t block, const bsa_neighborhood *nb,
                                         int32_t *row_ptr, int32_t *col_idx, int32_t *entry_flags,
                                         int64_t capacity, void *stream);
bsa_status bsa_forward_neighborhood(const bsa_tensor *q, const bsa_tensor *k, const bsa_tensor *v, int32_t block,
                                    const int32_t *row_ptr, const int32_t *col_idx, const int32_t *entry_flags,
                                    const bsa_neighborhood *nb, float scale, const bsa_tensor *o, float *lse,
                                    const bsa_split *split, void *stream);

/* bsa_forward_neighborhood_natural -- bsa_forward_neighborhood on Q, K, V
 * in natural order (text, then the grid row-major), with O and LSE written
 * in natural order: the kernel gathers each tile-major tile from its grid
 * rows and scatters its outputs, so no permutation pass is needed.  The
 * block list and flags are those of bsa_build_neighborhood_layout
 * (tile-major block indices).  Same errors as bsa_forward_neighborhood. */
bsa_status bsa_forward_neighborhood_natural(const bsa_tensor *q, const bsa_tensor *k, const bsa_tensor *v,
                                            int32_t block, const int32_t *row_ptr, const int32_t *col_idx,
                                            const int32_t *entry_flags, const bsa_neighborhood *nb, float scale,
                                            const bsa_tensor *o, float *lse, const bsa_split *split,
                                            void *stream);

/* bsa_backward_neighborhood -- bsa_backward for the 2-D neighbourhood
 * layout (GNA notes, 1.1 and 2.1): tile-major Q, K, V, O, dO and LSE as
 * bsa_forward_neighborhood produced them, its block list and entry flags
 * and the same geometry; partially covered entries are masked per token as
 * in the forward.  dQ, dK, dV come out in tile-major order (the caller
 * permutes them back with bsa_permute_tokens, inverse = 1).  Same
 * workspace, limits and errors as bsa_backward, plus the geometry checks of
 * bsa_forward_neighborhood. */
bsa_status bsa_backward_neighborhood(const bsa_tensor *q, const bsa_tensor *k, const bsa_tensor *v,
                                     const bsa_tensor *o, const bsa_tensor *dO, int32_t block,
                                     const int32_t *row_ptr, const int32_t *col_idx, const int32_t *entry_flags,
                                     const bsa_neighborhood *nb, const float *lse, float scale,
                                     const bsa_tensor *dq, const bsa_tensor *dk, const bsa_tensor *dv,
                                     void *workspace, size_t workspace_bytes, void *stream);

/* bsa_backward_neighborhood_natural -- bsa_backward_neighborhood with Q, K,
 * V, O, dO and LSE in natural order (as bsa_forward_neighborhood_natural
 * produced O and LSE) and dQ, dK, dV written in natural order: the kernels
 * gather the tile-major tiles from the grid rows and scatter the gradient
 * rows, so no permutation pass is needed.  Block list and flags as for
 * bsa_backward_neighborhood; same workspace, limits and errors. */
bsa_status bsa_backward_neighborhood_natural(const bsa_tensor *q, const bsa_tensor *k, const bsa_tensor *v,
                                             const bsa_tensor *o, const bsa_tensor *dO, int32_t block,
                                             const int32_t *row_ptr, const int32_t *col_idx,
                                             const int32_t *entry_flags, const bsa_neighborhood *nb,
                                             const float *lse, float scale, const bsa_tensor *dq,
                                             const bsa_tensor *dk, const bsa_tensor *dv, void *workspace,
                                             size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * FP8 forward (OCP E4M3 operands on the gfx950 FP8 matrix cores).
 *
 * The same operation as bsa_forward -- the dense softmax restricted to the
 * kept key blocks of every query block -- with Q, K, V held as E4M3 codes
 * and a scale per group, and P rounded to E4M3 for the P.V product.  This
 * is the FP8 throughput mode of block-sparse attention kernels (GNA sparse
 * attention write-up, section 2.1, mixed-precision support, and section
 * 1.2 for its FP16 / FP8 rates); results carry FP8 rounding error.
 *
 * bsa_quantize_fp8 fills a bsa_fp8_qkv from bf16 Q, K, V (same shapes and
 * conventions as bsa_forward), with max-abs scaling to +-448:
 *   q8 [B][H][N][D] uint8,  q_scale [B][H][N]        one scale per token,
 *   k8 [B][H][N][D] uint8,  k_scale [B][H][NT]       one per 64-key tile
 *                                                    (NT = ceil(N/64)),
 *   v8t [B][H][D][NP] uint8, v_scale [B][H][D]       one per channel,
 * with NP = 64*NT; v8t is V transposed, keys permuted inside each 64-key
 * group: key 64T + 32a + 8g + 4h + e (a, h in {0,1}, g, e in 0..3) sits at
 * column 64T + 32h + 16a + 4g + e; padding columns are 0.  For each group
 * scale = amax / 448 and code = E4M3(x * (448 / amax)), rounded to nearest
 * even, decided in fp32 (all 0 for an all-zero group).  All arrays are
 * caller-owned device memory, 16-byte aligned, contiguous as shown.  The
 * workspace (bsa_quantize_fp8_workspace_size bytes, 16-byte aligned) holds
 * the per-channel maxima.  Errors: INVALID_ARG, UNSUPPORTED (D not in
 * {64, 128}), WORKSPACE.
 *
 * bsa_forward_fp8 computes O (bf16, any strides as in bsa_forward) and LSE
 * (natural log, fp32 [B][H][N] or NULL) from a bsa_fp8_qkv with the CSR of
 * bsa_forward; scale <= 0 means 1/sqrt(D).  head_modes, o_cache, lse_cache
 * and split mean what they mean for bsa_forward: a SKIP head is copied from
 * the caches bit for bit ([D] head-wise caching), long rows may be cut into
 * chunks merged afterwards.  The row sum that normalises O and gives LSE is
 * the sum of the E4M3-rounded probabilities.  Errors: INVALID_ARG,
 * UNSUPPORTED (D not in {64, 128}, block not in {64, 128}), WORKSPACE.
 * ---------------------------------------------------------------------- */
typedef struct bsa_fp8_qkv {
    void *q8;
    float *q_scale;
    void *k8;
    float *k_scale;
    void *v8t;
    float *v_scale;
    int64_t B, H, N, D;
} bsa_fp8_qkv;

size_t bsa_quantize_fp8_workspace_size(int64_t B, int64_t H, int64_t N, int64_t D);
bsa_status bsa_quantize_fp8(const bsa_tensor *q, const bsa_tensor *k, const bsa_tensor *v,
                            const bsa_fp8_qkv *out, void *workspace, size_t workspace_bytes,
                            void *stream);
bsa_status bsa_forward_fp8(const bsa_fp8_qkv *in, int32_t block, const int32_t *row_ptr,
                           const int32_t *col_idx, const int8_t *head_modes, const bsa_tensor *o_cache,
                           const float *lse_cache, float scale, const bsa_tensor *o, float *lse,
                           const bsa_split *split, void *stream);

/* bsa_forward_fp8_neighborhood -- bsa_forward_fp8 for the 2-D neighbourhood
 * layout (GNA notes, 2.1: its FP8 mode): `in` quantised from tile-major Q,
 * K, V (bsa_permute_tokens, then bsa_quantize_fp8), the block list and
 * entry flags of bsa_build_neighborhood_layout and the same geometry;
 * partially covered entries are masked per token as in
 * bsa_forward_neighborhood.  O and LSE come out in tile-major order.
 * Errors as for bsa_forward_fp8 plus the geometry checks. */
bsa_status bsa_forward_fp8_neighborhood(const bsa_fp8_qkv *in, int32_t block, const int32_t *row_ptr,
                                        const int32_t *col_idx, const int32_t *entry_flags,
                                        const bsa_neighborhood *nb, float scale, const bsa_tensor *o, float *lse,
                                        void *stream);

/* bsa_quantize_fp8_neighborhood -- bsa_quantize_fp8 of natural-order Q, K,
 * V (text, then the grid row-major) whose codes come out in the tile-major
 * order of the geometry (block = tile_rows * tile_cols): the result equals,
 * bit for bit, bsa_permute_tokens of each tensor followed by
 * bsa_quantize_fp8 (GNA notes, 2.2: the permutation folded into a pass that
 * reads the tensors anyway).  Errors as for bsa_quantize_fp8 plus the
 * geometry checks.
 *
 * bsa_forward_fp8_neighborhood_natural -- bsa_forward_fp8_neighborhood
 * with O and LSE written in natural order (the kernel scatters each query
 * row to its grid position); `in` in tile-major order as above. */
bsa_status bsa_quantize_fp8_neighborhood(const bsa_tensor *q, const bsa_tensor *k, const bsa_tensor *v,
                                         int32_t block, const bsa_neighborhood *nb, const bsa_fp8_qkv *out,
                                         void *workspace, size_t workspace_bytes, void *stream);
bsa_status bsa_forward_fp8_neighborhood_natural(const bsa_fp8_qkv *in, int32_t block, const int32_t *row_ptr,
                                                const int32_t *col_idx, const int32_t *entry_flags,
                                                const bsa_neighborhood *nb, float scale, const bsa_tensor *o,
                                                float *lse, void *stream);

/* ------------------------------------------------------------------------
 * Diagnostics of sparse attention.
 *
 * bsa_output_rse: per-(b, h) relative squared error of an attention output
 * against a reference output (DiTFastAttnV2, head-wise arrow attention:
 * the single-layer RSE by which its compression plans are judged):
 *     rse[b*H + h] = sum (test - ref)^2 / sum (ref - mean(ref))^2
 * with sums and the mean over the head's N x D elements, accumulated in
 * fp64.  A reference with no spread gives +inf (0 when test == ref).  test
 * and ref are bf16 tensors as in bsa_forward (same shape, any strides);
 * rse is device memory, fp64 [B*H].  The workspace
 * (bsa_output_rse_workspace_size bytes, 16-byte aligned) holds per-chunk
 * partial sums.  Errors: INVALID_ARG, UNSUPPORTED (D not in {64, 128}),
 * WORKSPACE.
 *
 * bsa_mask_jaccard: per-(b, h) Jaccard similarity |A & B| / |A | B| of two
 * block masks given as CSR over rows (b*H + h)*n_blocks + i, n_blocks key
 * blocks per row (SparseD, sparse reuse: the stability of the reused mask
 * against each step's own selection).  Entries outside [0, n_blocks) are
 * ignored, repeated entries count once, two empty masks give 1.  All
 * arrays are device memory; jaccard is fp64 [B*H].  Errors: INVALID_ARG,
 * UNSUPPORTED (n_blocks > 65536 or B*H > 2^31 - 1).
 * ---------------------------------------------------------------------- */
size_t bsa_output_rse_workspace_size(int64_t B, int64_t H, int64_t N, int64_t D);
bsa_status bsa_output_rse(const bsa_tensor *test, const bsa_tensor *ref, double *rse, void *workspace,
                          size_t workspace_bytes, void *stream);
bsa_status bsa_mask_jaccard(int64_t B, int64_t H, int32_t n_blocks, const int32_t *row_ptr_a,
                            const int32_t *col_idx_a, const int32_t *row_ptr_b, const int32_t *col_idx_b,
                            double *jaccard, void *stream);

/* ------------------------------------------------------------------------
 * bsa_reuse_full_steps, bsa_reuse_step_action -- the select-once schedule
 * of [S] (skipping sparse, then sparse reuse) over `steps` denoising steps.
 * Steps 0 .. n_full-1 run full attention, n_full = floor(steps * skip); a
 * product that lands within 1e-9 below an integer counts as that integer
 * (10 x 0.3 gives 3).  Step n_full computes the exact avgpool scores,
 * selects the mask and runs sparse attention with it; every later step
 * reuses that mask.  Host only, nothing is enqueued.
 * bsa_reuse_full_steps returns n_full (0 .. steps), or -1 when steps < 1 or
 * skip is not in [0, 1] (NaN included).  bsa_reuse_step_action returns the
 * BSA_STEP_* action of step `step`, or -1 on the same errors or when step
 * is not in [0, steps).
 * ---------------------------------------------------------------------- */
enum { BSA_STEP_FULL = 0, BSA_STEP_SELECT = 1, BSA_STEP_SPARSE = 2 };
int32_t bsa_reuse_full_steps(int32_t steps, double skip);
int32_t bsa_reuse_step_action(int32_t steps, double skip, int32_t step);

/* ------------------------------------------------------------------------
 * Utilities.
 * ---------------------------------------------------------------------- */
/* Name of a status code (static string). */
const char *bsa_status_string(bsa_status status);
/* Message describing the most recent failure on the calling thread. */
const char *bsa_last_error(void);
/* Library version string. */
const char *bsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BSA_H */
