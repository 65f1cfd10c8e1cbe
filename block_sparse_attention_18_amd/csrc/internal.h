// Kernel parameter blocks and host launchers (one per kernel source file).
// Host-side only declarations; the C ABI in bsa_api.cpp validates every
// argument before calling a launcher.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsa {

constexpr int kMaxSkipHeads = 1024;   // bitmask of SKIP heads carried in kernel args
constexpr int kMaxArrowHeads = 256;   // per-head modes/windows carried in kernel args
constexpr int kMaxSelectBlocks = 1024;
constexpr int kExactSlots = 1024;     // persistent workgroups of the exact-score kernel

struct Tensor4 {
    const uint16_t *p;
    int64_t sb, sh, sn;
};

// Geometry of 2-D neighbourhood attention in tile-major token order: T text
// tokens (Tb blocks), then an R x C image grid cut into th x tw tiles (one
// block each, tw a power of two, tpr tiles per tile row), window kh x kw,
// stride sh x sw.  rep has bit x tw set for every x < 64 / tw (tw < 64),
// else only bit 0: multiplying a tw-bit pattern by it repeats the pattern
// across 64 bits.
struct NbGeom {
    int32_t T, Tb, R, C, th, tw, tw_log2, tpr, kh, kw, sh, sw;
    uint64_t rep;
};

// First position of the window of position i on an axis of length L
// (window k, stride s): the window of the centre of i's stride group,
// shifted inside the axis.
__host__ __device__ inline int32_t nb_start(int32_t i, int32_t L, int32_t k, int32_t s)
{
    const int32_t a = s * (i / s) + s / 2 - k / 2;
    return a < 0 ? 0 : (a > L - k ? L - k : a);
}

// Natural position of the token at tile-major position t (text tokens keep
// theirs), and the natural offset of tile-major row o inside a tile (o <
// block): the tile's rows are tw-token runs of the grid, C apart.
__host__ __device__ inline int32_t nb_rowoff(const NbGeom &g, int32_t o)
{
    return (o >> g.tw_log2) * g.C + (o & (g.tw - 1));
}

__host__ __device__ inline int32_t nb_natural(const NbGeom &g, int32_t block, int32_t t)
{
    if (t < g.T) return t;
    const int32_t pt = t - g.T, tile = pt / block, a = tile / g.tpr;
    return g.T + a * g.th * g.C + (tile - a * g.tpr) * g.tw + nb_rowoff(g, pt - tile * block);
}

#ifdef __HIPCC__
// Bits a .. b-1 of a 64-bit word (a, b clamped to 0..64; empty if b <= a).
__device__ __forceinline__ uint64_t bit_range64(int a, int b)
{
    a = min(max(a, 0), 64);
    b = min(max(b, 0), 64);
    const uint64_t hi = b >= 64 ? ~0ull : (1ull << b) - 1;
    const uint64_t lo = a >= 64 ? ~0ull : (1ull << a) - 1;
    return hi & ~lo;
}

// Which of 64 consecutive tokens of an image tile lie in a window of kh x kw
// grid positions: bit b stands for the token at offset s0 + b in the tile,
// kr / kc are the tile's first grid row / column minus the window's.  Tile
// row x holds offsets x tw .. x tw + tw - 1, so the window's rows form one
// run of bits and its columns a run repeated every tw bits.  s0 is a
// multiple of 64, or of 32 when only bits 0..31 are read.
__device__ __forceinline__ uint64_t nb_window_bits(const NbGeom &g, int s0, int kr, int kc, int kh, int kw)
{
    const int rlo = max(0, -kr), rhi = min(g.th, kh - kr);
    const uint64_t rows = rhi > rlo ? bit_range64(rlo * g.tw - s0, rhi * g.tw - s0) : 0ull;
    const int cs0 = s0 & (g.tw - 1);
    const int clo = max(0, -kc), chi = min(g.tw, kw - kc);
    const uint64_t cols = bit_range64(clo - cs0, chi - cs0) * g.rep;
    return rows & cols;
}
#endif

// Image query tile i (i >= Tb): the key tile ranges its queries' windows
// touch ([r0, r1) x [c0, c1) in tiles) and the token ranges every one of
// its queries sees ([ir0, ir1) x [ic0, ic1), possibly empty).
struct NbRow {
    int32_t r0, r1, c0, c1, ir0, ir1, ic0, ic1;
};

__host__ __device__ inline NbRow nb_row(const NbGeom &g, int32_t i)
{
    const int32_t tile = i - g.Tb, a = tile / g.tpr, b = tile - a * g.tpr;
    const int32_t q0 = a * g.th, q1 = q0 + g.th - 1, p0 = b * g.tw, p1 = p0 + g.tw - 1;
    NbRow w;
    const int32_t ur0 = nb_start(q0, g.R, g.kh, g.sh), ur1 = nb_start(q1, g.R, g.kh, g.sh) + g.kh;
    const int32_t uc0 = nb_start(p0, g.C, g.kw, g.sw), uc1 = nb_start(p1, g.C, g.kw, g.sw) + g.kw;
    w.r0 = ur0 / g.th;
    w.r1 = (ur1 + g.th - 1) / g.th;
    w.c0 = uc0 / g.tw;
    w.c1 = (uc1 + g.tw - 1) / g.tw;
    w.ir0 = nb_start(q1, g.R, g.kh, g.sh);
    w.ir1 = nb_start(q0, g.R, g.kh, g.sh) + g.kh;
    w.ic0 = nb_start(p1, g.C, g.kw, g.sw);
    w.ic1 = nb_start(p0, g.C, g.kw, g.sw) + g.kw;
    return w;
}

__host__ __device__ inline int64_t nb_row_len(const NbGeom &g, int32_t nB, int32_t i)
{
    if (i < g.Tb) return nB;
    const NbRow w = nb_row(g, i);
    return (int64_t)g.Tb + (int64_t)(w.r1 - w.r0) * (w.c1 - w.c0);
}

struct FwdParams {
    Tensor4 q, k, v;
    uint16_t *o;
    int64_t o_sb, o_sh, o_sn;
    float *lse;                 // [B][H][N] or null
    const int32_t *row_ptr;
    const int32_t *col_idx;
    int32_t B, H, N, nB;
    float scale_log2;           // softmax scale * log2(e)
    uint32_t skip_bits[kMaxSkipHeads / 32];
    // long-row splitting (items == null: one workgroup per row)
    const int4 *items;          // {row, chunk, chunks, split rank or -1}
    const int32_t *counts;      // [0] items, [1] split rows
    float *partials;            // [split rank * max_chunks + chunk] slots
    int32_t max_chunks;
    // 2-D neighbourhood masking (flags == null: none): per CSR entry 0 = every
    // (query, key) pair of the block pair kept, 1 = masked per token
    const int32_t *flags;
    NbGeom nb;
    int32_t natural;            // neighbourhood: Q, K, V, O, LSE in natural token order
    // SKIP heads: the workgroup of a SKIP row copies that row's cached
    // output (when copy_o) and LSE (when lse_src is set) instead of computing
    Tensor4 oc;                 // o_cache
    const float *lse_src;       // lse_cache [B][H][N] or null
    int32_t copy_o;
};

// Backward of the forward (see bsa_backward).  The dK/dV kernel keeps the
// list of query blocks of its key block in LDS beside the block's K and V
// and two Q/dO sub-tiles, which bounds the number of blocks per head.
constexpr int kBwdMaxBlocks = 7680;
struct BwdParams {
    Tensor4 q, k, v, o, dO;
    const float *lse;           // [B][H][N], natural log
    float *lse2, *delta;        // workspace: LSE * log2(e), rowsum(dO * O)
    const int32_t *row_ptr, *col_idx;
    const int32_t *flags;       // neighbourhood layouts: 1 = partially covered entry; else null
    NbGeom nb;
    uint16_t *dq, *dk, *dv;
    int64_t dq_sb, dq_sh, dq_sn, dk_sb, dk_sh, dk_sn, dv_sb, dv_sh, dv_sn;
    int32_t B, H, N, D, nB;
    float scale, scale_log2;
    // neighbourhood layouts: 0, or the block when every [B][H][N] tensor is in
    // natural token order (the kernels gather and scatter tile-major rows)
    int32_t natural;
};

// Tile-major token permutation (see bsa_permute_tokens).
struct PermuteParams {
    Tensor4 in;
    uint16_t *out;
    int64_t o_sb, o_sh, o_sn;
    const float *lse_in;
    float *lse_out;
    NbGeom nb;
    int32_t B, H, N, D, inverse;
};

// 2-D neighbourhood block layout (see bsa_build_neighborhood_layout).
struct NbLayoutParams {
    NbGeom nb;
    int32_t *row_ptr, *col_idx, *flags;
    int64_t capacity, per_head;  // per_head: entries of one head
    int32_t B, H, nB;
};

// Work-list builder for long-row splitting.
struct PlanParams {
    const int32_t *row_ptr;
    int4 *items;
    int32_t *counts;
    int2 *split_rows;           // [rank] = {row, chunks}
    int32_t BH, H, nB;
    int32_t chunk_blocks, max_chunks;
    int64_t max_split_rows;
    uint32_t skip_bits[kMaxSkipHeads / 32];   // rows of SKIP heads are never split
};

// Merges the partial results of split rows.
struct CombineParams {
    const float *partials;
    const int32_t *counts;
    const int2 *split_rows;
    uint16_t *o;
    int64_t o_sb, o_sh, o_sn;
    float *lse;
    int32_t H, N, nB, D, block;
    int32_t max_chunks;
    int32_t natural;            // neighbourhood: write O, LSE at natural token positions
    NbGeom nb;
};

struct SkipCopyParams {
    Tensor4 src;                // o_cache
    uint16_t *dst;
    int64_t d_sb, d_sh, d_sn;
    const float *lse_src;       // may be null
    float *lse_dst;             // may be null
    int32_t B, H, N, D;
    int32_t copy_o;             // 0 when o_cache aliases o
    uint32_t skip_bits[kMaxSkipHeads / 32];
};

struct PoolParams {
    Tensor4 x[2];               // q, k
    const float *w;             // [D][r]
    float *proj;                // [2][B*H*nB][r]
    float *mean;                // [2][B*H*nB][D] block means, or null
    int32_t B, H, N, nB, r;
};

// Gradient of the projected score (see bsa_score_grad); dW is summed from
// partials over chunks of kGradChunk blocks of a head.
constexpr int kGradChunk = 16;
struct ScoreGradParams {
    const float *proj;          // [2][BH*nB][r]   p_i, p'_j
    const float *mean;          // [2][BH*nB][D]   qbar_i, kbar_j
    const float *dS;            // [BH][nB][nB]
    const float *w;             // [D][r]
    float *g;                   // [2][BH*nB][r]   dL/dp_i, dL/dp'_j
    float *dpool[2];            // [BH*nB][D] dL/dqbar, dL/dkbar, or null
    float *wpart;               // [BH * chunks][D*r] partial dW per chunk of blocks
    float *dw;                  // [D][r]
    int32_t BH, nB, D, r;
};

struct ScoreParams {
    const float *proj;          // [2][B*H*nB][r]
    float *S;                   // [B*H][nB][nB]
    int32_t BH, nB, r;
};

struct ExactParams {
    Tensor4 q, k;
    float *S;                   // [B*H][nB][nB]
    float *scratch;             // [slots][nB][block] log2-domain block log-sum-exps
    int32_t B, H, N, nB;
    float scale_log2;
};

struct SelectParams {
    const float *S;             // [rows][nB]
    int32_t *row_ptr;           // counts written to row_ptr[r + 1] (direct: offsets)
    uint32_t *bits;             // [rows][words] (two-pass path only)
    int32_t *col_idx;           // direct path only
    int64_t rows, capacity;
    int32_t nB, words, text_blocks, n_groups;
    int32_t direct;             // row lengths known: write row_ptr and col_idx in place
    int32_t row_len;            // length of a non-text row on the direct path
    int32_t g_begin[8], g_end[8], g_k[8];
};

// Fused mean-pool / projection / score / top-k selection (see
// bsa_select_meanpool): the head's projections sit in LDS in phase 2.
constexpr int kMpsMaxBlocks = 256;     // blocks per head
constexpr int kMpsMaxProj = 4096;      // nB * r floats of one side's projections
struct MeanpoolSelectParams {
    Tensor4 q, k;
    const float *w;             // [D][r]
    float *proj;                // workspace [2][B*H*nB][r]: projected Q blocks, then K blocks
    float *scores;              // [B*H][nB][nB] or null
    int32_t *row_ptr, *col_idx;
    int64_t capacity;
    int32_t B, H, N, nB, r, text_blocks, n_groups, row_len;
    int32_t g_begin[8], g_end[8], g_k[8];
};

struct ExpandParams {
    const uint32_t *bits;
    const int32_t *row_ptr;
    int32_t *col_idx;
    int64_t rows, capacity;
    int32_t words;
};

struct ArrowParams {
    int32_t *row_ptr;
    int32_t *col_idx;
    int64_t capacity;
    int64_t per_batch;          // nnz of one batch entry (all heads)
    int32_t B, H, nB, text_blocks;
    int8_t mode[kMaxArrowHeads];
    int32_t window[kMaxArrowHeads];
};

// FP8 (E4M3) quantisation of Q, K, V (see bsa_quantize_fp8).
struct Fp8QuantParams {
    Tensor4 q, k, v;
    uint8_t *q8, *k8, *v8t;
    float *q_scale, *k_scale, *v_scale;
    float *vmax_part;           // [B*H][S][D] channel maxima of 256-key chunks
    float *v_inv;               // [B*H][D] 448 / amax
    int64_t BHN;
    int32_t B, H, N, NT, NP, S;
    // neighbourhood layouts: codes in tile-major order read from natural-order
    // inputs (nb_block = the block of the geometry nb; 0: no reordering)
    NbGeom nb;
    int32_t nb_block;
};

// FP8 forward (see bsa_forward_fp8).
struct Fp8FwdParams {
    const uint8_t *q8, *k8, *v8t;
    const float *q_scale, *k_scale, *v_scale;
    uint16_t *o;
    int64_t o_sb, o_sh, o_sn;
    float *lse;
    const int32_t *row_ptr;
    const int32_t *col_idx;
    const int32_t *flags;       // neighbourhood layouts: 1 = partially covered entry; else null
    NbGeom nb;
    int32_t B, H, N, nB, NT, NP;
    float scale_log2;
    int32_t natural;            // neighbourhood layouts: O and LSE written in natural token order
    uint32_t skip_bits[kMaxSkipHeads / 32];   // SKIP heads: nothing computed
    // long-row splitting (items == null: one workgroup per row), as in FwdParams
    const int4 *items;
    const int32_t *counts;
    float *partials;
    int32_t max_chunks;
};

// Per-head RSE of an output against a reference (see bsa_output_rse).
struct RseParams {
    Tensor4 test, ref;
    double *partials;           // [B*H][chunks][3]
    double *rse;                // [B*H]
    int32_t B, H, N, D, chunks, rows_per_chunk;
};

// Per-head Jaccard similarity of two block masks (see bsa_mask_jaccard).
struct JaccardParams {
    const int32_t *row_ptr_a, *col_idx_a, *row_ptr_b, *col_idx_b;
    double *jaccard;            // [B*H]
    int32_t B, H, nB;
};

hipError_t launch_forward(const FwdParams &p, int block, int D, int64_t grid, hipStream_t s);
hipError_t launch_output_rse(const RseParams &p, hipStream_t s);
hipError_t launch_permute_tokens(const PermuteParams &p, hipStream_t s);
hipError_t launch_backward(const BwdParams &p, int block, int D, hipStream_t s);   // masks when p.flags
hipError_t launch_neighborhood_layout(const NbLayoutParams &p, hipStream_t s);
hipError_t launch_mask_jaccard(const JaccardParams &p, hipStream_t s);
hipError_t launch_quantize_fp8(const Fp8QuantParams &p, int D, hipStream_t s);
hipError_t launch_forward_fp8(const Fp8FwdParams &p, int block, int D, int64_t grid, hipStream_t s);
hipError_t launch_skip_copy(const SkipCopyParams &p, hipStream_t s);
hipError_t launch_plan(const PlanParams &p, hipStream_t s);
hipError_t launch_combine(const CombineParams &p, int64_t grid, hipStream_t s);
// Work order of the kernels with one workgroup per (query block, head).
// Workgroup w runs on XCD w mod 8 (workgroups are dealt round-robin to the
// 8 XCDs, each with its own L2).  The first kLeadBlocks query blocks of
// every head -- the text rows of the multimodal layouts, the longest rows
// -- go first, query-block-major; the others are walked head by head on
// each XCD (XCD x takes heads x, x + 8, ...), so the key blocks that the
// rows of one head share stay in that XCD's L2.  With a head count that is
// not a multiple of 8 every row goes query-block-major.
constexpr int kLeadBlocks = 16;
#ifdef __HIPCC__
__device__ __forceinline__ void work_item(int w, int BH, int nB, int &i, int &bh)
{
    const int lead = nB < kLeadBlocks ? nB : kLeadBlocks;
    if ((BH & 7) == 0 && w >= lead * BH) {
        const int v = w - lead * BH;
        const int x = v & 7, sq = v >> 3, rows = nB - lead;
        const int hg = sq / rows;
        i = lead + sq - hg * rows;
        bh = hg * 8 + x;
    } else {
        i = w / BH;
        bh = w - i * BH;
    }
}
#endif

// floats of one partial-result slot: the unnormalised O as [D / 4][block]
// groups of four channels (query-minor, so that a wavefront's lanes, one
// query each, write and read consecutive 16-byte groups), then the
// reference max [block] and the sum [block]
__host__ __device__ inline int64_t partial_slot_floats(int block, int D) { return (int64_t)block * D + 2 * block; }
// float offset in a slot of channels c0 .. c0 + 3 (c0 a multiple of 4) of query tq
__host__ __device__ inline int64_t partial_o_index(int block, int c0, int tq)
{
    return ((int64_t)(c0 >> 2) * block + tq) * 4;
}
hipError_t launch_pool_proj(const PoolParams &p, int block, int D, hipStream_t s);
hipError_t launch_scores(const ScoreParams &p, hipStream_t s);
hipError_t launch_score_grad(const ScoreGradParams &p, hipStream_t s);
hipError_t launch_exact_scores(const ExactParams &p, int block, int D, int slots, hipStream_t s);
hipError_t launch_select(const SelectParams &p, hipStream_t s);
hipError_t launch_meanpool_select(const MeanpoolSelectParams &p, int block, int D, hipStream_t s);
hipError_t launch_scan(int32_t *row_ptr, int64_t rows, hipStream_t s);
hipError_t launch_expand(const ExpandParams &p, hipStream_t s);
hipError_t launch_arrow(const ArrowParams &p, hipStream_t s);

}  // namespace bsa
