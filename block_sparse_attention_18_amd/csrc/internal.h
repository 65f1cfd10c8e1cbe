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
    int32_t B, H, N, nB, r;
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
    int32_t *row_ptr;           // counts written to row_ptr[r + 1]
    uint32_t *bits;             // [rows][words]
    int64_t rows;
    int32_t nB, words, text_blocks, n_groups;
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
    int32_t B, H, N, nB, NT, NP;
    float scale_log2;
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
hipError_t launch_mask_jaccard(const JaccardParams &p, hipStream_t s);
hipError_t launch_quantize_fp8(const Fp8QuantParams &p, int D, hipStream_t s);
hipError_t launch_forward_fp8(const Fp8FwdParams &p, int block, int D, hipStream_t s);
hipError_t launch_skip_copy(const SkipCopyParams &p, hipStream_t s);
hipError_t launch_plan(const PlanParams &p, hipStream_t s);
hipError_t launch_combine(const CombineParams &p, int64_t grid, hipStream_t s);
// bytes of one partial-result slot (O [block][D] fp32, then max and sum [block])
__host__ __device__ inline int64_t partial_slot_floats(int block, int D) { return (int64_t)block * D + 2 * block; }
hipError_t launch_pool_proj(const PoolParams &p, int block, int D, hipStream_t s);
hipError_t launch_scores(const ScoreParams &p, hipStream_t s);
hipError_t launch_exact_scores(const ExactParams &p, int block, int D, int slots, hipStream_t s);
hipError_t launch_select(const SelectParams &p, hipStream_t s);
hipError_t launch_scan(int32_t *row_ptr, int64_t rows, hipStream_t s);
hipError_t launch_expand(const ExpandParams &p, hipStream_t s);
hipError_t launch_arrow(const ArrowParams &p, hipStream_t s);

}  // namespace bsa
