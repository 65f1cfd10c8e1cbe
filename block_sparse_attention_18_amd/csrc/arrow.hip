// Arrow block layout on gfx950 (DiTFastAttnV2 notes, "Head-wise Arrow
// Attention" and the fused kernel's per-head modes).
//
// The joint attention map splits into four regions: every region that
// involves text (text->text, text->vision, vision->text) stays dense and the
// vision->vision region keeps a diagonal window of +-w blocks.  Per head:
//   ARROW : keep(i, j) = i < T_b or j < T_b or |i - j| <= w
//   FULL  : keep every (i, j)
//   SKIP  : nothing is computed (empty rows)
// Everything is closed form, so every row is independent: one wavefront per
// row computes its offset (closed-form nnz of the heads before it plus the
// lengths of the earlier rows of its head), writes row_ptr and then its
// ascending columns.
#include "common.h"
#include "internal.h"

namespace bsa {

__device__ __forceinline__ int64_t arrow_row_len(int mode, int w, int nB, int tb, int i)
{
    if (mode == 2) return 0;                       // SKIP
    if (mode == 0 || i < tb) return nB;            // FULL or text row
    const int lo = max(tb, i - w);
    const int64_t hi = min((int64_t)nB - 1, (int64_t)i + w);
    const int64_t band = hi >= lo ? hi - lo + 1 : 0;
    return tb + band;
}

__device__ __forceinline__ int64_t arrow_head_nnz(int mode, int w, int nB, int tb)
{
    if (mode == 2) return 0;
    if (mode == 0) return (int64_t)nB * nB;
    const int64_t ni = nB - tb;
    int64_t band;
    if (ni <= 0) band = 0;
    else if ((int64_t)w >= ni - 1) band = ni * ni;
    else band = ni * (2 * (int64_t)w + 1) - (int64_t)w * (w + 1);
    return (int64_t)tb * nB + ni * tb + band;
}

// One wavefront per row (b, h, i).  The row's offset is the closed-form nnz
// of the batch entries and heads before it plus the lengths of the earlier
// rows of its head; lane 0 of row 0 also writes row_ptr[0].
__global__ __launch_bounds__(256) void arrow_kernel(const ArrowParams p)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t rows = (int64_t)p.B * p.H * p.nB;
    if (row >= rows) return;
    const int bh = (int)(row / p.nB), i = (int)(row - (int64_t)bh * p.nB);
    const int b = bh / p.H, hh = bh - b * p.H;
    const int mode = p.mode[hh], w = p.window[hh];

    // prefix: batch entries and heads before this one, then earlier rows of
    // this head (summed by the lanes, then reduced)
    int64_t part = 0;
    for (int h2 = lane; h2 < hh; h2 += 64) part += arrow_head_nnz(p.mode[h2], p.window[h2], p.nB, p.text_blocks);
    for (int i2 = lane; i2 < i; i2 += 64) part += arrow_row_len(mode, w, p.nB, p.text_blocks, i2);
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) part += __shfl_xor(part, d, 64);
    const int64_t base = (int64_t)b * p.per_batch + part;

    const int64_t len = arrow_row_len(mode, w, p.nB, p.text_blocks, i);
    if (lane == 0) {
        p.row_ptr[row + 1] = (int32_t)(base + len);
        if (row == 0) p.row_ptr[0] = 0;
    }
    const bool dense = (mode == 0) || (i < p.text_blocks);
    const int lo = max(p.text_blocks, i - w);
    for (int64_t e = lane; e < len; e += 64) {
        const int col = (dense || e < p.text_blocks) ? (int)e : lo + (int)(e - p.text_blocks);
        if (base + e < p.capacity) p.col_idx[base + e] = col;
    }
}

hipError_t launch_arrow(const ArrowParams &p, hipStream_t s)
{
    const int64_t rows = (int64_t)p.B * p.H * p.nB;
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL(arrow_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace bsa
