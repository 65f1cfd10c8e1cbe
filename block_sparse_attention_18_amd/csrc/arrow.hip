// Arrow block layout on gfx950 (DiTFastAttnV2 notes, "Head-wise Arrow
// Attention" and the fused kernel's per-head modes).
//
// The joint attention map splits into four regions: every region that
// involves text (text->text, text->vision, vision->text) stays dense and the
// vision->vision region keeps a diagonal window of +-w blocks.  Per head:
//   ARROW : keep(i, j) = i < T_b or j < T_b or |i - j| <= w
//   FULL  : keep every (i, j)
//   SKIP  : nothing is computed (empty rows)
// Everything is closed form, so one workgroup per (b, h) computes its row
// lengths, scans them, writes row_ptr and then the ascending columns.  The
// offset of a head is the closed-form nnz of every head before it.
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

__global__ __launch_bounds__(256) void arrow_kernel(const ArrowParams p)
{
    __shared__ int64_t wsum[4];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int bh = blockIdx.x;
    const int b = bh / p.H, hh = bh - b * p.H;
    const int mode = p.mode[hh], w = p.window[hh];

    int64_t base = (int64_t)b * p.per_batch;
    for (int h2 = 0; h2 < hh; ++h2) base += arrow_head_nnz(p.mode[h2], p.window[h2], p.nB, p.text_blocks);

    int32_t *rp = p.row_ptr + (int64_t)bh * p.nB;
    int64_t carry = 0;
    for (int i0 = 0; i0 < p.nB; i0 += 256) {
        const int i = i0 + tid;
        const int64_t len = i < p.nB ? arrow_row_len(mode, w, p.nB, p.text_blocks, i) : 0;
        // inclusive scan of 64-bit lengths across the workgroup
        int64_t x = len;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int64_t y = __shfl_up(x, d, 64);
            if (lane >= d) x += y;
        }
        if (lane == 63) wsum[wv] = x;
        __syncthreads();
        int64_t pre = 0, tot = 0;
        for (int v = 0; v < 4; ++v) {
            if (v < wv) pre += wsum[v];
            tot += wsum[v];
        }
        if (i < p.nB) rp[i + 1] = (int32_t)(base + carry + pre + x);
        carry += tot;
        __syncthreads();
    }
    if (bh == 0 && tid == 0) p.row_ptr[0] = 0;
    __syncthreads();   // row_ptr of this head is written (workgroup scope)

    // columns: one wavefront per row
    for (int i = wv; i < p.nB; i += 4) {
        const int64_t start = (i == 0) ? base : (int64_t)rp[i];
        const int64_t len = arrow_row_len(mode, w, p.nB, p.text_blocks, i);
        const bool dense = (mode == 0) || (i < p.text_blocks);
        const int lo = max(p.text_blocks, i - w);
        for (int64_t e = lane; e < len; e += 64) {
            int col;
            if (dense || e < p.text_blocks) col = (int)e;
            else col = lo + (int)(e - p.text_blocks);
            if (start + e < p.capacity) p.col_idx[start + e] = col;
        }
    }
}

hipError_t launch_arrow(const ArrowParams &p, hipStream_t s)
{
    const int64_t grid = (int64_t)p.B * p.H;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(arrow_kernel, dim3((unsigned)grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace bsa
