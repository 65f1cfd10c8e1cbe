// Top-k block selection on gfx950 (multimodal-DiT write-up, sections 2.2 and
// 2.3; SparseD notes, isolated selection).
//
// Three small kernels:
//  1. select: one wavefront per query-block row.  Text rows keep every
//     column; other rows keep the text columns plus, per column group, the
//     k best columns.  Only the k-th best score of a group is needed, not a
//     sorted order: each score becomes an order-preserving 32-bit key
//     (-0.0 folded onto +0.0, NaN mapped below -inf), the group's keys sit in
//     registers (lane l holds columns c + 64 e + l), and a bitwise search
//     from the top bit finds the largest key T with at least k keys >= T --
//     32 rounds of one compare and one ballot per register.  The row keeps
//     every key above T and, of the keys equal to T, the lowest columns up
//     to k (lane prefix counts of the equality ballots, taken in column
//     order).  The kept set is a per-row bitmask in LDS; its population
//     count is the row length.
//  2. scan: one workgroup turns the row lengths into row_ptr in place.
//  3. expand: one wavefront per row writes the set bits as ascending
//     column indices at row_ptr[row].
// When the column groups are pairwise disjoint and leave the text columns
// alone, every row's length is known beforehand (text rows nB, the others
// text_blocks + sum of k), so select writes its row_ptr entry and its
// column indices itself and the other two kernels are not launched.
#include "common.h"
#include "internal.h"
#include "topk.h"

namespace bsa {

__global__ __launch_bounds__(64) void select_kernel(const SelectParams p)
{
    __shared__ uint32_t wbits[kMaxSelectBlocks / 32];
    const int lane = threadIdx.x;
    const int64_t row = blockIdx.x;
    const int i = (int)(row % p.nB);
    const float *srow = p.S + row * p.nB;

    for (int w = lane; w < p.words; w += 64) {
        uint32_t v = 0u;
        const int lim = (i < p.text_blocks) ? p.nB : p.text_blocks;   // dense row / text columns
        const int lo = w * 32;
        if (lim >= lo + 32) v = 0xFFFFFFFFu;
        else if (lim > lo) v = (1u << (lim - lo)) - 1u;
        wbits[w] = v;
    }
    __syncthreads();
    if (i >= p.text_blocks) {
        for (int g = 0; g < p.n_groups; ++g) {
            const int c0 = p.g_begin[g], c1 = p.g_end[g], kk = p.g_k[g];
            const int width = c1 - c0;
            if (kk <= 0) continue;
            if (kk >= width) select_all(c0, c1, wbits);
            else if (width <= 64) select_group<1>(srow, c0, c1, kk, wbits, p.words);
            else if (width <= 128) select_group<2>(srow, c0, c1, kk, wbits, p.words);
            else if (width <= 256) select_group<4>(srow, c0, c1, kk, wbits, p.words);
            else if (width <= 512) select_group<8>(srow, c0, c1, kk, wbits, p.words);
            else select_group<16>(srow, c0, c1, kk, wbits, p.words);
        }
        __syncthreads();
    }
    if (p.direct) {
        // closed-form offsets: each head holds text_blocks rows of nB columns,
        // then nB - text_blocks rows of row_len columns
        const int64_t tb = p.text_blocks;
        const int64_t head = tb * p.nB + (int64_t)(p.nB - tb) * p.row_len;
        int64_t start = (row / p.nB) * head + (i < tb ? (int64_t)i * p.nB : tb * p.nB + (int64_t)(i - tb) * p.row_len);
        if (lane == 0) {
            p.row_ptr[row + 1] = (int32_t)(start + (i < tb ? p.nB : p.row_len));
            if (row == 0) p.row_ptr[0] = 0;
        }
        for (int w0 = 0; w0 < p.words; w0 += 64) {
            const int w = w0 + lane;
            uint32_t v = w < p.words ? wbits[w] : 0u;
            const int c = __popc(v);
            const int incl = wave_incl_scan(c);
            int64_t pos = start + incl - c;
            while (v) {
                const int bit = __ffs(v) - 1;
                v &= v - 1u;
                if (pos < p.capacity) p.col_idx[pos] = w * 32 + bit;
                ++pos;
            }
            start += __shfl(incl, 63, 64);
        }
        return;
    }
    int cnt = 0;
    for (int w = lane; w < p.words; w += 64) {
        const uint32_t v = wbits[w];
        p.bits[row * p.words + w] = v;
        cnt += __popc(v);
    }
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) cnt += __shfl_xor(cnt, d, 64);
    if (lane == 0) {
        p.row_ptr[row + 1] = cnt;
        if (row == 0) p.row_ptr[0] = 0;
    }
}

hipError_t launch_select(const SelectParams &p, hipStream_t s)
{
    if (p.rows == 0) return hipSuccess;
    hipLaunchKernelGGL(select_kernel, dim3((unsigned)p.rows), dim3(64), 0, s, p);
    return hipGetLastError();
}

// In-place inclusive scan of row_ptr[1 .. rows] by one workgroup.
__global__ __launch_bounds__(1024) void scan_kernel(int32_t *rp, int64_t rows)
{
    constexpr int PER = 4;
    __shared__ int wsum[16];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int carry = 0;
    for (int64_t base = 0; base < rows; base += 1024 * PER) {
        int v[PER];
        int tsum = 0;
#pragma unroll
        for (int a = 0; a < PER; ++a) {
            const int64_t idx = base + (int64_t)tid * PER + a;
            v[a] = idx < rows ? rp[1 + idx] : 0;
            tsum += v[a];
        }
        const int incl = wave_incl_scan(tsum);
        if (lane == 63) wsum[wv] = incl;
        __syncthreads();
        int wpre = 0, total = 0;
        for (int x = 0; x < 16; ++x) {
            if (x < wv) wpre += wsum[x];
            total += wsum[x];
        }
        int run = carry + wpre + incl - tsum;
#pragma unroll
        for (int a = 0; a < PER; ++a) {
            const int64_t idx = base + (int64_t)tid * PER + a;
            run += v[a];
            if (idx < rows) rp[1 + idx] = run;
        }
        carry += total;
        __syncthreads();
    }
    if (tid == 0) rp[0] = 0;
}

hipError_t launch_scan(int32_t *row_ptr, int64_t rows, hipStream_t s)
{
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, row_ptr, rows);
    return hipGetLastError();
}

__global__ __launch_bounds__(64) void expand_kernel(const ExpandParams p)
{
    const int lane = threadIdx.x;
    const int64_t row = blockIdx.x;
    int64_t start = p.row_ptr[row];
    for (int w0 = 0; w0 < p.words; w0 += 64) {
        const int w = w0 + lane;
        uint32_t v = w < p.words ? p.bits[row * p.words + w] : 0u;
        const int cnt = __popc(v);
        const int incl = wave_incl_scan(cnt);
        int64_t pos = start + incl - cnt;
        while (v) {
            const int bit = __ffs(v) - 1;
            v &= v - 1u;
            if (pos < p.capacity) p.col_idx[pos] = w * 32 + bit;
            ++pos;
        }
        start += __shfl(incl, 63, 64);
    }
}

hipError_t launch_expand(const ExpandParams &p, hipStream_t s)
{
    if (p.rows == 0) return hipSuccess;
    hipLaunchKernelGGL(expand_kernel, dim3((unsigned)p.rows), dim3(64), 0, s, p);
    return hipGetLastError();
}

}  // namespace bsa
