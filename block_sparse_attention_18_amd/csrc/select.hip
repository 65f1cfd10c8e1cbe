// Top-k block selection on gfx950 (multimodal-DiT write-up, sections 2.2 and
// 2.3; SparseD notes, isolated selection).
//
// Three small kernels:
//  1. select: one wavefront per query-block row, four to a workgroup; the
//     row's scores are staged in LDS in one round trip.  Text rows keep every
//     column; other rows keep the text columns plus, per column group, the
//     k best columns.  Only the k-th best score of a group is needed, not a
//     sorted order: each score becomes an order-preserving 32-bit key
//     (-0.0 folded onto +0.0, NaN mapped below -inf), the group's keys sit in
//     registers (lane l holds columns c + 64 e + l), and a bitwise search
//     from the top bit finds the largest key T with at least k keys >= T --
//     at most 32 rounds of one compare and one ballot per register (it stops
//     early at a probe with exactly k keys at or above it).  The row keeps
//     every key above T and, of the keys equal to T, the lowest columns up
//     to k (lane prefix counts of the equality ballots, taken in column
//     order).  On the two-pass path below the kept set is a per-row
//     bitmask in LDS; its population count is the row length.
//  2. scan: one workgroup turns the row lengths into row_ptr in place.
//  3. expand: one wavefront per row writes the set bits as ascending
//     column indices at row_ptr[row].
// When the column groups are pairwise disjoint and leave the text columns
// alone, every row's length is known beforehand (text rows nB, the others
// text_blocks + sum of k), so select writes its row_ptr entry and its
// column indices itself and the other two kernels are not launched: the
// groups arrive in ascending column order, and each group's kept columns
// are written as soon as its search ends (positions from ballot prefix
// counts), with no bitmask.
#include "common.h"
#include "internal.h"
#include "topk.h"

namespace bsa {

namespace sel {
constexpr int RW = 4;                                   // rows (wavefronts) per workgroup
constexpr int LU = kMaxSelectBlocks / 64;               // score loads per lane, at most
}

__global__ __launch_bounds__(256) void select_kernel(const SelectParams p)
{
    __shared__ float srow_s[sel::RW][kMaxSelectBlocks];
    __shared__ uint32_t wbits_s[sel::RW][kMaxSelectBlocks / 32];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nB = p.nB;
    // a workgroup holds RW consecutive rows of one head
    const uint32_t per_head = (uint32_t)(nB + sel::RW - 1) / sel::RW;
    const uint32_t bh = blockIdx.x / per_head;
    const int i = (int)(blockIdx.x - bh * per_head) * sel::RW + wv;
    const bool live = i < nB;
    const int64_t row = (int64_t)bh * nB + i;
    float *srow = srow_s[wv];
    uint32_t *wbits = wbits_s[wv];
    // the whole score row in one round trip: every load issued before the
    // first LDS write (loads past the row re-read its last element)
    if (live) {
        const float *g = p.S + row * nB;
        float v[sel::LU] = {};
#pragma unroll
        for (int u = 0; u < sel::LU; ++u)
            if (u * 64 < nB) v[u] = g[min(u * 64 + lane, nB - 1)];
#pragma unroll
        for (int u = 0; u < sel::LU; ++u) asm volatile("" ::"v"(v[u]));
#pragma unroll
        for (int u = 0; u < sel::LU; ++u)
            if (u * 64 + lane < nB) srow[u * 64 + lane] = v[u];
        if (!p.direct) {
            const int lim = (i < p.text_blocks) ? nB : p.text_blocks;   // dense row / text columns
            for (int w = lane; w < p.words; w += 64) {
                const int lo = w * 32;
                wbits[w] = lim >= lo + 32 ? 0xFFFFFFFFu : (lim > lo ? (1u << (lim - lo)) - 1u : 0u);
            }
        }
    }
    __syncthreads();
    if (p.direct) {
        // closed-form offsets: each head holds text_blocks rows of nB columns,
        // then nB - text_blocks rows of row_len columns.  The groups come in
        // ascending column order, after the text columns, so the row's
        // columns are written in order as they are chosen.
        if (!live) return;
        const int64_t tb = p.text_blocks;
        const int64_t head = tb * nB + (int64_t)(nB - tb) * p.row_len;
        int64_t pos = (int64_t)bh * head + (i < tb ? (int64_t)i * nB : tb * nB + (int64_t)(i - tb) * p.row_len);
        if (lane == 0) {
            p.row_ptr[row + 1] = (int32_t)(pos + (i < tb ? nB : p.row_len));
            if (row == 0) p.row_ptr[0] = 0;
        }
        const int lead = i < tb ? nB : (int)tb;   // dense row / text columns
        for (int c = lane; c < lead; c += 64)
            if (pos + c < p.capacity) p.col_idx[pos + c] = c;
        if (i < tb) return;
        pos += tb;
        for (int g = 0; g < p.n_groups; ++g) {
            const int c0 = p.g_begin[g], c1 = p.g_end[g], kk = p.g_k[g];
            const int width = c1 - c0;
            if (kk <= 0) continue;
            if (kk >= width) {
                for (int c = lane; c < width; c += 64)
                    if (pos + c < p.capacity) p.col_idx[pos + c] = c0 + c;
                pos += width;
                continue;
            }
            if (width <= 64) topk_write<1>(srow, c0, c1, kk, p.col_idx, pos, p.capacity);
            else if (width <= 128) topk_write<2>(srow, c0, c1, kk, p.col_idx, pos, p.capacity);
            else if (width <= 256) topk_write<4>(srow, c0, c1, kk, p.col_idx, pos, p.capacity);
            else if (width <= 512) topk_write<8>(srow, c0, c1, kk, p.col_idx, pos, p.capacity);
            else topk_write<16>(srow, c0, c1, kk, p.col_idx, pos, p.capacity);
            pos += kk;
        }
        return;
    }
    if (live && i >= p.text_blocks) {
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
    }
    __syncthreads();
    if (!live) return;
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
    if (p.nB > kMaxSelectBlocks) return hipErrorInvalidValue;
    const int64_t heads = p.rows / p.nB, per_head = (p.nB + sel::RW - 1) / sel::RW;
    if (heads * per_head >= (1ll << 31)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(select_kernel, dim3((unsigned)(heads * per_head)), dim3(256), 0, s, p);
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
