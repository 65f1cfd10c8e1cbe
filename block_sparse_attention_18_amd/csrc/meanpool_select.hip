// Content-driven block selection in two short kernels (multimodal-DiT
// write-up, section 2.2 for the score -- mean-pool, one small projection,
// dot product, top-k -- and 2.3 for the dense text rows and columns; the
// write-up's tip that scoring must stay a small fraction of the attention
// is why the steps are fused this far).
//
// The pooling kernel of bsa_pool_scores (mean-pool in one streaming pass,
// project by W [D][r]) parks the projections in the workspace.  Then
// score_select_kernel, one workgroup per four rows of a head and one row
// per wavefront: with the head's projected key blocks in LDS, lane j
// computes the scores of column j (+64 e) in registers (and writes them to
// the optional score output); text rows keep every column, other rows the
// text columns plus each group's k best (the threshold search of the
// selection kernel), and each row's CSR entry and ascending columns are
// written at their closed-form offsets.  The score matrix itself never goes
// to memory.  (Four rows per wavefront searched in lockstep, 16 per
// workgroup, measured 1.7x slower at the content-driven DiT shape: too few
// wavefronts to fill the chip.)
#include "common.h"
#include "internal.h"
#include "topk.h"

namespace bsa {

namespace mps {
constexpr int NT = 256;             // threads per score-select workgroup
constexpr int NW = NT / 64;
constexpr int ROWS = NW;            // rows per workgroup, one per wavefront
}

// Scores and selection of ROWS query-block rows of one head: the head's
// projected key blocks in LDS transposed ([r][nB | 1], r padded to a
// multiple of 4 with zero rows), the workgroup's projected query blocks
// beside them.
template <int E>
__global__ __launch_bounds__(256) void score_select_kernel(const MeanpoolSelectParams p)
{
    __shared__ __attribute__((aligned(16))) float pkt[kMpsMaxProj + 64];
    __shared__ __attribute__((aligned(16))) float pq[mps::ROWS][64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nB = p.nB, r = p.r, r4 = (r + 3) & ~3;
    const int ld = nB | 1;              // odd LDS row stride: the transposing writes hit distinct banks
    const int tiles = (nB + mps::ROWS - 1) / mps::ROWS;
    const int bh = blockIdx.x / tiles, row_base = (blockIdx.x - bh * tiles) * mps::ROWS;
    const int64_t rows_all = (int64_t)p.B * p.H * nB;
    const float *proj_q = p.proj + (int64_t)bh * nB * r;
    const float *proj_k = p.proj + (rows_all + (int64_t)bh * nB) * r;
    const float inv_r = 1.0f / (float)r;
    // Staging: every load is issued before the first LDS write (indices
    // past the end re-read a valid element, dropped after), so it costs one
    // memory round trip.
    constexpr int QU = mps::ROWS * 64 / mps::NT;
    float vq[QU];
#pragma unroll
    for (int u = 0; u < QU; ++u) {
        const int x = u * mps::NT + tid, rr = x >> 6, m = x & 63;
        const bool ok = row_base + rr < nB && m < r;
        vq[u] = proj_q[ok ? (int64_t)(row_base + rr) * r + m : 0];
    }
    constexpr int KU = kMpsMaxProj / mps::NT;
    const int nk = nB * r;
    float vk[KU];
#pragma unroll
    for (int u = 0; u < KU; ++u) vk[u] = proj_k[min(u * mps::NT + tid, nk - 1)];
    // the loads stay here, not sunk into the guarded writes below
#pragma unroll
    for (int u = 0; u < KU; ++u) asm volatile("" ::"v"(vk[u]));
#pragma unroll
    for (int u = 0; u < KU; ++u) {
        const int x = u * mps::NT + tid;
        const int j = div_small(x, inv_r), m = x - j * r;
        if (x < nk) pkt[m * ld + j] = vk[u];
    }
    for (int x = r * ld + tid; x < r4 * ld; x += mps::NT) pkt[x] = 0.f;
#pragma unroll
    for (int u = 0; u < QU; ++u) {
        const int x = u * mps::NT + tid, rr = x >> 6, m = x & 63;
        pq[rr][m] = (row_base + rr < nB && m < r) ? vq[u] : 0.f;
    }
    __syncthreads();
    const int tb = p.text_blocks;
    const int64_t head = (int64_t)tb * nB + (int64_t)(nB - tb) * p.row_len;
    const int row = row_base + wv;
    if (row >= nB) return;
    // lane j scores column j + 64 e of the row
    float s[E];
#pragma unroll
    for (int e = 0; e < E; ++e) s[e] = 0.f;
    for (int mm = 0; mm < r4; mm += 4) {
        float kv[4][E];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int e = 0; e < E; ++e) kv[t][e] = (e * 64 + lane < nB) ? pkt[(mm + t) * ld + e * 64 + lane] : 0.f;
        const float4 v = *reinterpret_cast<const float4 *>(&pq[wv][mm]);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            s[e] = __builtin_fmaf(v.x, kv[0][e], s[e]);
            s[e] = __builtin_fmaf(v.y, kv[1][e], s[e]);
            s[e] = __builtin_fmaf(v.z, kv[2][e], s[e]);
            s[e] = __builtin_fmaf(v.w, kv[3][e], s[e]);
        }
    }
    if (p.scores)
#pragma unroll
        for (int e = 0; e < E; ++e)
            if (e * 64 + lane < nB) p.scores[((int64_t)bh * nB + row) * nB + e * 64 + lane] = s[e];
    // closed-form offset of the row (text rows nB columns, others row_len);
    // the text columns, then each group's columns in ascending order (the
    // groups come sorted by column and lie past the text columns)
    int64_t pos = bh * head + (row < tb ? (int64_t)row * nB : (int64_t)tb * nB + (int64_t)(row - tb) * p.row_len);
    if (lane == 0) {
        p.row_ptr[(int64_t)bh * nB + row + 1] = (int32_t)(pos + (row < tb ? nB : p.row_len));
        if (bh == 0 && row == 0) p.row_ptr[0] = 0;
    }
    const int lead = row < tb ? nB : tb;
    for (int c = lane; c < lead; c += 64)
        if (pos + c < p.capacity) p.col_idx[pos + c] = c;
    if (row < tb) return;
    pos += tb;
    for (int g = 0; g < p.n_groups; ++g) {
        const int c0 = p.g_begin[g], c1 = p.g_end[g], kk = p.g_k[g];
        if (kk <= 0) continue;
        if (kk >= c1 - c0) {
            for (int c = lane; c < c1 - c0; c += 64)
                if (pos + c < p.capacity) p.col_idx[pos + c] = c0 + c;
            pos += c1 - c0;
            continue;
        }
        uint32_t key[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int col = e * 64 + lane;
            key[e] = (col >= c0 && col < c1) ? score_key(s[e]) : 0u;
        }
        topk_keys_write<E>(key, 0, c0, c1, kk, p.col_idx, pos, p.capacity);
        pos += kk;
    }
}

hipError_t launch_meanpool_select(const MeanpoolSelectParams &p, int block, int D, hipStream_t s)
{
    const int64_t items = (int64_t)p.B * p.H * p.nB;
    if (items == 0) return hipSuccess;
    PoolParams pp{};
    pp.x[0] = p.q;
    pp.x[1] = p.k;
    pp.w = p.w;
    pp.proj = p.proj;
    pp.B = p.B; pp.H = p.H; pp.N = p.N; pp.nB = p.nB; pp.r = p.r;
    hipError_t e = launch_pool_proj(pp, block, D, s);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)((int64_t)((p.nB + mps::ROWS - 1) / mps::ROWS) * p.B * p.H)), thr(mps::NT);
    switch ((p.nB + 63) / 64) {
    case 1: hipLaunchKernelGGL(score_select_kernel<1>, grid, thr, 0, s, p); break;
    case 2: hipLaunchKernelGGL(score_select_kernel<2>, grid, thr, 0, s, p); break;
    case 3: hipLaunchKernelGGL(score_select_kernel<3>, grid, thr, 0, s, p); break;
    case 4: hipLaunchKernelGGL(score_select_kernel<4>, grid, thr, 0, s, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace bsa
