// Content-driven block selection in two short kernels (multimodal-DiT
// write-up, section 2.2 for the score -- mean-pool, one small projection,
// dot product, top-k -- and 2.3 for the dense text rows and columns; the
// write-up's tip that scoring must stay a small fraction of the attention
// is why the steps are fused this far).
//
// meanpool_project_kernel, one workgroup per block i of a head: waves 0-7
// mean-pool block i of Q, waves 8-15 block i of K (one streaming pass,
// 16-byte loads all issued before any sum), the two means are projected by
// W [D][r], and the projections are parked in the workspace (K side
// transposed, [r][nB] per head).
// score_select_kernel, one workgroup per head: with the head's projections
// in LDS it scores and selects four rows per wave at a time -- lane j
// computes the scores of column j (+64 e) in registers (and writes them to
// the optional score output), text rows keep every column, other rows the
// text columns plus each group's k best (the threshold search of the
// selection kernel, run for the four rows in lockstep so that their
// dependency chains overlap), and each row's CSR entry and ascending
// columns are written at their closed-form offsets.  The kernel boundary
// makes the projections of every block visible to the scoring workgroup.
#include "common.h"
#include "internal.h"
#include "topk.h"

namespace bsa {

namespace mps {
constexpr int NT = 1024;            // threads per workgroup
constexpr int NW = NT / 64;
constexpr int R = 4;                // rows a wave selects at a time
}

template <int BETA, int D>
__global__ __launch_bounds__(1024) void meanpool_project_kernel(const MeanpoolSelectParams p)
{
    constexpr int CH = D / 8;                  // 16-byte chunks per token row
    constexpr int RS = 512 / CH;               // row slots of one tensor's 512 threads
    constexpr int IT = (BETA + RS - 1) / RS;   // rows per thread
    // phase 1 partial sums and phase 2 projections share this space
    __shared__ __attribute__((aligned(16))) float buf[2 * kMpsMaxProj];
    __shared__ float mean[2][D];
    static_assert(2 * RS * D <= 2 * kMpsMaxProj, "partial sums fit the shared buffer");
    static_assert(2 * 8 * 64 <= 2 * kMpsMaxProj, "projection partials fit the shared buffer");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nB = p.nB, r = p.r;
    const int item = blockIdx.x;               // (b * H + h) * nB + i
    const int bh = item / nB, i = item - bh * nB;
    const int b = bh / p.H, hh = bh - b * p.H;

    // pool block i of Q (sel 0) and of K (sel 1), project
    {
        const int sel = tid >> 9, t9 = tid & 511;
        const Tensor4 X = sel ? p.k : p.q;
        const uint16_t *base = X.p + b * X.sb + hh * X.sh;
        const int cc = t9 % CH, rs = t9 / CH;
        const int t0 = i * BETA, n_i = min(BETA, p.N - t0);
        uint4 u[IT];
#pragma unroll
        for (int a = 0; a < IT; ++a) {
            const int t = rs + a * RS;
            u[a] = t < n_i ? ld_g16(base + (int64_t)(t0 + t) * X.sn + cc * 8) : zero_u4();
        }
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
        for (int a = 0; a < IT; ++a) {
            const uint32_t wd[4] = {u[a].x, u[a].y, u[a].z, u[a].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] += __uint_as_float(wd[e] << 16);
                acc[2 * e + 1] += __uint_as_float(wd[e] & 0xFFFF0000u);
            }
        }
        float *red = buf + sel * RS * D;       // [RS][D] per tensor
#pragma unroll
        for (int e = 0; e < 8; ++e) red[rs * D + cc * 8 + e] = acc[e];
        __syncthreads();
        if (tid < 2 * D) {
            const int s = tid / D, d = tid - s * D;
            const float *rd = buf + s * RS * D;
            float sum = 0.f;
            for (int x = 0; x < RS; ++x) sum += rd[x * D + d];
            mean[s][d] = sum / (float)n_i;
        }
        __syncthreads();
        // projection: thread (sel, part, m) sums the part-th eighth of d
        const int m = t9 & 63, part = t9 >> 6;
        float a = 0.f;
        if (m < r) {
#pragma unroll 4
            for (int d = part * (D / 8); d < (part + 1) * (D / 8); ++d)
                a = __builtin_fmaf(p.w[d * r + m], mean[sel][d], a);
        }
        float *pp = buf;                       // [2][8][64] partials: the sums are dead past this barrier
        __syncthreads();
        pp[(sel * 8 + part) * 64 + m] = a;
        __syncthreads();
        if (t9 < r) {
            float s = 0.f;
#pragma unroll
            for (int x = 0; x < 8; ++x) s += pp[(sel * 8 + x) * 64 + t9];
            if (sel == 0) p.proj_q[(int64_t)item * r + t9] = s;
            else p.proj_kt[((int64_t)bh * r + t9) * nB + i] = s;
        }
    }
}

template <int E>
__global__ __launch_bounds__(1024) void score_select_kernel(const MeanpoolSelectParams p)
{
    __shared__ __attribute__((aligned(16))) float buf[2 * kMpsMaxProj];
    __shared__ uint32_t bits[mps::NW][mps::R][kMpsMaxBlocks / 32];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nB = p.nB, r = p.r;
    const int bh = blockIdx.x;
    float *pq = buf, *pkt = buf + kMpsMaxProj;
    for (int x = tid; x < nB * r; x += mps::NT) {
        pq[x] = p.proj_q[(int64_t)bh * nB * r + x];
        pkt[x] = p.proj_kt[(int64_t)bh * r * nB + x];
    }
    __syncthreads();
    const int tb = p.text_blocks, words = (nB + 31) >> 5;
    const int64_t head = (int64_t)tb * nB + (int64_t)(nB - tb) * p.row_len;
    uint32_t *wb[mps::R];
#pragma unroll
    for (int q = 0; q < mps::R; ++q) wb[q] = bits[wv][q];
    for (int row0 = wv * mps::R; row0 < nB; row0 += mps::NW * mps::R) {
        // scores of rows row0 .. row0 + R - 1 (rows past nB score 0 and are dropped)
        float s[mps::R][E];
#pragma unroll
        for (int q = 0; q < mps::R; ++q)
#pragma unroll
            for (int e = 0; e < E; ++e) s[q][e] = 0.f;
        for (int mm = 0; mm < r; ++mm) {
            float kv[E];
#pragma unroll
            for (int e = 0; e < E; ++e) kv[e] = (e * 64 + lane < nB) ? pkt[mm * nB + e * 64 + lane] : 0.f;
#pragma unroll
            for (int q = 0; q < mps::R; ++q) {
                const float qv = row0 + q < nB ? pq[(row0 + q) * r + mm] : 0.f;
#pragma unroll
                for (int e = 0; e < E; ++e) s[q][e] = __builtin_fmaf(qv, kv[e], s[q][e]);
            }
        }
#pragma unroll
        for (int q = 0; q < mps::R; ++q) {
            const int row = row0 + q;
            if (row >= nB) break;
            if (p.scores)
#pragma unroll
                for (int e = 0; e < E; ++e)
                    if (e * 64 + lane < nB) p.scores[((int64_t)bh * nB + row) * nB + e * 64 + lane] = s[q][e];
            if (lane < words) {
                const int lim = row < tb ? nB : tb, lo = lane * 32;
                wb[q][lane] = lim >= lo + 32 ? 0xFFFFFFFFu : (lim > lo ? (1u << (lim - lo)) - 1u : 0u);
            }
        }
        // the batch is selected when it holds a non-text row (a text row's
        // mask is already dense, so the selection's bits leave it unchanged)
        if (row0 + mps::R > tb) {
            for (int g = 0; g < p.n_groups; ++g) {
                const int c0 = p.g_begin[g], c1 = p.g_end[g], kk = p.g_k[g];
                if (kk <= 0) continue;
                if (kk >= c1 - c0) {
#pragma unroll
                    for (int q = 0; q < mps::R; ++q)
                        if (row0 + q >= tb && row0 + q < nB) select_all(c0, c1, wb[q]);
                } else {
                    select_rows<E, mps::R>(s, c0, c1, kk, wb);
                }
            }
        }
#pragma unroll
        for (int q = 0; q < mps::R; ++q) {
            const int row = row0 + q;
            if (row >= nB) break;
            // closed-form offset of the row (text rows nB columns, others row_len)
            int64_t start = bh * head + (row < tb ? (int64_t)row * nB : (int64_t)tb * nB + (int64_t)(row - tb) * p.row_len);
            if (lane == 0) {
                p.row_ptr[(int64_t)bh * nB + row + 1] = (int32_t)(start + (row < tb ? nB : p.row_len));
                if (bh == 0 && row == 0) p.row_ptr[0] = 0;
            }
            for (int w0 = 0; w0 < words; w0 += 64) {
                const int w = w0 + lane;
                uint32_t v = w < words ? wb[q][w] : 0u;
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
        }
    }
}

hipError_t launch_meanpool_select(const MeanpoolSelectParams &p, int block, int D, hipStream_t s)
{
    const int64_t items = (int64_t)p.B * p.H * p.nB;
    if (items == 0) return hipSuccess;
    const dim3 thr(mps::NT);
    if (block == 64 && D == 64) hipLaunchKernelGGL((meanpool_project_kernel<64, 64>), dim3((unsigned)items), thr, 0, s, p);
    else if (block == 64 && D == 128) hipLaunchKernelGGL((meanpool_project_kernel<64, 128>), dim3((unsigned)items), thr, 0, s, p);
    else if (block == 128 && D == 64) hipLaunchKernelGGL((meanpool_project_kernel<128, 64>), dim3((unsigned)items), thr, 0, s, p);
    else if (block == 128 && D == 128) hipLaunchKernelGGL((meanpool_project_kernel<128, 128>), dim3((unsigned)items), thr, 0, s, p);
    else return hipErrorInvalidValue;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 heads((unsigned)(p.B * p.H));
    switch ((p.nB + 63) / 64) {
    case 1: hipLaunchKernelGGL(score_select_kernel<1>, heads, thr, 0, s, p); break;
    case 2: hipLaunchKernelGGL(score_select_kernel<2>, heads, thr, 0, s, p); break;
    case 3: hipLaunchKernelGGL(score_select_kernel<3>, heads, thr, 0, s, p); break;
    case 4: hipLaunchKernelGGL(score_select_kernel<4>, heads, thr, 0, s, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace bsa
