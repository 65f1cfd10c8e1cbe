// Gradient of the content-driven block score.  The block-sparse DiT
// write-up (section 2.2) scores query block i against key block j by
//   S_ij = p_i . p'_j,   p_i = W^T qbar_i,   p'_j = W^T kbar_j
// (qbar, kbar: block means of Q and K; W: one small projection trained
// jointly with the model).  For an upstream gradient dS = dL/dS this gives
//   g_i  = dL/dp_i  = sum_j dS_ij p'_j,   g'_j = dL/dp'_j = sum_i dS_ij p_i,
//   dL/dW = sum over heads and blocks of qbar_i g_i^T + kbar_j g'_j^T,
//   dL/dqbar_i = W g_i,   dL/dkbar_j = W g'_j.
// Three small kernels, deterministic (fixed summation orders, no atomics):
//  * score_grad_p_kernel: g (row i of dS) and g' (column j of dS), and the
//    pooled gradients W g, W g' when asked for;
//  * score_grad_w_kernel: partial dW over a chunk of 16 blocks of a head;
//  * score_grad_reduce_kernel: dW as the sum of the partials in a fixed
//    order.
// The block means and projections come from the scoring's own pooling
// kernel.  All of it is a few MFLOP: plain fp32 vector code.
#include "common.h"
#include "internal.h"

namespace bsa {

// grid (BH*nB, 2), 256 threads; blockIdx.y 0: g_i over row i of dS against
// the key projections, 1: g'_j over column j against the query projections.
// Lane m of each wave owns output m; the four waves split the summation
// index and their partial sums are added in a fixed order.
__global__ __launch_bounds__(256) void score_grad_p_kernel(const ScoreGradParams p)
{
    __shared__ float part[4][64];
    __shared__ float g[64];
    const int tid = threadIdx.x, m = tid & 63, wv = tid >> 6;
    const int item = blockIdx.x, which = blockIdx.y;
    const int bh = item / p.nB, x = item - bh * p.nB;
    const int64_t rows = (int64_t)p.BH * p.nB;
    const float *other = p.proj + ((int64_t)(1 - which) * rows + (int64_t)bh * p.nB) * p.r;
    const float *ds = p.dS + (int64_t)bh * p.nB * p.nB;
    const int64_t step_row = which == 0 ? 1 : p.nB;             // dS stride along the summed index
    const float *dsx = ds + (which == 0 ? (int64_t)x * p.nB : (int64_t)x);
    float acc = 0.f;
    if (m < p.r)
#pragma unroll 4
        for (int y = wv; y < p.nB; y += 4)
            acc = __builtin_fmaf(dsx[y * step_row], other[(int64_t)y * p.r + m], acc);
    part[wv][m] = acc;
    __syncthreads();
    if (tid < p.r) {
        const float v = (part[0][tid] + part[1][tid]) + (part[2][tid] + part[3][tid]);
        g[tid] = v;
        p.g[((int64_t)which * rows + item) * p.r + tid] = v;
    }
    __syncthreads();
    float *dp = p.dpool[which];
    if (dp && tid < p.D) {
        float a = 0.f;
#pragma unroll 8
        for (int mm = 0; mm < p.r; ++mm) a = __builtin_fmaf(p.w[tid * p.r + mm], g[mm], a);
        dp[(int64_t)item * p.D + tid] = a;
    }
}

// Partial dW of a chunk of kGradChunk blocks of one head (workgroup
// bh * chunks + c): wpart[wg][d*r + m] = sum over the chunk's blocks x of
// qbar_x[d] g_x[m] + kbar_x[d] g'_x[m], the chunk staged in LDS.  Thread t
// owns entries t, t+256, ... of the D*r <= 64*D outputs.
template <int D>
__global__ __launch_bounds__(256) void score_grad_w_kernel(const ScoreGradParams p)
{
    constexpr int CH = kGradChunk;
    constexpr int MAXE = D * 64 / 256;
    __shared__ float sm[2][CH][D];
    __shared__ float sg[2][CH][64];
    const int tid = threadIdx.x;
    const int chunks = (p.nB + CH - 1) / CH;
    const int bh = blockIdx.x / chunks, ch = blockIdx.x - bh * chunks;
    const int x0 = ch * CH, n = min(CH, p.nB - x0);
    const int r = p.r, E = D * r;
    const int64_t rows = (int64_t)p.BH * p.nB;
    const int64_t base = (int64_t)bh * p.nB + x0;
    for (int i = tid; i < 2 * CH * D; i += 256) {
        const int w = i / (CH * D), c = (i / D) % CH, d = i % D;
        sm[w][c][d] = c < n ? p.mean[((int64_t)w * rows + base + c) * D + d] : 0.f;
    }
    for (int i = tid; i < 2 * CH * 64; i += 256) {
        const int w = i / (CH * 64), c = (i / 64) % CH, m = i % 64;
        sg[w][c][m] = (c < n && m < r) ? p.g[((int64_t)w * rows + base + c) * r + m] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < MAXE; ++k) {
        const int e = tid + 256 * k;
        if (k * 256 >= E) break;                              // uniform: no entries left
        const int d = e < E ? e / r : 0, m = e < E ? e - d * r : 0;
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            acc = __builtin_fmaf(sm[0][c][d], sg[0][c][m], acc);
            acc = __builtin_fmaf(sm[1][c][d], sg[1][c][m], acc);
        }
        if (e < E) p.wpart[(int64_t)blockIdx.x * E + e] = acc;
    }
}

// dW[e] = sum of the partials: 64 entries per workgroup, each summed by four
// waves over interleaved partials and the four sums added in a fixed order.
__global__ __launch_bounds__(256) void score_grad_reduce_kernel(const ScoreGradParams p)
{
    __shared__ float part[4][64];
    const int E = p.D * p.r;
    const int l = threadIdx.x & 63, grp = threadIdx.x >> 6;
    const int e = blockIdx.x * 64 + l;
    const int P = p.BH * ((p.nB + kGradChunk - 1) / kGradChunk);
    float s = 0.f;
    if (e < E)
#pragma unroll 8
        for (int i = grp; i < P; i += 4) s += p.wpart[(int64_t)i * E + e];
    part[grp][l] = s;
    __syncthreads();
    if (grp == 0 && e < E) p.dw[e] = (part[0][l] + part[1][l]) + (part[2][l] + part[3][l]);
}

hipError_t launch_score_grad(const ScoreGradParams &p, hipStream_t s)
{
    const int64_t items = (int64_t)p.BH * p.nB;
    if (items <= 0 || p.r < 1 || p.r > 64) return hipErrorInvalidValue;
    if (p.D != 64 && p.D != 128) return hipErrorInvalidValue;
    hipLaunchKernelGGL(score_grad_p_kernel, dim3((unsigned)items, 2), dim3(256), 0, s, p);
    const int64_t parts = (int64_t)p.BH * ((p.nB + kGradChunk - 1) / kGradChunk);
    if (p.D == 128)
        hipLaunchKernelGGL(score_grad_w_kernel<128>, dim3((unsigned)parts), dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL(score_grad_w_kernel<64>, dim3((unsigned)parts), dim3(256), 0, s, p);
    hipLaunchKernelGGL(score_grad_reduce_kernel, dim3((unsigned)((p.D * p.r + 63) / 64)), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace bsa
