// Diagnostics of sparse attention: the per-head relative squared error of
// an output against a reference (DiTFastAttnV2, single-layer RSE, the
// measure its compression plans are judged by) and the per-head Jaccard
// similarity of two block masks (SparseD, sparse reuse: how stable a mask
// chosen at one denoising step stays at later steps).
//
// RSE: one pass over both tensors, HBM-bound; each workgroup sums a chunk of
// one head in fp64 (squared error, sum and sum of squares of the
// reference), a second small kernel combines the chunks in a fixed order
// (deterministic, no atomics).  Jaccard: one workgroup per head; each wave
// takes one block row at a time, marks both masks' columns in LDS bitmaps
// and counts the bits of their AND and OR.
#include "common.h"
#include "internal.h"

namespace bsa {

// Sum over 256 threads of three doubles (result valid in thread 0).
__device__ __forceinline__ void block_sum3(double &a, double &b, double &c)
{
    __shared__ double red[3][4];
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        a += __shfl_xor(a, d, 64);
        b += __shfl_xor(b, d, 64);
        c += __shfl_xor(c, d, 64);
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        red[0][w] = a;
        red[1][w] = b;
        red[2][w] = c;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        a = red[0][0] + red[0][1] + red[0][2] + red[0][3];
        b = red[1][0] + red[1][1] + red[1][2] + red[1][3];
        c = red[2][0] + red[2][1] + red[2][2] + red[2][3];
    }
}

// Grid (B*H, chunks): chunk c of head bh covers rows [c*rows, (c+1)*rows).
__global__ __launch_bounds__(256) void rse_partial_kernel(const RseParams p)
{
    const int bh = blockIdx.x, c = blockIdx.y;
    const int b = bh / p.H, h = bh - b * p.H;
    const int lpr = p.D / 8;                     // lanes per row (16 bytes each)
    const int rpi = 256 / lpr;                   // rows per iteration
    const int lr = threadIdx.x / lpr, ch = threadIdx.x % lpr;
    const int t0 = c * p.rows_per_chunk, t1 = min(p.N, t0 + p.rows_per_chunk);
    const uint16_t *tb = p.test.p + b * p.test.sb + h * p.test.sh;
    const uint16_t *rb = p.ref.p + b * p.ref.sb + h * p.ref.sh;
    double se = 0.0, sr = 0.0, srr = 0.0;
    for (int t = t0 + lr; t < t1; t += rpi) {
        const uint4 a = ld_g16(tb + (int64_t)t * p.test.sn + 8 * ch);
        const uint4 r = ld_g16(rb + (int64_t)t * p.ref.sn + 8 * ch);
        const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, rw[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int hi = 0; hi < 2; ++hi) {
                const double x = (double)__uint_as_float(hi ? (aw[j] & 0xFFFF0000u) : (aw[j] << 16));
                const double y = (double)__uint_as_float(hi ? (rw[j] & 0xFFFF0000u) : (rw[j] << 16));
                const double d = x - y;
                se = __builtin_fma(d, d, se);
                sr += y;
                srr = __builtin_fma(y, y, srr);
            }
        }
    }
    block_sum3(se, sr, srr);
    if (threadIdx.x == 0) {
        double *o = p.partials + ((int64_t)bh * p.chunks + c) * 3;
        o[0] = se;
        o[1] = sr;
        o[2] = srr;
    }
}

// One thread per head: RSE = se / (srr - sr^2 / n); 0/0 -> 0, x/0 -> inf.
__global__ __launch_bounds__(256) void rse_final_kernel(const RseParams p)
{
    const int64_t bh = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (bh >= (int64_t)p.B * p.H) return;
    double se = 0.0, sr = 0.0, srr = 0.0;
    for (int c = 0; c < p.chunks; ++c) {
        const double *o = p.partials + (bh * p.chunks + c) * 3;
        se += o[0];
        sr += o[1];
        srr += o[2];
    }
    const double n = (double)p.N * p.D;
    const double den = fmax(srr - sr * sr / n, 0.0);
    p.rse[bh] = den > 0.0 ? se / den : (se == 0.0 ? 0.0 : INFINITY);
}

hipError_t launch_output_rse(const RseParams &p, hipStream_t s)
{
    const int64_t BH = (int64_t)p.B * p.H;
    hipLaunchKernelGGL(rse_partial_kernel, dim3((unsigned)BH, (unsigned)p.chunks), dim3(256), 0, s, p);
    hipLaunchKernelGGL(rse_final_kernel, dim3((unsigned)((BH + 255) / 256)), dim3(256), 0, s, p);
    return hipGetLastError();
}

// One workgroup (4 waves) per head; wave w takes block rows w, w + 4, ...
// Dynamic LDS: per wave two bitmaps of nW = ceil(nB / 32) words.
__global__ __launch_bounds__(256) void jaccard_kernel(const JaccardParams p)
{
    extern __shared__ uint32_t bits[];
    const int bh = blockIdx.x;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int nB = p.nB, nW = (nB + 31) / 32;
    uint32_t *ba = bits + wv * 2 * nW, *bb = ba + nW;
    uint64_t inter = 0, uni = 0;
    for (int i0 = 0; i0 < nB; i0 += 4) {
        const int i = i0 + wv;                  // every wave runs the same number of iterations
        for (int x = lane; x < nW; x += 64) {
            ba[x] = 0u;
            bb[x] = 0u;
        }
        __syncthreads();
        if (i < nB) {
            const int64_t r = (int64_t)bh * nB + i;
            const int a0 = p.row_ptr_a[r], a1 = p.row_ptr_a[r + 1];
            for (int e = a0 + lane; e < a1; e += 64) {
                const int j = p.col_idx_a[e];
                if ((unsigned)j < (unsigned)nB) atomicOr(&ba[j >> 5], 1u << (j & 31));
            }
            const int b0 = p.row_ptr_b[r], b1 = p.row_ptr_b[r + 1];
            for (int e = b0 + lane; e < b1; e += 64) {
                const int j = p.col_idx_b[e];
                if ((unsigned)j < (unsigned)nB) atomicOr(&bb[j >> 5], 1u << (j & 31));
            }
        }
        __syncthreads();
        if (i < nB) {
            for (int x = lane; x < nW; x += 64) {
                inter += __popc(ba[x] & bb[x]);
                uni += __popc(ba[x] | bb[x]);
            }
        }
        __syncthreads();
    }
    double a = (double)inter, u = (double)uni, z = 0.0;
    block_sum3(a, u, z);
    if (threadIdx.x == 0) p.jaccard[bh] = u > 0.0 ? a / u : 1.0;
}

hipError_t launch_mask_jaccard(const JaccardParams &p, hipStream_t s)
{
    const int64_t BH = (int64_t)p.B * p.H;
    const size_t lds = (size_t)4 * 2 * ((p.nB + 31) / 32) * sizeof(uint32_t);
    hipLaunchKernelGGL(jaccard_kernel, dim3((unsigned)BH), dim3(256), lds, s, p);
    return hipGetLastError();
}

}  // namespace bsa
