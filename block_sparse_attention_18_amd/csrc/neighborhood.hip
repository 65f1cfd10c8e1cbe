// 2-D neighbourhood attention on the latent grid (GNA notes, sections 1.1
// and 2.1-2.2): each image query attends to the keys of a window around it
// on the R x C grid, with a stride by which groups of queries share one
// window; regions involving text stay dense.
//
// Two kernels here:
//  * permute_kernel: text tokens stay first, the image tokens move from
//    row-major to tile-major order (th x tw tiles, one block each; tiles
//    row-major, tokens row-major inside a tile), or back.  Then every block
//    of the sequence is one 2-D tile, and a window covers whole tiles plus
//    a rim of partially covered ones.  One 16-byte chunk per thread; each
//    tile row is a contiguous run of tw tokens on both sides.
//  * layout_kernel: the block list of that order, closed form per query
//    tile.  A key tile is kept when some query of the query tile sees some
//    key of it (the windows of a tile's queries span the product of their
//    row and column ranges); it is "full" (flag 0) when every query sees
//    every key, else "partial" (flag 1) and the forward masks it per token.
#include "common.h"
#include "internal.h"

namespace bsa {

__device__ __forceinline__ int nb_natural(const NbGeom &g, int beta, int t)
{
    if (t < g.T) return t;
    const int q = t - g.T, tile = q / beta, o = q - tile * beta;
    const int a = tile / g.tpr, b = tile - a * g.tpr;
    return g.T + (a * g.th + (o >> g.tw_log2)) * g.C + b * g.tw + (o & (g.tw - 1));
}

// Grid (chunks / 256, B*H): chunk x of a head is token x / (D/8), 16 bytes
// at channel 8 (x % (D/8)).
__global__ __launch_bounds__(256) void permute_kernel(const PermuteParams p)
{
    const int bh = blockIdx.y, b = bh / p.H, h = bh - b * p.H;
    const int cpt = p.D / 8;
    const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (x >= (int64_t)p.N * cpt) return;
    const int t = (int)(x / cpt), c = (int)(x - (int64_t)t * cpt);
    const int nat = nb_natural(p.nb, p.nb.th * p.nb.tw, t);
    const int src = p.inverse ? t : nat, dst = p.inverse ? nat : t;
    const uint4 v = ld_g16(p.in.p + b * p.in.sb + h * p.in.sh + (int64_t)src * p.in.sn + 8 * c);
    *reinterpret_cast<uint4 *>(p.out + b * p.o_sb + h * p.o_sh + (int64_t)dst * p.o_sn + 8 * c) = v;
    if (c == 0 && p.lse_in && p.lse_out)
        p.lse_out[(int64_t)bh * p.N + dst] = p.lse_in[(int64_t)bh * p.N + src];
}

hipError_t launch_permute_tokens(const PermuteParams &p, hipStream_t s)
{
    const int64_t chunks = (int64_t)p.N * (p.D / 8);
    hipLaunchKernelGGL(permute_kernel, dim3((unsigned)((chunks + 255) / 256), (unsigned)(p.B * p.H)), dim3(256), 0,
                       s, p);
    return hipGetLastError();
}

// One wavefront per row (b, h, i): its offset is the entries of the heads
// before it plus the lengths of the earlier rows of its head (summed by the
// lanes); then its ascending columns and flags.
__global__ __launch_bounds__(256) void nb_layout_kernel(const NbLayoutParams p)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t rows = (int64_t)p.B * p.H * p.nB;
    if (row >= rows) return;
    const int64_t bh = row / p.nB;
    const int i = (int)(row - bh * p.nB);
    int64_t part = 0;
    for (int i2 = lane; i2 < i; i2 += 64) part += nb_row_len(p.nb, p.nB, i2);
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) part += __shfl_xor(part, d, 64);
    const int64_t base = bh * p.per_head + part;
    const int64_t len = nb_row_len(p.nb, p.nB, i);
    if (lane == 0) {
        p.row_ptr[row + 1] = (int32_t)(base + len);
        if (row == 0) p.row_ptr[0] = 0;
    }
    const NbGeom &g = p.nb;
    NbRow w{};
    if (i >= g.Tb) w = nb_row(g, i);
    const int nc = w.c1 - w.c0;
    for (int64_t e = lane; e < len; e += 64) {
        int col, flag = 0;
        if (i < g.Tb || e < g.Tb) {
            col = (int)e;
        } else {
            const int x = (int)(e - g.Tb), a = w.r0 + x / nc, b = w.c0 + x % nc;
            col = g.Tb + a * g.tpr + b;
            const bool full = a * g.th >= w.ir0 && a * g.th + g.th <= w.ir1 && b * g.tw >= w.ic0 &&
                              b * g.tw + g.tw <= w.ic1;
            flag = full ? 0 : 1;
        }
        if (base + e < p.capacity) {
            p.col_idx[base + e] = col;
            p.flags[base + e] = flag;
        }
    }
}

hipError_t launch_neighborhood_layout(const NbLayoutParams &p, hipStream_t s)
{
    const int64_t rows = (int64_t)p.B * p.H * p.nB;
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL(nb_layout_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace bsa
