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
//    a rim of partially covered ones.  One workgroup per tile; each tile
//    row is a contiguous run of tw tokens on both sides.
//  * layout_kernel: the block list of that order, closed form per query
//    tile.  A key tile is kept when some query of the query tile sees some
//    key of it (the windows of a tile's queries span the product of their
//    row and column ranges); it is "full" (flag 0) when every query sees
//    every key, else "partial" (flag 1) and the forward masks it per token.
#include "common.h"
#include "internal.h"

namespace bsa {

// Grid (blocks of the sequence, B*H): workgroup (i, bh) moves block i of
// head bh -- a text block unchanged, or image tile i - Tb -- as 16-byte
// chunks, 8 per thread.  Tile coordinates are worked out once per
// workgroup; inside a tile, token o sits at grid row o / tw, column o % tw
// (shifts: tw and D / 8 are powers of two).
template <int D>
__global__ __launch_bounds__(256) void permute_kernel(const PermuteParams p)
{
    constexpr int CPT = D / 8;                      // chunks per token
    const NbGeom &g = p.nb;
    const int beta = g.th * g.tw;
    const int i = blockIdx.x, bh = blockIdx.y, b = bh / p.H, h = bh - b * p.H;
    int base;                                       // natural index of the block's token 0
    int tile_row_stride;                            // natural-index step between the tile's rows
    if (i < g.Tb) {
        base = i * beta;
        tile_row_stride = g.tw;                     // a text block: contiguous
    } else {
        const int tile = i - g.Tb, a = tile / g.tpr;
        base = g.T + a * g.th * g.C + (tile - a * g.tpr) * g.tw;
        tile_row_stride = g.C;
    }
    const uint16_t *__restrict__ inb = p.in.p + b * p.in.sb + h * p.in.sh;
    uint16_t *__restrict__ outb = p.out + b * p.o_sb + h * p.o_sh;
    // all loads of the thread first, then the stores (up to 8 chunks in flight)
    constexpr int MAXU = 128 * CPT / 256;
    const int nu = beta * CPT / 256;
    uint4 v[MAXU];
    int dst[MAXU];
#pragma unroll
    for (int u = 0; u < MAXU; ++u) {
        if (u < nu) {
            const int x = threadIdx.x + 256 * u;
            const int o = x / CPT, c = x - o * CPT;
            const int t = i * beta + o;                                         // tile-major index
            const int nat = base + (o >> g.tw_log2) * tile_row_stride + (o & (g.tw - 1));
            const int src = p.inverse ? t : nat;
            dst[u] = p.inverse ? nat : t;
            v[u] = ld_g16(inb + (int64_t)src * p.in.sn + 8 * c);
            if (c == 0 && p.lse_in && p.lse_out)
                p.lse_out[(int64_t)bh * p.N + dst[u]] = p.lse_in[(int64_t)bh * p.N + src];
        }
    }
#pragma unroll
    for (int u = 0; u < MAXU; ++u) {
        if (u < nu) {
            const int c = (threadIdx.x + 256 * u) % CPT;
            *reinterpret_cast<uint4 *>(outb + (int64_t)dst[u] * p.o_sn + 8 * c) = v[u];
        }
    }
}

hipError_t launch_permute_tokens(const PermuteParams &p, hipStream_t s)
{
    const int nblk = p.N / (p.nb.th * p.nb.tw);
    const dim3 grid((unsigned)nblk, (unsigned)(p.B * p.H));
    if (p.D == 128) hipLaunchKernelGGL(permute_kernel<128>, grid, dim3(256), 0, s, p);
    else if (p.D == 64) hipLaunchKernelGGL(permute_kernel<64>, grid, dim3(256), 0, s, p);
    else return hipErrorInvalidValue;
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
