// Block-sparse attention forward on gfx950.
//
// Computes, for every query token t of a non-skipped head, the softmax
// attention restricted to the key blocks listed in the CSR row of t's query
// block, with an online (running max / running sum) softmax over the blocks
// in list order -- the FlashAttention-style kernel over block indices of the
// multimodal-DiT write-up (section 3.1) and the fused full / arrow kernel of
// DiTFastAttnV2 ("Fused Kernel").  Kept blocks are dense: nothing is masked
// inside a block except keys past N in a partial last block.
//
// Mapping onto CDNA4:
//  * one workgroup per (query block i, head); BETA/32 waves, each owning 32
//    query rows.  Work items are ordered query-block-major so that the long
//    text rows of every head are dispatched first, and consecutive
//    workgroups (which the dispatcher deals round-robin to the 8 XCDs) walk
//    different heads, so each XCD's L2 keeps a few heads' K/V windows.
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 d from LDS,
//    B = 16 d x 32 queries held in registers for the whole kernel).  K rows
//    are fed in a permuted order (bits 2 and 3 of the row index swapped)
//    so that the fp32 accumulator of S^T, converted to bf16, is already the
//    B operand (16 keys x 32 queries) of O^T = V^T P^T.  Each lane therefore
//    owns one query: the running max, running sum and the O rescale are
//    lane-local, and only the max needs one cross-half exchange per block.
//  * K is staged row-major and V transposed ([d][key]) in LDS with XOR
//    swizzles of 16-byte chunks, so the 128-bit operand reads and the
//    staging writes stay (near) conflict-free without padding.
//  * exp is exp2 with scale*log2(e) folded into one FMA.
#include "common.h"
#include "internal.h"

namespace bsa {

template <int BETA, int D>
struct FwdShape {
    static constexpr int NW = BETA / 32;          // waves per workgroup
    static constexpr int NT = NW * 64;            // threads per workgroup
    static constexpr int KT = BETA / 32;          // 32-key sub-tiles per block
    static constexpr int QS = D / 16;             // k-steps of S^T over d
    static constexpr int DT = D / 32;             // 32-row d tiles of O^T
    static constexpr int KCH = D / 8;             // 16-byte chunks per K row
    static constexpr int VCH = BETA / 8;          // 16-byte chunks per V^T row
    static constexpr int K_ITEMS = BETA * KCH;    // 16-byte chunks per K tile
    static constexpr int V_ITEMS = (BETA / 4) * (D / 8);   // (4 keys x 8 d) items per V tile
    static constexpr size_t LDS_BYTES = 2u * BETA * D * sizeof(uint16_t);
    static_assert(K_ITEMS % NT == 0 && V_ITEMS % NT == 0, "tile split");
};

// Row of the K tile fed to A-operand row n of a 32-key sub-tile.
__device__ __forceinline__ int perm_row(int n)
{
    return (n & ~12) | ((n & 4) << 1) | ((n & 8) >> 1);
}

__device__ __forceinline__ uint32_t u4_word(const uint4 &u, int w)
{
    return w == 0 ? u.x : (w == 1 ? u.y : (w == 2 ? u.z : u.w));
}

template <int BETA, int D>
__global__ __launch_bounds__(BETA / 32 * 64) void fwd_kernel(const FwdParams p)
{
    using Sh = FwdShape<BETA, D>;
    extern __shared__ __align__(16) uint16_t lds[];
    uint16_t *Ks = lds;                 // [BETA][D], chunk c of row r at (c ^ r % KCH)
    uint16_t *Vt = lds + BETA * D;      // [D][BETA], chunk c of row d at (c ^ d % VCH)

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int hl = lane >> 5;           // lane half
    const int n = lane & 31;

    const int BH = p.B * p.H;
    const int i = blockIdx.x / BH;
    const int bh = blockIdx.x - i * BH;
    const int b = bh / p.H;
    const int hh = bh - b * p.H;
    if ((p.skip_bits[hh >> 5] >> (hh & 31)) & 1u) return;

    const int64_t row = (int64_t)bh * p.nB + i;
    const int e0 = p.row_ptr[row];
    const int e1 = p.row_ptr[row + 1];

    const uint16_t *qb = p.q.p + b * p.q.sb + hh * p.q.sh;
    const uint16_t *kb = p.k.p + b * p.k.sb + hh * p.k.sh;
    const uint16_t *vb = p.v.p + b * p.v.sb + hh * p.v.sh;

    // Q^T fragments: lane (hl, n) holds query row n, d = 16 s + 8 hl .. +7.
    const int qrow = i * BETA + wv * 32 + n;
    bf16x8 qf[Sh::QS];
#pragma unroll
    for (int s = 0; s < Sh::QS; ++s) {
        uint4 u = qrow < p.N ? ld_g16(qb + (int64_t)qrow * p.q.sn + 16 * s + 8 * hl) : zero_u4();
        qf[s] = as_bf16x8(u);
    }

    f32x16 oacc[Sh::DT];
#pragma unroll
    for (int t = 0; t < Sh::DT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[t][r] = 0.f;
    float m_run = -INFINITY;   // running max, log2-scaled domain
    float l_run = 0.f;         // running sum over this lane's keys
    const float c = p.scale_log2;

    for (int e = e0; e < e1; ++e) {
        const int j = p.col_idx[e];
        if ((unsigned)j >= (unsigned)p.nB) continue;
        const int key0 = j * BETA;

        __syncthreads();   // every wave is done reading the previous tile
#pragma unroll
        for (int it = 0; it < Sh::K_ITEMS / Sh::NT; ++it) {
            const int c16 = tid + it * Sh::NT;
            const int r = c16 / Sh::KCH, cc = c16 % Sh::KCH;
            const int key = key0 + r;
            uint4 u = key < p.N ? ld_g16(kb + (int64_t)key * p.k.sn + cc * 8) : zero_u4();
            *reinterpret_cast<uint4 *>(Ks + r * D + ((cc ^ (r % Sh::KCH)) * 8)) = u;
        }
#pragma unroll
        for (int it = 0; it < Sh::V_ITEMS / Sh::NT; ++it) {
            const int item = tid + it * Sh::NT;
            const int q4 = (item % 16) + 16 * (item / (16 * (D / 8)));   // key quad
            const int cd = (item / 16) % (D / 8);                        // d chunk
            uint4 x[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int key = key0 + 4 * q4 + a;
                x[a] = key < p.N ? ld_g16(vb + (int64_t)key * p.v.sn + cd * 8) : zero_u4();
            }
#pragma unroll
            for (int ee = 0; ee < 8; ++ee) {
                const int wd = ee >> 1;
                uint32_t lo, hi;
                if (ee & 1) {
                    lo = (u4_word(x[0], wd) >> 16) | (u4_word(x[1], wd) & 0xFFFF0000u);
                    hi = (u4_word(x[2], wd) >> 16) | (u4_word(x[3], wd) & 0xFFFF0000u);
                } else {
                    lo = (u4_word(x[0], wd) & 0xFFFFu) | (u4_word(x[1], wd) << 16);
                    hi = (u4_word(x[2], wd) & 0xFFFFu) | (u4_word(x[3], wd) << 16);
                }
                const int d = cd * 8 + ee;
                const int pos = q4 ^ (2 * (d % Sh::VCH));
                *reinterpret_cast<uint2 *>(Vt + d * BETA + 4 * pos) = make_uint2(lo, hi);
            }
        }
        __syncthreads();

        // S^T (keys x queries) for the BETA keys of this block
        f32x16 sacc[Sh::KT];
#pragma unroll
        for (int kt = 0; kt < Sh::KT; ++kt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.f;
            const int r = kt * 32 + perm_row(n);
#pragma unroll
            for (int s = 0; s < Sh::QS; ++s) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
                    Ks + r * D + (((2 * s + hl) ^ (r % Sh::KCH)) * 8));
                sacc[kt] = mfma32x32x16(a, qf[s], sacc[kt]);
            }
        }
        if (key0 + BETA > p.N) {   // partial last block: keys past N do not exist
#pragma unroll
            for (int kt = 0; kt < Sh::KT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = key0 + kt * 32 + perm_row(8 * (r >> 2) + 4 * hl + (r & 3));
                    if (key >= p.N) sacc[kt][r] = -INFINITY;
                }
        }

        // online softmax for this lane's query
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < Sh::KT; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kt][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx * c);
        const float alpha = (m_run == m_new) ? 1.f : fast_exp2(m_run - m_new);
        m_run = m_new;
        float ls = 0.f;
#pragma unroll
        for (int kt = 0; kt < Sh::KT; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float pr = fast_exp2(__builtin_fmaf(sacc[kt][r], c, -m_new));
                sacc[kt][r] = pr;
                ls += pr;
            }
        l_run = l_run * alpha + ls;
#pragma unroll
        for (int t = 0; t < Sh::DT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[t][r] *= alpha;

        // O^T += V^T P^T
#pragma unroll
        for (int kt = 0; kt < Sh::KT; ++kt) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                uint4 pk;
                pk.x = pack_bf16x2(sacc[kt][8 * u + 0], sacc[kt][8 * u + 1]);
                pk.y = pack_bf16x2(sacc[kt][8 * u + 2], sacc[kt][8 * u + 3]);
                pk.z = pack_bf16x2(sacc[kt][8 * u + 4], sacc[kt][8 * u + 5]);
                pk.w = pack_bf16x2(sacc[kt][8 * u + 6], sacc[kt][8 * u + 7]);
                const bf16x8 pf = as_bf16x8(pk);
                const int key8 = 4 * kt + 2 * u + hl;
#pragma unroll
                for (int t = 0; t < Sh::DT; ++t) {
                    const int d = t * 32 + n;
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
                        Vt + d * BETA + 8 * (key8 ^ (d % Sh::VCH)));
                    oacc[t] = mfma32x32x16(a, pf, oacc[t]);
                }
            }
        }
    }

    // epilogue: normalise and store O (bf16) and LSE (natural log)
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (qrow < p.N) {
        uint16_t *orow = p.o + b * p.o_sb + hh * p.o_sh + (int64_t)qrow * p.o_sn;
#pragma unroll
        for (int t = 0; t < Sh::DT; ++t)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                uint2 st;
                st.x = pack_bf16x2(oacc[t][4 * g + 0] * inv, oacc[t][4 * g + 1] * inv);
                st.y = pack_bf16x2(oacc[t][4 * g + 2] * inv, oacc[t][4 * g + 3] * inv);
                *reinterpret_cast<uint2 *>(orow + t * 32 + 8 * g + 4 * hl) = st;
            }
        if (p.lse && hl == 0) {
            const float lse = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
            p.lse[(int64_t)bh * p.N + qrow] = lse;
        }
    }
}

template <int BETA, int D>
static hipError_t launch_fwd_t(const FwdParams &p, hipStream_t s)
{
    using Sh = FwdShape<BETA, D>;
    auto kern = fwd_kernel<BETA, D>;
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         (int)Sh::LDS_BYTES);
    if (err != hipSuccess) return err;
    const unsigned grid = (unsigned)((int64_t)p.B * p.H * p.nB);
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(Sh::NT), Sh::LDS_BYTES, s, p);
    return hipGetLastError();
}

hipError_t launch_forward(const FwdParams &p, int block, int D, hipStream_t s)
{
    if (block == 128 && D == 128) return launch_fwd_t<128, 128>(p, s);
    if (block == 128 && D == 64) return launch_fwd_t<128, 64>(p, s);
    if (block == 64 && D == 128) return launch_fwd_t<64, 128>(p, s);
    if (block == 64 && D == 64) return launch_fwd_t<64, 64>(p, s);
    return hipErrorInvalidValue;
}

// SKIP heads: copy the cached output (and LSE) of the head unchanged
// (DiTFastAttnV2, "Head-wise Caching").  16-byte chunks; grid.y = head.
__global__ __launch_bounds__(256) void skip_copy_kernel(const SkipCopyParams p)
{
    const int bh = blockIdx.y;
    const int b = bh / p.H, hh = bh - b * p.H;
    if (!((p.skip_bits[hh >> 5] >> (hh & 31)) & 1u)) return;
    const int chunks_per_row = p.D / 8;
    const int64_t total = (int64_t)p.N * chunks_per_row;
    for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < total;
         x += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = x / chunks_per_row;
        const int cc = (int)(x - t * chunks_per_row);
        if (p.copy_o) {
            const uint16_t *src = p.src.p + b * p.src.sb + hh * p.src.sh + t * p.src.sn + cc * 8;
            uint16_t *dst = p.dst + b * p.d_sb + hh * p.d_sh + t * p.d_sn + cc * 8;
            *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(src);
        }
        if (cc == 0 && p.lse_src && p.lse_dst)
            p.lse_dst[(int64_t)bh * p.N + t] = p.lse_src[(int64_t)bh * p.N + t];
    }
}

hipError_t launch_skip_copy(const SkipCopyParams &p, hipStream_t s)
{
    const int64_t chunks = (int64_t)p.N * (p.D / 8);
    int gx = (int)((chunks + 255) / 256);
    if (gx > 1024) gx = 1024;
    if (gx < 1) gx = 1;
    hipLaunchKernelGGL(skip_copy_kernel, dim3(gx, p.B * p.H), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace bsa
