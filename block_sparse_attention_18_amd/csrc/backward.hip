// Backward of the block-sparse forward on gfx950: dQ, dK, dV of the softmax
// restricted to the kept blocks (the gradient a training step needs, e.g.
// for training the selection's projection jointly with the model, as the
// multimodal-DiT write-up does in section 2.2).  With P recomputed from the
// forward's LSE, dP = dO V^T, Delta = rowsum(dO * O) and dS = P (dP - Delta):
//   dV = P^T dO,   dK = scale dS^T Q,   dQ = scale dS K.
//
// Three kernels, all deterministic (no atomics):
//  * bwd_prep_kernel: Delta and LSE * log2(e) per query token.
//  * bwd_dq_kernel: one workgroup per (query block, head), laid out like the
//    forward (each wave owns 32 queries; K and V tiles of 64 keys stream
//    through LDS with double-buffered LDS-DMA copies).  S^T = K Q^T and
//    dP^T = V dO^T on bf16 MFMA with Q and dO in registers; dS^T, packed to
//    bf16, is directly the B operand of dQ^T += K^T dS^T (K^T by
//    transposing LDS reads).
//  * bwd_dkdv_kernel: one workgroup per (key block, head) of 2 * block / 32
//    waves, each wave owning 32 keys and one 32-query half of every 64-query
//    sub-tile; the block's K and V sit in LDS.  The workgroup first lists,
//    by binary search in each block row (columns ascend), the query blocks
//    that keep its key block; their Q and dO sub-tiles stream through LDS.
//    S = Q K^T and dP = dO V^T with the query rows in the permuted order, so
//    that P and dS packed to bf16 are the B operands of dV^T += dO^T P and
//    dK^T += Q^T dS (dO^T, Q^T by transposing LDS reads); the two query
//    halves' partial sums are added through LDS at the end.
// Tiles read both by rows and transposed use one XOR swizzle of the 16-byte
// chunk index that keeps both read patterns on distinct bank slots.
// With a 2-D neighbourhood layout (NBM), the scores of partially covered
// entries are masked per token as in the forward: dQ tests each key of a
// sub-tile against its lane's query window; dK/dV, whose lanes own keys,
// tests each query against the range of query rows and columns whose
// windows hold the lane's key (window starts do not decrease along an axis,
// so that range is an interval, found once by binary search).
#include "common.h"
#include "internal.h"

namespace bsa {

template <int BETA, int D>
struct BwShape {
    static constexpr int NW = BETA / 32;
    static constexpr int NT = NW * 64;
    static constexpr int SUB = BETA / 64;
    static constexpr int QS = D / 16;
    static constexpr int DT = D / 32;
    static constexpr int KCH = D / 8;
    static constexpr int TILE = 64 * D;
    static constexpr int DMA = 64 * KCH / NT;
    static_assert(64 * KCH % NT == 0, "tile split");
};

// Chunk swizzle of a tile row: injective over the 16 rows a quarter-wave
// reads as MFMA rows, and constant-plus-distinct over the 4 consecutive rows
// of a transposing read.
template <int D>
__device__ __forceinline__ int bswz(int r)
{
    return D == 128 ? ((4 * (r & 3)) ^ ((r >> 2) & 3)) : ((4 * ((r >> 1) & 1)) | ((r >> 2) & 3));
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_prep_kernel(const BwdParams p)
{
    const int lpt = p.D / 8, tpb = 256 / lpt;
    const int g = threadIdx.x / lpt, c = threadIdx.x % lpt;
    const int64_t tok = (int64_t)blockIdx.x * tpb + g;
    const bool ok = tok < (int64_t)p.B * p.H * p.N;
    float acc = 0.f;
    if (ok) {
        const int64_t bh = tok / p.N, t = tok - bh * p.N;
        const int b = (int)(bh / p.H), h = (int)(bh - (int64_t)b * p.H);
        // natural-order tensors: the row of tile-major token t
        const int64_t tn = p.natural ? nb_natural(p.nb, p.natural, (int)t) : t;
        const uint4 a = ld_g16(p.dO.p + b * p.dO.sb + h * p.dO.sh + tn * p.dO.sn + 8 * c);
        const uint4 o = ld_g16(p.o.p + b * p.o.sb + h * p.o.sh + tn * p.o.sn + 8 * c);
        const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, ow[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc += __uint_as_float(aw[j] << 16) * __uint_as_float(ow[j] << 16);
            acc += __uint_as_float(aw[j] & 0xFFFF0000u) * __uint_as_float(ow[j] & 0xFFFF0000u);
        }
    }
    for (int d = 1; d < lpt; d <<= 1) acc += __shfl_xor(acc, d, 64);
    if (ok && c == 0) {
        const int64_t bh = tok / p.N, t = tok - bh * p.N;
        const int64_t tn = p.natural ? nb_natural(p.nb, p.natural, (int)t) : t;
        p.delta[tok] = acc;                              // workspace: tile-major order
        p.lse2[tok] = p.lse[bh * p.N + tn] * kLog2e;
    }
}

// ---------------------------------------------------------------------------
// shared pieces
// ---------------------------------------------------------------------------
// Copy of a 64-row tile (rows from r0 of a [N][D] bf16 matrix with row
// stride sn) into LDS, slot s = (x*NW + wave)*64 + lane holding row s / KCH,
// chunk (s % KCH) ^ bswz(row); rows past N repeat row N-1.  nat: the matrix
// is in natural token order and tile-major row r0 + r is gathered from its
// natural position.
template <int BETA, int D>
__device__ __forceinline__ void bw_load_tile(uint16_t *__restrict__ dst, __amdgpu_buffer_rsrc_t rs, int64_t sn,
                                             int r0, int N, int wv, int lane, bool nat = false,
                                             const NbGeom &g = NbGeom{})
{
    using Sh = BwShape<BETA, D>;
    // one opaque LDS base per call: each copy's destination is a scalar add
    __attribute__((address_space(3))) char *lbase = (__attribute__((address_space(3))) char *)(lds_void *)(dst + wv * 64 * 8);
    asm volatile("" : "+s"(lbase));
    if (nat && r0 >= g.T) {
        // the tile's 64 rows gathered from natural order: a scalar base (the
        // first row's position) plus a per-lane offset that is the same for
        // every tile (the row offsets add over the disjoint bits of r0 mod
        // BETA, a multiple of 64, and r < 64)
        const int b0 = r0 & ~(BETA - 1);
        const uint32_t so = (uint32_t)((nb_natural(g, BETA, b0) + nb_rowoff(g, r0 - b0)) * sn * 2);
#pragma unroll
        for (int x = 0; x < Sh::DMA; ++x) {
            const int slot = (x * Sh::NW + wv) * 64 + lane;
            const int r = slot / Sh::KCH, ps = slot % Sh::KCH;
            const uint32_t o = (uint32_t)(nb_rowoff(g, r) * sn * 2 + ((ps ^ bswz<D>(r)) * 16));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(lbase + x * Sh::NW * 64 * 16), 16, o, so, 0, 0);
        }
        return;
    }
#pragma unroll
    for (int x = 0; x < Sh::DMA; ++x) {
        const int slot = (x * Sh::NW + wv) * 64 + lane;
        const int r = slot / Sh::KCH, ps = slot % Sh::KCH;
        const int src = max(0, min(r0 + r, N - 1));
        const uint32_t o = (uint32_t)(src * sn * 2 + ((ps ^ bswz<D>(r)) * 16));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(lbase + x * Sh::NW * 64 * 16), 16, o, 0, 0, 0);
    }
}

// Byte offsets of a lane's MFMA operand reads in a tile: rows (A operand of
// 32 rows x 16 columns fed in perm_row order; k-step s: ^ KSTEP * s), and
// transposing reads (A operand of 32 columns x 16 rows; pp selects rows
// +0 / +4 of the 4-row group; 32-column group d: ^ VSTEP * d).
template <int D>
struct BwOffsets {
    uint32_t rows;
    uint32_t tr[2];
};

template <int D>
__device__ __forceinline__ BwOffsets<D> bw_offsets(int lane)
{
    BwOffsets<D> o;
    const int hl = lane >> 5, n = lane & 31;
    const int r0 = perm_row(n);
    o.rows = (uint32_t)(r0 * D * 2 + 16 * (hl ^ bswz<D>(r0)));
    const int G = lane >> 4, jl = lane & 15;
    const int vr0 = 8 * (G >> 1) + (jl >> 2);
    const int dc = 16 * (G & 1) + 4 * (jl & 3);
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
        const int r = vr0 + 4 * pp;
        o.tr[pp] = (uint32_t)(r * D * 2 + (((dc >> 3) ^ bswz<D>(r)) * 16) + (dc & 4) * 2);
    }
    return o;
}

// acc[kt] = sum_s X[kt*32 + perm rows][16 s ..] * frag[s]  (two 32x32 tiles)
template <int D>
__device__ __forceinline__ void bw_rows_mfma(const uint16_t *__restrict__ X, uint32_t rows, const bf16x8 (&frag)[D / 16],
                                             f32x16 (&acc)[2])
{
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[kt][r] = 0.f;
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            const bf16x8 a = *lds_at<bf16x8>(X + kt * 32 * D, rows ^ (KSTEP * s));
            acc[kt] = mfma32x32x16(a, frag[s], acc[kt]);
        }
}

// out[d] += X^T (rows d of 32-column group d) * pf, over the 64 tile rows
template <int D>
__device__ __forceinline__ void bw_tr_mfma(const uint16_t *__restrict__ X, const BwOffsets<D> &off,
                                           const bf16x8 (&pf)[2][2], f32x16 (&out)[D / 32])
{
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int d = 0; d < D / 32; ++d) {
                s16x4 h2[2];
#pragma unroll
                for (int pp = 0; pp < 2; ++pp) {
                    const uint16_t *rowp = X + (kt * 32 + 16 * u) * D;
                    h2[pp] = __builtin_bit_cast(
                        s16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                   (__attribute__((address_space(3))) bf16x4 *)lds_at<uint16_t>(rowp, off.tr[pp] ^ (VSTEP * d))));
                }
                const bf16x8 a =
                    __builtin_bit_cast(bf16x8, __builtin_shufflevector(h2[0], h2[1], 0, 1, 2, 3, 4, 5, 6, 7));
                out[d] = mfma32x32x16(a, pf[kt][u], out[d]);
            }
}

// pack 8 consecutive accumulator values (kt, u) of a two-tile accumulator
__device__ __forceinline__ bf16x8 pack8(const f32x16 (&x)[2], int kt, int u)
{
    uint4 pk;
    pk.x = pack_bf16x2(x[kt][8 * u + 0], x[kt][8 * u + 1]);
    pk.y = pack_bf16x2(x[kt][8 * u + 2], x[kt][8 * u + 3]);
    pk.z = pack_bf16x2(x[kt][8 * u + 4], x[kt][8 * u + 5]);
    pk.w = pack_bf16x2(x[kt][8 * u + 6], x[kt][8 * u + 7]);
    return as_bf16x8(pk);
}

// ---------------------------------------------------------------------------
// 2-D neighbourhood helpers
// ---------------------------------------------------------------------------
// Grid row and column of the image token at tile-major position t >= T.
template <int BETA>
__device__ __forceinline__ void nb_pos(const NbGeom &g, int t, int &r, int &c)
{
    const int pt = t - g.T, tile = pt / BETA, o = pt - tile * BETA;
    const int a = tile / g.tpr;
    r = a * g.th + (o >> g.tw_log2);
    c = (tile - a * g.tpr) * g.tw + (o & (g.tw - 1));
}

// The positions i in [0, L) whose window [start(i), start(i) + k) holds x:
// start(i) does not decrease with i, so they form [lo, hi] (empty: lo > hi).
__device__ __forceinline__ void nb_seen_by(int x, int L, int k, int s, int &lo, int &hi)
{
    int a = 0, b = L;
    while (a < b) {
        const int m = (a + b) >> 1;
        if (nb_start(m, L, k, s) <= x) a = m + 1;
        else b = m;
    }
    hi = a - 1;
    a = 0;
    b = L;
    while (a < b) {
        const int m = (a + b) >> 1;
        if (nb_start(m, L, k, s) + k <= x) a = m + 1;
        else b = m;
    }
    lo = a;
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per (query block, head)
// ---------------------------------------------------------------------------
template <int BETA, int D, bool NBM>
__global__ __launch_bounds__(BETA / 32 * 64, 2) void bwd_dq_kernel(const BwdParams p)
{
    using Sh = BwShape<BETA, D>;
    __shared__ __attribute__((aligned(16))) uint16_t smem[4 * Sh::TILE];   // two (K, V) buffers
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hl = lane >> 5, n = lane & 31;
    const int BH = p.B * p.H;
    int i, bh;
    work_item((int)blockIdx.x, BH, p.nB, i, bh);
    const int b = bh / p.H, hh = bh - b * p.H;
    const int64_t row = (int64_t)bh * p.nB + i;
    const int e0 = p.row_ptr[row], e1 = p.row_ptr[row + 1];
    const int T = (e1 > e0 ? e1 - e0 : 0) * Sh::SUB;

    const int qrow = i * BETA + wv * 32 + n;
    const bool qok = qrow < p.N;
    // natural-order tensors: rows are gathered from (and dQ scattered to)
    // the natural positions of the tile-major tokens
    const bool nat = NBM && p.natural;
    const int qpos = (nat && qok) ? nb_natural(p.nb, BETA, qrow) : qrow;
    bf16x8 qf[Sh::QS], dof[Sh::QS];
    {
        const uint16_t *qb = p.q.p + b * p.q.sb + hh * p.q.sh + (int64_t)qpos * p.q.sn;
        const uint16_t *gb = p.dO.p + b * p.dO.sb + hh * p.dO.sh + (int64_t)qpos * p.dO.sn;
#pragma unroll
        for (int s = 0; s < Sh::QS; ++s) {
            qf[s] = as_bf16x8(qok ? ld_g16(qb + 16 * s + 8 * hl) : zero_u4());
            dof[s] = as_bf16x8(qok ? ld_g16(gb + 16 * s + 8 * hl) : zero_u4());
        }
    }
    // neighbourhood: the window of the lane's query (image queries only)
    int wr0 = 0, wc0 = 0;
    const bool qimg = NBM && qok && qrow >= p.nb.T;
    if (qimg) {
        int rq, cq;
        nb_pos<BETA>(p.nb, qrow, rq, cq);
        wr0 = nb_start(rq, p.nb.R, p.nb.kh, p.nb.sh);
        wc0 = nb_start(cq, p.nb.C, p.nb.kw, p.nb.sw);
    }
    const __attribute__((address_space(4))) int32_t *cflag =
        (const __attribute__((address_space(4))) int32_t *)(NBM ? p.flags + e0 : p.col_idx);
    const int64_t qtok = (int64_t)bh * p.N + (qok ? qrow : 0);
    const float lse2 = qok ? p.lse2[qtok] : 0.f;
    const float delta = qok ? p.delta[qtok] : 0.f;
    const float c = p.scale_log2;
    f32x16 dq[Sh::DT];
#pragma unroll
    for (int d = 0; d < Sh::DT; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) dq[d][r] = 0.f;

    const BwOffsets<D> off = bw_offsets<D>(lane);
    const uint16_t *kb = p.k.p + b * p.k.sb + hh * p.k.sh;
    const uint16_t *vb = p.v.p + b * p.v.sb + hh * p.v.sh;
    const __amdgpu_buffer_rsrc_t krs = buffer_desc(kb, (uint32_t)(((int64_t)(p.N - 1) * p.k.sn + D) * 2));
    const __amdgpu_buffer_rsrc_t vrs = buffer_desc(vb, (uint32_t)(((int64_t)(p.N - 1) * p.v.sn + D) * 2));
    const __attribute__((address_space(4))) int32_t *cidx =
        (const __attribute__((address_space(4))) int32_t *)(p.col_idx + e0);
    auto key0 = [&](int t, bool &valid) {
        const int j = cidx[t / Sh::SUB];
        valid = (unsigned)j < (unsigned)p.nB;
        return (valid ? j * BETA : 0) + 64 * (t % Sh::SUB);
    };

    if (T > 0) {
        bool vcur;
        int kcur = key0(0, vcur);
        bw_load_tile<BETA, D>(smem, krs, p.k.sn, kcur, p.N, wv, lane, nat, p.nb);
        bw_load_tile<BETA, D>(smem + Sh::TILE, vrs, p.v.sn, kcur, p.N, wv, lane, nat, p.nb);
        for (int t = 0; t < T; ++t) {
            uint16_t *Kc = smem + (t & 1) * 2 * Sh::TILE, *Vc = Kc + Sh::TILE;
            bool vnxt = false;
            int knxt = 0;
            wait_tile_copies();
            __syncthreads();   // tile t in LDS; buffer (t+1)&1 free
            if (t + 1 < T) {
                knxt = key0(t + 1, vnxt);
                uint16_t *Kn = smem + ((t + 1) & 1) * 2 * Sh::TILE;
                bw_load_tile<BETA, D>(Kn, krs, p.k.sn, knxt, p.N, wv, lane, nat, p.nb);
                bw_load_tile<BETA, D>(Kn + Sh::TILE, vrs, p.v.sn, knxt, p.N, wv, lane, nat, p.nb);
            }
            f32x16 s[2], dp[2];
            bw_rows_mfma<D>(Kc, off.rows, qf, s);
            bw_rows_mfma<D>(Vc, off.rows, dof, dp);
            if (!vcur || kcur + 64 > p.N) mask_keys(s, (vcur ? p.N - kcur : 0) - 8 * hl);
            if (NBM && vcur && cflag[t / Sh::SUB] != 0) {
                // a partially covered entry: keys outside the lane's query window
                const int jj = kcur / BETA;
                if (jj >= p.nb.Tb) {
                    const int tk = jj - p.nb.Tb, ak = tk / p.nb.tpr;
                    uint64_t bits = nb_window_bits(p.nb, kcur - jj * BETA, ak * p.nb.th - wr0,
                                                   (tk - ak * p.nb.tpr) * p.nb.tw - wc0, p.nb.kh, p.nb.kw);
                    bits = qimg ? bits >> (8 * hl) : ~0ull;   // bit kt*32 + koff(r): register r of chain kt
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt) {
                        const uint32_t w = (uint32_t)(bits >> (32 * kt));
#pragma unroll
                        for (int r = 0; r < 16; ++r) s[kt][r] = keep_if_bit(s[kt][r], w, koff(r));
                    }
                }
            }
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float pr = fast_exp2(__builtin_fmaf(s[kt][r], c, -lse2));
                    s[kt][r] = pr * (dp[kt][r] - delta);   // dS^T
                }
            bf16x8 pf[2][2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int u = 0; u < 2; ++u) pf[kt][u] = pack8(s, kt, u);
            bw_tr_mfma<D>(Kc, off, pf, dq);
            vcur = vnxt;
            kcur = knxt;
        }
    }
    if (qok) {
        const float sc = p.scale;
        uint16_t *orow = p.dq + b * p.dq_sb + hh * p.dq_sh + (int64_t)qpos * p.dq_sn;
#pragma unroll
        for (int d = 0; d < Sh::DT; ++d)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                uint2 sv;
                sv.x = pack_bf16x2(dq[d][4 * g + 0] * sc, dq[d][4 * g + 1] * sc);
                sv.y = pack_bf16x2(dq[d][4 * g + 2] * sc, dq[d][4 * g + 3] * sc);
                *reinterpret_cast<uint2 *>(orow + d * 32 + 8 * g + 4 * hl) = sv;
            }
    }
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per (key block, head)
// ---------------------------------------------------------------------------
// P and dS of one 32-query half (rows 32 h + 8 hl + koff(r) of the
// sub-tile) from its S and dP, in place (s <- P, dp <- dS), packed to bf16
// as the B operands (two 16-query k-steps) of dV^T += dO^T P and
// dK^T += Q^T dS.  Query rows past N carry -inf scores (masked before).
__device__ __forceinline__ void bw_probs_half(f32x16 &s, f32x16 &dp, const float *stats, int h, float c, int hl,
                                              bf16x8 (&pp)[2], bf16x8 (&ps)[2])
{
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int r0 = 32 * h + 8 * hl + koff(4 * g);
        const float4 l2 = *reinterpret_cast<const float4 *>(stats + r0);
        const float4 dl = *reinterpret_cast<const float4 *>(stats + 64 + r0);
        const float lv[4] = {l2.x, l2.y, l2.z, l2.w};
        const float dv4[4] = {dl.x, dl.y, dl.z, dl.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            const float pr = fast_exp2(__builtin_fmaf(s[r], c, -lv[e]));
            s[r] = pr;
            dp[r] = pr * (dp[r] - dv4[e]);
        }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        uint4 a, b;
        a.x = pack_bf16x2(s[8 * u + 0], s[8 * u + 1]);
        a.y = pack_bf16x2(s[8 * u + 2], s[8 * u + 3]);
        a.z = pack_bf16x2(s[8 * u + 4], s[8 * u + 5]);
        a.w = pack_bf16x2(s[8 * u + 6], s[8 * u + 7]);
        b.x = pack_bf16x2(dp[8 * u + 0], dp[8 * u + 1]);
        b.y = pack_bf16x2(dp[8 * u + 2], dp[8 * u + 3]);
        b.z = pack_bf16x2(dp[8 * u + 4], dp[8 * u + 5]);
        b.w = pack_bf16x2(dp[8 * u + 6], dp[8 * u + 7]);
        pp[u] = as_bf16x8(a);
        ps[u] = as_bf16x8(b);
    }
}

// out[d] += X^T (32-column group d, rows 32 h .. 32 h + 31) * pf
template <int D>
__device__ __forceinline__ void bw_tr_half(const uint16_t *__restrict__ X, const BwOffsets<D> &off, int h,
                                           const bf16x8 (&pf)[2], f32x16 (&out)[D / 32])
{
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int d = 0; d < D / 32; ++d) {
            s16x4 h2[2];
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                const uint16_t *rowp = X + (h * 32 + 16 * u) * D;
                h2[pp] = __builtin_bit_cast(
                    s16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                               (__attribute__((address_space(3))) bf16x4 *)lds_at<uint16_t>(rowp, off.tr[pp] ^ (VSTEP * d))));
            }
            const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(h2[0], h2[1], 0, 1, 2, 3, 4, 5, 6, 7));
            out[d] = mfma32x32x16(a, pf[u], out[d]);
        }
}

// ---------------------------------------------------------------------------
// dK, dV with two waves per key group: one workgroup per (key block, head)
// of 2 * BETA / 32 waves; wave w owns the 32 keys of group w % (BETA / 32)
// and the 32-query half w / (BETA / 32) of every 64-query sub-tile.  The
// key block's K and V stay in LDS (B operands read per MFMA), which keeps a
// wave within 256 registers (two waves per SIMD).  The two halves' partial
// dK, dV are added through LDS at the end.
// ---------------------------------------------------------------------------
template <int BETA, int D>
struct DkShape {
    static constexpr int NKG = BETA / 32;
    static constexpr int NW = 2 * NKG;
    static constexpr int NT = NW * 64;
    static constexpr int QS = D / 16;
    static constexpr int DT = D / 32;
    static constexpr int KCH = D / 8;
    static constexpr int KV = BETA * D;          // bf16 elements of the block's K (or V)
    static constexpr int QT = 64 * D;            // bf16 elements of a 64-query tile
    static constexpr int BUF = 2 * QT + 256;     // Q, dO, then 2 x 64 fp32 statistics
    static constexpr int SMEM = 2 * KV + 2 * BUF;
};

// Copy of R rows (from r0; rows past N repeat row N-1) into LDS with the
// backward's chunk swizzle; NT threads, 16 bytes each per copy.  nat: the
// matrix is in natural token order (rows gathered as in bw_load_tile;
// blocks of BETA tokens).
template <int R, int D, int NT, int BETA>
__device__ __forceinline__ void bw_load_rows(uint16_t *__restrict__ dst, __amdgpu_buffer_rsrc_t rs, int64_t sn,
                                              int r0, int N, int tid, bool nat = false, const NbGeom &g = NbGeom{})
{
    constexpr int KCH = D / 8, CP = R * KCH / NT;
    static_assert(R * KCH % NT == 0, "tile split");
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    __attribute__((address_space(3))) char *lbase = (__attribute__((address_space(3))) char *)(lds_void *)(dst + wv * 64 * 8);
    asm volatile("" : "+s"(lbase));
    if (nat && r0 >= g.T) {
        // natural order: scalar base plus a per-lane offset, as in bw_load_tile
        // (r0 mod BETA is a multiple of R, and r < R)
        const int b0 = r0 & ~(BETA - 1);
        const uint32_t so = (uint32_t)((nb_natural(g, BETA, b0) + nb_rowoff(g, r0 - b0)) * sn * 2);
#pragma unroll
        for (int x = 0; x < CP; ++x) {
            const int slot = (x * (NT / 64) + wv) * 64 + lane;
            const int r = slot / KCH, ps = slot % KCH;
            const uint32_t o = (uint32_t)(nb_rowoff(g, r) * sn * 2 + ((ps ^ bswz<D>(r)) * 16));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(lbase + x * (NT / 64) * 64 * 16), 16, o, so, 0,
                                                     0);
        }
        return;
    }
#pragma unroll
    for (int x = 0; x < CP; ++x) {
        const int slot = (x * (NT / 64) + wv) * 64 + lane;
        const int r = slot / KCH, ps = slot % KCH;
        const int src = max(0, min(r0 + r, N - 1));
        const uint32_t o = (uint32_t)(src * sn * 2 + ((ps ^ bswz<D>(r)) * 16));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(lbase + x * (NT / 64) * 64 * 16), 16, o, 0, 0, 0);
    }
}

template <int BETA, int D, bool NBM>
__global__ __launch_bounds__(2 * BETA / 32 * 64, 2) void bwd_dkdv_kernel(const BwdParams p)
{
    using G = DkShape<BETA, D>;
    __shared__ __attribute__((aligned(16))) uint16_t dsm[G::SMEM];
    extern __shared__ int qlist[];   // query blocks keeping this key block (bit 30: partial entry)
    uint16_t *const Kt = dsm, *const Vt = dsm + G::KV;
    uint16_t *const Bf0 = dsm + 2 * G::KV;
    __shared__ int wcount[G::NW];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = wv % G::NKG, qh = wv / G::NKG;
    const int hl = lane >> 5, n = lane & 31;
    const int BH = p.B * p.H;
    int j, bh;
    work_item((int)blockIdx.x, BH, p.nB, j, bh);   // key block j
    const int b = bh / p.H, hh = bh - b * p.H;
    // natural-order tensors: rows gathered from (and dK, dV scattered to)
    // the natural positions of the tile-major tokens
    const bool nat = NBM && p.natural;

    // query blocks whose row lists j, ascending
    int count = 0;
    for (int base = 0; base < p.nB; base += G::NT) {
        int i = base + tid;
        bool f = false;
        if (i < p.nB) {
            const int64_t r = (int64_t)bh * p.nB + i;
            int lo = p.row_ptr[r], hi = p.row_ptr[r + 1];
            const int end = hi;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (p.col_idx[mid] < j) lo = mid + 1;
                else hi = mid;
            }
            f = lo < end && p.col_idx[lo] == j;
            if (NBM && f && p.flags[lo] != 0) i |= 1 << 30;
        }
        const uint64_t m = __ballot(f);
        if (lane == 0) wcount[wv] = __popcll(m);
        __syncthreads();
        int pre = count, tot = 0;
        for (int w = 0; w < G::NW; ++w) {
            if (w < wv) pre += wcount[w];
            tot += wcount[w];
        }
        if (f) qlist[pre + __popcll(m & ((1ull << lane) - 1))] = i;
        __syncthreads();
        count += tot;
    }
    const int T = count * (BETA / 64);

    const uint16_t *kb = p.k.p + b * p.k.sb + hh * p.k.sh;
    const uint16_t *vb = p.v.p + b * p.v.sb + hh * p.v.sh;
    const uint16_t *qb = p.q.p + b * p.q.sb + hh * p.q.sh;
    const uint16_t *gb = p.dO.p + b * p.dO.sb + hh * p.dO.sh;
    const __amdgpu_buffer_rsrc_t krs = buffer_desc(kb, (uint32_t)(((int64_t)(p.N - 1) * p.k.sn + D) * 2));
    const __amdgpu_buffer_rsrc_t vrs = buffer_desc(vb, (uint32_t)(((int64_t)(p.N - 1) * p.v.sn + D) * 2));
    const __amdgpu_buffer_rsrc_t qrs = buffer_desc(qb, (uint32_t)(((int64_t)(p.N - 1) * p.q.sn + D) * 2));
    const __amdgpu_buffer_rsrc_t grs = buffer_desc(gb, (uint32_t)(((int64_t)(p.N - 1) * p.dO.sn + D) * 2));
    const __amdgpu_buffer_rsrc_t lrs = buffer_desc(p.lse2 + (int64_t)bh * p.N, (uint32_t)p.N * 4);
    const __amdgpu_buffer_rsrc_t drs = buffer_desc(p.delta + (int64_t)bh * p.N, (uint32_t)p.N * 4);
    auto qblock = [&](int t) { return qlist[t / (BETA / 64)] & ((1 << 30) - 1); };
    auto qstart = [&](int t) { return qblock(t) * BETA + 64 * (t % (BETA / 64)); };
    auto buf = [&](int t) { return Bf0 + (t & 1) * G::BUF; };
    auto load = [&](int t) {
        const int q0 = qstart(t);
        uint16_t *B0 = buf(t);
        bw_load_rows<64, D, G::NT, BETA>(B0, qrs, p.q.sn, q0, p.N, tid, nat, p.nb);
        bw_load_rows<64, D, G::NT, BETA>(B0 + G::QT, grs, p.dO.sn, q0, p.N, tid, nat, p.nb);
        if (wv == 0) {
            float *st = reinterpret_cast<float *>(B0 + 2 * G::QT);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(lrs, (lds_void *)st, 4, (uint32_t)lane * 4, (uint32_t)q0 * 4, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(drs, (lds_void *)(st + 64), 4, (uint32_t)lane * 4,
                                                     (uint32_t)q0 * 4, 0, 0);
        }
    };

    f32x16 dk[G::DT], dv[G::DT];
#pragma unroll
    for (int d = 0; d < G::DT; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            dk[d][r] = 0.f;
            dv[d][r] = 0.f;
        }
    const float c = p.scale_log2;
    const BwOffsets<D> off = bw_offsets<D>(lane);
    // B operand rows of the wave's keys in Kt / Vt (natural order)
    const int krow_l = kg * 32 + n;
    // neighbourhood: the query rows [qr0, qr1] and columns [qc0, qc1] whose
    // windows hold the lane's key (image keys only)
    int qr0 = 0, qr1 = -1, qc0 = 0, qc1 = -1;
    const bool kimg = NBM && j >= p.nb.Tb;
    if (kimg) {
        int kr, kc;
        nb_pos<BETA>(p.nb, j * BETA + krow_l, kr, kc);
        nb_seen_by(kr, p.nb.R, p.nb.kh, p.nb.sh, qr0, qr1);
        nb_seen_by(kc, p.nb.C, p.nb.kw, p.nb.sw, qc0, qc1);
    }
    const uint32_t brow = (uint32_t)(krow_l * D * 2 + 16 * (hl ^ bswz<D>(krow_l)));

    if (T > 0) {
        bw_load_rows<BETA, D, G::NT, BETA>(Kt, krs, p.k.sn, j * BETA, p.N, tid, nat, p.nb);
        bw_load_rows<BETA, D, G::NT, BETA>(Vt, vrs, p.v.sn, j * BETA, p.N, tid, nat, p.nb);
        load(0);
        for (int t = 0; t < T; ++t) {
            wait_tile_copies();
            __syncthreads();                  // sub-tile t in LDS; buffer (t+1)&1 free
            if (t + 1 < T) load(t + 1);
            const uint16_t *Qc = buf(t), *Gc = Qc + G::QT;
            const float *stats = reinterpret_cast<const float *>(Qc + 2 * G::QT);
            const int q0 = qstart(t) + 32 * qh;
            f32x16 s, dp;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[r] = 0.f;
                dp[r] = 0.f;
            }
#pragma unroll
            for (int k = 0; k < G::QS; ++k) {
                const bf16x8 aq = *lds_at<bf16x8>(Qc + qh * 32 * D, off.rows ^ (KSTEP * k));
                const bf16x8 bk = *lds_at<bf16x8>(Kt, brow ^ (KSTEP * k));
                s = mfma32x32x16(aq, bk, s);
                const bf16x8 ag = *lds_at<bf16x8>(Gc + qh * 32 * D, off.rows ^ (KSTEP * k));
                const bf16x8 bv = *lds_at<bf16x8>(Vt, brow ^ (KSTEP * k));
                dp = mfma32x32x16(ag, bv, dp);
            }
            if (q0 + 32 > p.N) {
                const int lim = p.N - q0 - 8 * hl;
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (koff(r) >= lim) s[r] = -INFINITY;
            }
            bf16x8 pp[2], ps[2];
            if (NBM && kimg && (qlist[t / (BETA / 64)] >> 30) != 0 && qblock(t) >= p.nb.Tb) {
                // a partially covered entry (an image query block): queries
                // whose window misses the lane's key are masked.  The queries
                // that see it, [qr0, qr1] x [qc0, qc1], act as a window over
                // the query tile; register r holds query 8 hl + koff(r).
                const int i = qblock(t), tq = i - p.nb.Tb, aq = tq / p.nb.tpr;
                const uint32_t w = (uint32_t)(nb_window_bits(p.nb, q0 - i * BETA, aq * p.nb.th - qr0,
                                                             (tq - aq * p.nb.tpr) * p.nb.tw - qc0, qr1 - qr0 + 1,
                                                             qc1 - qc0 + 1) >> (8 * hl));
#pragma unroll
                for (int r = 0; r < 16; ++r) s[r] = keep_if_bit(s[r], w, koff(r));
            }
            bw_probs_half(s, dp, stats, qh, c, hl, pp, ps);
            bw_tr_half<D>(Gc, off, qh, pp, dv);
            bw_tr_half<D>(Qc, off, qh, ps, dk);
        }
    }

    // add the two query halves' partial sums through LDS: the second half's
    // waves park theirs, the first half's add them and store
    __syncthreads();
    float *park = reinterpret_cast<float *>(dsm);
    const int slot0 = (kg * G::DT) * 64 + lane;
    if (qh == 1) {
#pragma unroll
        for (int d = 0; d < G::DT; ++d)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                *reinterpret_cast<float4 *>(park + ((slot0 + d * 64) * 2 * 4 + g) * 4) =
                    make_float4(dk[d][4 * g], dk[d][4 * g + 1], dk[d][4 * g + 2], dk[d][4 * g + 3]);
                *reinterpret_cast<float4 *>(park + ((slot0 + d * 64) * 2 * 4 + 4 + g) * 4) =
                    make_float4(dv[d][4 * g], dv[d][4 * g + 1], dv[d][4 * g + 2], dv[d][4 * g + 3]);
            }
    }
    __syncthreads();
    const int krow = j * BETA + kg * 32 + n;
    if (qh == 0 && krow < p.N) {
        const int kpos = nat ? nb_natural(p.nb, BETA, krow) : krow;
        const float sc = p.scale;
        uint16_t *rk = p.dk + b * p.dk_sb + hh * p.dk_sh + (int64_t)kpos * p.dk_sn;
        uint16_t *rv = p.dv + b * p.dv_sb + hh * p.dv_sh + (int64_t)kpos * p.dv_sn;
#pragma unroll
        for (int d = 0; d < G::DT; ++d)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 ok = *reinterpret_cast<const float4 *>(park + ((slot0 + d * 64) * 2 * 4 + g) * 4);
                const float4 ov = *reinterpret_cast<const float4 *>(park + ((slot0 + d * 64) * 2 * 4 + 4 + g) * 4);
                uint2 a, v2;
                a.x = pack_bf16x2((dk[d][4 * g + 0] + ok.x) * sc, (dk[d][4 * g + 1] + ok.y) * sc);
                a.y = pack_bf16x2((dk[d][4 * g + 2] + ok.z) * sc, (dk[d][4 * g + 3] + ok.w) * sc);
                v2.x = pack_bf16x2(dv[d][4 * g + 0] + ov.x, dv[d][4 * g + 1] + ov.y);
                v2.y = pack_bf16x2(dv[d][4 * g + 2] + ov.z, dv[d][4 * g + 3] + ov.w);
                *reinterpret_cast<uint2 *>(rk + d * 32 + 8 * g + 4 * hl) = a;
                *reinterpret_cast<uint2 *>(rv + d * 32 + 8 * g + 4 * hl) = v2;
            }
    }
}

template <int BETA, int D, bool NBM>
static hipError_t launch_bwd_t(const BwdParams &p, hipStream_t s)
{
    using Sh = BwShape<BETA, D>;
    const int64_t grid = (int64_t)p.B * p.H * p.nB;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((bwd_dq_kernel<BETA, D, NBM>), dim3((unsigned)grid), dim3(Sh::NT), 0, s, p);
    using G = DkShape<BETA, D>;
    static_assert(G::SMEM * 2 + G::NW * 4 + kBwdMaxBlocks * 4 <= 160 * 1024, "dK/dV LDS");
    if (p.nB > kBwdMaxBlocks) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_dkdv_kernel<BETA, D, NBM>), dim3((unsigned)grid), dim3(G::NT),
                       (size_t)p.nB * sizeof(int), s, p);
    return hipGetLastError();
}

template <int BETA, int D>
static hipError_t launch_bwd_t(const BwdParams &p, hipStream_t s)
{
    return p.flags ? launch_bwd_t<BETA, D, true>(p, s) : launch_bwd_t<BETA, D, false>(p, s);
}

hipError_t launch_backward(const BwdParams &p, int block, int D, hipStream_t s)
{
    const int64_t toks = (int64_t)p.B * p.H * p.N;
    const int tpb = 256 / (D / 8);
    hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)((toks + tpb - 1) / tpb)), dim3(256), 0, s, p);
    if (block == 128 && D == 128) return launch_bwd_t<128, 128>(p, s);
    if (block == 128 && D == 64) return launch_bwd_t<128, 64>(p, s);
    if (block == 64 && D == 128) return launch_bwd_t<64, 128>(p, s);
    if (block == 64 && D == 64) return launch_bwd_t<64, 64>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace bsa
