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
//  * bwd_dkdv_kernel: one workgroup per (key block, head), each wave owning
//    32 keys, K and V in registers.  The workgroup first lists, by binary
//    search in each block row (columns ascend), the query blocks that keep
//    its key block; their Q and dO tiles stream through LDS.  S = Q K^T and
//    dP = dO V^T with the query rows in the permuted order, so that P and
//    dS packed to bf16 are the B operands of dV^T += dO^T P and
//    dK^T += Q^T dS (dO^T, Q^T by transposing LDS reads).
// Tiles read both by rows and transposed use one XOR swizzle of the 16-byte
// chunk index that keeps both read patterns on distinct bank slots.
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
        const uint4 a = ld_g16(p.dO.p + b * p.dO.sb + h * p.dO.sh + t * p.dO.sn + 8 * c);
        const uint4 o = ld_g16(p.o.p + b * p.o.sb + h * p.o.sh + t * p.o.sn + 8 * c);
        const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, ow[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc += __uint_as_float(aw[j] << 16) * __uint_as_float(ow[j] << 16);
            acc += __uint_as_float(aw[j] & 0xFFFF0000u) * __uint_as_float(ow[j] & 0xFFFF0000u);
        }
    }
    for (int d = 1; d < lpt; d <<= 1) acc += __shfl_xor(acc, d, 64);
    if (ok && c == 0) {
        p.delta[tok] = acc;
        p.lse2[tok] = p.lse[tok] * kLog2e;
    }
}

// ---------------------------------------------------------------------------
// shared pieces
// ---------------------------------------------------------------------------
// Copy of a 64-row tile (rows from r0 of a [N][D] bf16 matrix with row
// stride sn) into LDS, slot s = (x*NW + wave)*64 + lane holding row s / KCH,
// chunk (s % KCH) ^ bswz(row); rows past N repeat row N-1.
template <int BETA, int D>
__device__ __forceinline__ void bw_load_tile(uint16_t *__restrict__ dst, __amdgpu_buffer_rsrc_t rs, int64_t sn,
                                             int r0, int N, int wv, int lane)
{
    using Sh = BwShape<BETA, D>;
    // one opaque LDS base per call: each copy's destination is a scalar add
    __attribute__((address_space(3))) char *lbase = (__attribute__((address_space(3))) char *)(lds_void *)(dst + wv * 64 * 8);
    asm volatile("" : "+s"(lbase));
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
// dQ: one workgroup per (query block, head)
// ---------------------------------------------------------------------------
template <int BETA, int D>
__global__ __launch_bounds__(BETA / 32 * 64, 2) void bwd_dq_kernel(const BwdParams p)
{
    using Sh = BwShape<BETA, D>;
    __shared__ __attribute__((aligned(16))) uint16_t smem[4 * Sh::TILE];   // two (K, V) buffers
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hl = lane >> 5, n = lane & 31;
    const int BH = p.B * p.H;
    const int i = blockIdx.x / BH, bh = blockIdx.x - i * BH;
    const int b = bh / p.H, hh = bh - b * p.H;
    const int64_t row = (int64_t)bh * p.nB + i;
    const int e0 = p.row_ptr[row], e1 = p.row_ptr[row + 1];
    const int T = (e1 > e0 ? e1 - e0 : 0) * Sh::SUB;

    const int qrow = i * BETA + wv * 32 + n;
    const bool qok = qrow < p.N;
    bf16x8 qf[Sh::QS], dof[Sh::QS];
    {
        const uint16_t *qb = p.q.p + b * p.q.sb + hh * p.q.sh + (int64_t)qrow * p.q.sn;
        const uint16_t *gb = p.dO.p + b * p.dO.sb + hh * p.dO.sh + (int64_t)qrow * p.dO.sn;
#pragma unroll
        for (int s = 0; s < Sh::QS; ++s) {
            qf[s] = as_bf16x8(qok ? ld_g16(qb + 16 * s + 8 * hl) : zero_u4());
            dof[s] = as_bf16x8(qok ? ld_g16(gb + 16 * s + 8 * hl) : zero_u4());
        }
    }
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
        bw_load_tile<BETA, D>(smem, krs, p.k.sn, kcur, p.N, wv, lane);
        bw_load_tile<BETA, D>(smem + Sh::TILE, vrs, p.v.sn, kcur, p.N, wv, lane);
        for (int t = 0; t < T; ++t) {
            uint16_t *Kc = smem + (t & 1) * 2 * Sh::TILE, *Vc = Kc + Sh::TILE;
            bool vnxt = false;
            int knxt = 0;
            __syncthreads();   // tile t in LDS; buffer (t+1)&1 free
            if (t + 1 < T) {
                knxt = key0(t + 1, vnxt);
                uint16_t *Kn = smem + ((t + 1) & 1) * 2 * Sh::TILE;
                bw_load_tile<BETA, D>(Kn, krs, p.k.sn, knxt, p.N, wv, lane);
                bw_load_tile<BETA, D>(Kn + Sh::TILE, vrs, p.v.sn, knxt, p.N, wv, lane);
            }
            f32x16 s[2], dp[2];
            bw_rows_mfma<D>(Kc, off.rows, qf, s);
            bw_rows_mfma<D>(Vc, off.rows, dof, dp);
            if (!vcur || kcur + 64 > p.N) mask_keys(s, (vcur ? p.N - kcur : 0) - 8 * hl);
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
        uint16_t *orow = p.dq + b * p.dq_sb + hh * p.dq_sh + (int64_t)qrow * p.dq_sn;
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
template <int BETA, int D>
__global__ __launch_bounds__(BETA / 32 * 64, 1) void bwd_dkdv_kernel(const BwdParams p)
{
    using Sh = BwShape<BETA, D>;
    __shared__ __attribute__((aligned(16))) uint16_t smem[4 * Sh::TILE];   // two (Q, dO) buffers
    __shared__ int wcount[Sh::NW];
    extern __shared__ int qlist[];                                          // query blocks keeping this key block
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hl = lane >> 5, n = lane & 31;
    const int BH = p.B * p.H;
    const int j = blockIdx.x / BH, bh = blockIdx.x - j * BH;
    const int b = bh / p.H, hh = bh - b * p.H;

    // the query blocks whose row lists j (binary search: columns ascend),
    // in ascending order
    int count = 0;
    for (int base = 0; base < p.nB; base += Sh::NT) {
        const int i = base + tid;
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
        }
        const uint64_t m = __ballot(f);
        if (lane == 0) wcount[wv] = __popcll(m);
        __syncthreads();
        int pre = count, tot = 0;
        for (int w = 0; w < Sh::NW; ++w) {
            if (w < wv) pre += wcount[w];
            tot += wcount[w];
        }
        if (f) qlist[pre + __popcll(m & ((1ull << lane) - 1))] = i;
        __syncthreads();
        count += tot;
    }
    const int T = count * Sh::SUB;

    const int krow = j * BETA + wv * 32 + n;   // the lane's key
    const bool kok = krow < p.N;
    bf16x8 kf[Sh::QS], vf[Sh::QS];
    {
        const uint16_t *kb = p.k.p + b * p.k.sb + hh * p.k.sh + (int64_t)krow * p.k.sn;
        const uint16_t *vb = p.v.p + b * p.v.sb + hh * p.v.sh + (int64_t)krow * p.v.sn;
#pragma unroll
        for (int s = 0; s < Sh::QS; ++s) {
            kf[s] = as_bf16x8(kok ? ld_g16(kb + 16 * s + 8 * hl) : zero_u4());
            vf[s] = as_bf16x8(kok ? ld_g16(vb + 16 * s + 8 * hl) : zero_u4());
        }
    }
    f32x16 dk[Sh::DT], dv[Sh::DT];
#pragma unroll
    for (int d = 0; d < Sh::DT; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            dk[d][r] = 0.f;
            dv[d][r] = 0.f;
        }
    const float c = p.scale_log2;
    const BwOffsets<D> off = bw_offsets<D>(lane);
    const uint16_t *qb = p.q.p + b * p.q.sb + hh * p.q.sh;
    const uint16_t *gb = p.dO.p + b * p.dO.sb + hh * p.dO.sh;
    const __amdgpu_buffer_rsrc_t qrs = buffer_desc(qb, (uint32_t)(((int64_t)(p.N - 1) * p.q.sn + D) * 2));
    const __amdgpu_buffer_rsrc_t grs = buffer_desc(gb, (uint32_t)(((int64_t)(p.N - 1) * p.dO.sn + D) * 2));
    const float *lse2 = p.lse2 + (int64_t)bh * p.N;
    const float *delta = p.delta + (int64_t)bh * p.N;
    auto qstart = [&](int t) { return qlist[t / Sh::SUB] * BETA + 64 * (t % Sh::SUB); };
    const bool vec_stats = ((int64_t)bh * p.N) % 4 == 0;   // 16-byte aligned rows of lse2, delta

    if (T > 0) {
        int q0 = qstart(0);
        bw_load_tile<BETA, D>(smem, qrs, p.q.sn, q0, p.N, wv, lane);
        bw_load_tile<BETA, D>(smem + Sh::TILE, grs, p.dO.sn, q0, p.N, wv, lane);
        for (int t = 0; t < T; ++t) {
            uint16_t *Qc = smem + (t & 1) * 2 * Sh::TILE, *Gc = Qc + Sh::TILE;
            __syncthreads();
            int qn = 0;
            if (t + 1 < T) {
                qn = qstart(t + 1);
                uint16_t *Qn = smem + ((t + 1) & 1) * 2 * Sh::TILE;
                bw_load_tile<BETA, D>(Qn, qrs, p.q.sn, qn, p.N, wv, lane);
                bw_load_tile<BETA, D>(Qn + Sh::TILE, grs, p.dO.sn, qn, p.N, wv, lane);
            }
            // row statistics of the lane's 32 accumulator rows: query
            // q0 + 32 kt + 8 hl + koff(r), in groups of 4 consecutive rows
            // (16-byte loads when the head's rows are 16-byte aligned)
            float4 l2[2][4], dl[2][4];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int r0 = q0 + 32 * kt + 8 * hl + koff(4 * g);
                    if (vec_stats && r0 + 4 <= p.N) {
                        l2[kt][g] = *reinterpret_cast<const float4 *>(lse2 + r0);
                        dl[kt][g] = *reinterpret_cast<const float4 *>(delta + r0);
                    } else {
                        float4 a = make_float4(0.f, 0.f, 0.f, 0.f), d4 = a;
                        if (r0 + 0 < p.N) { a.x = lse2[r0 + 0]; d4.x = delta[r0 + 0]; }
                        if (r0 + 1 < p.N) { a.y = lse2[r0 + 1]; d4.y = delta[r0 + 1]; }
                        if (r0 + 2 < p.N) { a.z = lse2[r0 + 2]; d4.z = delta[r0 + 2]; }
                        if (r0 + 3 < p.N) { a.w = lse2[r0 + 3]; d4.w = delta[r0 + 3]; }
                        l2[kt][g] = a;
                        dl[kt][g] = d4;
                    }
                }
            f32x16 s[2], dp[2];
            bw_rows_mfma<D>(Qc, off.rows, kf, s);
            bw_rows_mfma<D>(Gc, off.rows, vf, dp);
            if (q0 + 64 > p.N) mask_keys(s, p.N - q0 - 8 * hl);   // query rows past N
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const float lv[4] = {l2[kt][g].x, l2[kt][g].y, l2[kt][g].z, l2[kt][g].w};
                    const float dv4[4] = {dl[kt][g].x, dl[kt][g].y, dl[kt][g].z, dl[kt][g].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * g + e;
                        const float pr = fast_exp2(__builtin_fmaf(s[kt][r], c, -lv[e]));
                        s[kt][r] = pr;                              // P
                        dp[kt][r] = pr * (dp[kt][r] - dv4[e]);      // dS
                    }
                }
            bf16x8 pp[2][2], ps[2][2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    pp[kt][u] = pack8(s, kt, u);
                    ps[kt][u] = pack8(dp, kt, u);
                }
            bw_tr_mfma<D>(Gc, off, pp, dv);
            bw_tr_mfma<D>(Qc, off, ps, dk);
            q0 = qn;
        }
    }
    if (kok) {
        const float sc = p.scale;
        uint16_t *krow_k = p.dk + b * p.dk_sb + hh * p.dk_sh + (int64_t)krow * p.dk_sn;
        uint16_t *krow_v = p.dv + b * p.dv_sb + hh * p.dv_sh + (int64_t)krow * p.dv_sn;
#pragma unroll
        for (int d = 0; d < Sh::DT; ++d)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                uint2 a, v2;
                a.x = pack_bf16x2(dk[d][4 * g + 0] * sc, dk[d][4 * g + 1] * sc);
                a.y = pack_bf16x2(dk[d][4 * g + 2] * sc, dk[d][4 * g + 3] * sc);
                v2.x = pack_bf16x2(dv[d][4 * g + 0], dv[d][4 * g + 1]);
                v2.y = pack_bf16x2(dv[d][4 * g + 2], dv[d][4 * g + 3]);
                *reinterpret_cast<uint2 *>(krow_k + d * 32 + 8 * g + 4 * hl) = a;
                *reinterpret_cast<uint2 *>(krow_v + d * 32 + 8 * g + 4 * hl) = v2;
            }
    }
}

template <int BETA, int D>
static hipError_t launch_bwd_t(const BwdParams &p, hipStream_t s)
{
    using Sh = BwShape<BETA, D>;
    const int64_t grid = (int64_t)p.B * p.H * p.nB;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((bwd_dq_kernel<BETA, D>), dim3((unsigned)grid), dim3(Sh::NT), 0, s, p);
    hipLaunchKernelGGL((bwd_dkdv_kernel<BETA, D>), dim3((unsigned)grid), dim3(Sh::NT), (size_t)p.nB * sizeof(int), s,
                       p);
    return hipGetLastError();
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
