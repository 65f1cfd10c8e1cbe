// Block scores for content-driven selection on gfx950.
//
// MEANPOOL_PROJ (multimodal-DiT write-up, section 2.2): each block of Q and
// K is mean-pooled to one vector and projected by one small linear map W
// [D][r]; the score of (query block i, key block j) is the dot product of
// the two projected vectors.  Pool + projection is one streaming pass over
// Q and K (HBM-bound: every byte read once, 16-byte coalesced loads); the
// score product is a tiny nB x nB x r kernel.
//
// EXACT_AVGPOOL (SparseD notes, isolated selection): the block average of
// the post-softmax attention map over all N keys, computed per query block
// without materialising A.  One pass over the key blocks: for every query
// token t and key block j the kernel forms the block log-sum-exp
//   l_tj = log2 sum_{s in j} 2^{c z_ts}   (c = scale * log2 e)
// with QK^T on bf16 MFMA, keeps a running log-sum-exp over j, and parks
// l_tj in a per-workgroup scratch slot.  Once the row's full log-sum-exp
// L_t is known, S_ij = 1/(n_i n_j) sum_t 2^{l_tj - L_t}.  The QK^T product is
// therefore done once, not twice.
#include "common.h"
#include "internal.h"

namespace bsa {

// ---------------------------------------------------------------------------
// mean-pool + projection: grid (B*H*nB, 2), 256 threads
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void pool_proj_kernel(const PoolParams p, int beta)
{
    constexpr int CH = D / 8;          // 16-byte chunks per row
    constexpr int RS = 256 / CH;       // row slots
    __shared__ float red[RS][D];
    __shared__ float mean[D];

    const int tid = threadIdx.x;
    const int item = blockIdx.x;
    const int which = blockIdx.y;
    const int bh = item / p.nB, i = item - bh * p.nB;
    const int b = bh / p.H, hh = bh - b * p.H;
    const Tensor4 X = p.x[which];
    const uint16_t *base = X.p + b * X.sb + hh * X.sh;
    const int cc = tid % CH, rs = tid / CH;
    const int t0 = i * beta;
    const int n_i = min(beta, p.N - t0);

    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    for (int t = rs; t < n_i; t += RS) {
        const uint4 u = ld_g16(base + (int64_t)(t0 + t) * X.sn + cc * 8);
        const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] += __uint_as_float(wd[e] << 16);
            acc[2 * e + 1] += __uint_as_float(wd[e] & 0xFFFF0000u);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[rs][cc * 8 + e] = acc[e];
    __syncthreads();
    if (tid < D) {
        float s = 0.f;
        for (int r = 0; r < RS; ++r) s += red[r][tid];
        mean[tid] = s / (float)n_i;
    }
    __syncthreads();
    if (tid < p.r) {
        float a = 0.f;
        for (int d = 0; d < D; ++d) a = __builtin_fmaf(p.w[d * p.r + tid], mean[d], a);
        const int64_t rows = (int64_t)p.B * p.H * p.nB;
        p.proj[((int64_t)which * rows + item) * p.r + tid] = a;
    }
}

hipError_t launch_pool_proj(const PoolParams &p, int block, int D, hipStream_t s)
{
    const int64_t items = (int64_t)p.B * p.H * p.nB;
    if (items == 0) return hipSuccess;
    if (D == 128)
        hipLaunchKernelGGL(pool_proj_kernel<128>, dim3((unsigned)items, 2), dim3(256), 0, s, p, block);
    else if (D == 64)
        hipLaunchKernelGGL(pool_proj_kernel<64>, dim3((unsigned)items, 2), dim3(256), 0, s, p, block);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// S_ij = p_i . p'_j : one workgroup per query-block row
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void scores_kernel(const ScoreParams p)
{
    __shared__ float pq[64];
    const int item = blockIdx.x;
    const int bh = item / p.nB;
    const int64_t rows = (int64_t)p.BH * p.nB;
    if (threadIdx.x < p.r) pq[threadIdx.x] = p.proj[(int64_t)item * p.r + threadIdx.x];
    __syncthreads();
    for (int j = threadIdx.x; j < p.nB; j += blockDim.x) {
        const float *pk = p.proj + (rows + (int64_t)bh * p.nB + j) * p.r;
        float s = 0.f;
        for (int m = 0; m < p.r; ++m) s = __builtin_fmaf(pq[m], pk[m], s);
        p.S[(int64_t)item * p.nB + j] = s;
    }
}

hipError_t launch_scores(const ScoreParams &p, hipStream_t s)
{
    const int64_t items = (int64_t)p.BH * p.nB;
    if (items == 0) return hipSuccess;
    hipLaunchKernelGGL(scores_kernel, dim3((unsigned)items), dim3(256), 0, s, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// exact avgpool scores: persistent workgroups, one query block per item
// ---------------------------------------------------------------------------
template <int BETA, int D>
struct ExactShape {
    static constexpr int NW = BETA / 32;            // waves, 32 query rows each
    static constexpr int NT = NW * 64;
    static constexpr int SUB = BETA / 64;           // 64-key sub-tiles per key block
    static constexpr int QS = D / 16;               // k-steps over d
    static constexpr int KCH = D / 8;               // 16-byte chunks per K row
    static constexpr int TILE = 64 * D;             // bf16 elements of one 64-key K tile
    static constexpr int DMA = 64 * KCH / NT;       // 16-byte copies per lane per tile
    static constexpr int ROWS_PER_COPY = NT / KCH;
    static constexpr bool UNIFORM_COPY = ROWS_PER_COPY % 16 == 0;
    static_assert(64 * KCH % NT == 0, "tile split");
};

// Copy one 64-key K tile (rows from key k0) straight into LDS; lane l of
// copy x writes slot (x*NW + wave)*64 + l = (row, chunk XOR the row's
// swizzle).  A partial tile repeats its last key (those scores are masked).
template <int BETA, int D>
__device__ __forceinline__ void exact_load_k(uint16_t *__restrict__ dst, __amdgpu_buffer_rsrc_t rs,
                                             int64_t sn, uint32_t off0, int N, int k0, int wv, int lane)
{
    using Sh = ExactShape<BETA, D>;
    const int rows = N - k0;
    const uint32_t so = (uint32_t)((int64_t)k0 * sn * 2);
    const uint32_t step = (uint32_t)((int64_t)Sh::ROWS_PER_COPY * sn * 2);
#pragma unroll
    for (int x = 0; x < Sh::DMA; ++x) {
        uint32_t o = off0, sx = so + x * step;
        if (rows < 64 || !Sh::UNIFORM_COPY) {
            const int slot = (x * Sh::NW + wv) * 64 + lane;
            const int r = slot / Sh::KCH, ps = slot % Sh::KCH;
            o = (uint32_t)(min(r, rows - 1) * sn * 2 + ((ps ^ kswz<D>(r)) * 16));
            sx = so;
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(dst + (x * Sh::NW + wv) * 64 * 8), 16, o,
                                                 sx, 0, 0);
    }
}

// Per-lane state: the 32 queries' Q^T fragments, the running log2-sum-exp
// over key blocks (M, L), the current key block's partial (bm, bl), and
// the lane's constant LDS / global offsets.
template <int BETA, int D>
struct ExactState {
    bf16x8 qf[ExactShape<BETA, D>::QS];
    float M, L, bm, bl;
    uint32_t kread[ExactShape<BETA, D>::QS];
    uint32_t kdma;
};

// One step: copy the next sub-tile into the other buffer, then fold the
// current 64 keys (starting at k0) into the block partial; at the end of a
// key block, park its log2-sum-exp in the scratch slot and update (M, L).
template <int BETA, int D>
__device__ __forceinline__ void exact_step(const uint16_t *__restrict__ Kc, uint16_t *__restrict__ Kn,
                                           bool prefetch, int k0n, int k0, bool first_half, bool last_half,
                                           int j, __amdgpu_buffer_rsrc_t krs, const ExactParams &p,
                                           float *slot, int wv, int lane, ExactState<BETA, D> &st)
{
    using Sh = ExactShape<BETA, D>;
    if (prefetch) exact_load_k<BETA, D>(Kn, krs, p.k.sn, st.kdma, p.N, k0n, wv, lane);
    const int hl = lane >> 5, n = lane & 31;
    const float c = p.scale_log2;
    f32x16 sacc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.f;
#pragma unroll
        for (int s = 0; s < Sh::QS; ++s) {
            const bf16x8 a = *lds_at<bf16x8>(Kc + kt * 32 * D, st.kread[s]);
            sacc[kt] = mfma32x32x16(a, st.qf[s], sacc[kt]);
        }
    }
    if (k0 + 64 > p.N) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = k0 + kt * 32 + perm_row(8 * (r >> 2) + 4 * hl + (r & 3));
                if (key >= p.N) sacc[kt][r] = -INFINITY;
            }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kt][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * c;   // at least one key of a tile exists
    float ls = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) ls += fast_exp2(__builtin_fmaf(sacc[kt][r], c, -mx));
    ls += __shfl_xor(ls, 32, 64);
    if (first_half) {
        st.bm = mx;
        st.bl = ls;
    } else {
        const float m2 = fmaxf(st.bm, mx);
        st.bl = st.bl * fast_exp2(st.bm - m2) + ls * fast_exp2(mx - m2);
        st.bm = m2;
    }
    if (last_half) {
        const float lj = st.bm + __log2f(st.bl);   // block log2-sum-exp of this token
        const float Mn = fmaxf(st.M, lj);
        st.L = st.L * ((st.M == Mn) ? 1.f : fast_exp2(st.M - Mn)) + fast_exp2(lj - Mn);
        st.M = Mn;
        if (hl == 0) slot[(int64_t)j * BETA + wv * 32 + n] = lj;
    }
}

template <int BETA, int D>
__global__ __launch_bounds__(BETA / 32 * 64, 4) void exact_scores_kernel(const ExactParams p)
{
    using Sh = ExactShape<BETA, D>;
    __shared__ __attribute__((aligned(16))) uint16_t kbuf[2 * Sh::TILE];
    __shared__ float lse2[BETA];
    uint16_t *const K0 = kbuf, *const K1 = kbuf + Sh::TILE;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hl = lane >> 5;
    const int n = lane & 31;
    float *slot = p.scratch + (int64_t)blockIdx.x * p.nB * BETA;   // [nB][BETA]
    const int64_t items = (int64_t)p.B * p.H * p.nB;
    const int T = p.nB * Sh::SUB;   // 64-key sub-tiles per item

    ExactState<BETA, D> st;
    {
        const int r0 = perm_row(n);
#pragma unroll
        for (int s = 0; s < Sh::QS; ++s)
            st.kread[s] = (uint32_t)(r0 * D * 2 + (((2 * s + hl) ^ kswz<D>(r0)) * 16));
        const int sl = wv * 64 + lane;
        const int r = sl / Sh::KCH, ps = sl % Sh::KCH;
        st.kdma = (uint32_t)(r * p.k.sn * 2 + ((ps ^ kswz<D>(r)) * 16));
    }

    for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
        const int bh = (int)(item / p.nB);
        const int i = (int)(item - (int64_t)bh * p.nB);
        const int b = bh / p.H, hh = bh - b * p.H;
        const uint16_t *qb = p.q.p + b * p.q.sb + hh * p.q.sh;
        const uint16_t *kb = p.k.p + b * p.k.sb + hh * p.k.sh;
        const __amdgpu_buffer_rsrc_t krs =
            buffer_desc(kb, (uint32_t)(((int64_t)(p.N - 1) * p.k.sn + D) * 2));
        const int qrow = i * BETA + wv * 32 + n;
#pragma unroll
        for (int s = 0; s < Sh::QS; ++s) {
            uint4 u = qrow < p.N ? ld_g16(qb + (int64_t)qrow * p.q.sn + 16 * s + 8 * hl) : zero_u4();
            st.qf[s] = as_bf16x8(u);
        }
        st.M = -INFINITY;
        st.L = 0.f;

        __syncthreads();   // the previous item is done with K0 / K1 and lse2
        exact_load_k<BETA, D>(K0, krs, p.k.sn, st.kdma, p.N, 0, wv, lane);
        __syncthreads();   // sub-tile 0 in LDS
        // even sub-tiles in K0, odd in K1 (the loop is unrolled by two)
        for (int t = 0; t < T; t += 2) {
            const int k0 = t * 64;
            exact_step<BETA, D>(K0, K1, t + 1 < T, k0 + 64, k0, (t % Sh::SUB) == 0,
                                (t % Sh::SUB) == Sh::SUB - 1, t / Sh::SUB, krs, p, slot, wv, lane, st);
            __syncthreads();
            if (t + 1 >= T) break;
            exact_step<BETA, D>(K1, K0, t + 2 < T, k0 + 128, k0 + 64, ((t + 1) % Sh::SUB) == 0,
                                ((t + 1) % Sh::SUB) == Sh::SUB - 1, (t + 1) / Sh::SUB, krs, p, slot, wv,
                                lane, st);
            __syncthreads();
        }
        if (hl == 0) lse2[wv * 32 + n] = st.M + __log2f(st.L);
        __syncthreads();   // slot and lse2 complete for this item

        // S_ij = 1/(n_i n_j) sum_t 2^(l_tj - L_t), one wave per key block j
        const int n_i = min(BETA, p.N - i * BETA);
        for (int j = wv; j < p.nB; j += Sh::NW) {
            float sum = 0.f;
#pragma unroll
            for (int t = lane; t < BETA; t += 64)
                if (t < n_i) sum += fast_exp2(slot[(int64_t)j * BETA + t] - lse2[t]);
#pragma unroll
            for (int d = 32; d > 0; d >>= 1) sum += __shfl_xor(sum, d, 64);
            if (lane == 0) {
                const int n_j = min(BETA, p.N - j * BETA);
                p.S[item * p.nB + j] = sum / ((float)n_i * (float)n_j);
            }
        }
    }
}

template <int BETA, int D>
static hipError_t launch_exact_t(const ExactParams &p, int slots, hipStream_t s)
{
    using Sh = ExactShape<BETA, D>;
    auto kern = exact_scores_kernel<BETA, D>;
    hipLaunchKernelGGL(kern, dim3(slots), dim3(Sh::NT), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_exact_scores(const ExactParams &p, int block, int D, int slots, hipStream_t s)
{
    if (slots <= 0) return hipSuccess;
    if (block == 128 && D == 128) return launch_exact_t<128, 128>(p, slots, s);
    if (block == 128 && D == 64) return launch_exact_t<128, 64>(p, slots, s);
    if (block == 64 && D == 128) return launch_exact_t<64, 128>(p, slots, s);
    if (block == 64 && D == 64) return launch_exact_t<64, 64>(p, slots, s);
    return hipErrorInvalidValue;
}

}  // namespace bsa
