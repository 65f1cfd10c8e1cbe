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
    static constexpr int NW = BETA / 32;
    static constexpr int NT = NW * 64;
    static constexpr int KT = BETA / 32;
    static constexpr int QS = D / 16;
    static constexpr int KCH = D / 8;
    static constexpr int K_ITEMS = BETA * KCH;
    static constexpr size_t LDS_BYTES = (size_t)BETA * D * sizeof(uint16_t) + BETA * sizeof(float);
    static_assert(K_ITEMS % NT == 0, "tile split");
};

__device__ __forceinline__ int exact_perm_row(int n)
{
    return (n & ~12) | ((n & 4) << 1) | ((n & 8) >> 1);
}

template <int BETA, int D>
__global__ __launch_bounds__(BETA / 32 * 64) void exact_scores_kernel(const ExactParams p)
{
    using Sh = ExactShape<BETA, D>;
    extern __shared__ __align__(16) uint16_t lds[];
    uint16_t *Ks = lds;
    float *lse2 = reinterpret_cast<float *>(lds + BETA * D);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int hl = lane >> 5;
    const int n = lane & 31;
    const float c = p.scale_log2;
    float *slot = p.scratch + (int64_t)blockIdx.x * p.nB * BETA;   // [nB][BETA]
    const int64_t items = (int64_t)p.B * p.H * p.nB;

    for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
        const int bh = (int)(item / p.nB);
        const int i = (int)(item - (int64_t)bh * p.nB);
        const int b = bh / p.H, hh = bh - b * p.H;
        const uint16_t *qb = p.q.p + b * p.q.sb + hh * p.q.sh;
        const uint16_t *kb = p.k.p + b * p.k.sb + hh * p.k.sh;
        const int tq = wv * 32 + n;           // query token within the block
        const int qrow = i * BETA + tq;

        bf16x8 qf[Sh::QS];
#pragma unroll
        for (int s = 0; s < Sh::QS; ++s) {
            uint4 u = qrow < p.N ? ld_g16(qb + (int64_t)qrow * p.q.sn + 16 * s + 8 * hl) : zero_u4();
            qf[s] = as_bf16x8(u);
        }
        float M = -INFINITY, L = 0.f;     // running log2-sum-exp over key blocks

        for (int j = 0; j < p.nB; ++j) {
            const int key0 = j * BETA;
            __syncthreads();
#pragma unroll
            for (int it = 0; it < Sh::K_ITEMS / Sh::NT; ++it) {
                const int c16 = tid + it * Sh::NT;
                const int r = c16 / Sh::KCH, cc = c16 % Sh::KCH;
                const int key = key0 + r;
                uint4 u = key < p.N ? ld_g16(kb + (int64_t)key * p.k.sn + cc * 8) : zero_u4();
                *reinterpret_cast<uint4 *>(Ks + r * D + ((cc ^ (r % Sh::KCH)) * 8)) = u;
            }
            __syncthreads();

            f32x16 sacc[Sh::KT];
#pragma unroll
            for (int kt = 0; kt < Sh::KT; ++kt) {
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.f;
                const int r = kt * 32 + exact_perm_row(n);
#pragma unroll
                for (int s = 0; s < Sh::QS; ++s) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
                        Ks + r * D + (((2 * s + hl) ^ (r % Sh::KCH)) * 8));
                    sacc[kt] = mfma32x32x16(a, qf[s], sacc[kt]);
                }
            }
            if (key0 + BETA > p.N) {
#pragma unroll
                for (int kt = 0; kt < Sh::KT; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = key0 + kt * 32 + exact_perm_row(8 * (r >> 2) + 4 * hl + (r & 3));
                        if (key >= p.N) sacc[kt][r] = -INFINITY;
                    }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < Sh::KT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kt][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float mb = mx * c;
            float ls = 0.f;
#pragma unroll
            for (int kt = 0; kt < Sh::KT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) ls += fast_exp2(__builtin_fmaf(sacc[kt][r], c, -mb));
            ls += __shfl_xor(ls, 32, 64);
            const float lj = mb + __log2f(ls);        // block log2-sum-exp of this token
            const float Mn = fmaxf(M, lj);
            L = L * ((M == Mn) ? 1.f : fast_exp2(M - Mn)) + fast_exp2(lj - Mn);
            M = Mn;
            if (hl == 0) slot[(int64_t)j * BETA + tq] = lj;
        }
        if (hl == 0) lse2[tq] = M + __log2f(L);
        __syncthreads();   // slot and lse2 complete for this item

        const int n_i = min(BETA, p.N - i * BETA);
        for (int j = wv; j < p.nB; j += Sh::NW) {
            float s = 0.f;
#pragma unroll
            for (int t = lane; t < BETA; t += 64)
                if (t < n_i) s += fast_exp2(slot[(int64_t)j * BETA + t] - lse2[t]);
#pragma unroll
            for (int d = 32; d > 0; d >>= 1) s += __shfl_xor(s, d, 64);
            if (lane == 0) {
                const int n_j = min(BETA, p.N - j * BETA);
                p.S[item * p.nB + j] = s / ((float)n_i * (float)n_j);
            }
        }
    }
}

template <int BETA, int D>
static hipError_t launch_exact_t(const ExactParams &p, int slots, hipStream_t s)
{
    using Sh = ExactShape<BETA, D>;
    auto kern = exact_scores_kernel<BETA, D>;
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         (int)Sh::LDS_BYTES);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(kern, dim3(slots), dim3(Sh::NT), Sh::LDS_BYTES, s, p);
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
