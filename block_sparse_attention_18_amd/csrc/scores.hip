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
// with QK^T on bf16 MFMA.  Sums are kept against a per-query reference that
// only moves when a score exceeds it by about 2^6 (log2 units); l_tj is
// parked in a per-workgroup scratch slot and the running total gives the
// row's log-sum-exp L_t.  Then S_ij = 1/(n_i n_j) sum_t 2^{l_tj - L_t}.  The
// QK^T product is done once, not twice; the exp2 / sum work of one 32-key
// half runs between the MFMAs of the next half, four waves per SIMD.
#include "common.h"
#include "internal.h"

namespace bsa {

// ---------------------------------------------------------------------------
// mean-pool + projection: grid (B*H*nB, 2), 256 threads, one block of Q or K
// per workgroup.  Every 16-byte load of the block is issued first (BETA * D
// / 2048 per thread: 8 at block 128, D 128), and the thread's slice of W is
// fetched while they are in flight.  The column sums are reduced across the
// wavefront's row slots with lane shuffles, across the four wavefronts
// through LDS; the projection is split over all 256 threads (output m =
// tid / 8, every eighth dimension), so the tail after the last load is a
// few dozen instructions.
// ---------------------------------------------------------------------------
template <int BETA, int D>
__global__ __launch_bounds__(256) void pool_proj_kernel(const PoolParams p)
{
    constexpr int CH = D / 8;          // 16-byte chunks per row
    constexpr int RS = 256 / CH;       // row slots
    constexpr int IT = BETA / RS;      // rows per thread
    constexpr int DP = D / 8;          // dimensions per projection thread
    static_assert(BETA % RS == 0 && CH <= 64, "rows split evenly");
    __shared__ float red[4][D];
    __shared__ float mean[D];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int item = blockIdx.x;
    const int which = blockIdx.y;
    const int bh = item / p.nB, i = item - bh * p.nB;
    const int b = bh / p.H, hh = bh - b * p.H;
    const Tensor4 X = p.x[which];
    const uint16_t *base = X.p + b * X.sb + hh * X.sh;
    const int cc = tid % CH, rs = tid / CH;
    const int t0 = i * BETA;
    const int n_i = min(BETA, p.N - t0);

    // rows past the end of a ragged last block re-read its last row (no
    // branch around a load, so none waits for another) and are zeroed after
    uint4 u[IT];
#pragma unroll
    for (int a = 0; a < IT; ++a) {
        const int t = min(rs + a * RS, n_i - 1);
        u[a] = ld_g16(base + (int64_t)(t0 + t) * X.sn + cc * 8);
    }
    const int m = tid >> 3, part = tid & 7;
    float wm[DP];
    const int mc = min(m, p.r - 1);          // lanes of outputs past r load a valid column, zeroed below
#pragma unroll
    for (int t = 0; t < DP; ++t) wm[t] = p.w[(part + 8 * t) * p.r + mc];
    // keep every load above this point: none may be issued after the first wait
    __builtin_amdgcn_sched_barrier(0);

    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
    for (int a = 0; a < IT; ++a) {
        const uint32_t live = rs + a * RS < n_i ? 0xFFFFFFFFu : 0u;
        const uint32_t wd[4] = {u[a].x & live, u[a].y & live, u[a].z & live, u[a].w & live};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] += __uint_as_float(wd[e] << 16);
            acc[2 * e + 1] += __uint_as_float(wd[e] & 0xFFFF0000u);
        }
    }
    // lanes l and l ^ x (x >= CH) hold the same columns of other rows
#pragma unroll
    for (int x = CH; x < 64; x <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], x, 64);
    if (lane < CH)
#pragma unroll
        for (int e = 0; e < 8; ++e) red[wv][lane * 8 + e] = acc[e];
    __syncthreads();
    if (tid < D) {
        const float s = (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
        mean[tid] = s / (float)n_i;
        if (p.mean) p.mean[((int64_t)which * p.B * p.H * p.nB + item) * D + tid] = mean[tid];
    }
    __syncthreads();
    const int64_t out = ((int64_t)which * p.B * p.H * p.nB + item) * p.r;
    float a = 0.f;
#pragma unroll
    for (int t = 0; t < DP; ++t) a = __builtin_fmaf(m < p.r ? wm[t] : 0.f, mean[part + 8 * t], a);
    a += __shfl_xor(a, 1, 64);
    a += __shfl_xor(a, 2, 64);
    a += __shfl_xor(a, 4, 64);
    if (part == 0 && m < p.r) p.proj[out + m] = a;
    // outputs 32 .. r-1 (r > 32): a second pass, the eight lanes of an output together
    for (int m2 = m + 32; m2 < p.r; m2 += 32) {
        float c = 0.f;
#pragma unroll
        for (int t = 0; t < DP; ++t) c = __builtin_fmaf(p.w[(part + 8 * t) * p.r + m2], mean[part + 8 * t], c);
        c += __shfl_xor(c, 1, 64);
        c += __shfl_xor(c, 2, 64);
        c += __shfl_xor(c, 4, 64);
        if (part == 0) p.proj[out + m2] = c;
    }
}

// Small blocks (BETA * D <= 8192 elements, 16 KB): one wavefront per block,
// four blocks to a workgroup, so a workgroup still streams 32-64 KB.  W
// [D][r] is staged in LDS once per workgroup (its loads issued first, so the
// wait for them leaves the block's loads in flight); each wavefront sums its
// block in registers, reduces across its row slots with lane shuffles, parks
// the mean in LDS and projects it: lane m + 32 h sums half h of the
// dimensions for output m, one shuffle adds the halves.  No workgroup
// barrier after the one for W.
template <int BETA, int D>
__global__ __launch_bounds__(256) void pool_wave_kernel(const PoolParams p)
{
    constexpr int CH = D / 8;          // 16-byte chunks per row
    constexpr int RSW = 64 / CH;       // row slots per wavefront
    constexpr int IT = BETA / RSW;     // rows per lane
    static_assert(BETA * D <= 8192 && BETA % RSW == 0, "block fits one wavefront");
    extern __shared__ __attribute__((aligned(16))) float smem[];
    float *w_s = smem;                               // [D][r]
    float *mean_s = smem + D * p.r;                  // [4][D]
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t items = (uint32_t)(p.B * p.H * p.nB);
    const uint32_t gidx = blockIdx.x * 4u + (uint32_t)wv;     // over [2][items]
    const bool live = gidx < 2u * items;
    const int which = live && gidx >= items ? 1 : 0;
    const uint32_t item = live ? gidx - (uint32_t)which * items : 0u;
    const uint32_t bh = item / (uint32_t)p.nB;
    const int i = (int)(item - bh * (uint32_t)p.nB);
    const int b = (int)(bh / (uint32_t)p.H), hh = (int)bh - b * p.H;
    const Tensor4 X = p.x[which];
    const uint16_t *base = X.p + b * X.sb + hh * X.sh;
    const int t0 = i * BETA, n_i = min(BETA, p.N - t0);
    const int cc = lane % CH, rs = lane / CH;
    const int nw = D * p.r;

    // W first (every thread a share), then the block: waiting for W leaves
    // the block's loads in flight
    constexpr int WU = 8192 / 256;                   // D * r <= 128 * 64
    float wv_r[WU];
#pragma unroll
    for (int u = 0; u < WU; ++u)
        if (u * 256 < nw) wv_r[u] = p.w[min(u * 256 + tid, nw - 1)];
    uint4 x[IT];
#pragma unroll
    for (int a = 0; a < IT; ++a) {
        const int t = min(rs + a * RSW, n_i - 1);
        x[a] = ld_g16(base + (int64_t)(t0 + t) * X.sn + cc * 8);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < WU; ++u)
        if (u * 256 + tid < nw) w_s[u * 256 + tid] = wv_r[u];
    __syncthreads();
    if (!live) return;

    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
    for (int a = 0; a < IT; ++a) {
        const uint32_t keep = rs + a * RSW < n_i ? 0xFFFFFFFFu : 0u;
        const uint32_t wd[4] = {x[a].x & keep, x[a].y & keep, x[a].z & keep, x[a].w & keep};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] += __uint_as_float(wd[e] << 16);
            acc[2 * e + 1] += __uint_as_float(wd[e] & 0xFFFF0000u);
        }
    }
#pragma unroll
    for (int xm = CH; xm < 64; xm <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], xm, 64);
    float *mean = mean_s + wv * D;
    const float inv_n = 1.0f / (float)n_i;
    const int64_t slot = (int64_t)which * items + item;
    if (lane < CH) {
#pragma unroll
        for (int e = 0; e < 8; ++e) mean[lane * 8 + e] = acc[e] * inv_n;
        if (p.mean)
#pragma unroll
            for (int e = 0; e < 8; ++e) p.mean[slot * D + lane * 8 + e] = acc[e] * inv_n;
    }
    // the wavefront's own LDS writes are visible to its later reads
    const int m0 = lane & 31, h = lane >> 5;
    for (int m = m0; m < p.r; m += 32) {
        float s = 0.f;
#pragma unroll 8
        for (int d = h * (D / 2); d < (h + 1) * (D / 2); ++d) s = __builtin_fmaf(w_s[d * p.r + m], mean[d], s);
        s += __shfl_xor(s, 32, 64);
        if (h == 0) p.proj[slot * p.r + m] = s;
    }
}

hipError_t launch_pool_proj(const PoolParams &p, int block, int D, hipStream_t s)
{
    const int64_t items = (int64_t)p.B * p.H * p.nB;
    if (items == 0) return hipSuccess;
    if (p.r < 1 || p.r > 64 || 2 * items >= (1ll << 31)) return hipErrorInvalidValue;
    const dim3 grid((unsigned)items, 2), thr(256);
    const dim3 wgrid((unsigned)((2 * items + 3) / 4));
    const size_t wsh = (size_t)(D * p.r + 4 * D) * sizeof(float);
    if (block == 128 && D == 128) hipLaunchKernelGGL((pool_proj_kernel<128, 128>), grid, thr, 0, s, p);
    else if (block == 128 && D == 64) hipLaunchKernelGGL((pool_wave_kernel<128, 64>), wgrid, thr, wsh, s, p);
    else if (block == 64 && D == 128) hipLaunchKernelGGL((pool_wave_kernel<64, 128>), wgrid, thr, wsh, s, p);
    else if (block == 64 && D == 64) hipLaunchKernelGGL((pool_wave_kernel<64, 64>), wgrid, thr, wsh, s, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// S_ij = p_i . p'_j: one workgroup (256 threads) per head, QR query blocks
// and CB key blocks.  The projected key blocks are staged in LDS transposed
// ([m][j], rows padded by one word against bank conflicts), the projected
// query blocks beside them (read as 4-wide broadcasts); every load of the
// staging is issued before the first LDS write, so it costs one memory
// round trip.  Thread t computes column t % CB of QR / 2 rows; each row of
// S is written as coalesced runs.
// ---------------------------------------------------------------------------
namespace sc {
constexpr int QR = 16;              // query blocks per workgroup
constexpr int CB = 128;             // key blocks per workgroup
constexpr int RP = 64;              // r padded (r <= 64)
constexpr int KU = CB * RP / 256;   // staged key values per thread at most
constexpr int QU = QR * RP / 256;   // staged query values per thread
}

__global__ __launch_bounds__(256) void scores_kernel(const ScoreParams p)
{
    __shared__ __attribute__((aligned(16))) float pkt[sc::RP][sc::CB + 1];
    __shared__ __attribute__((aligned(16))) float pq[sc::QR][sc::RP];
    const int tid = threadIdx.x;
    const int nB = p.nB, r = p.r, r4 = (r + 3) & ~3;
    const int rt = (nB + sc::QR - 1) / sc::QR, ct = (nB + sc::CB - 1) / sc::CB;
    const int bh = blockIdx.x / (rt * ct), rest = blockIdx.x - bh * (rt * ct);
    const int i0 = (rest / ct) * sc::QR, j0 = (rest % ct) * sc::CB;
    const int nq = min(sc::QR, nB - i0), nj = min(sc::CB, nB - j0), nk = nj * r;
    const int64_t rows = (int64_t)p.BH * nB;
    const float *proj_q = p.proj + ((int64_t)bh * nB + i0) * r;
    const float *proj_k = p.proj + (rows + (int64_t)bh * nB + j0) * r;
    const float inv_r = 1.0f / (float)r;
    // indices past the end re-read a valid element, dropped after
    float vk[sc::KU], vq[sc::QU];
#pragma unroll
    for (int u = 0; u < sc::QU; ++u) {
        const int x = u * 256 + tid, q = x / sc::RP, m = x % sc::RP;
        vq[u] = proj_q[(q < nq && m < r) ? q * r + m : 0];
    }
#pragma unroll
    for (int u = 0; u < sc::KU; ++u) vk[u] = proj_k[min(u * 256 + tid, nk - 1)];
    // the loads stay here, not sunk into the guarded writes below
#pragma unroll
    for (int u = 0; u < sc::KU; ++u) asm volatile("" ::"v"(vk[u]));
#pragma unroll
    for (int u = 0; u < sc::KU; ++u) {
        const int x = u * 256 + tid;
        const int j = div_small(x, inv_r), m = x - j * r;
        if (x < nk) pkt[m][j] = vk[u];
    }
    for (int x = tid; x < (r4 - r) * sc::CB; x += 256) pkt[r + x / sc::CB][x % sc::CB] = 0.f;
#pragma unroll
    for (int u = 0; u < sc::QU; ++u) {
        const int x = u * 256 + tid, q = x / sc::RP, m = x % sc::RP;
        pq[q][m] = (q < nq && m < r) ? vq[u] : 0.f;
    }
    __syncthreads();
    const int col = tid % sc::CB, q0 = (tid / sc::CB) * (sc::QR / 2);
    if (col >= nj) return;
    float acc[sc::QR / 2];
#pragma unroll
    for (int q = 0; q < sc::QR / 2; ++q) acc[q] = 0.f;
    for (int m = 0; m < r4; m += 4) {
        const float k0 = pkt[m][col], k1 = pkt[m + 1][col], k2 = pkt[m + 2][col], k3 = pkt[m + 3][col];
#pragma unroll
        for (int q = 0; q < sc::QR / 2; ++q) {
            const float4 v = *reinterpret_cast<const float4 *>(&pq[q0 + q][m]);
            acc[q] = __builtin_fmaf(v.x, k0, acc[q]);
            acc[q] = __builtin_fmaf(v.y, k1, acc[q]);
            acc[q] = __builtin_fmaf(v.z, k2, acc[q]);
            acc[q] = __builtin_fmaf(v.w, k3, acc[q]);
        }
    }
    float *out = p.S + ((int64_t)bh * nB + i0 + q0) * nB + j0 + col;
#pragma unroll
    for (int q = 0; q < sc::QR / 2; ++q)
        if (q0 + q < nq) out[(int64_t)q * nB] = acc[q];
}

hipError_t launch_scores(const ScoreParams &p, hipStream_t s)
{
    if ((int64_t)p.BH * p.nB == 0) return hipSuccess;
    if (p.r < 1 || p.r > sc::RP) return hipErrorInvalidValue;
    const int64_t wgs = (int64_t)((p.nB + sc::QR - 1) / sc::QR) * ((p.nB + sc::CB - 1) / sc::CB) * p.BH;
    if (wgs >= (1ll << 31)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(scores_kernel, dim3((unsigned)wgs), dim3(256), 0, s, p);
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
// swizzle).  A partial tile repeats its last key (those scores are masked);
// a full tile is copy 0 moved by x * ROWS_PER_COPY rows.
template <int BETA, int D>
__device__ __forceinline__ void exact_load_k(uint16_t *__restrict__ dst, __amdgpu_buffer_rsrc_t rs,
                                             int64_t sn, uint32_t off0, int N, int k0, int wv, int lane)
{
    using Sh = ExactShape<BETA, D>;
    const int rows = N - k0;
    const uint32_t so = (uint32_t)((int64_t)k0 * sn * 2);
    if (Sh::UNIFORM_COPY && rows >= 64) {
        const uint32_t step = (uint32_t)((int64_t)Sh::ROWS_PER_COPY * sn * 2);
#pragma unroll
        for (int x = 0; x < Sh::DMA; ++x)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(dst + (x * Sh::NW + wv) * 64 * 8), 16,
                                                     off0, so + x * step, 0, 0);
        return;
    }
#pragma unroll
    for (int x = 0; x < Sh::DMA; ++x) {
        const int slot = (x * Sh::NW + wv) * 64 + lane;
        const int r = slot / Sh::KCH, ps = slot % Sh::KCH;
        const uint32_t o = (uint32_t)(min(r, rows - 1) * sn * 2 + ((ps ^ kswz<D>(r)) * 16));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(dst + (x * Sh::NW + wv) * 64 * 8), 16, o, so,
                                                 0, 0);
    }
}

// Per-lane state: the 32 queries' Q^T fragments; the reference max m_ref
// (log2 domain, equal in both lane halves of a query); bl, the current key
// block's sum of 2^(c z - m_ref) over this lane's keys; L, the sum over the
// finished key blocks (both halves), relative to m_ref; the lane's constant
// LDS / global offsets.
template <int BETA, int D>
struct ExactState {
    bf16x8 qf[ExactShape<BETA, D>::QS];
    float m_ref, bl, L;
    uint32_t kread;              // K operand of k-step 0; k-step s: ^ KSTEP * s
    uint32_t kdma;
};

// S^T of one 32-key half (kt) of a 64-key sub-tile: 32 keys x 32 queries.
template <int BETA, int D>
__device__ __forceinline__ void exact_qk_half(const uint16_t *__restrict__ Kc, int kt, const ExactState<BETA, D> &st,
                                              f32x16 &acc)
{
    using Sh = ExactShape<BETA, D>;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int s = 0; s < Sh::QS; ++s) {
        const bf16x8 a = *lds_at<bf16x8>(Kc + kt * 32 * D, st.kread ^ (KSTEP * s));
        acc = mfma32x32x16(a, st.qf[s], acc);
    }
}

// Fold the scores of one 32-key half into the current block's sum.  The
// common path has no max: it sums 2^(c z - m_ref) against the current
// reference and returns that partial; exact_fold_fix, taken (wave-uniform)
// when some lane's partial exceeds 2^64 or overflowed, recomputes the half
// against the exact max and rescales the running sums.  The reference thus
// only moves when a score exceeds it by about 2^6 log2 units, and the sums
// stay far from the fp32 range.
template <int BETA, int D>
__device__ __forceinline__ float exact_fold_sum(const f32x16 &sv, float c, const ExactState<BETA, D> &st)
{
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
        s0 += fast_exp2(__builtin_fmaf(sv[r], c, -st.m_ref));
        s1 += fast_exp2(__builtin_fmaf(sv[r + 1], c, -st.m_ref));
    }
    return s0 + s1;
}

constexpr float kExactBig = 18446744073709551616.0f;   // 2^64

// One region with an explicit instruction order: S^T of half kt of the
// sub-tile in Kc into acc, and the fold sum of the scores sv of another half.
// Slot s issues the K read of k-step s+2, the MFMA of k-step s, and the
// fma / exp2 / add of scores 2s and 2s+1; a full scheduling barrier between
// slots keeps the order, so the vector work runs under the MFMAs.
template <int BETA, int D>
__device__ __forceinline__ float exact_region(const uint16_t *__restrict__ Kc, int kt, const ExactState<BETA, D> &st,
                                              f32x16 &acc, const f32x16 &sv, float c)
{
    using Sh = ExactShape<BETA, D>;
    static_assert(Sh::QS == 8 || Sh::QS == 4, "k-steps");
    constexpr int PER = 16 / Sh::QS;   // scores folded per slot
    const uint16_t *kt_base = Kc + kt * 32 * D;
    bf16x8 a[Sh::QS];
    a[0] = *lds_at<bf16x8>(kt_base, st.kread);
    a[1] = *lds_at<bf16x8>(kt_base, st.kread ^ KSTEP);
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    float s0 = 0.f, s1 = 0.f;
    const float m = st.m_ref;
#pragma unroll
    for (int s = 0; s < Sh::QS; ++s) {
        if (s + 2 < Sh::QS) a[s + 2] = *lds_at<bf16x8>(kt_base, st.kread ^ (KSTEP * (s + 2)));
        acc = mfma32x32x16(a[s], st.qf[s], acc);
#pragma unroll
        for (int e = 0; e < PER; e += 2) {
            s0 += fast_exp2(__builtin_fmaf(sv[PER * s + e], c, -m));
            s1 += fast_exp2(__builtin_fmaf(sv[PER * s + e + 1], c, -m));
        }
        // pin the partial sums to this slot: pure arithmetic is otherwise
        // free to move past the scheduling barrier towards its only use
        asm volatile("" ::"v"(s0), "v"(s1));
        __builtin_amdgcn_sched_barrier(0);
    }
    return s0 + s1;
}


template <int BETA, int D>
__device__ __forceinline__ void exact_fold_commit(float part, const f32x16 &sv, float c, ExactState<BETA, D> &st)
{
    if (__ballot(!(part <= kExactBig))) {
        float m = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) m = fmaxf(m, sv[r]);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
        const float mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * c;
        const float m_new = fmaxf(st.m_ref, mx);
        const float alpha = fast_exp2(st.m_ref - m_new);
        st.bl *= alpha;
        st.L *= alpha;
        st.m_ref = m_new;
        part = exact_fold_sum<BETA, D>(sv, c, st);
    }
    st.bl += part;
}

// End of key block j: its log2-sum-exp l_tj = m_ref + log2(bl over both
// halves) is parked in the scratch slot and the block joins L.
template <int BETA, int D>
__device__ __forceinline__ void exact_finish_block(int j, float *slot, int wv, int lane, ExactState<BETA, D> &st)
{
    const float bt = half_sum(st.bl);
    st.L += bt;
    st.bl = 0.f;
    if ((lane >> 5) == 0) slot[(int64_t)j * BETA + wv * 32 + (lane & 31)] = st.m_ref + __log2f(bt);
}

// Keys of half kt of the sub-tile at k0 that lie past N become -inf.
__device__ __forceinline__ void exact_mask_half(int k0, int kt, int N, int lane, f32x16 &sv)
{
    if (k0 + 64 > N) {
        const int lim = N - k0 - 32 * kt - 8 * (lane >> 5);
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (koff(r) >= lim) sv[r] = -INFINITY;
    }
}

// Step t over the 64-key sub-tile in Kc (keys from k0), pipelined at
// 32-key granularity: region 1 computes S^T of half 0 of t while folding
// half 1 of t-1 (sb, carried over from the previous step); region 2
// computes S^T of half 1 of t (into sb) while folding half 0 of t (sa).
// Both halves' scores are 16 registers each.  Masks and the end of a key
// block are handled between the regions, so no branch splits a region.
template <int BETA, int D>
__device__ __forceinline__ void exact_step(const uint16_t *__restrict__ Kc, uint16_t *__restrict__ Kn, bool load_k,
                                           int k0_k, int k0, bool finish_prev, int j_prev,
                                           __amdgpu_buffer_rsrc_t krs, const ExactParams &p, float *slot, int wv,
                                           int lane, ExactState<BETA, D> &st, f32x16 &sa, f32x16 &sb)
{
    const float c = p.scale_log2;
    if (load_k) exact_load_k<BETA, D>(Kn, krs, p.k.sn, st.kdma, p.N, k0_k, wv, lane);
    exact_mask_half(k0 - 64, 1, p.N, lane, sb);
    float part = exact_region<BETA, D>(Kc, 0, st, sa, sb, c);
    exact_fold_commit<BETA, D>(part, sb, c, st);
    if (finish_prev) exact_finish_block<BETA, D>(j_prev, slot, wv, lane, st);
    exact_mask_half(k0, 0, p.N, lane, sa);
    part = exact_region<BETA, D>(Kc, 1, st, sb, sa, c);
    exact_fold_commit<BETA, D>(part, sa, c, st);
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
        st.kread = (uint32_t)(r0 * D * 2 + ((hl ^ kswz<D>(r0)) * 16));
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
        st.m_ref = -1.0e30f;   // finite: the first sub-tile moves it with alpha = 0
        st.bl = 0.f;
        st.L = 0.f;

        __syncthreads();   // the previous item is done with K0 / K1 and lse2
        exact_load_k<BETA, D>(K0, krs, p.k.sn, st.kdma, p.N, 0, wv, lane);
        wait_tile_copies();
        __syncthreads();   // K(0) in LDS
        // sub-tile t in K[t&1]; step t copies K(t+1) into the other buffer.
        // Step 0 (no previous half to fold) is peeled.
        f32x16 sa, sb;
        if (T > 1) exact_load_k<BETA, D>(K1, krs, p.k.sn, st.kdma, p.N, 64, wv, lane);
        exact_qk_half<BETA, D>(K0, 0, st, sa);
        exact_mask_half(0, 0, p.N, lane, sa);
        exact_qk_half<BETA, D>(K0, 1, st, sb);
        exact_fold_commit<BETA, D>(exact_fold_sum<BETA, D>(sa, p.scale_log2, st), sa, p.scale_log2, st);
        wait_tile_copies();
        __syncthreads();
        for (int t = 1; t < T; t += 2) {
            exact_step<BETA, D>(K1, K0, t + 1 < T, (t + 1) * 64, t * 64, ((t - 1) % Sh::SUB) == Sh::SUB - 1,
                                (t - 1) / Sh::SUB, krs, p, slot, wv, lane, st, sa, sb);
            wait_tile_copies();
            __syncthreads();
            if (t + 1 >= T) break;
            exact_step<BETA, D>(K0, K1, t + 2 < T, (t + 2) * 64, (t + 1) * 64, (t % Sh::SUB) == Sh::SUB - 1,
                                t / Sh::SUB, krs, p, slot, wv, lane, st, sa, sb);
            wait_tile_copies();
            __syncthreads();
        }
        // half 1 of the last sub-tile, then the last key block
        exact_mask_half((T - 1) * 64, 1, p.N, lane, sb);
        exact_fold_commit<BETA, D>(exact_fold_sum<BETA, D>(sb, p.scale_log2, st), sb, p.scale_log2, st);
        exact_finish_block<BETA, D>(p.nB - 1, slot, wv, lane, st);
        if (hl == 0) lse2[wv * 32 + n] = st.m_ref + __log2f(st.L);
        __syncthreads();   // slot and lse2 complete for this item

        // S_ij = 1/(n_i n_j) sum_t 2^(l_tj - L_t), one wave per key block j
        const int n_i = min(BETA, p.N - i * BETA);
        for (int j = wv; j < p.nB; j += Sh::NW) {
            float sum = 0.f;
#pragma unroll
            for (int tq = lane; tq < BETA; tq += 64)
                if (tq < n_i) sum += fast_exp2(slot[(int64_t)j * BETA + tq] - lse2[tq]);
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
