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
    static constexpr int SUB = BETA / 64;         // 64-key sub-tiles per block
    static constexpr int QS = D / 16;             // k-steps of S^T over d
    static constexpr int DT = D / 32;             // 32-row d tiles of O^T
    static constexpr int KCH = D / 8;             // 16-byte chunks per K / V row
    static constexpr int TILE = 64 * D;           // bf16 elements of one 64-key K or V tile
    static constexpr int DMA = 64 * KCH / NT;     // 16-byte loads per lane per tile
    static constexpr int ROWS_PER_COPY = NT / KCH; // tile rows covered by one copy of all lanes
    static_assert(64 * KCH % NT == 0, "tile split");
    // when the swizzles ignore the row bits a copy step changes, the per-lane
    // source offset of copy x is that of copy 0 plus x rows-per-copy rows
    static constexpr bool UNIFORM_COPY = ROWS_PER_COPY % 16 == 0;
};

// Lazy rescaling: the running reference max only moves when a sub-tile's max
// exceeds it by more than this (log2 units), so the O rescale is skipped for
// most sub-tiles; probabilities stay below 2^8 relative to the reference.
constexpr float kRescaleSlack = 8.0f;

// Per-lane state of one wave: its 32 queries' Q^T fragments, O^T
// accumulators, online-softmax statistics, and the lane's LDS / global byte
// offsets, which are the same for every sub-tile.
template <int BETA, int D>
struct WaveState {
    using Sh = FwdShape<BETA, D>;
    bf16x8 qf[Sh::QS];
    f32x16 oacc[Sh::DT];
    float m_run;                 // reference max, log2-scaled domain
    float l_run;                 // running sum over this lane's keys
    uint32_t kread[Sh::QS];      // K operand of k-step s, key sub-tile 0 (bytes in a tile)
    uint32_t vread[Sh::DT];      // V^T operand of d tile d, keys 0..3 (bytes in a tile)
    uint32_t kdma, vdma;         // source offset of the lane's first 16-byte copy of a tile
};

template <int BETA, int D>
__device__ __forceinline__ void init_offsets(WaveState<BETA, D> &st, const FwdParams &p, int wv, int lane)
{
    using Sh = FwdShape<BETA, D>;
    const int hl = lane >> 5, n = lane & 31;
    const int r0 = perm_row(n);
#pragma unroll
    for (int s = 0; s < Sh::QS; ++s)
        st.kread[s] = (uint32_t)(r0 * D * 2 + (((2 * s + hl) ^ kswz<D>(r0)) * 16));
    // transposing V reads: lane 4r + c of each 16-lane group names row r,
    // columns 4c..4c+3; lane x of the group receives column x of rows 0..3
    const int G = lane >> 4, jl = lane & 15;
    const int vr0 = 8 * (G >> 1) + (jl >> 2);
#pragma unroll
    for (int d = 0; d < Sh::DT; ++d) {
        const int dc = 32 * d + 16 * (G & 1) + 4 * (jl & 3);
        st.vread[d] = (uint32_t)(vr0 * D * 2 + (((dc >> 3) ^ vswz<D>(vr0)) * 16) + (dc & 4) * 2);
    }
    // copy x of a lane covers tile row r0 + x * ROWS_PER_COPY with the same
    // chunk: the swizzles only use row bits that the step leaves unchanged
    const int slot = wv * 64 + lane;
    const int r = slot / Sh::KCH, ps = slot % Sh::KCH;
    st.kdma = (uint32_t)(r * p.k.sn * 2 + ((ps ^ kswz<D>(r)) * 16));
    st.vdma = (uint32_t)(r * p.v.sn * 2 + ((ps ^ vswz<D>(r)) * 16));
}


// S^T (64 keys x 32 queries) of one sub-tile from the K tile Kc.
template <int BETA, int D>
__device__ __forceinline__ void qk_mfma(const uint16_t *__restrict__ Kc, const WaveState<BETA, D> &st,
                                        f32x16 (&sacc)[2])
{
    using Sh = FwdShape<BETA, D>;
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
}

// Keys past N in a partial last tile do not exist: their scores become -inf.
template <int BETA, int D>
__device__ __forceinline__ void mask_tail(int k0, int N, int lane, f32x16 (&sacc)[2])
{
    const int hl = lane >> 5;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = k0 + kt * 32 + perm_row(8 * (r >> 2) + 4 * hl + (r & 3));
            if (key >= N) sacc[kt][r] = -INFINITY;
        }
}

// Online softmax, part 1: the sub-tile's row max (both lane halves) and the
// lazy rescale of the running state when it exceeds the reference by more
// than the slack.
template <int BETA, int D>
__device__ __forceinline__ void softmax_rescale(const f32x16 (&sacc)[2], float c, WaveState<BETA, D> &st)
{
    using Sh = FwdShape<BETA, D>;
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kt][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * c;
    if (__ballot(mx > st.m_run + kRescaleSlack)) {
        const float m_new = fmaxf(st.m_run, mx);
        const float alpha = (st.m_run == m_new) ? 1.f : fast_exp2(st.m_run - m_new);
        st.m_run = m_new;
        st.l_run *= alpha;
#pragma unroll
        for (int d = 0; d < Sh::DT; ++d)
#pragma unroll
            for (int r = 0; r < 16; ++r) st.oacc[d][r] *= alpha;
    }
}

// Online softmax, part 2: probabilities relative to the reference max,
// summed and packed to bf16 as the B operand of each 16-key k-step.
template <int BETA, int D>
__device__ __forceinline__ void softmax_probs(const f32x16 (&sacc)[2], float c, WaveState<BETA, D> &st,
                                              bf16x8 (&pf)[2][2])
{
    const float mr = st.m_run;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            float pr[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pr[e] = fast_exp2(__builtin_fmaf(sacc[kt][8 * u + e], c, -mr));
                st.l_run += pr[e];
            }
            uint4 pk;
            pk.x = pack_bf16x2(pr[0], pr[1]);
            pk.y = pack_bf16x2(pr[2], pr[3]);
            pk.z = pack_bf16x2(pr[4], pr[5]);
            pk.w = pack_bf16x2(pr[6], pr[7]);
            pf[kt][u] = as_bf16x8(pk);
        }
}

// O^T += V^T P^T with the V tile Vc.  V^T operands come from row-major V by
// transposing LDS reads.
template <int BETA, int D>
__device__ __forceinline__ void pv_mfma(const uint16_t *__restrict__ Vc, const bf16x8 (&pf)[2][2],
                                        WaveState<BETA, D> &st)
{
    using Sh = FwdShape<BETA, D>;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
            for (int d = 0; d < Sh::DT; ++d) {
                s16x4 h2[2];
#pragma unroll
                for (int pp = 0; pp < 2; ++pp) {
                    const uint16_t *rowp = Vc + (kt * 32 + 16 * u + 4 * pp) * D;
                    h2[pp] = __builtin_bit_cast(
                        s16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                   (__attribute__((address_space(3))) bf16x4 *)lds_at<uint16_t>(rowp, st.vread[d])));
                }
                const bf16x8 a =
                    __builtin_bit_cast(bf16x8, __builtin_shufflevector(h2[0], h2[1], 0, 1, 2, 3, 4, 5, 6, 7));
                st.oacc[d] = mfma32x32x16(a, pf[kt][u], st.oacc[d]);
            }
        }
    }
}

// Issue the copy of one 64-key tile (K or V rows from key k0) into LDS.
// Lane l of copy x writes the 16-byte slot (x*NW + wave)*64 + l; slot s holds
// tile row s / KCH, chunk (s % KCH) XOR the row's swizzle.  A partial tile
// repeats its last key (those scores are masked).
template <int BETA, int D>
__device__ __forceinline__ void load_tile(uint16_t *__restrict__ dst, __amdgpu_buffer_rsrc_t rs, int64_t sn,
                                          uint32_t off0, bool is_v, const FwdParams &p, int k0, int wv,
                                          int lane)
{
    using Sh = FwdShape<BETA, D>;
    const int rows = p.N - k0;
    const uint32_t so = (uint32_t)((int64_t)k0 * sn * 2);
    const uint32_t step = (uint32_t)((int64_t)Sh::ROWS_PER_COPY * sn * 2);
#pragma unroll
    for (int x = 0; x < Sh::DMA; ++x) {
        uint32_t o = off0, sx = so + x * step;
        if (rows < 64 || !Sh::UNIFORM_COPY) {
            const int slot = (x * Sh::NW + wv) * 64 + lane;
            const int r = slot / Sh::KCH, ps = slot % Sh::KCH;
            const int rr = min(r, rows - 1);
            o = (uint32_t)(rr * sn * 2 + ((ps ^ (is_v ? vswz<D>(r) : kswz<D>(r))) * 16));
            sx = so;
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(dst + (x * Sh::NW + wv) * 64 * 8), 16,
                                                 o, sx, 0, 0);
    }
}

// One pipeline step: start copying the next sub-tile (K and V) into the
// other buffer pair, then fold the current sub-tile (keys k0 .. k0+63 in
// Kc / Vc) into the wave's online softmax.  The restrict-qualified buffers
// tell the compiler that the copies in flight do not alias the tiles read.
template <int BETA, int D>
__device__ __forceinline__ void pipeline_step(
    const uint16_t *__restrict__ Kc, const uint16_t *__restrict__ Vc, uint16_t *__restrict__ Kn,
    uint16_t *__restrict__ Vn, bool prefetch, int k0n, bool compute, int k0,
    __amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs, const FwdParams &p, int wv, int lane,
    WaveState<BETA, D> &st)
{
    if (prefetch) {
        load_tile<BETA, D>(Kn, krs, p.k.sn, st.kdma, false, p, k0n, wv, lane);
        load_tile<BETA, D>(Vn, vrs, p.v.sn, st.vdma, true, p, k0n, wv, lane);
    }
    if (!compute) return;
    const float c = p.scale_log2;
    f32x16 sacc[2];
    qk_mfma<BETA, D>(Kc, st, sacc);
    if (k0 + 64 > p.N) mask_tail<BETA, D>(k0, p.N, lane, sacc);
    softmax_rescale<BETA, D>(sacc, c, st);
    bf16x8 pf[2][2];
    softmax_probs<BETA, D>(sacc, c, st, pf);
    pv_mfma<BETA, D>(Vc, pf, st);
}

template <int BETA, int D>
__global__ __launch_bounds__(BETA / 32 * 64, BETA == 128 ? 2 : 1) void fwd_kernel(const FwdParams p)
{
    using Sh = FwdShape<BETA, D>;
    // two buffers, each a 64-key K tile and a 64-key V tile
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * 2 * Sh::TILE];
    uint16_t *const K0 = smem, *const V0 = smem + Sh::TILE;
    uint16_t *const K1 = smem + 2 * Sh::TILE, *const V1 = smem + 3 * Sh::TILE;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hl = lane >> 5;           // lane half
    const int n = lane & 31;

    const int BH = p.B * p.H;
    int i, bh, chunk = 0, chunks = 1, rank = -1;
    if (p.items) {   // one item of the long-row splitting work list
        if ((int)blockIdx.x >= p.counts[0]) return;
        const int4 it = p.items[blockIdx.x];
        bh = it.x / p.nB;
        i = it.x - bh * p.nB;
        chunk = it.y;
        chunks = it.z;
        rank = it.w;
    } else {         // query-block-major: every head's text rows first
        i = blockIdx.x / BH;
        bh = blockIdx.x - i * BH;
    }
    const int b = bh / p.H;
    const int hh = bh - b * p.H;
    if ((p.skip_bits[hh >> 5] >> (hh & 31)) & 1u) return;

    const int64_t row = (int64_t)bh * p.nB + i;
    int e0 = p.row_ptr[row];
    int e1 = p.row_ptr[row + 1];
    if (chunks > 1) {   // this workgroup takes one contiguous chunk of the row
        const int len = e1 > e0 ? e1 - e0 : 0;
        const int cs = (len + chunks - 1) / chunks;
        const int lo = e0 + min(len, chunk * cs);
        e1 = e0 + min(len, (chunk + 1) * cs);
        e0 = lo;
    }
    const int T = (e1 > e0 ? e1 - e0 : 0) * Sh::SUB;   // 64-key sub-tiles to visit

    const uint16_t *qb = p.q.p + b * p.q.sb + hh * p.q.sh;
    const uint16_t *kb = p.k.p + b * p.k.sb + hh * p.k.sh;
    const uint16_t *vb = p.v.p + b * p.v.sb + hh * p.v.sh;

    WaveState<BETA, D> st;
    // Q^T fragments: lane (hl, n) holds query row n, d = 16 s + 8 hl .. +7.
    const int qrow = i * BETA + wv * 32 + n;
#pragma unroll
    for (int s = 0; s < Sh::QS; ++s) {
        uint4 u = qrow < p.N ? ld_g16(qb + (int64_t)qrow * p.q.sn + 16 * s + 8 * hl) : zero_u4();
        st.qf[s] = as_bf16x8(u);
    }
#pragma unroll
    for (int d = 0; d < Sh::DT; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.oacc[d][r] = 0.f;
    st.m_run = -INFINITY;
    st.l_run = 0.f;
    init_offsets<BETA, D>(st, p, wv, lane);

    const __amdgpu_buffer_rsrc_t krs = buffer_desc(kb, (uint32_t)(((int64_t)(p.N - 1) * p.k.sn + D) * 2));
    const __amdgpu_buffer_rsrc_t vrs = buffer_desc(vb, (uint32_t)(((int64_t)(p.N - 1) * p.v.sn + D) * 2));

    // Sub-tile t: key block col_idx[e0 + t / SUB], keys 64 (t % SUB) .. +63.
    // An entry outside [0, nB) is ignored: its copies read block 0 and its
    // compute is skipped.
    auto tile_key0 = [&](int t, bool &valid) {
        const int j = __builtin_amdgcn_readfirstlane(p.col_idx[e0 + t / Sh::SUB]);
        valid = (unsigned)j < (unsigned)p.nB;
        return (valid ? j * BETA : 0) + 64 * (t % Sh::SUB);
    };

    bool valid = false;
    int k0 = 0;
    if (T > 0) {
        k0 = tile_key0(0, valid);
        load_tile<BETA, D>(K0, krs, p.k.sn, st.kdma, false, p, k0, wv, lane);
        load_tile<BETA, D>(V0, vrs, p.v.sn, st.vdma, true, p, k0, wv, lane);
    }
    __syncthreads();   // Q in registers; sub-tile 0 in LDS

    // Even sub-tiles live in buffer 0, odd ones in buffer 1; the loop is
    // unrolled by two so that every LDS address is a per-lane offset plus a
    // compile-time constant.
    for (int t = 0; t < T; t += 2) {
        bool valid_n = false;
        int k0n = 0;
        bool prefetch = t + 1 < T;
        if (prefetch) k0n = tile_key0(t + 1, valid_n);
        pipeline_step<BETA, D>(K0, V0, K1, V1, prefetch, k0n, valid, k0, krs, vrs, p, wv, lane, st);
        __syncthreads();   // sub-tile t + 1 landed for every wave; buffer 0 is free
        if (!prefetch) break;
        valid = valid_n;
        k0 = k0n;
        prefetch = t + 2 < T;
        if (prefetch) k0n = tile_key0(t + 2, valid_n);
        pipeline_step<BETA, D>(K1, V1, K0, V0, prefetch, k0n, valid, k0, krs, vrs, p, wv, lane, st);
        __syncthreads();   // sub-tile t + 2 landed for every wave; buffer 1 is free
        valid = valid_n;
        k0 = k0n;
    }

    const float l_tot = st.l_run + __shfl_xor(st.l_run, 32, 64);
    if (rank >= 0) {
        // a chunk of a split row: park the unnormalised output and the
        // (reference max, sum) of every query for the combine step
        float *slot = p.partials + ((int64_t)rank * p.max_chunks + chunk) * partial_slot_floats(BETA, D);
        const int tq = wv * 32 + n;
#pragma unroll
        for (int d = 0; d < Sh::DT; ++d)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *reinterpret_cast<float4 *>(slot + tq * D + d * 32 + 8 * g + 4 * hl) =
                    make_float4(st.oacc[d][4 * g + 0], st.oacc[d][4 * g + 1], st.oacc[d][4 * g + 2],
                                st.oacc[d][4 * g + 3]);
        if (hl == 0) {
            slot[BETA * D + tq] = st.m_run;
            slot[BETA * D + BETA + tq] = l_tot;
        }
        return;
    }
    // epilogue: normalise and store O (bf16) and LSE (natural log)
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (qrow < p.N) {
        uint16_t *orow = p.o + b * p.o_sb + hh * p.o_sh + (int64_t)qrow * p.o_sn;
#pragma unroll
        for (int d = 0; d < Sh::DT; ++d)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                uint2 sv;
                sv.x = pack_bf16x2(st.oacc[d][4 * g + 0] * inv, st.oacc[d][4 * g + 1] * inv);
                sv.y = pack_bf16x2(st.oacc[d][4 * g + 2] * inv, st.oacc[d][4 * g + 3] * inv);
                *reinterpret_cast<uint2 *>(orow + d * 32 + 8 * g + 4 * hl) = sv;
            }
        if (p.lse && hl == 0) {
            const float lse = l_tot > 0.f ? (st.m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
            p.lse[(int64_t)bh * p.N + qrow] = lse;
        }
    }
}

template <int BETA, int D>
static hipError_t launch_fwd_t(const FwdParams &p, int64_t grid, hipStream_t s)
{
    using Sh = FwdShape<BETA, D>;
    if (grid == 0) return hipSuccess;
    auto kern = fwd_kernel<BETA, D>;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(Sh::NT), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_forward(const FwdParams &p, int block, int D, int64_t grid, hipStream_t s)
{
    if (block == 128 && D == 128) return launch_fwd_t<128, 128>(p, grid, s);
    if (block == 128 && D == 64) return launch_fwd_t<128, 64>(p, grid, s);
    if (block == 64 && D == 128) return launch_fwd_t<64, 128>(p, grid, s);
    if (block == 64 && D == 64) return launch_fwd_t<64, 64>(p, grid, s);
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Long-row splitting.  One workgroup walks the rows query-block-major (the
// order the forward dispatches them in), cuts every row longer than
// chunk_blocks into min(max_chunks, ceil(len / chunk_blocks)) chunks, ranks
// the split rows (at most max_split_rows; later long rows stay whole) and
// writes the work list.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void plan_kernel(const PlanParams p)
{
    __shared__ int ws_split[16], ws_items[16];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t rows = (int64_t)p.BH * p.nB;
    int carry_split = 0, carry_items = 0;
    for (int64_t base = 0; base < rows; base += 1024) {
        const int64_t g = base + tid;   // query-block-major position
        int len = 0, row = 0;
        if (g < rows) {
            const int i = (int)(g / p.BH), bh = (int)(g % p.BH);
            row = bh * p.nB + i;
            len = max(0, p.row_ptr[row + 1] - p.row_ptr[row]);
        }
        int want = 1;
        const int hh = (int)((g % p.BH) % p.H);
        const bool skip_head = (p.skip_bits[hh >> 5] >> (hh & 31)) & 1u;
        if (g < rows && !skip_head && len > p.chunk_blocks)
            want = min(p.max_chunks, (len + p.chunk_blocks - 1) / p.chunk_blocks);
        int split = (g < rows && want > 1) ? 1 : 0;
        // rank of this split row
        int incl = wave_incl_scan(split);
        if (lane == 63) ws_split[wv] = incl;
        __syncthreads();
        int pre = 0, tot_split = 0;
        for (int x = 0; x < 16; ++x) {
            if (x < wv) pre += ws_split[x];
            tot_split += ws_split[x];
        }
        const int rank = carry_split + pre + incl - split;
        if (split && rank >= p.max_split_rows) {   // pool full: run this row whole
            split = 0;
            want = 1;
        }
        const int items = g < rows ? want : 0;
        int incl2 = wave_incl_scan(items);
        if (lane == 63) ws_items[wv] = incl2;
        __syncthreads();
        int pre2 = 0, tot_items = 0;
        for (int x = 0; x < 16; ++x) {
            if (x < wv) pre2 += ws_items[x];
            tot_items += ws_items[x];
        }
        const int first = carry_items + pre2 + incl2 - items;
        for (int c = 0; c < items; ++c) p.items[first + c] = make_int4(row, c, want, split ? rank : -1);
        if (split) p.split_rows[rank] = make_int2(row, want);
        carry_split += tot_split;
        carry_items += tot_items;
        __syncthreads();
    }
    if (tid == 0) {
        p.counts[0] = carry_items;
        p.counts[1] = (int)min((int64_t)carry_split, p.max_split_rows);
    }
}

hipError_t launch_plan(const PlanParams &p, hipStream_t s)
{
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, s, p);
    return hipGetLastError();
}

// Merge the chunks of one split row: with reference maxima m_c and sums l_c,
// M = max m_c, L = sum l_c 2^(m_c - M), O = sum O_c 2^(m_c - M) / L and
// LSE = (M + log2 L) ln 2.  One workgroup per split row, two threads per
// query (half the head dimension each).
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(const CombineParams p)
{
    constexpr int HALF = D / 2;
    if ((int)blockIdx.x >= p.counts[1]) return;
    const int2 sr = p.split_rows[blockIdx.x];
    const int row = sr.x, chunks = sr.y;
    const int bh = row / p.nB, i = row - bh * p.nB;
    const int b = bh / p.H, hh = bh - b * p.H;
    const int64_t slot_floats = partial_slot_floats(p.block, D);
    const float *base = p.partials + (int64_t)blockIdx.x * p.max_chunks * slot_floats;
    for (int x = threadIdx.x; x < 2 * p.block; x += blockDim.x) {
        const int tq = x >> 1, d0 = (x & 1) * HALF;
        const int t = i * p.block + tq;
        if (t >= p.N) continue;
        float M = -INFINITY;
        for (int c = 0; c < chunks; ++c) M = fmaxf(M, base[c * slot_floats + p.block * D + tq]);
        float L = 0.f;
        float acc[HALF];
#pragma unroll
        for (int d = 0; d < HALF; ++d) acc[d] = 0.f;
        for (int c = 0; c < chunks; ++c) {
            const float *slot = base + c * slot_floats;
            const float mc = slot[p.block * D + tq];
            const float w = (mc == -INFINITY) ? 0.f : fast_exp2(mc - M);
            L += slot[p.block * D + p.block + tq] * w;
            const float *src = slot + tq * D + d0;
#pragma unroll
            for (int d = 0; d < HALF; d += 4) {
                const float4 a = *reinterpret_cast<const float4 *>(src + d);
                acc[d] += a.x * w;
                acc[d + 1] += a.y * w;
                acc[d + 2] += a.z * w;
                acc[d + 3] += a.w * w;
            }
        }
        const float inv = L > 0.f ? 1.f / L : 0.f;
        uint16_t *orow = p.o + b * p.o_sb + hh * p.o_sh + (int64_t)t * p.o_sn + d0;
#pragma unroll
        for (int d = 0; d < HALF; d += 8) {
            uint4 st;
            st.x = pack_bf16x2(acc[d] * inv, acc[d + 1] * inv);
            st.y = pack_bf16x2(acc[d + 2] * inv, acc[d + 3] * inv);
            st.z = pack_bf16x2(acc[d + 4] * inv, acc[d + 5] * inv);
            st.w = pack_bf16x2(acc[d + 6] * inv, acc[d + 7] * inv);
            *reinterpret_cast<uint4 *>(orow + d) = st;
        }
        if (p.lse && (x & 1) == 0)
            p.lse[(int64_t)bh * p.N + t] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
    }
}

hipError_t launch_combine(const CombineParams &p, int64_t grid, hipStream_t s)
{
    if (grid <= 0) return hipSuccess;
    if (p.D == 128)
        hipLaunchKernelGGL(combine_kernel<128>, dim3((unsigned)grid), dim3(256), 0, s, p);
    else if (p.D == 64)
        hipLaunchKernelGGL(combine_kernel<64>, dim3((unsigned)grid), dim3(256), 0, s, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
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
