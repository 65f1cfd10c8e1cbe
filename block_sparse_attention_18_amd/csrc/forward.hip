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
//    query rows.  The leading query blocks of every head (the long text
//    rows) are dispatched first; the other rows go head by head on each of
//    the 8 XCDs, so an XCD's L2 holds the key blocks one head's rows share
//    (work_item).
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 d from LDS,
//    B = 16 d x 32 queries held in registers for the whole kernel).  K rows
//    are fed in a permuted order (bits 2 and 3 of the row index swapped)
//    so that the fp32 accumulator of S^T, converted to bf16, is already the
//    B operand (16 keys x 32 queries) of O^T = V^T P^T.  Each lane therefore
//    owns one query: the running max, running sum and the O rescale are
//    lane-local, and only the max needs one cross-half exchange per block.
//  * K and V are copied row-major into LDS by buffer loads that write LDS
//    directly, double-buffered in 64-key sub-tiles, with XOR swizzles of
//    16-byte chunks so that the 128-bit K reads and the transposing V reads
//    are conflict-free without padding.
//  * Software pipeline: step t computes S^T of sub-tile t while it finishes
//    the softmax and O update of sub-tile t-1, and the vector work (exp2
//    with scale*log2(e) folded into one FMA, row sums, bf16 packing, row
//    max) is spread between the MFMAs of the same wave.
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
    uint32_t kread;              // K operand of k-step 0 (bytes in a tile); k-step s: ^ KSTEP * s
    uint32_t vread;              // V^T operand of d tile 0, keys 0..3; d tile d: ^ VSTEP * d
    uint32_t kdma, vdma;         // source offset of the lane's first 16-byte copy of a tile
    uint32_t knat, vnat;         // the same in natural token order (neighbourhood image tiles)
};

template <int BETA, int D>
__device__ __forceinline__ void init_offsets(WaveState<BETA, D> &st, const FwdParams &p, int wv, int lane)
{
    using Sh = FwdShape<BETA, D>;
    const int hl = lane >> 5, n = lane & 31;
    const int r0 = perm_row(n);
    st.kread = (uint32_t)(r0 * D * 2 + ((hl ^ kswz<D>(r0)) * 16));
    // transposing V reads: lane 4r + c of each 16-lane group names row r,
    // columns 4c..4c+3; lane x of the group receives column x of rows 0..3
    const int G = lane >> 4, jl = lane & 15;
    const int vr0 = 8 * (G >> 1) + (jl >> 2);
    const int dc = 16 * (G & 1) + 4 * (jl & 3);
    st.vread = (uint32_t)(vr0 * D * 2 + (((dc >> 3) ^ vswz<D>(vr0)) * 16) + (dc & 4) * 2);
    // copy x of a lane covers tile row r0 + x * ROWS_PER_COPY with the same
    // chunk: the swizzles only use row bits that the step leaves unchanged
    const int slot = wv * 64 + lane;
    const int r = slot / Sh::KCH, ps = slot % Sh::KCH;
    st.kdma = (uint32_t)(r * p.k.sn * 2 + ((ps ^ kswz<D>(r)) * 16));
    st.vdma = (uint32_t)(r * p.v.sn * 2 + ((ps ^ vswz<D>(r)) * 16));
    const int rn = nb_rowoff(p.nb, r);
    st.knat = (uint32_t)(rn * p.k.sn * 2 + ((ps ^ kswz<D>(r)) * 16));
    st.vnat = (uint32_t)(rn * p.v.sn * 2 + ((ps ^ vswz<D>(r)) * 16));
}


// S^T (64 keys x 32 queries) of one sub-tile from the K tile Kc; the two
// 32-key accumulator chains alternate so consecutive MFMAs are independent.
template <int BETA, int D>
__device__ __forceinline__ void qk_mfma(const uint16_t *__restrict__ Kc, const WaveState<BETA, D> &st,
                                        f32x16 (&sacc)[2])
{
    using Sh = FwdShape<BETA, D>;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.f;
#pragma unroll
    for (int s = 0; s < Sh::QS; ++s)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            const bf16x8 a = *lds_at<bf16x8>(Kc + kt * 32 * D, st.kread ^ (KSTEP * s));
            sacc[kt] = mfma32x32x16(a, st.qf[s], sacc[kt]);
        }
}

// Keys past N in a partial last tile do not exist: their scores become -inf.
template <int BETA, int D>
__device__ __forceinline__ void mask_tail(int k0, int N, int lane, f32x16 (&sacc)[2])
{
    mask_keys(sacc, N - k0 - 8 * (lane >> 5));
}

// Online softmax, part 1: the lazy rescale of the running state when the
// sub-tile's row max (tile_max) exceeds the reference by more than the slack.
template <int BETA, int D>
__device__ __forceinline__ void lazy_rescale(float mx, WaveState<BETA, D> &st)
{
    using Sh = FwdShape<BETA, D>;
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
// summed and packed to bf16 as the B operand of each 16-key k-step.  Groups
// G0 .. G1-1 of the four (kt, u) groups are done.
template <int BETA, int D, int G0 = 0, int G1 = 4>
__device__ __forceinline__ void softmax_probs(const f32x16 (&sacc)[2], float c, WaveState<BETA, D> &st,
                                              bf16x8 (&pf)[2][2])
{
    const float mr = st.m_run;
#pragma unroll
    for (int g = G0; g < G1; ++g) {
        const int kt = g >> 1, u = g & 1;
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
template <int BETA, int D, int KT0 = 0, int KT1 = 2>
__device__ __forceinline__ void pv_mfma(const uint16_t *__restrict__ Vc, const bf16x8 (&pf)[2][2],
                                        WaveState<BETA, D> &st)
{
    using Sh = FwdShape<BETA, D>;
#pragma unroll
    for (int kt = KT0; kt < KT1; ++kt) {
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
                                   (__attribute__((address_space(3))) bf16x4 *)lds_at<uint16_t>(rowp, st.vread ^ (VSTEP * d))));
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
// repeats its last key (those scores are masked).  NAT: with natural-order
// inputs an image tile is gathered from its grid rows (tile row o sits
// nb_rowoff(o) tokens after the tile's first token; a copy step adds the
// same to every lane, so the source stays a per-lane offset offn plus a
// scalar one).
template <int BETA, int D, bool NAT = false>
__device__ __forceinline__ void load_tile(uint16_t *__restrict__ dst, __amdgpu_buffer_rsrc_t rs, int64_t sn,
                                          uint32_t off0, uint32_t offn, bool is_v, const FwdParams &p, int k0,
                                          int wv, int lane)
{
    using Sh = FwdShape<BETA, D>;
    const int rows = p.N - k0;
    const uint32_t so = (uint32_t)((int64_t)k0 * sn * 2);
    // the LDS destination of the wave's first copy, opaque to the compiler
    // so that every copy's address is this base plus a constant (one scalar
    // add), rather than a loop-invariant value of its own kept in a register
    __attribute__((address_space(3))) char *lbase = (__attribute__((address_space(3))) char *)(lds_void *)(dst + wv * 64 * 8);
    asm volatile("" : "+s"(lbase));
    if (NAT && p.natural && k0 >= p.nb.T) {
        // whole tiles only (text and grid are whole numbers of blocks)
        const uint32_t sn0 = (uint32_t)((int64_t)nb_natural(p.nb, BETA, k0) * sn * 2);
        if (Sh::UNIFORM_COPY) {
#pragma unroll
            for (int x = 0; x < Sh::DMA; ++x)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rs, (lds_void *)(lbase + x * Sh::NW * 64 * 16), 16, offn,
                    sn0 + (uint32_t)((int64_t)nb_rowoff(p.nb, x * Sh::ROWS_PER_COPY) * sn * 2), 0, 0);
        } else {
#pragma unroll
            for (int x = 0; x < Sh::DMA; ++x) {
                const int slot = (x * Sh::NW + wv) * 64 + lane;
                const int r = slot / Sh::KCH, ps = slot % Sh::KCH;
                const uint32_t o = (uint32_t)(nb_rowoff(p.nb, r) * sn * 2 +
                                              ((ps ^ (is_v ? vswz<D>(r) : kswz<D>(r))) * 16));
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(lbase + x * Sh::NW * 64 * 16), 16, o, sn0,
                                                         0, 0);
            }
        }
        return;
    }
    if (Sh::UNIFORM_COPY && rows >= 64) {
        // full tile: copy x is copy 0 moved by x * ROWS_PER_COPY rows
        const uint32_t step = (uint32_t)((int64_t)Sh::ROWS_PER_COPY * sn * 2);
#pragma unroll
        for (int x = 0; x < Sh::DMA; ++x)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(lbase + x * Sh::NW * 64 * 16), 16,
                                                     off0, so + x * step, 0, 0);
        return;
    }
#pragma unroll
    for (int x = 0; x < Sh::DMA; ++x) {
        const int slot = (x * Sh::NW + wv) * 64 + lane;
        const int r = slot / Sh::KCH, ps = slot % Sh::KCH;
        const int rr = min(r, rows - 1);
        const uint32_t o = (uint32_t)(rr * sn * 2 + ((ps ^ (is_v ? vswz<D>(r) : kswz<D>(r))) * 16));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(lbase + x * Sh::NW * 64 * 16), 16, o, so, 0, 0);
    }
}

// 2-D neighbourhood masking of a partially covered key tile: the score of
// (query, key) survives when the key's grid position lies in the query's
// window, whose first grid row and column are wr0, wc0 (wr0 < 0: a text
// query, never masked; text keys are never masked either).  The window test
// of the sub-tile's 64 keys is one bitmap per lane, read bit by bit.
template <int BETA, int D>
__device__ __forceinline__ void mask_window(const FwdParams &p, int k0, int wr0, int wc0, int lane, f32x16 (&sacc)[2])
{
    const NbGeom &g = p.nb;
    const int j = k0 / BETA;
    if (j < g.Tb) return;
    const int tk = j - g.Tb, ak = tk / g.tpr;
    uint64_t bits = nb_window_bits(g, k0 - j * BETA, ak * g.th - wr0, (tk - ak * g.tpr) * g.tw - wc0, g.kh, g.kw);
    bits = wr0 < 0 ? ~0ull : bits >> (8 * (lane >> 5));   // bit kt*32 + koff(r): register r of chain kt
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
        const uint32_t w = (uint32_t)(bits >> (32 * kt));
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kt][r] = keep_if_bit(sacc[kt][r], w, koff(r));
    }
}

// Scores of a sub-tile whose block index is invalid, or of keys past N in
// the last tile, are masked out; so are those outside the windows in a
// partially covered tile of a neighbourhood layout.
template <int BETA, int D>
__device__ __forceinline__ void mask_scores(bool valid, int k0, int N, int lane, f32x16 (&sacc)[2])
{
    if (!valid || k0 + 64 > N) mask_tail<BETA, D>(k0, valid ? N : k0, lane, sacc);
}

// Steady-state step t: S^T of sub-tile t (K tile Kc) and the softmax and O
// update of sub-tile t-1 (scores s_prev, V tile Vp).  Copies of K(t+1) into
// Kn (when there is one) and V(t) into Vn are issued first.  Three scheduled
// regions:
//   A: QK^T(t)               with probabilities of keys 0..47 of t-1
//                            (0..31 at β = 64, D = 64)
//   B: PV(t-1), keys 0..31   with the rest of t-1's probabilities
//   C: PV(t-1), keys 32..63  with the row max of t
// then the lazy rescale for t.  t's scores are masked at the next step.
template <int BETA, int D, bool NBM>
__device__ __forceinline__ void fused_step(
    const uint16_t *__restrict__ Kc, const uint16_t *__restrict__ Vp, uint16_t *__restrict__ Kn,
    uint16_t *__restrict__ Vn, bool valid, int k0, bool valid_p, int k0_p, bool load_k, int k0_k,
    __amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs, const FwdParams &p, int wv, int lane,
    WaveState<BETA, D> &st, f32x16 (&s_cur)[2], f32x16 (&s_prev)[2], bool partial_p, int wr0, int wc0)
{
    using Sh = FwdShape<BETA, D>;
    // masking of t-1's scores first: a branch here does not split the
    // scheduled regions, and t's scores are not live yet
    mask_scores<BETA, D>(valid_p, k0_p, p.N, lane, s_prev);
    if (NBM && partial_p) mask_window<BETA, D>(p, k0_p, wr0, wc0, lane, s_prev);
    if (load_k) load_tile<BETA, D, NBM>(Kn, krs, p.k.sn, st.kdma, st.knat, false, p, k0_k, wv, lane);
    load_tile<BETA, D, NBM>(Vn, vrs, p.v.sn, st.vdma, st.vnat, true, p, k0, wv, lane);
    const float c = p.scale_log2;
    bf16x8 pf[2][2];
    constexpr int PV_HALF = 2 * Sh::DT;        // MFMAs of PV over 32 keys
    constexpr int QK = 2 * Sh::QS;             // MFMAs of QK^T
    // Probability groups (16 keys: 8 exp2, ~20 other vector instructions
    // each) done in region A, the rest in B, and LDS reads issued ahead of
    // each P.V region; at β = 64, D = 64 (four MFMAs a region half) a 2 / 2
    // split and reads two ahead measured 4-5 % faster than the 3 / 1, four
    // ahead that suits the longer regions of D = 128.
    constexpr bool SHORT = BETA == 64 && D == 64;
    constexpr int GA = SHORT ? 2 : 3;
    constexpr int PRE_PV = SHORT ? 2 : 4;
    qk_mfma<BETA, D>(Kc, st, s_cur);
    softmax_probs<BETA, D, 0, GA>(s_prev, c, st, pf);
    interleave<3, QK, 1, (20 * GA + QK - 1) / QK, (8 * GA + QK - 1) / QK>();
    __builtin_amdgcn_sched_barrier(0);
    pv_mfma<BETA, D, 0, 1>(Vp, pf, st);
    softmax_probs<BETA, D, GA, 4>(s_prev, c, st, pf);
    interleave<PRE_PV, PV_HALF, 2, (20 * (4 - GA) + PV_HALF - 1) / PV_HALF, (8 * (4 - GA) + PV_HALF - 1) / PV_HALF>();
    __builtin_amdgcn_sched_barrier(0);
    pv_mfma<BETA, D, 1, 2>(Vp, pf, st);
    // the rows of a partial tile past N repeat its last key, so the max over
    // the unmasked scores is the max over the keys that exist; a sub-tile
    // with no key below N (the second half of a last block of <= 64 keys)
    // or with an invalid block index has none
    const bool has_keys = valid && k0 < p.N;
    const float mx = tile_max(s_cur, c) + (has_keys ? 0.f : -INFINITY);   // no branch
    interleave<PRE_PV, PV_HALF, 2, (24 + PV_HALF - 1) / PV_HALF, 0>();
    __builtin_amdgcn_sched_barrier(0);
    lazy_rescale<BETA, D>(mx, st);
}

// First step: S^T of sub-tile 0 and its row max; copies K(1) and V(0).
template <int BETA, int D, bool NBM>
__device__ __forceinline__ void first_step(
    const uint16_t *__restrict__ Kc, uint16_t *__restrict__ Kn, uint16_t *__restrict__ Vn, bool valid,
    int k0, bool load_k, int k0_k, __amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs,
    const FwdParams &p, int wv, int lane, WaveState<BETA, D> &st, f32x16 (&s_cur)[2])
{
    if (load_k) load_tile<BETA, D, NBM>(Kn, krs, p.k.sn, st.kdma, st.knat, false, p, k0_k, wv, lane);
    load_tile<BETA, D, NBM>(Vn, vrs, p.v.sn, st.vdma, st.vnat, true, p, k0, wv, lane);
    qk_mfma<BETA, D>(Kc, st, s_cur);
    lazy_rescale<BETA, D>((valid && k0 < p.N) ? tile_max(s_cur, p.scale_log2) : -INFINITY, st);
}

// Last step: softmax and O update of the last sub-tile.
template <int BETA, int D, bool NBM>
__device__ __forceinline__ void last_step(const uint16_t *__restrict__ Vp, bool valid_p, int k0_p,
                                          const FwdParams &p, int lane, WaveState<BETA, D> &st,
                                          f32x16 (&s_prev)[2], bool partial_p, int wr0, int wc0)
{
    mask_scores<BETA, D>(valid_p, k0_p, p.N, lane, s_prev);
    if (NBM && partial_p) mask_window<BETA, D>(p, k0_p, wr0, wc0, lane, s_prev);
    bf16x8 pf[2][2];
    softmax_probs<BETA, D>(s_prev, p.scale_log2, st, pf);
    pv_mfma<BETA, D>(Vp, pf, st);
}

// A SKIP row (DiTFastAttnV2, "Head-wise Caching"): the rows of query block i
// of head (b, hh) take the cached output bit for bit, 16 bytes a copy, and
// the cached LSE when one is given.
template <int BETA, int D>
__device__ __forceinline__ void skip_row_copy(const FwdParams &p, int b, int hh, int bh, int i, int tid)
{
    constexpr int NT = FwdShape<BETA, D>::NT;
    constexpr int CH = D / 8;                  // 16-byte chunks per row
    const int t0 = i * BETA, rows = min(BETA, p.N - t0);
    if (p.copy_o) {
        const uint16_t *src = p.oc.p + b * p.oc.sb + hh * p.oc.sh;
        uint16_t *dst = p.o + b * p.o_sb + hh * p.o_sh;
        for (int x = tid; x < rows * CH; x += NT) {
            const int r = x / CH, c = x - r * CH;
            const int64_t t = t0 + r;
            *reinterpret_cast<uint4 *>(dst + t * p.o_sn + 8 * c) =
                *reinterpret_cast<const uint4 *>(src + t * p.oc.sn + 8 * c);
        }
    }
    if (p.lse_src && p.lse)
        for (int r = tid; r < rows; r += NT) p.lse[(int64_t)bh * p.N + t0 + r] = p.lse_src[(int64_t)bh * p.N + t0 + r];
}

// Occupancy: two waves per SIMD at β=128 (two 4-wave workgroups per CU).
// β=64, D=64 asks for three: the register budget of 168 holds its state
// without spilling (at two the allocator spends all 256 and still spills),
// and five 2-wave workgroups, whose 32 KB of tiles fit the LDS five times,
// share a CU.  The launch bound's second argument is waves per SIMD.
template <int BETA, int D>
constexpr int fwd_waves_per_simd() { return (BETA == 64 && D == 64) ? 3 : 2; }

// NBM: neighbourhood masking of the tiles the layout flags as partial.
template <int BETA, int D, bool NBM>
__global__ __launch_bounds__(BETA / 32 * 64, (fwd_waves_per_simd<BETA, D>())) void fwd_kernel(const FwdParams p)
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
    } else {         // the text rows of every head first, then head by head per XCD
        work_item((int)blockIdx.x, BH, p.nB, i, bh);
    }
    const int b = bh / p.H;
    const int hh = bh - b * p.H;
    if ((p.skip_bits[hh >> 5] >> (hh & 31)) & 1u) {
        skip_row_copy<BETA, D>(p, b, hh, bh, i, tid);
        return;
    }

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
    // natural-order neighbourhood inputs: the query's natural position
    const int qpos = (NBM && p.natural && qrow < p.N) ? nb_natural(p.nb, BETA, qrow) : qrow;
    // neighbourhood layouts: the window origin of an image query (-1: none)
    int wr0 = -1, wc0 = 0;
    if (NBM && qrow >= p.nb.T && qrow < p.N) {
        const NbGeom &g = p.nb;
        const int pq = qrow - g.T, tq = pq / BETA, oq = pq - tq * BETA, aq = tq / g.tpr;
        wr0 = nb_start(aq * g.th + (oq >> g.tw_log2), g.R, g.kh, g.sh);
        wc0 = nb_start((tq - aq * g.tpr) * g.tw + (oq & (g.tw - 1)), g.C, g.kw, g.sw);
    }
#pragma unroll
    for (int s = 0; s < Sh::QS; ++s) {
        uint4 u = qrow < p.N ? ld_g16(qb + (int64_t)qpos * p.q.sn + 16 * s + 8 * hl) : zero_u4();
        st.qf[s] = as_bf16x8(u);
    }
#pragma unroll
    for (int d = 0; d < Sh::DT; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.oacc[d][r] = 0.f;
    st.m_run = -1.0e30f;   // finite: a fully masked tile gives p = 0, never NaN
    st.l_run = 0.f;
    init_offsets<BETA, D>(st, p, wv, lane);

    const __amdgpu_buffer_rsrc_t krs = buffer_desc(kb, (uint32_t)(((int64_t)(p.N - 1) * p.k.sn + D) * 2));
    const __amdgpu_buffer_rsrc_t vrs = buffer_desc(vb, (uint32_t)(((int64_t)(p.N - 1) * p.v.sn + D) * 2));

    // Sub-tile t: key block col_idx[e0 + t / SUB], keys 64 (t % SUB) .. +63.
    // The index is wave-uniform, so it is read through the constant address
    // space (a scalar load, which leaves the vector memory counter to the
    // tile copies).  An entry outside [0, nB) is ignored: its copies read
    // block 0 and its scores are masked.
    const __attribute__((address_space(4))) int32_t *cidx =
        (const __attribute__((address_space(4))) int32_t *)(p.col_idx + e0);
    auto tile_key0 = [&](int t, bool &valid) {
        const int j = cidx[t / Sh::SUB];
        valid = (unsigned)j < (unsigned)p.nB;
        return (valid ? j * BETA : 0) + 64 * (t % Sh::SUB);
    };
    // neighbourhood layouts: per-entry flag of a partially covered key tile
    const __attribute__((address_space(4))) int32_t *cflag =
        (const __attribute__((address_space(4))) int32_t *)(NBM ? p.flags + e0 : p.col_idx + e0);
    auto tile_partial = [&](int t, bool valid) { return NBM && valid && cflag[t / Sh::SUB] != 0; };

    // Step t computes S^T of sub-tile t and finishes sub-tile t-1.  K(t) sits
    // in K[t&1], V(t) in V[t&1]; step t copies K(t+1) and V(t), so a V tile
    // lands one step after its K tile.  Steps 0 and T are peeled; the loop
    // is unrolled by two so that every LDS address is a per-lane offset plus
    // a compile-time constant.  An entry whose block index is invalid is
    // read from block 0 and fully masked.
    f32x16 sa[2], sb[2];
    if (T > 0) {
        // (valid, first key) of sub-tiles t-1 (prv), t (cur), t+1 (nxt); the
        // index of t+2 is read during step t, a full step before its use
        bool v_cur = false, v_nxt = false, v_prv;
        int k_cur = tile_key0(0, v_cur), k_nxt = 0, k_prv;
        if (T > 1) k_nxt = tile_key0(1, v_nxt);
        bool f_cur = tile_partial(0, v_cur), f_nxt = T > 1 && tile_partial(1, v_nxt), f_prv;
        load_tile<BETA, D, NBM>(K0, krs, p.k.sn, st.kdma, st.knat, false, p, k_cur, wv, lane);
        __syncthreads();   // Q in registers; K(0) in LDS
        first_step<BETA, D, NBM>(K0, K1, V0, v_cur, k_cur, T > 1, k_nxt, krs, vrs, p, wv, lane, st, sa);
        __syncthreads();
        v_prv = v_cur; k_prv = k_cur; f_prv = f_cur;
        v_cur = v_nxt; k_cur = k_nxt; f_cur = f_nxt;
        for (int t = 1; t < T; t += 2) {
            // odd step t: K(t) in K1, V(t-1) in V0; copies K(t+1) -> K0, V(t) -> V1
            v_nxt = false; k_nxt = 0; f_nxt = false;
            if (t + 1 < T) {
                k_nxt = tile_key0(t + 1, v_nxt);
                f_nxt = tile_partial(t + 1, v_nxt);
            }
            fused_step<BETA, D, NBM>(K1, V0, K0, V1, v_cur, k_cur, v_prv, k_prv, t + 1 < T, k_nxt, krs, vrs, p, wv,
                                lane, st, sb, sa, f_prv, wr0, wc0);
            __syncthreads();
            v_prv = v_cur; k_prv = k_cur; f_prv = f_cur;
            v_cur = v_nxt; k_cur = k_nxt; f_cur = f_nxt;
            if (t + 1 >= T) break;
            // even step t+1: K(t+1) in K0, V(t) in V1; copies K(t+2) -> K1, V(t+1) -> V0
            v_nxt = false; k_nxt = 0; f_nxt = false;
            if (t + 2 < T) {
                k_nxt = tile_key0(t + 2, v_nxt);
                f_nxt = tile_partial(t + 2, v_nxt);
            }
            fused_step<BETA, D, NBM>(K0, V1, K1, V0, v_cur, k_cur, v_prv, k_prv, t + 2 < T, k_nxt, krs, vrs, p, wv,
                                lane, st, sa, sb, f_prv, wr0, wc0);
            __syncthreads();
            v_prv = v_cur; k_prv = k_cur; f_prv = f_cur;
            v_cur = v_nxt; k_cur = k_nxt; f_cur = f_nxt;
        }
        // finish sub-tile T-1 (V(T-1) in V[(T-1)&1])
        if (T & 1) last_step<BETA, D, NBM>(V0, v_prv, k_prv, p, lane, st, sa, f_prv, wr0, wc0);
        else last_step<BETA, D, NBM>(V1, v_prv, k_prv, p, lane, st, sb, f_prv, wr0, wc0);
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
                *reinterpret_cast<float4 *>(slot + partial_o_index(BETA, d * 32 + 8 * g + 4 * hl, tq)) =
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
        uint16_t *orow = p.o + b * p.o_sb + hh * p.o_sh + (int64_t)qpos * p.o_sn;
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
            p.lse[(int64_t)bh * p.N + qpos] = lse;
        }
    }
}

template <int BETA, int D>
static hipError_t launch_fwd_t(const FwdParams &p, int64_t grid, hipStream_t s)
{
    using Sh = FwdShape<BETA, D>;
    if (grid == 0) return hipSuccess;
    if (p.flags)
        hipLaunchKernelGGL((fwd_kernel<BETA, D, true>), dim3((unsigned)grid), dim3(Sh::NT), 0, s, p);
    else
        hipLaunchKernelGGL((fwd_kernel<BETA, D, false>), dim3((unsigned)grid), dim3(Sh::NT), 0, s, p);
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
// LSE = (M + log2 L) ln 2.  One workgroup per split row, 256 / BETA threads
// per query, each a share of the head dimension's groups of four channels.
template <int BETA, int D>
__global__ __launch_bounds__(256) void combine_kernel(const CombineParams p)
{
    constexpr int TPQ = 256 / BETA;     // threads per query
    constexpr int NG = D / 4 / TPQ;     // groups of four channels per thread
    if ((int)blockIdx.x >= p.counts[1]) return;
    const int2 sr = p.split_rows[blockIdx.x];
    const int row = sr.x, chunks = sr.y;
    const int bh = row / p.nB, i = row - bh * p.nB;
    const int b = bh / p.H, hh = bh - b * p.H;
    const int64_t slot_floats = partial_slot_floats(BETA, D);
    const float *base = p.partials + (int64_t)blockIdx.x * p.max_chunks * slot_floats;
    // thread x owns query x mod BETA and the channel groups x / BETA + TPQ g:
    // for each g the threads read consecutive 16-byte groups of a slot
    const int tq = threadIdx.x % BETA, part = threadIdx.x / BETA;
    const int t = i * BETA + tq;
    if (t >= p.N) return;
    const int tpos = p.natural ? nb_natural(p.nb, BETA, t) : t;
    float M = -INFINITY;
    for (int c = 0; c < chunks; ++c) M = fmaxf(M, base[c * slot_floats + BETA * D + tq]);
    float L = 0.f;
    float4 acc[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) acc[g] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int c = 0; c < chunks; ++c) {
        const float *slot = base + c * slot_floats;
        const float mc = slot[BETA * D + tq];
        const float w = (mc == -INFINITY) ? 0.f : fast_exp2(mc - M);
        L += slot[BETA * D + BETA + tq] * w;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const float4 a = *reinterpret_cast<const float4 *>(slot + partial_o_index(BETA, 4 * (part + TPQ * g), tq));
            acc[g].x += a.x * w;
            acc[g].y += a.y * w;
            acc[g].z += a.z * w;
            acc[g].w += a.w * w;
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    uint16_t *orow = p.o + b * p.o_sb + hh * p.o_sh + (int64_t)tpos * p.o_sn;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        uint2 st;
        st.x = pack_bf16x2(acc[g].x * inv, acc[g].y * inv);
        st.y = pack_bf16x2(acc[g].z * inv, acc[g].w * inv);
        *reinterpret_cast<uint2 *>(orow + 4 * (part + TPQ * g)) = st;
    }
    if (p.lse && part == 0)
        p.lse[(int64_t)bh * p.N + tpos] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
}

hipError_t launch_combine(const CombineParams &p, int64_t grid, hipStream_t s)
{
    if (grid <= 0) return hipSuccess;
    if (p.block == 128 && p.D == 128)
        hipLaunchKernelGGL((combine_kernel<128, 128>), dim3((unsigned)grid), dim3(256), 0, s, p);
    else if (p.block == 128 && p.D == 64)
        hipLaunchKernelGGL((combine_kernel<128, 64>), dim3((unsigned)grid), dim3(256), 0, s, p);
    else if (p.block == 64 && p.D == 128)
        hipLaunchKernelGGL((combine_kernel<64, 128>), dim3((unsigned)grid), dim3(256), 0, s, p);
    else if (p.block == 64 && p.D == 64)
        hipLaunchKernelGGL((combine_kernel<64, 64>), dim3((unsigned)grid), dim3(256), 0, s, p);
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
