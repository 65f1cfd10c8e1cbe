// FP8 (OCP E4M3) path on gfx950: quantisation of Q, K, V with max-abs
// scales, and the block-sparse forward on v_mfma_f32_32x32x64_f8f6f4 (the
// FP8 mixed-precision mode of block-sparse attention kernels, GNA sparse
// attention write-up, section 2.1).
//
// E4M3: bias 7, largest finite value 448, subnormals m * 2^-9, NaN only.
// v_cvt_pk_fp8_f32 rounds to nearest even and does not saturate, so every
// scaled value is kept within +-448 by its group's scale.
//
// The FP8 MFMA multiplies byte j of A-lane (row m, half h) with byte j of
// B-lane (column n, half h) for every j and h, so both operands only have
// to agree on one bijection (h, j) -> k:
//  * S^T = K Q^T: k is the channel d = 64 ks + 32 h + j; K rows are the
//    keys, Q^T columns the queries (Q codes held in registers);
//  * O^T = V^T P^T: the fp32 S^T accumulator of lane (n, h) holds keys
//    32 a + 8 g + 4 h + e (a = accumulator tile, r = 4 g + e); packed to
//    E4M3 as byte j = 16 a + r it is directly the B operand.  V^T is stored
//    with the matching key order (key 32a + 8g + 4h + e at column
//    32 h + 16 a + 4 g + e of its 64-key group), so each A operand is 32
//    contiguous bytes of one V^T row.
#include "common.h"
#include "internal.h"

namespace bsa {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr float kFp8Max = 448.0f;

__device__ __forceinline__ void fp8_group_scale(float amax, float &scale, float &inv)
{
    if (amax > 0.f) {
        scale = amax / kFp8Max;
        inv = kFp8Max / amax;
    } else {
        scale = 0.f;
        inv = 0.f;
    }
}

// Four floats -> four E4M3 bytes (byte 0 = a).  The first conversion keeps
// the upper half of its destination, which the second one overwrites: any
// dying value serves as that destination (no zeroing move).
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d)
{
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

__device__ __forceinline__ void unpack_bf16x8(const uint4 &u, float (&x)[8])
{
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}

// Column of key k (0..63) inside its 64-key group of V^T.
__device__ __forceinline__ int fp8_vcol(int k)
{
    const int a = k >> 5, g = (k >> 3) & 3, h = (k >> 2) & 1, e = k & 3;
    return 32 * h + 16 * a + 4 * g + e;
}

// ---------------------------------------------------------------------------
// quantisation
// ---------------------------------------------------------------------------
// Input row of the token at position t of the codes: t itself, or with a
// neighbourhood geometry the natural position of tile-major position t.
__device__ __forceinline__ int64_t quant_src(const Fp8QuantParams &p, int t)
{
    return p.nb_block ? nb_natural(p.nb, p.nb_block, t) : t;
}

// Q: one scale per token; D/8 lanes per token, 16 bytes of bf16 each.
template <int D>
__global__ __launch_bounds__(256) void quant_q_kernel(const Fp8QuantParams p)
{
    constexpr int LPT = D / 8, TPB = 256 / LPT;
    const int tid = threadIdx.x, g = tid / LPT, c = tid % LPT;
    const int64_t tok = (int64_t)blockIdx.x * TPB + g;   // (b*H + h)*N + t
    const bool ok = tok < p.BHN;
    float x[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float amax = 0.f;
    if (ok) {
        const int64_t bh = tok / p.N, t = tok - bh * p.N;
        const int b = (int)(bh / p.H), h = (int)(bh - (int64_t)b * p.H);
        unpack_bf16x8(ld_g16(p.q.p + b * p.q.sb + h * p.q.sh + quant_src(p, (int)t) * p.q.sn + 8 * c), x);
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
    }
#pragma unroll
    for (int d = 1; d < LPT; d <<= 1) amax = fmaxf(amax, __shfl_xor(amax, d, 64));
    float sc, inv;
    fp8_group_scale(amax, sc, inv);
    if (ok) {
        uint2 w;
        w.x = pack_fp8x4(x[0] * inv, x[1] * inv, x[2] * inv, x[3] * inv);
        w.y = pack_fp8x4(x[4] * inv, x[5] * inv, x[6] * inv, x[7] * inv);
        *reinterpret_cast<uint2 *>(p.q8 + tok * D + 8 * c) = w;
        if (c == 0) p.q_scale[tok] = sc;
    }
}

// K: one scale per 64-key tile; one workgroup per (b, h, tile).
template <int D>
__global__ __launch_bounds__(256) void quant_k_kernel(const Fp8QuantParams p)
{
    constexpr int CH = D / 8, CPT = 64 * CH / 256;
    __shared__ float red[4];
    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.x / p.NT;
    const int T = (int)(blockIdx.x - bh * p.NT);
    const int b = (int)(bh / p.H), h = (int)(bh - (int64_t)b * p.H);
    float x[CPT][8];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int slot = i * 256 + tid, row = slot / CH, c = slot % CH;
        const int t = T * 64 + row;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[i][e] = 0.f;
        if (t < p.N) unpack_bf16x8(ld_g16(p.k.p + b * p.k.sb + h * p.k.sh + quant_src(p, t) * p.k.sn + 8 * c), x[i]);
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[i][e]));
    }
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) amax = fmaxf(amax, __shfl_xor(amax, d, 64));
    if ((tid & 63) == 0) red[tid >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    float sc, inv;
    fp8_group_scale(amax, sc, inv);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int slot = i * 256 + tid, row = slot / CH, c = slot % CH;
        const int t = T * 64 + row;
        if (t < p.N) {
            uint2 w;
            w.x = pack_fp8x4(x[i][0] * inv, x[i][1] * inv, x[i][2] * inv, x[i][3] * inv);
            w.y = pack_fp8x4(x[i][4] * inv, x[i][5] * inv, x[i][6] * inv, x[i][7] * inv);
            *reinterpret_cast<uint2 *>(p.k8 + (bh * p.N + t) * D + 8 * c) = w;
        }
    }
    if (tid == 0) p.k_scale[bh * p.NT + T] = sc;
}

// V, pass 1: channel maxima of 256-key chunks.  Grid (B*H, S).  The
// maxima over all keys do not depend on their order, so the chunks are
// read in input order also when the codes are reordered.
template <int D>
__global__ __launch_bounds__(256) void vmax_kernel(const Fp8QuantParams p)
{
    constexpr int CH = D / 8, ST = 256 / CH;   // chunks per row, key stripes
    __shared__ float red[ST][D];
    const int tid = threadIdx.x, c = tid % CH, st = tid / CH;
    const int64_t bh = blockIdx.x;
    const int s = blockIdx.y;
    const int b = (int)(bh / p.H), h = (int)(bh - (int64_t)b * p.H);
    float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int i = 0; i < 256 / ST; ++i) {
        const int t = s * 256 + st + i * ST;
        if (t < p.N) {
            float x[8];
            unpack_bf16x8(ld_g16(p.v.p + b * p.v.sb + h * p.v.sh + (int64_t)t * p.v.sn + 8 * c), x);
#pragma unroll
            for (int e = 0; e < 8; ++e) m[e] = fmaxf(m[e], fabsf(x[e]));
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[st][8 * c + e] = m[e];
    __syncthreads();
    if (tid < D) {
        float a = 0.f;
        for (int i = 0; i < ST; ++i) a = fmaxf(a, red[i][tid]);
        p.vmax_part[(bh * p.S + s) * D + tid] = a;
    }
}

// V, pass 2: per-channel scales (and their reciprocals for pass 3).
template <int D>
__global__ __launch_bounds__(D) void vscale_kernel(const Fp8QuantParams p)
{
    const int64_t bh = blockIdx.x;
    const int d = threadIdx.x;
    // four independent maxima keep four loads in flight (the chunks' maxima
    // are non-negative, and max is exact in any order)
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    const float *mp = p.vmax_part + bh * p.S * D + d;
    int s = 0;
    for (; s + 4 <= p.S; s += 4) {
        a0 = fmaxf(a0, mp[(int64_t)(s + 0) * D]);
        a1 = fmaxf(a1, mp[(int64_t)(s + 1) * D]);
        a2 = fmaxf(a2, mp[(int64_t)(s + 2) * D]);
        a3 = fmaxf(a3, mp[(int64_t)(s + 3) * D]);
    }
    for (; s < p.S; ++s) a0 = fmaxf(a0, mp[(int64_t)s * D]);
    const float a = fmaxf(fmaxf(a0, a1), fmaxf(a2, a3));
    float sc, inv;
    fp8_group_scale(a, sc, inv);
    p.v_scale[bh * D + d] = sc;
    p.v_inv[bh * D + d] = inv;
}

// V, pass 3: codes of one 64-key tile, transposed to [d][key] with the key
// order of the P operand, through LDS.  One workgroup per (b, h, tile).
template <int D>
__global__ __launch_bounds__(256) void quant_v_kernel(const Fp8QuantParams p)
{
    constexpr int CH = D / 8, CPT = 64 * CH / 256;
    __shared__ __attribute__((aligned(16))) uint8_t tile[D * 64];
    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.x / p.NT;
    const int T = (int)(blockIdx.x - bh * p.NT);
    const int b = (int)(bh / p.H), h = (int)(bh - (int64_t)b * p.H);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int slot = i * 256 + tid, row = slot / CH, c = slot % CH;
        const int t = T * 64 + row;
        float x[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (t < p.N) unpack_bf16x8(ld_g16(p.v.p + b * p.v.sb + h * p.v.sh + quant_src(p, t) * p.v.sn + 8 * c), x);
        const float4 i0 = *reinterpret_cast<const float4 *>(p.v_inv + bh * D + 8 * c);
        const float4 i1 = *reinterpret_cast<const float4 *>(p.v_inv + bh * D + 8 * c + 4);
        const uint32_t w0 = pack_fp8x4(x[0] * i0.x, x[1] * i0.y, x[2] * i0.z, x[3] * i0.w);
        const uint32_t w1 = pack_fp8x4(x[4] * i1.x, x[5] * i1.y, x[6] * i1.z, x[7] * i1.w);
        const int col = fp8_vcol(row);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            tile[(8 * c + e) * 64 + col] = (uint8_t)(w0 >> (8 * e));
            tile[(8 * c + 4 + e) * 64 + col] = (uint8_t)(w1 >> (8 * e));
        }
    }
    __syncthreads();
    for (int slot = tid; slot < D * 4; slot += 256) {
        const int d = slot >> 2, cc = slot & 3;
        *reinterpret_cast<uint4 *>(p.v8t + (bh * D + d) * p.NP + T * 64 + 16 * cc) =
            *reinterpret_cast<const uint4 *>(tile + d * 64 + 16 * cc);
    }
}

hipError_t launch_quantize_fp8(const Fp8QuantParams &p, int D, hipStream_t s)
{
    const int64_t BH = (int64_t)p.B * p.H;
    if (BH == 0) return hipSuccess;
    if (D == 128) {
        hipLaunchKernelGGL(quant_q_kernel<128>, dim3((unsigned)((p.BHN + 15) / 16)), dim3(256), 0, s, p);
        hipLaunchKernelGGL(quant_k_kernel<128>, dim3((unsigned)(BH * p.NT)), dim3(256), 0, s, p);
        hipLaunchKernelGGL(vmax_kernel<128>, dim3((unsigned)BH, (unsigned)p.S), dim3(256), 0, s, p);
        hipLaunchKernelGGL(vscale_kernel<128>, dim3((unsigned)BH), dim3(128), 0, s, p);
        hipLaunchKernelGGL(quant_v_kernel<128>, dim3((unsigned)(BH * p.NT)), dim3(256), 0, s, p);
    } else if (D == 64) {
        hipLaunchKernelGGL(quant_q_kernel<64>, dim3((unsigned)((p.BHN + 31) / 32)), dim3(256), 0, s, p);
        hipLaunchKernelGGL(quant_k_kernel<64>, dim3((unsigned)(BH * p.NT)), dim3(256), 0, s, p);
        hipLaunchKernelGGL(vmax_kernel<64>, dim3((unsigned)BH, (unsigned)p.S), dim3(256), 0, s, p);
        hipLaunchKernelGGL(vscale_kernel<64>, dim3((unsigned)BH), dim3(64), 0, s, p);
        hipLaunchKernelGGL(quant_v_kernel<64>, dim3((unsigned)(BH * p.NT)), dim3(256), 0, s, p);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
template <int BETA, int D>
struct F8Shape {
    static constexpr int NW = BETA / 32;          // waves per workgroup
    static constexpr int NT = NW * 64;            // threads per workgroup
    static constexpr int SUB = BETA / 64;         // 64-key sub-tiles per block
    static constexpr int KS = D / 64;             // k-steps of S^T over d
    static constexpr int DT = D / 32;             // 32-row d tiles of O^T
    static constexpr int TILE = 64 * D;           // bytes of a 64-key K tile or V^T tile
    static constexpr int KCH = D / 16;            // 16-byte chunks per K row
    static constexpr int DMA = TILE / 16 / NT;    // 16-byte copies per lane per tile
    static_assert(TILE / 16 % NT == 0, "tile split");
};

// XOR swizzles of the 16-byte chunk index within a row: K rows are D bytes,
// V^T rows 64 bytes.  The 16 rows read by one quarter-wave land on 16
// distinct chunk slots of the 256-byte bank window.
template <int D>
__device__ __forceinline__ int k8swz(int row)
{
    return D == 128 ? ((row >> 1) & 7) : ((row >> 2) & 3);
}
__device__ __forceinline__ int v8swz(int row) { return (row >> 2) & 3; }

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8 &a, const i32x8 &b, const f32x16 &c)
{
    // scale operands 0 select the unscaled E4M3 x E4M3 product
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

template <int BETA, int D>
struct F8State {
    using Sh = F8Shape<BETA, D>;
    i32x8 qf[Sh::KS];            // Q^T codes: query n, channels 64 ks + 32 h .. +31
    f32x16 oacc[Sh::DT];         // O^T in V code units
    f32x16 lacc;                 // row sums of the E4M3 probabilities (all 16 equal)
    i32x8 ones;                  // E4M3 1.0 in every byte: A operand of the row sums
    float m_run;                 // reference max, log2-scaled domain
    float cq;                    // scale * log2(e) * q_scale of the lane's query
    uint32_t kread;              // K operand, k-step 0, first 16 bytes; (ks, x): ^ (64 ks + 16 x)
    uint32_t vread;              // V^T operand, d tile 0, first 16 bytes; x: ^ 16
    uint32_t kdma, vdma;         // source offset of the lane's first copy of a tile
    int wr0, wc0;                // neighbourhood: window start (row, column) of the lane's query
    bool qimg;                   // neighbourhood: the lane's query is an image token
};

__device__ __forceinline__ i32x8 lds_i32x8(const uint8_t *base, uint32_t o0, uint32_t o1)
{
    const uint4 a = *reinterpret_cast<const uint4 *>(base + o0);
    const uint4 b = *reinterpret_cast<const uint4 *>(base + o1);
    i32x8 r;
    r[0] = (int)a.x; r[1] = (int)a.y; r[2] = (int)a.z; r[3] = (int)a.w;
    r[4] = (int)b.x; r[5] = (int)b.y; r[6] = (int)b.z; r[7] = (int)b.w;
    return r;
}

// S^T (64 keys x 32 queries) of one sub-tile; accumulator tile a holds keys
// 32 a + 8 g + 4 h + e at register 4 g + e of lane half h.
template <int BETA, int D>
__device__ __forceinline__ void qk8(const uint8_t *__restrict__ Kc, const F8State<BETA, D> &st,
                                    f32x16 (&sacc)[2])
{
    using Sh = F8Shape<BETA, D>;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[a][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < Sh::KS; ++ks)
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            const uint8_t *t = Kc + a * 32 * D;
            const i32x8 k = lds_i32x8(t, st.kread ^ (64 * ks), st.kread ^ (64 * ks + 16));
            sacc[a] = mfma_fp8(k, st.qf[ks], sacc[a]);
        }
}

// Keys at sub-tile offset >= lim do not exist (or their block is invalid).
__device__ __forceinline__ void mask8(f32x16 (&sacc)[2], int lim)
{
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (32 * a + 8 * (r >> 2) + (r & 3) >= lim) sacc[a][r] = -INFINITY;
}

__device__ __forceinline__ void mask_scores8(bool valid, int k0, int N, int lane, f32x16 (&sacc)[2])
{
    if (!valid || k0 + 64 > N) mask8(sacc, (valid ? N - k0 : 0) - 4 * (lane >> 5));
}

// 2-D neighbourhood masking of a partially covered key tile (image keys
// only): a score survives when the key's grid position lies in the window
// (row start wr0, column start wc0) of the lane's image query.  The window
// test of the sub-tile's 64 keys is one bitmap per lane, read bit by bit.
template <int BETA>
__device__ __forceinline__ void mask_window8(const NbGeom &g, int k0, int wr0, int wc0, int lane, f32x16 (&sacc)[2])
{
    const int j = k0 / BETA;
    if (j < g.Tb) return;
    const int tk = j - g.Tb, ak = tk / g.tpr;
    // register r of chain a holds key 32 a + 8 (r >> 2) + 4 hl + (r & 3)
    const uint64_t bits =
        nb_window_bits(g, k0 - j * BETA, ak * g.th - wr0, (tk - ak * g.tpr) * g.tw - wc0, g.kh, g.kw) >> (4 * (lane >> 5));
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        const uint32_t w = (uint32_t)(bits >> (32 * a));
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[a][r] = keep_if_bit(sacc[a][r], w, 8 * (r >> 2) + (r & 3));
    }
}

template <int BETA, int D>
__device__ __forceinline__ bool lazy_rescale8(float mx, F8State<BETA, D> &st)
{
    using Sh = F8Shape<BETA, D>;
    if (!__ballot(mx > st.m_run + 8.0f)) return false;
    const float m_new = fmaxf(st.m_run, mx);
    const float alpha = (st.m_run == m_new) ? 1.f : fast_exp2(st.m_run - m_new);
    st.m_run = m_new;
#pragma unroll
    for (int r = 0; r < 16; ++r) st.lacc[r] *= alpha;
#pragma unroll
    for (int d = 0; d < Sh::DT; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.oacc[d][r] *= alpha;
    return true;
}

// Probabilities of accumulator tile A of a sub-tile (keys 32 A + 8 g + 4 h
// + e) relative to the reference max (at most 2^8 under the lazy rescale,
// inside the E4M3 range), rounded to E4M3 and packed into bytes 16 A + r of
// the B operand of O^T += V^T P^T.
template <int A>
__device__ __forceinline__ void probs_half(const f32x16 (&sacc)[2], float c, float m, i32x8 &pf)
{
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = fast_exp2(__builtin_fmaf(sacc[A][4 * g + e], c, -m));
        pf[4 * A + g] = (int)pack_fp8x4(x[0], x[1], x[2], x[3]);
    }
}

// O^T += V^T P^T (one MFMA per 32-row d tile) and the row sums of P (an
// MFMA with an all-ones A operand: every row of its output is the column
// sum of P^T).
template <int BETA, int D>
__device__ __forceinline__ void pv8(const uint8_t *__restrict__ Vc, const i32x8 &pf, F8State<BETA, D> &st)
{
    using Sh = F8Shape<BETA, D>;
#pragma unroll
    for (int d = 0; d < Sh::DT; ++d) {
        const uint8_t *t = Vc + d * 32 * 64;
        const i32x8 v = lds_i32x8(t, st.vread, st.vread ^ 16);
        st.oacc[d] = mfma_fp8(v, pf, st.oacc[d]);
    }
    st.lacc = mfma_fp8(st.ones, pf, st.lacc);
}

// Copy of one 64-key K tile (keys from k0; rows past N repeat key N-1) into
// LDS: lane l of copy x fills the 16-byte slot (x*NW + wave)*64 + l, slot s
// holding row s / KCH, chunk (s % KCH) ^ k8swz(row).
template <int BETA, int D>
__device__ __forceinline__ void load_k8(uint8_t *__restrict__ dst, __amdgpu_buffer_rsrc_t rs, uint32_t kdma,
                                        int N, int k0, int wv, int lane)
{
    using Sh = F8Shape<BETA, D>;
    constexpr int RPC = Sh::NT / Sh::KCH;   // rows per copy
    // one opaque LDS base per call: each copy's destination is a scalar add
    __attribute__((address_space(3))) char *lbase = (__attribute__((address_space(3))) char *)(lds_void *)(dst + wv * 64 * 16);
    asm volatile("" : "+s"(lbase));
    if (k0 + 64 <= N) {
#pragma unroll
        for (int x = 0; x < Sh::DMA; ++x)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(lbase + x * Sh::NW * 64 * 16), 16,
                                                     kdma + x * RPC * D, k0 * D, 0, 0);
        return;
    }
#pragma unroll
    for (int x = 0; x < Sh::DMA; ++x) {
        const int slot = (x * Sh::NW + wv) * 64 + lane;
        const int r = slot / Sh::KCH, ps = slot % Sh::KCH;
        const int key = max(0, min(k0 + r, N - 1));
        const uint32_t o = (uint32_t)(key * D + ((ps ^ k8swz<D>(r)) * 16));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(lbase + x * Sh::NW * 64 * 16), 16, o, 0, 0, 0);
    }
}

// Copy of the V^T tile of keys k0 .. k0+63 (D rows of 64 bytes, columns
// k0.. of the padded V^T; k0 is clamped to the last tile).
template <int BETA, int D>
__device__ __forceinline__ void load_v8(uint8_t *__restrict__ dst, __amdgpu_buffer_rsrc_t rs, uint32_t vdma,
                                        uint32_t vstep, int NP, int k0, int wv)
{
    using Sh = F8Shape<BETA, D>;
    const int c0 = min(k0, NP - 64);
    __attribute__((address_space(3))) char *lbase = (__attribute__((address_space(3))) char *)(lds_void *)(dst + wv * 64 * 16);
    asm volatile("" : "+s"(lbase));
#pragma unroll
    for (int x = 0; x < Sh::DMA; ++x)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(lbase + x * Sh::NW * 64 * 16), 16,
                                                 vdma + x * vstep, c0, 0, 0);
}

struct F8Tile {
    int k0;        // first key of the sub-tile
    bool valid;    // block index in range
    float c;       // scale * log2(e) * q_scale * k_scale of the tile (> 0)
    bool partial;  // neighbourhood layouts: a partially covered entry
};

// Steady-state step t, two scheduled regions of MFMAs with the vector work
// spread between them:
//   A: S^T(t) = K(t) Q^T            with the probabilities of keys 32..63 of t-1
//   B: O^T += V^T(t-1) P^T(t-1)     with the row max of t and the
//                                   probabilities of keys 0..31 of t
// Keys 0..31 of t are exponentiated against the reference max before the
// max of t is known; when the lazy rescale then moves the reference (rare:
// the first sub-tile of a row, or a max that grows by more than 2^8) they
// are recomputed.  Masking of t's scores sits between the two regions.
template <int BETA, int D, bool NBM>
__device__ __forceinline__ void step8(const uint8_t *__restrict__ Kc, const uint8_t *__restrict__ Vp,
                                      uint8_t *__restrict__ Kn, uint8_t *__restrict__ Vn, const F8Tile &cur,
                                      const F8Tile &prv, bool load_k, int k0_k, __amdgpu_buffer_rsrc_t krs,
                                      __amdgpu_buffer_rsrc_t vrs, uint32_t vstep, const Fp8FwdParams &p, int wv,
                                      int lane, F8State<BETA, D> &st, f32x16 (&s_cur)[2], f32x16 (&s_prev)[2],
                                      i32x8 &pf_prev, i32x8 &pf_cur)
{
    using Sh = F8Shape<BETA, D>;
    if (load_k) load_k8<BETA, D>(Kn, krs, st.kdma, p.N, k0_k, wv, lane);
    load_v8<BETA, D>(Vn, vrs, st.vdma, vstep, p.NP, cur.k0, wv);
    constexpr int QK = 2 * Sh::KS, PV = Sh::DT + 1;
    qk8<BETA, D>(Kc, st, s_cur);
    probs_half<1>(s_prev, prv.c, st.m_run, pf_prev);        // 16 exp, ~24 other
    interleave<2, QK, 2, (24 + QK - 1) / QK, (16 + QK - 1) / QK>();
    __builtin_amdgcn_sched_barrier(0);
    // the packed probabilities are used after the masking branch; without
    // this use the compiler sinks their computation past it, out of region A
    asm volatile("" ::"v"(pf_prev));
    mask_scores8(cur.valid, cur.k0, p.N, lane, s_cur);
    if (NBM && cur.partial && st.qimg) mask_window8<BETA>(p.nb, cur.k0, st.wr0, st.wc0, lane, s_cur);
    pv8<BETA, D>(Vp, pf_prev, st);
    const bool has_keys = cur.valid && cur.k0 < p.N;
    const float mx = tile_max(s_cur, cur.c) + (has_keys ? 0.f : -INFINITY);
    probs_half<0>(s_cur, cur.c, st.m_run, pf_cur);           // 16 exp, ~44 other with the max
    interleave<2, PV, 2, (44 + PV - 1) / PV, (16 + PV - 1) / PV>();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::"v"(pf_cur), "v"(mx));
    if (lazy_rescale8<BETA, D>(mx, st)) probs_half<0>(s_cur, cur.c, st.m_run, pf_cur);
}

// Occupancy target (waves per SIMD): two, so that a wave's accumulators,
// scores of two sub-tiles and Q codes fit its registers without spilling.
template <int BETA, int D, bool NBM>
__global__ __launch_bounds__(BETA / 32 * 64, 2) void fwd8_kernel(const Fp8FwdParams p)
{
    using Sh = F8Shape<BETA, D>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[4 * Sh::TILE];
    uint8_t *const K0 = smem, *const V0 = smem + Sh::TILE;
    uint8_t *const K1 = smem + 2 * Sh::TILE, *const V1 = smem + 3 * Sh::TILE;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hl = lane >> 5;
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
    const int b = bh / p.H, hh = bh - b * p.H;
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
    const int T = (e1 > e0 ? e1 - e0 : 0) * Sh::SUB;

    F8State<BETA, D> st;
    const int qrow = i * BETA + wv * 32 + n;
    const int64_t qtok = (int64_t)bh * p.N + qrow;
    float qs = 0.f;
#pragma unroll
    for (int ks = 0; ks < Sh::KS; ++ks)
#pragma unroll
        for (int j = 0; j < 8; ++j) st.qf[ks][j] = 0;
    if (qrow < p.N) {
        const uint8_t *qp = p.q8 + qtok * D + 32 * hl;
#pragma unroll
        for (int ks = 0; ks < Sh::KS; ++ks)
            st.qf[ks] = lds_i32x8(qp + 64 * ks, 0, 16);   // (global: plain 16-byte loads)
        qs = p.q_scale[qtok];
    }
    st.cq = p.scale_log2 * qs;
    st.qimg = NBM && qrow < p.N && qrow >= p.nb.T;
    st.wr0 = st.wc0 = 0;
    if (NBM && st.qimg) {
        const int pq = qrow - p.nb.T, tq = pq / BETA, oq = pq - tq * BETA, aq = tq / p.nb.tpr;
        const int rq = aq * p.nb.th + (oq >> p.nb.tw_log2), cq = (tq - aq * p.nb.tpr) * p.nb.tw + (oq & (p.nb.tw - 1));
        st.wr0 = nb_start(rq, p.nb.R, p.nb.kh, p.nb.sh);
        st.wc0 = nb_start(cq, p.nb.C, p.nb.kw, p.nb.sw);
    }
#pragma unroll
    for (int d = 0; d < Sh::DT; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.oacc[d][r] = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) st.lacc[r] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) st.ones[j] = 0x38383838;
    // opaque to the compiler: otherwise it keeps one copy and rebuilds the
    // 8-register operand before every row-sum MFMA
    asm volatile("" : "+v"(st.ones));
    st.m_run = -1.0e30f;

    st.kread = (uint32_t)(n * D + 16 * (k8swz<D>(n) ^ (2 * hl)));
    st.vread = (uint32_t)(n * 64 + 16 * (v8swz(n) ^ (2 * hl)));
    {
        const int slot = wv * 64 + lane;
        const int kr = slot / Sh::KCH, kp = slot % Sh::KCH;
        st.kdma = (uint32_t)(kr * D + 16 * (kp ^ k8swz<D>(kr)));
        const int vr = slot >> 2, vp = slot & 3;
        st.vdma = (uint32_t)(vr * p.NP + 16 * (vp ^ v8swz(vr)));
    }
    const uint32_t vstep = (uint32_t)(Sh::NT / 4) * (uint32_t)p.NP;

    const __amdgpu_buffer_rsrc_t krs = buffer_desc(p.k8 + (int64_t)bh * p.N * D, (uint32_t)(p.N * D));
    const __amdgpu_buffer_rsrc_t vrs = buffer_desc(p.v8t + (int64_t)bh * D * p.NP, (uint32_t)(D * p.NP));

    // wave-uniform block indices and K tile scales through scalar loads
    const __attribute__((address_space(4))) int32_t *cidx =
        (const __attribute__((address_space(4))) int32_t *)(p.col_idx + e0);
    const __attribute__((address_space(4))) int32_t *cflag =
        (const __attribute__((address_space(4))) int32_t *)(NBM ? p.flags + e0 : p.col_idx);
    const __attribute__((address_space(4))) float *kscl =
        (const __attribute__((address_space(4))) float *)(p.k_scale + (int64_t)bh * p.NT);
    auto tile = [&](int t) {
        F8Tile x;
        const int j = cidx[t / Sh::SUB];
        x.valid = (unsigned)j < (unsigned)p.nB;
        x.k0 = (x.valid ? j * BETA : 0) + 64 * (t % Sh::SUB);
        const float ks = kscl[min(x.k0 >> 6, p.NT - 1)];
        // a zero scale means all-zero codes; any positive c gives the same
        // scores and keeps -inf * c a -inf for masked keys
        x.c = fmaxf(st.cq * ks, 1.17549435e-38f);
        x.partial = NBM && cflag[t / Sh::SUB] != 0;
        return x;
    };
    const F8Tile none = {0, false, 1.f, false};

    f32x16 sa[2], sb[2];
    i32x8 pa, pb;
    if (T > 0) {
        F8Tile cur = tile(0), nxt = none, prv;
        if (T > 1) nxt = tile(1);
        load_k8<BETA, D>(K0, krs, st.kdma, p.N, cur.k0, wv, lane);
        __syncthreads();
        // first step: S^T(0), its max and the probabilities of keys 0..31;
        // copies K(1) and V(0)
        if (T > 1) load_k8<BETA, D>(K1, krs, st.kdma, p.N, nxt.k0, wv, lane);
        load_v8<BETA, D>(V0, vrs, st.vdma, vstep, p.NP, cur.k0, wv);
        qk8<BETA, D>(K0, st, sa);
        mask_scores8(cur.valid, cur.k0, p.N, lane, sa);
        if (NBM && cur.partial && st.qimg) mask_window8<BETA>(p.nb, cur.k0, st.wr0, st.wc0, lane, sa);
        lazy_rescale8<BETA, D>((cur.valid && cur.k0 < p.N) ? tile_max(sa, cur.c) : -INFINITY, st);
        probs_half<0>(sa, cur.c, st.m_run, pa);
        __syncthreads();
        prv = cur;
        cur = nxt;
        for (int t = 1; t < T; t += 2) {
            nxt = none;
            if (t + 1 < T) nxt = tile(t + 1);
            step8<BETA, D, NBM>(K1, V0, K0, V1, cur, prv, t + 1 < T, nxt.k0, krs, vrs, vstep, p, wv, lane, st, sb, sa,
                           pa, pb);
            __syncthreads();
            prv = cur;
            cur = nxt;
            if (t + 1 >= T) break;
            nxt = none;
            if (t + 2 < T) nxt = tile(t + 2);
            step8<BETA, D, NBM>(K0, V1, K1, V0, cur, prv, t + 2 < T, nxt.k0, krs, vrs, vstep, p, wv, lane, st, sa, sb,
                           pb, pa);
            __syncthreads();
            prv = cur;
            cur = nxt;
        }
        // last sub-tile: keys 32..63 of its probabilities and the O update
        // (V(T-1) in V[(T-1)&1], scores already masked)
        if (T & 1) {
            probs_half<1>(sa, prv.c, st.m_run, pa);
            pv8<BETA, D>(V0, pa, st);
        } else {
            probs_half<1>(sb, prv.c, st.m_run, pb);
            pv8<BETA, D>(V1, pb, st);
        }
    }

    const float l_tot = st.lacc[0];
    if (rank >= 0) {
        // a chunk of a split row: park the output (channel scales applied,
        // not normalised) and the (reference max, sum) of every query
        float *slot = p.partials + ((int64_t)rank * p.max_chunks + chunk) * partial_slot_floats(BETA, D);
        const int tq = wv * 32 + n;
        const float *vs = p.v_scale + (int64_t)bh * D;
#pragma unroll
        for (int d = 0; d < Sh::DT; ++d)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c0 = d * 32 + 8 * g + 4 * hl;
                const float4 s4 = *reinterpret_cast<const float4 *>(vs + c0);
                *reinterpret_cast<float4 *>(slot + partial_o_index(BETA, c0, tq)) =
                    make_float4(st.oacc[d][4 * g + 0] * s4.x, st.oacc[d][4 * g + 1] * s4.y,
                                st.oacc[d][4 * g + 2] * s4.z, st.oacc[d][4 * g + 3] * s4.w);
            }
        if (hl == 0) {
            slot[BETA * D + tq] = st.m_run;
            slot[BETA * D + BETA + tq] = l_tot;
        }
        return;
    }
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (qrow < p.N) {
        // natural-order outputs of a neighbourhood layout: the query's grid position
        const int qpos = (NBM && p.natural) ? nb_natural(p.nb, BETA, qrow) : qrow;
        uint16_t *orow = p.o + b * p.o_sb + hh * p.o_sh + (int64_t)qpos * p.o_sn;
        const float *vs = p.v_scale + (int64_t)bh * D;
#pragma unroll
        for (int d = 0; d < Sh::DT; ++d)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c0 = d * 32 + 8 * g + 4 * hl;
                const float4 s4 = *reinterpret_cast<const float4 *>(vs + c0);
                uint2 sv;
                sv.x = pack_bf16x2(st.oacc[d][4 * g + 0] * (s4.x * inv), st.oacc[d][4 * g + 1] * (s4.y * inv));
                sv.y = pack_bf16x2(st.oacc[d][4 * g + 2] * (s4.z * inv), st.oacc[d][4 * g + 3] * (s4.w * inv));
                *reinterpret_cast<uint2 *>(orow + c0) = sv;
            }
        if (p.lse && hl == 0)
            p.lse[(int64_t)bh * p.N + qpos] = l_tot > 0.f ? (st.m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
}

template <int BETA, int D>
static hipError_t launch_fwd8_t(const Fp8FwdParams &p, int64_t grid, hipStream_t s)
{
    using Sh = F8Shape<BETA, D>;
    if (grid == 0) return hipSuccess;
    if (p.flags)
        hipLaunchKernelGGL((fwd8_kernel<BETA, D, true>), dim3((unsigned)grid), dim3(Sh::NT), 0, s, p);
    else
        hipLaunchKernelGGL((fwd8_kernel<BETA, D, false>), dim3((unsigned)grid), dim3(Sh::NT), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_forward_fp8(const Fp8FwdParams &p, int block, int D, int64_t grid, hipStream_t s)
{
    if (block == 128 && D == 128) return launch_fwd8_t<128, 128>(p, grid, s);
    if (block == 128 && D == 64) return launch_fwd8_t<128, 64>(p, grid, s);
    if (block == 64 && D == 128) return launch_fwd8_t<64, 128>(p, grid, s);
    if (block == 64 && D == 64) return launch_fwd8_t<64, 64>(p, grid, s);
    return hipErrorInvalidValue;
}

}  // namespace bsa
