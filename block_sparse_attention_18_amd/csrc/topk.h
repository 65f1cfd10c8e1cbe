// Top-k of a column group inside one wavefront (see select.hip): device
// helpers shared by the selection kernel and the fused pool-score-select
// kernel.
#pragma once

#include "common.h"

namespace bsa {

// Order-preserving key of a score: larger score, larger key; -0.0 ranks
// equal to +0.0; NaN ranks below every number (key 0, like padding).
__device__ __forceinline__ uint32_t score_key(float s)
{
    if (s == 0.f) s = 0.f;
    uint32_t u = __float_as_uint(s);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return (s != s) ? 0u : u;
}

__device__ __forceinline__ int ballot_count(bool x) { return __popcll(__ballot(x)); }

__device__ __forceinline__ int lanes_below(uint64_t m)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

// AND and OR of a value over the 64 lanes of a wavefront (uniform results):
// each 16-lane row folds into its lane 15 by DPP row shifts (a shifted-in
// lane reads the identity), lanes 15 and 31 are broadcast into the rows
// above them, and lane 63 holds the result.
__device__ __forceinline__ void wave_and_or(uint32_t &a, uint32_t &o)
{
    a &= __builtin_amdgcn_update_dpp(~0u, a, 0x111, 0xf, 0xf, false);     // row_shr:1
    o |= __builtin_amdgcn_update_dpp(0u, o, 0x111, 0xf, 0xf, false);
    a &= __builtin_amdgcn_update_dpp(~0u, a, 0x112, 0xf, 0xf, false);     // row_shr:2
    o |= __builtin_amdgcn_update_dpp(0u, o, 0x112, 0xf, 0xf, false);
    a &= __builtin_amdgcn_update_dpp(~0u, a, 0x114, 0xf, 0xf, false);     // row_shr:4
    o |= __builtin_amdgcn_update_dpp(0u, o, 0x114, 0xf, 0xf, false);
    a &= __builtin_amdgcn_update_dpp(~0u, a, 0x118, 0xf, 0xf, false);     // row_shr:8
    o |= __builtin_amdgcn_update_dpp(0u, o, 0x118, 0xf, 0xf, false);
    a &= __builtin_amdgcn_update_dpp(~0u, a, 0x142, 0xa, 0xf, false);     // row_bcast:15
    o |= __builtin_amdgcn_update_dpp(0u, o, 0x142, 0xa, 0xf, false);
    a &= __builtin_amdgcn_update_dpp(~0u, a, 0x143, 0xc, 0xf, false);     // row_bcast:31
    o |= __builtin_amdgcn_update_dpp(0u, o, 0x143, 0xc, 0xf, false);
    a = __builtin_amdgcn_readlane(a, 63);
    o = __builtin_amdgcn_readlane(o, 63);
}

// Number of keys >= cand over the wavefront.  Each register's compare gives
// a 64-lane mask in scalar registers; for a group of four or more registers
// the scalar unit (one per CU, shared by its four SIMDs) counts half of the
// masks and the vector unit the other half (v_bcnt of the two mask halves
// into a lane-uniform sum), so that the two issue ports split the work of a
// search round; one or two registers are counted by the scalar unit alone
// (a shorter dependency chain).
template <int E>
__device__ __forceinline__ int count_at_least(const uint32_t (&key)[E], uint32_t cand)
{
    constexpr int EV = E >= 4 ? E / 2 : 0;
    int s = 0;
    uint32_t acc = 0u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const uint64_t m = __ballot(key[e] >= cand);
        if (e < E - EV) {
            s += __popcll(m);
        } else {
            // the mask was just written by a vector compare: a vector read of
            // it needs two wait states, which the compiler does not insert
            // ahead of an asm statement
            asm("s_nop 1\n\tv_bcnt_u32_b32 %0, %1, %0\n\tv_bcnt_u32_b32 %0, %2, %0"
                : "+v"(acc)
                : "s"((uint32_t)m), "s"((uint32_t)(m >> 32)));
        }
    }
    if (EV > 0) s += __builtin_amdgcn_readfirstlane(acc);
    return s;
}

// Top kk of the column group [c0, c1) (0 < kk < c1 - c0), written as
// ascending column indices from col_idx[pos] (entries at or past capacity
// are dropped).  key[e] is the key of column cbase + 64 e + lane, 0 for a
// column outside the group (no probe, which is >= 1, counts it).
//
// The bits of T, the kk-th largest key, are decided from the top: a probe
// cand = T | bit is taken when at least kk keys are >= cand.  Alongside, the
// search keeps the number of keys whose leading (decided) bits exceed T's:
// it becomes the count of a rejected probe and is unchanged by a taken one,
// so after the last bit it is the number of keys > T, and the keys equal to
// T that are kept (lowest columns first) need no further count.  The search
// stops early at a probe with exactly kk keys at or above it: the kept set
// is then the keys >= T.
template <int E>
__device__ void topk_keys_write(const uint32_t (&key)[E], int cbase, int c0, int c1, int kk, int32_t *col_idx,
                                int64_t pos, int64_t capacity)
{
    const int lane = threadIdx.x & 63;
    // Above the highest bit where two of the group's keys differ, every probe
    // is decided without a count: all keys share those bits, so T has them
    // too and no key exceeds T there.  The search starts at that bit.
    uint32_t a = ~0u, o = 0u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int col = cbase + e * 64 + lane;
        a &= ((col >= c0) & (col < c1)) ? key[e] : ~0u;
        o |= key[e];                            // 0 outside the group
    }
    wave_and_or(a, o);
    const uint32_t dx = a ^ o;
    uint32_t T, probe;
    int above = 0, cnt;
    if (dx == 0u) {                             // all keys equal: the first kk columns
        T = a;
        probe = 0u;
        cnt = c1 - c0;
    } else {
        const int h = 31 - __builtin_clz(dx);
        T = a & ~((2u << h) - 1u);
        probe = 1u << h;
    }
    while (probe != 0u) {
        const uint32_t cand = __builtin_amdgcn_readfirstlane(T | probe);
        cnt = count_at_least<E>(key, cand);
        const bool take = cnt >= kk;
        T = take ? cand : T;
        above = take ? above : cnt;
        probe = cnt == kk ? 0u : probe >> 1;
        asm("" : "+s"(probe));      // one scalar test ends the loop
    }
    // keys equal to T to keep, lowest columns first (all of them when exact)
    int need = cnt == kk ? 0x7fffffff : kk - above;
    int at0 = (int)pos;                         // CSR positions fit in int32
    const int cap = (int)min(capacity, (int64_t)0x7fffffff);
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int col = cbase + e * 64 + lane;
        const bool eq = (col >= c0) & (col < c1) & (key[e] == T);
        const uint64_t me = __ballot(eq);
        const bool keep = (key[e] > T) | (eq & (lanes_below(me) < need));
        need -= __popcll(me);
        const uint64_t K = __ballot(keep);
        const int at = at0 + lanes_below(K);
        if (keep & (at < cap)) col_idx[at] = col;
        at0 += __popcll(K);
    }
}

// topk_keys_write for a group whose scores sit in LDS (srow[c] is column c):
// lane l takes columns c0 + 64 e + l.
template <int E>
__device__ void topk_write(const float *srow, int c0, int c1, int kk, int32_t *col_idx, int64_t pos,
                           int64_t capacity)
{
    const int lane = threadIdx.x & 63;
    uint32_t key[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int col = c0 + e * 64 + lane;
        key[e] = col < c1 ? score_key(srow[col]) : 0u;
    }
    topk_keys_write<E>(key, c0, c0, c1, kk, col_idx, pos, capacity);
}

// Keep the kk best columns of [c0, c1) (kk < c1 - c0): set their bits in the
// row bitmask wbits.  Columns past c1 are padding with key 0 and the highest
// columns, so they never reach the kept set.
template <int E>
__device__ void select_group(const float *srow, int c0, int c1, int kk, uint32_t *wbits, int words)
{
    const int lane = threadIdx.x & 63;
    uint32_t key[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int col = c0 + e * 64 + lane;
        key[e] = col < c1 ? score_key(srow[col]) : 0u;
    }
    // T = the kk-th largest key: the largest value with >= kk keys at or
    // above it.  The search may stop at the first probe with exactly kk keys
    // at or above it: the kept set (below) is then those kk keys.
    uint32_t T = 0u;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = T | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) cnt += ballot_count(key[e] >= cand);
        if (cnt >= kk) {
            T = cand;
            if (cnt == kk) break;
        }
    }
    int need = kk;
#pragma unroll
    for (int e = 0; e < E; ++e) need -= ballot_count(key[e] > T);
    // keys above T, then keys equal to T in column order until kk are kept
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const uint64_t eq = __ballot(key[e] == T);
        const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(eq >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)eq, 0));
        const bool keep = key[e] > T || (key[e] == T && rank < need);
        need -= __popcll(eq);
        const uint64_t K = __ballot(keep);
        // bits 0..63 of K stand for columns c0 + 64 e .. +63: or them into
        // the (up to three) bitmask words they straddle
        const int pos = c0 + e * 64, w0 = pos >> 5, sh = pos & 31;
        const uint64_t lo = K << sh;
        const uint32_t hi = sh ? (uint32_t)(K >> (64 - sh)) : 0u;
        if (K != 0ull && lane < 3) {
            const uint32_t v = lane == 0 ? (uint32_t)lo : lane == 1 ? (uint32_t)(lo >> 32) : hi;
            if (v && w0 + lane < words) atomicOr(&wbits[w0 + lane], v);
        }
    }
}

// Keep every column of [c0, c1).
__device__ void select_all(int c0, int c1, uint32_t *wbits)
{
    for (int col = c0 + (int)(threadIdx.x & 63); col < c1; col += 64) atomicOr(&wbits[col >> 5], 1u << (col & 31));
}

}  // namespace bsa
