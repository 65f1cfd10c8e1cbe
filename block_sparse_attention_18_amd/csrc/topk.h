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

// Top-k of the column group [c0, c1) (kk < c1 - c0) for R rows at once,
// with the scores in registers in absolute column order: s[q][e] is the
// score of row q at column 64 e + lane.  Columns outside the group get key
// 0 and are never counted (every probe value is at least 1) nor kept.
// Sets the kept bits of row q in wb[q] (words of 32 columns).
template <int E, int R>
__device__ void select_rows(const float (&s)[R][E], int c0, int c1, int kk, uint32_t *const (&wb)[R])
{
    const int lane = threadIdx.x & 63;
    uint32_t key[R][E];
#pragma unroll
    for (int q = 0; q < R; ++q)
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int col = e * 64 + lane;
            key[q][e] = (col >= c0 && col < c1) ? score_key(s[q][e]) : 0u;
        }
    uint32_t T[R];
    bool live[R];
#pragma unroll
    for (int q = 0; q < R; ++q) {
        T[q] = 0u;
        live[q] = true;
    }
    // the rows' searches run in lockstep; a row stops at its first probe
    // with exactly kk keys at or above it (as in select_group)
    for (int bit = 31; bit >= 0; --bit) {
        bool any = false;
#pragma unroll
        for (int q = 0; q < R; ++q) {
            if (!live[q]) continue;
            const uint32_t cand = T[q] | (1u << bit);
            int cnt = 0;
#pragma unroll
            for (int e = 0; e < E; ++e) cnt += ballot_count(key[q][e] >= cand);
            if (cnt >= kk) {
                T[q] = cand;
                live[q] = cnt != kk;
            }
            any = any || live[q];
        }
        if (!any) break;
    }
#pragma unroll
    for (int q = 0; q < R; ++q) {
        int need = kk;
#pragma unroll
        for (int e = 0; e < E; ++e) need -= ballot_count(key[q][e] > T[q]);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int col = e * 64 + lane;
            const bool inside = col >= c0 && col < c1;
            const uint64_t eq = __ballot(inside && key[q][e] == T[q]);
            const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(eq >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)eq, 0));
            const bool keep = inside && (key[q][e] > T[q] || (key[q][e] == T[q] && rank < need));
            need -= __popcll(eq);
            const uint64_t K = __ballot(keep);
            if (K != 0ull && lane < 2) {
                const uint32_t v = lane == 0 ? (uint32_t)K : (uint32_t)(K >> 32);
                if (v) atomicOr(&wb[q][2 * e + lane], v);
            }
        }
    }
}

// Write the set bits of a row bitmask of nB columns as ascending column
// indices from col_idx[start] (entries at or past capacity are dropped): a
// lane per column, 64 columns a round, each position from the lanes below.
__device__ __forceinline__ void write_row_columns(const uint32_t *wb, int nB, int64_t start, int32_t *col_idx,
                                                  int64_t capacity)
{
    const int lane = threadIdx.x & 63;
    for (int c0 = 0; c0 < nB; c0 += 64) {
        const int col = c0 + lane;
        const bool on = col < nB && ((wb[col >> 5] >> (col & 31)) & 1u);
        const uint64_t m = __ballot(on);
        const int64_t pos =
            start + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
        if (on && pos < capacity) col_idx[pos] = col;
        start += __popcll(m);
    }
}

}  // namespace bsa
