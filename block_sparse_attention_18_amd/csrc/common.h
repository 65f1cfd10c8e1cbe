// Device-side helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b)
{
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even float -> bfloat16 pair packed in one dword
// (lowers to v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v;
    v[0] = static_cast<__bf16>(lo);
    v[1] = static_cast<__bf16>(hi);
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wait for this wave's outstanding vector-memory operations, its
// global-to-LDS tile copies among them.  Every wave calls it right before
// the barrier that hands a copied tile to the other waves: the barrier does
// not wait for copies in flight, and the compiler does not place this wait
// by itself in every loop shape (without it, a wave could read a tile whose
// copy by another wave had not landed).
__device__ __forceinline__ void wait_tile_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8 &a, const bf16x8 &b, const f32x16 &c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint4 zero_u4() { return make_uint4(0u, 0u, 0u, 0u); }

// 16-byte global load of 8 bfloat16 values.
__device__ __forceinline__ uint4 ld_g16(const uint16_t *p)
{
    return *reinterpret_cast<const uint4 *>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4 &u) { return __builtin_bit_cast(bf16x8, u); }

// Wave-wide (64 lanes) inclusive prefix sum of an int.
// x / r for 0 <= x < 2^20 and 1 <= r <= 64 by one fp32 multiply: (x + 0.5)
// / r lies at least 0.5 / r from every integer, far more than the rounding
// of the product and of inv_r = 1 / r.
__device__ __forceinline__ int div_small(int x, float inv_r)
{
    return (int)(((float)x + 0.5f) * inv_r);
}

__device__ __forceinline__ int wave_incl_scan(int x)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    return x;
}

// Row of the K tile fed to A-operand row n of a 32-key sub-tile.
__device__ __forceinline__ int perm_row(int n)
{
    return (n & ~12) | ((n & 4) << 1) | ((n & 8) >> 1);
}

// XOR swizzles of the 16-byte chunk index within a row of the K and V tiles.
// K: the 16 rows read by one quarter-wave land on 16 distinct chunk slots.
// V: the 4 rows x 4 chunks read by one half-wave transpose load land on 16
// distinct chunk slots.  (Rows are 256 B for D = 128, 128 B for D = 64.)
template <int D>
__device__ __forceinline__ int kswz(int row)
{
    return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int vswz(int row)
{
    return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// Raw buffer resource over `bytes` bytes from `base` (gfx9 format word).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_desc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}


template <typename T>
__device__ __forceinline__ const T *lds_at(const uint16_t *base, uint32_t byte_off)
{
    return reinterpret_cast<const T *>(reinterpret_cast<const char *>(base) + byte_off);
}

// The swizzles XOR the chunk index with row bits, so stepping the chunk by
// a power of two that the swizzle also touches is an XOR of the byte offset:
// K k-step s moves 2 chunks (32 bytes), V d tile d moves 4 chunks (64 bytes).
constexpr uint32_t KSTEP = 32, VSTEP = 64;

// Accumulator row r of half-wave hl of a 32x32 S^T tile (K rows fed in the
// perm_row order) holds key 8 hl + koff(r) of its 32 keys.
__device__ __forceinline__ constexpr int koff(int r) { return (r & 3) + 4 * ((r >> 2) & 1) + 16 * ((r >> 3) & 1); }

// x if bit c of w is set, else -inf, without a branch: the sign-extended
// bit selects between the two bit patterns.
__device__ __forceinline__ float keep_if_bit(float x, uint32_t w, int c)
{
    const int m = (int)(w << (31 - c)) >> 31;
    return __int_as_float((__float_as_int(x) & m) | ((int)0xff800000 & ~m));
}

// Scores of keys at offset >= lim (per lane: key offset within the 64-key
// sub-tile minus 8 hl) become -inf.
__device__ __forceinline__ void mask_keys(f32x16 (&sacc)[2], int lim)
{
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (kt * 32 + koff(r) >= lim) sacc[kt][r] = -INFINITY;
}

// Max over a 64-key sub-tile of S^T for the lane's query, times c: the two
// lane halves hold the two key halves of every query and are combined by a
// lane swap (a VALU op, no LDS round trip).
__device__ __forceinline__ float tile_max(const f32x16 (&sacc)[2], float c)
{
    float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        m0 = fmaxf(m0, sacc[0][r]);
        m1 = fmaxf(m1, sacc[1][r]);
    }
    const float mx = fmaxf(m0, m1);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * c;
}

// Sum of a value over the two lane halves (lanes l and l ^ 32).
__device__ __forceinline__ float half_sum(float x)
{
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// Instruction interleave of one scheduled region: NPRE LDS reads first, then
// NM groups of one MFMA, NR LDS reads, NV vector and NE transcendental
// instructions.  A waiting MFMA holds the SIMD's issue stage, so vector work
// is spread between the MFMAs of the same wave rather than run beside a
// back-to-back MFMA chain.
template <int NPRE, int NM, int NR, int NV, int NE>
__device__ __forceinline__ void interleave()
{
    __builtin_amdgcn_sched_group_barrier(0x100, NPRE, 0);
#pragma unroll
    for (int x = 0; x < NM; ++x) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
        __builtin_amdgcn_sched_group_barrier(0x400, NE, 0);
    }
}

}  // namespace bsa
