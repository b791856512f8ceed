// Device helpers shared by the gfx950 kernels of libep_mi355x (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ep {

constexpr int kWave = 64;   // CDNA wavefront width

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// A 16-byte chunk: 8 bf16 channels, or 16 FP8 codes. NT selects the non-temporal form, which
// streams past the caches; whether it pays depends on the access pattern (measured per kernel).
template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4 *p)
{
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

template <bool NT>
__device__ __forceinline__ void store16(u32x4 *p, u32x4 v)
{
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// bf16 pattern in the low / high half of a 32-bit word -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 pattern, round to nearest even. Adding 0x7FFF plus the kept LSB carries into
// the upper half exactly when the dropped half is above the midpoint, or at it with an odd
// LSB; overflow past the largest finite value carries into the infinity pattern. Every NaN
// gives the one quiet NaN 0x7FC0 (the sign and payload of a NaN that an fp32 sum produces are
// not fixed by IEEE 754, so a NaN result is written as that single pattern).
__device__ __forceinline__ uint32_t bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    return ((u & 0x7FFFFFFFu) > 0x7F800000u) ? 0x7FC0u : r;
}

// fp32 -> OCP E4M3 code, round to nearest even, saturating at +-448 (NaN -> S.1111.111).
//  * |v| >= 448 (or inf): 0x7E.
//  * normal range [2^-6, 448): keep 3 mantissa bits by adding half an E4M3 ulp (2^19 in the
//    fp32 mantissa) minus one plus the kept LSB, then shifting; a carry moves into the
//    exponent, which is then rebiased from 127 to 7 (subtract 120 << 3).
//  * below 2^-6 the E4M3 step is 2^-9: the code is the integer nearest to |v| * 2^9 (exact
//    scaling), rounded half to even by v_rndne; 8 gives 0x08, the smallest normal.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float v)
{
    uint32_t u = __float_as_uint(v);
    uint32_t sign = (u >> 24) & 0x80u;
    uint32_t a = u & 0x7FFFFFFFu;
    uint32_t code;
    if (a > 0x7F800000u) {
        code = 0x7Fu;
    } else if (a >= 0x43E00000u) {              // 448.0f
        code = 0x7Eu;
    } else if (a >= 0x3C800000u) {              // 2^-6
        uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
        code = r - (120u << 3);
    } else {
        code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
    }
    return sign | code;
}

// OCP E4M3 codes of four fp32 values, packed little-endian (v0 in the low byte), by gfx950's
// conversion instruction (round to nearest even). Checked over all 2^32 fp32 inputs on MI355X:
// equal to e4m3_rne_sat for every finite |v| <= 464, including e4m3 subnormals and fp32
// denormals; it differs only for NaN (always 0xFF) and |v| > 464 (NaN instead of saturating),
// which its callers never pass.
__device__ __forceinline__ uint32_t e4m3_pack4(float v0, float v1, float v2, float v3)
{
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, lo, true);
}

// RN(x / d) for d > 0 given y = RN(1 / d), without a division: q = x*y, then two remainder
// corrections q += (x - d*q)*y, each remainder exact by FMA. After the first, q is within one
// ulp of x/d; then, with y the correctly rounded reciprocal, the second gives the correctly
// rounded quotient (Markstein's theorem on division by FMA). It needs the remainders not to
// underflow: true when |x / d| >= 2^-11 and d >= 2^-60 / 448; below that the result is still
// within a denormal step of x/d. The sign is x's (a zero sum in a correction rounds to +0).
__device__ __forceinline__ float div_by_rcp(float x, float d, float y)
{
    float q = __fmul_rn(x, y);
    q = __builtin_fmaf(__builtin_fmaf(-d, q, x), y, q);
    q = __builtin_fmaf(__builtin_fmaf(-d, q, x), y, q);
    return __builtin_copysignf(q, x);
}

// Row of pair (e, s) in the receive buffer, or -1 if it is not kept: e*C + s in the padded
// [E][C] layout, offset[e] + s (below `rows`) in a packed one.
__device__ __forceinline__ int pair_row(int e, int s, int E, int C, const int32_t *offset,
                                        int rows)
{
    if ((unsigned)e >= (unsigned)E || (unsigned)s >= (unsigned)C) return -1;
    if (!offset) return e * C + s;
    const int r = offset[e] + s;
    return (unsigned)r < (unsigned)rows ? r : -1;
}

// Number of set bits of `mask` in lanes below this one (v_mbcnt).
__device__ __forceinline__ int count_below(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// DPP move of `v` from the lane n below within the same row of 16 lanes; 0 past the row start.
template <int N>
__device__ __forceinline__ int row_shr(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, 0x110 + N, 0xF, 0xF, true);
}

// Inclusive prefix sum within each row of 16 lanes (4 DPP steps, no LDS).
__device__ __forceinline__ int row16_inclusive_sum(int v)
{
    v += row_shr<1>(v);
    v += row_shr<2>(v);
    v += row_shr<4>(v);
    v += row_shr<8>(v);
    return v;
}

// Inclusive prefix sum across the 64 lanes: per-row scans, then the last lane of row 0 (row
// 2) is broadcast into row 1 (row 3) and the last lane of row 1 into rows 2 and 3.
__device__ __forceinline__ int wave_inclusive_sum(int v)
{
    v = row16_inclusive_sum(v);
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31
    return v;
}

// Max over aligned groups of 8 lanes, with DPP moves: swap neighbours (quad_perm 1,0,3,2),
// swap pairs (quad_perm 2,3,0,1), then mirror within each half-row of 8 lanes.
__device__ __forceinline__ float group8_max(float v)
{
    int x = __float_as_int(v);
    x = max(x, __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false));
    x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false));
    x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x141, 0xF, 0xF, false));
    return __int_as_float(x);   // inputs are non-negative floats: integer order = value order
}

// The tile this workgroup takes. Workgroups go to the 8 XCDs round-robin (blockIdx mod 8), some
// XCDs write more slowly than others, and a tile's layout pass grows with its position.
// ORDER = 1: the odd XCDs take the first half of the tiles (the cheaper layouts) and the even
// ones the second half; ORDER = 2 the other way round; each XCD's tiles interleaved with its
// three peers'. A bijection on [0, gridDim.x) when gridDim.x is a multiple of 8, else the
// identity; ORDER = 0: the identity.
template <int ORDER>
__device__ __forceinline__ int xcd_tile()
{
    if constexpr (ORDER != 0) {
        const int n = gridDim.x, b = blockIdx.x;
        if ((n & 7) != 0) return b;
        const int x = b & 7, i = b >> 3;
        const bool first_half = (x & 1) == (ORDER == 1 ? 1 : 0);
        return (first_half ? 0 : n / 2) + 4 * i + (x >> 1);
    }
    return blockIdx.x;
}

}  // namespace ep
