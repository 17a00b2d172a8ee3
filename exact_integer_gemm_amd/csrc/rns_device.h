// Device helpers shared by the gfx950 kernels of librns_gemm: vector types,
// the exact rounding steps that reduce mod q, and byte packing.
//
// Every reduction mod q is one exact rounding step: t - q * round(t / q) is
// the balanced residue of t for odd q.  round(t / q) is formed from fl(1/q) by
// a fused multiply-add with 1.5 * 2^52 (binary64, any int32 t: the relative
// error 2^-53 moves t/q by less than 2^-22, while t/q stays at least 1/(2q)
// from every half-integer) or with 1.5 * 2^23 (binary32, |t| < 2^22), which
// leaves the rounded quotient in the low bits of the result.  q = 2 is
// handled separately (the low bit).
#pragma once

#include <hip/hip_runtime.h>

#include "rns_internal.h"

namespace rns {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

// The residue split reduces values |t| < 2^22, for which binary32 suffices:
// fl(1/q) moves t/q by less than 1/(4q), and adding 1.5 * 2^23 in the fused
// multiply-add leaves 0x400000 + round(t/q) in the low 24 bits of the result,
// which __mul24 reads as a signed 24-bit value.  The result is t - q *
// round(t/q) - q * 2^22, exact in its low byte (q * 2^22 = 0 mod 256).
__device__ __forceinline__ int reduce_low_byte_f32(int t, int q, float inv) {
    return __mul24(__float_as_int(__builtin_fmaf((float)t, inv, kRoundMagic32)), -q) + t;
}

// round(t / q) as a 32-bit integer, for |t| < 2^31 and odd q (exact).
__device__ __forceinline__ int round_div(int t, double inv) {
    const double g = __builtin_fma((double)t, inv, kRoundMagic);
    return (int)(uint32_t)__double_as_longlong(g);
}

// t - q * round(t / q): the balanced residue of t, exact for |t| < 2^23 and odd q.
__device__ __forceinline__ int reduce_exact(int t, int q, double inv) {
    return __mul24(round_div(t, inv), -q) + t;
}

// The same expression for any |t| < 2^31: the 24-bit product wraps, but
// only mod 2^24, so the low byte (the int8 residue that is stored) is exact.
__device__ __forceinline__ int reduce_low_byte(int t, int q, double inv) {
    return __mul24(round_div(t, inv), -q) + t;
}

// floor(x * 2^F) for the binary64 value with bit pattern `bits`, as L
// little-endian two's-complement limbs (the caller guarantees the result
// fits).  A finite x is m * 2^e2 with m < 2^53 (hidden bit for normal
// numbers; subnormals share the smallest normal exponent), so the magnitude
// is m shifted by e2 + F; a right shift that drops set bits moves the floor of
// a negative value one further from zero.
template <int L>
__device__ __forceinline__ void fp64_floor_scaled(uint64_t bits, int F, uint64_t (&limb)[L]) {
    const uint64_t a = bits & 0x7fffffffffffffffull;
    const int ef = (int)(a >> 52);
    const uint64_t frac = a & ((1ull << 52) - 1);
    const uint64_t m = ef ? (frac | (1ull << 52)) : frac;
    const int e2 = ef ? ef - 1075 : -1074;
#pragma unroll
    for (int l = 0; l < L; l++) limb[l] = 0;
    bool dropped = false;
    if (a != 0) {
        const int shift = e2 + F;
        if (shift >= 0) {
            const int li = shift >> 6, off = shift & 63;
#pragma unroll
            for (int l = 0; l < L; l++) {
                uint64_t w = 0;
                if (l == li) w = m << off;
                if (l == li + 1 && off) w = m >> (64 - off);
                limb[l] = w;
            }
        } else if (shift > -64) {
            limb[0] = m >> -shift;
            dropped = (m & ((1ull << -shift) - 1)) != 0;
        } else {
            dropped = true;
        }
    }
    if (bits >> 63) {
        // -(magnitude + dropped) = ~magnitude + 1 - dropped
        uint64_t carry = dropped ? 0 : 1;
#pragma unroll
        for (int l = 0; l < L; l++) {
            const uint64_t w = ~limb[l] + carry;
            carry = (carry && w == 0) ? 1 : 0;
            limb[l] = w;
        }
    }
}

__device__ __forceinline__ uint32_t pack4(int b0, int b1, int b2, int b3) {
    // low bytes of four ints -> one word (byte 0 = b0)
    uint32_t lo = __builtin_amdgcn_perm((uint32_t)b1, (uint32_t)b0, 0x0c0c0400u);
    uint32_t hi = __builtin_amdgcn_perm((uint32_t)b3, (uint32_t)b2, 0x0c0c0400u);
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

}  // namespace rns
