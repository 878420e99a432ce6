// codec_device.h -- device-side minifloat conversions for the closed KV profiles.
//
// Formats (published definitions): FP8 E4M3FN -- OCP 8-bit floating point,
// bias 7, 3 mantissa bits, no infinities, 0x7F/0xFF NaN, max 448; FP4 E2M1 --
// OCP MX, values {0, .5, 1, 1.5, 2, 3, 4, 6}.  Encoders round half to even
// and saturate; the sign of the fp32 input is kept (so -0 keeps its sign bit).
// Every step is exact fp32 or integer arithmetic, so the results are the
// correctly rounded conversions the profiles call for.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace kvs {

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t u16) { return __uint_as_float(u16 << 16); }

// fp32 -> E4M3FN, round half to even on the 3-bit mantissa, saturate to 448
// (NaN too).  Both the subnormal and the normal result are formed and one is
// selected, so a wave takes no branch.
__device__ __forceinline__ uint32_t f32_to_e4m3fn(float y) {
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    // |y| < 2^-6: subnormal step 2^-9; |y| * 2^9 is exact (a power-of-two
    // scale of a value >= 2^-149 * 2^9), rounded half to even (code 8 is 2^-6)
    const uint32_t sub = uint32_t(__builtin_rintf(__uint_as_float(a) * 512.0f));
    // normal: exponent in [-6, 8]; keep 3 of 23 mantissa bits, round half to
    // even; a carry out of the mantissa steps the exponent (e * 8 + 8)
    const uint32_t e = (a >> 23) - 127u + 7u;             // biased E4M3 exponent, 1..15
    const uint32_t mant = a & 0x7FFFFFu;
    const uint32_t q = mant >> 20;
    const uint32_t rem = mant & 0xFFFFFu;
    const uint32_t nrm = (e << 3) + q + ((rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ? 1u : 0u);
    const uint32_t r = a >= 0x43E00000u ? 0x7Eu : (a < 0x3C800000u ? sub : nrm);   // |y| >= 448 (or NaN)
    return sign | r;                                      // |y| < 448 keeps this <= 0x7E
}

// E4M3FN -> fp32 (NaN code never produced by the encoder).
__device__ __forceinline__ float e4m3fn_to_f32(uint32_t c) {
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    float v;
    if (e == 0u) v = float(m) * 0.001953125f;             // m * 2^-9
    else v = __uint_as_float(((e + 120u) << 23) | (m << 20));
    return (c & 0x80u) ? -v : v;
}

// fp32 -> E2M1 nibble (sign in bit 3): thresholds at the midpoints of the
// grid, a tie goes to the neighbour with an even code.  The code counts the
// thresholds |y| passes: above 0.25, from 0.75, above 1.25, from 1.75, above
// 2.5, from 3.5, above 5; NaN passes all of them (6.0, as a saturation).
__device__ __forceinline__ uint32_t f32_to_e2m1(float y) {
    const uint32_t sign = (__float_as_uint(y) >> 28) & 8u;
    const float a = __builtin_fabsf(y);
    const uint32_t c = uint32_t(!(a <= 0.25f)) + uint32_t(!(a < 0.75f)) + uint32_t(!(a <= 1.25f)) +
                       uint32_t(!(a < 1.75f)) + uint32_t(!(a <= 2.5f)) + uint32_t(!(a < 3.5f)) +
                       uint32_t(!(a <= 5.0f));
    return sign | c;
}

__device__ __forceinline__ float e2m1_to_f32(uint32_t nib) {
    const uint32_t m = nib & 7u;
    // 0, .5, 1, 1.5, 2, 3, 4, 6: exponent/mantissa form of E2M1
    const float v = (m < 2u) ? 0.5f * float(m) : __uint_as_float(((m >> 1) + 126u) << 23) * (1.0f + 0.5f * float(m & 1u));
    return (nib & 8u) ? -v : v;
}

}  // namespace kvs
