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

// fp32 -> E4M3FN, round half to even on the 3-bit mantissa, saturate to 448.
__device__ __forceinline__ uint32_t f32_to_e4m3fn(float y) {
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a >= 0x43E00000u) return sign | 0x7Eu;           // |y| >= 448 (or NaN): saturate
    if (a < 0x3C800000u) {                                // |y| < 2^-6: subnormal step 2^-9
        // |y| * 2^9 is exact (power-of-two scale of a value >= 2^-149 * 2^9)
        const float m = __builtin_rintf(__uint_as_float(a) * 512.0f);
        return sign | uint32_t(m);                        // m == 8 encodes 2^-6 (0x08)
    }
    // normal: exponent e in [-6, 8]; keep 3 of 23 mantissa bits, round half to even
    uint32_t e = (a >> 23) - 127u + 7u;                   // biased E4M3 exponent, 1..15
    uint32_t mant = a & 0x7FFFFFu;
    uint32_t q = mant >> 20;
    const uint32_t rem = mant & 0xFFFFFu;
    q += (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ? 1u : 0u;
    if (q == 8u) { q = 0u; e += 1u; }
    return sign | (e << 3) | q;                           // |y| < 448 keeps this <= 0x7E
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
// grid, a tie goes to the neighbour with an even code.
__device__ __forceinline__ uint32_t f32_to_e2m1(float y) {
    const uint32_t sign = (__float_as_uint(y) >> 28) & 8u;
    const float a = __builtin_fabsf(y);
    uint32_t c;
    if (a <= 0.25f) c = 0;         // tie 0.25 -> 0 (code 0)
    else if (a < 0.75f) c = 1;     // 0.5
    else if (a <= 1.25f) c = 2;    // tie 0.75 -> 1.0 (code 2); tie 1.25 -> 1.0
    else if (a < 1.75f) c = 3;     // 1.5
    else if (a <= 2.5f) c = 4;     // tie 1.75 -> 2.0; tie 2.5 -> 2.0
    else if (a < 3.5f) c = 5;      // 3.0
    else if (a <= 5.0f) c = 6;     // tie 3.5 -> 4.0; tie 5 -> 4.0
    else c = 7;                    // 6.0 and saturation
    return sign | c;
}

__device__ __forceinline__ float e2m1_to_f32(uint32_t nib) {
    const uint32_t m = nib & 7u;
    // 0, .5, 1, 1.5, 2, 3, 4, 6: exponent/mantissa form of E2M1
    const float v = (m < 2u) ? 0.5f * float(m) : __uint_as_float(((m >> 1) + 126u) << 23) * (1.0f + 0.5f * float(m & 1u));
    return (nib & 8u) ? -v : v;
}

}  // namespace kvs
