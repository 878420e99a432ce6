// codec_write.h -- quantize one K or V row of the closed KV profiles and
// store its codes and scales (the persistent codec of the "Paged KV Context
// Store" page: BF16 stored as is; INT8-G64; FP8-E4M3FN-row; NVFP4-G16).
// Rounding follows this library's reading of the page: fp32 arithmetic,
// correctly rounded division, round half to even, saturating FP8/FP4, a zero
// scale gives zero codes; no contraction into fused multiply-adds, whatever
// the including file's flags.
//
// One 64-lane wave writes one row: lane l owns elements [l*EPL, (l+1)*EPL)
// with EPL = D/64, so the code stores of a wave are contiguous, and group
// maxima (64, 16 or D elements) are butterfly reductions over the lanes that
// hold the group.  The append kernel and the quantized page stream (which
// writes the step's rows itself) share these functions, so both produce the
// same bytes.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <type_traits>

#include "codec_device.h"
#include "internal.h"

namespace kvs {

// The maximum over aligned groups of W lanes, in every lane of the group:
// lane exchanges within quads, half rows and rows (DPP), then across rows
// (permlane swaps), so no step goes through the LDS.  fmaxf is commutative
// and associative (a NaN operand yields the other one), so the order of the
// exchanges does not change the result.
template <int W>
__device__ __forceinline__ float group_max(float x) {
    static_assert(W == 1 || W == 2 || W == 4 || W == 8 || W == 16 || W == 32 || W == 64, "group width");
    auto dpp = [](float v, auto ctrl) __attribute__((always_inline)) {
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), decltype(ctrl)::value, 0xf, 0xf, false));
    };
    if constexpr (W >= 2) x = fmaxf(x, dpp(x, std::integral_constant<int, 0xB1>{}));    // quad_perm 1,0,3,2
    if constexpr (W >= 4) x = fmaxf(x, dpp(x, std::integral_constant<int, 0x4E>{}));    // quad_perm 2,3,0,1
    if constexpr (W >= 8) x = fmaxf(x, dpp(x, std::integral_constant<int, 0x141>{}));   // row_half_mirror
    if constexpr (W >= 16) x = fmaxf(x, dpp(x, std::integral_constant<int, 0x140>{}));  // row_mirror
    if constexpr (W >= 32) {
        const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    }
    if constexpr (W >= 64) {
        const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
    }
    return x;
}

template <int EPL>
__device__ __forceinline__ void load_row(const uint16_t* src, int lane, float (&x)[EPL], uint32_t (&bits)[EPL]) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        bits[e] = src[lane * EPL + e];
        x[e] = bf16_bits_to_f32(bits[e]);
    }
}

// The same row as raw bf16 bits in one load per lane (EPL = 1: 16 bits, 2:
// 32, 4: 64), and its elements as fp32.
template <int EPL>
__device__ __forceinline__ uint2 load_row_bits(const uint16_t* src, int lane) {
    if constexpr (EPL == 4) return *reinterpret_cast<const uint2*>(src + lane * 4);
    else if constexpr (EPL == 2) return make_uint2(*reinterpret_cast<const uint32_t*>(src + lane * 2), 0u);
    else return make_uint2(src[lane], 0u);
}

template <int EPL>
__device__ __forceinline__ void row_floats(uint2 bits, float (&x)[EPL]) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) x[e] = bf16_bits_to_f32(((e < 2 ? bits.x : bits.y) >> (16 * (e & 1))) & 0xFFFFu);
}

// A scale as stored: fp32 (SB = 4) or binary16 (SB = 2: the quotient
// saturated at 65504, then rounded half to even): its bits, and the value the
// codes are taken against.
template <int SB>
__device__ __forceinline__ uint32_t scale_bits(float s32) {
    if constexpr (SB == 4) return __float_as_uint(s32);
    else return __builtin_bit_cast(uint16_t, static_cast<_Float16>(fminf(s32, 65504.0f)));
}

template <int SB>
__device__ __forceinline__ float scale_value(uint32_t bits) {
    if constexpr (SB == 4) return __uint_as_float(bits);
    else return static_cast<float>(__builtin_bit_cast(_Float16, uint16_t(bits)));
}

// One lane's share of a quantized row: its code bytes (EPL of them for INT8 /
// FP8, EPL / 2 for NVFP4, lowest address in the low byte; at D = 64 NVFP4
// even lanes hold the byte of their pair) and the bits of the scale of its
// group, which the group's first lane stores.
struct RowCode {
    uint32_t code;
    uint32_t scale;
};

// Quantize one row of a quantized side (EPL elements per lane, loaded by
// load_row).
template <int D, int CODEC, int SB>
__device__ __forceinline__ RowCode quantize_side(const float (&x)[D / 64], int lane) {
#pragma clang fp contract(off)
    constexpr int EPL = D / 64;
    static_assert(CODEC != CODEC_BF16, "quantized sides");
    RowCode rc{0u, 0u};
    float a = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) a = fmaxf(a, __builtin_fabsf(x[e]));
    if constexpr (CODEC == CODEC_INT8_G64) {
        a = group_max<64 / EPL>(a);                       // 64-element group
        rc.scale = scale_bits<SB>(a / 127.0f);
        const float s = scale_value<SB>(rc.scale);
#pragma unroll
        for (int e = 0; e < EPL; ++e) {            // the quotient is formed whatever s (selected away at 0)
            const float q = s != 0.f ? fminf(fmaxf(__builtin_rintf(x[e] / s), -127.f), 127.f) : 0.f;
            rc.code |= (uint32_t(int(q)) & 0xFFu) << (8 * e);
        }
    } else if constexpr (CODEC == CODEC_FP8_ROW) {
        a = group_max<64>(a);                             // the whole row
        rc.scale = scale_bits<SB>(a / 448.0f);
        const float s = scale_value<SB>(rc.scale);
#pragma unroll
        for (int e = 0; e < EPL; ++e) rc.code |= (s != 0.f ? f32_to_e4m3fn(x[e] / s) : 0u) << (8 * e);
    } else {  // CODEC_NVFP4_G16
        a = group_max<16 / EPL>(a);                       // 16-element group
        rc.scale = f32_to_e4m3fn(a / 6.0f);
        const float vs = e4m3fn_to_f32(rc.scale);
        uint32_t nib[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) nib[e] = vs != 0.f ? f32_to_e2m1(x[e] / vs) : 0u;
        if constexpr (EPL == 1) {
            rc.code = nib[0] | (uint32_t(__shfl_xor(int(nib[0]), 1, 64)) << 4);
        } else {
#pragma unroll
            for (int e = 0; e < EPL; e += 2) rc.code |= (nib[e] | (nib[e + 1] << 4)) << (4 * e);
        }
    }
    return rc;
}

// Store a quantized row at row `slot` of its code and scale planes.
template <int D, int CODEC, int SB>
__device__ __forceinline__ void store_side(void* code, void* scale, size_t slot, const RowCode& rc, int lane) {
    constexpr int EPL = D / 64;
    constexpr int GL = CODEC == CODEC_INT8_G64 ? 64 / EPL : (CODEC == CODEC_FP8_ROW ? 64 : 16 / EPL);
    constexpr int CB = CODEC == CODEC_NVFP4_G16 ? EPL / 2 : EPL;   // code bytes per lane
    char* c = static_cast<char*>(code) + slot * (CODEC == CODEC_NVFP4_G16 ? D / 2 : D) + lane * CB;
    if constexpr (CB == 0) {                              // NVFP4 at D = 64: even lanes, one byte each
        if ((lane & 1) == 0) *reinterpret_cast<uint8_t*>(c + lane / 2) = uint8_t(rc.code);
    } else if constexpr (CB == 1) {
        *reinterpret_cast<uint8_t*>(c) = uint8_t(rc.code);
    } else if constexpr (CB == 2) {
        *reinterpret_cast<uint16_t*>(c) = uint16_t(rc.code);
    } else {
        *reinterpret_cast<uint32_t*>(c) = rc.code;
    }
    if (lane % GL == 0) {
        constexpr int GROUPS = 64 / GL;                   // scale elements per row
        const size_t idx = slot * GROUPS + lane / GL;
        if constexpr (CODEC == CODEC_NVFP4_G16) static_cast<uint8_t*>(scale)[idx] = uint8_t(rc.scale);
        else if constexpr (SB == 4) static_cast<uint32_t*>(scale)[idx] = rc.scale;
        else static_cast<uint16_t*>(scale)[idx] = uint16_t(rc.scale);
    }
}

// Quantize and store one row (EPL elements per lane, loaded by load_row) of
// one side.
template <int D, int CODEC, int SB>
__device__ __forceinline__ void write_side(void* code, void* scale, size_t slot, const float (&x)[D / 64],
                                           const uint32_t (&bits)[D / 64], int lane) {
    constexpr int EPL = D / 64;
    if constexpr (CODEC == CODEC_BF16) {
        uint16_t* c = static_cast<uint16_t*>(code) + slot * D + lane * EPL;
#pragma unroll
        for (int e = 0; e < EPL; ++e) c[e] = uint16_t(bits[e]);
    } else {
        store_side<D, CODEC, SB>(code, scale, slot, quantize_side<D, CODEC, SB>(x, lane), lane);
    }
}

}  // namespace kvs
