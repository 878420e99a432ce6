// kv_read.h -- dequantizing readers of plane rows.
//
// A plane row is the X elements of one (page group g, KV head h, column o),
// at row index slot = (g * sg + h * sh) * 64 + o of every plane of the layer
// (page group diagram: one id selects slice g of every grouped plane;
// page-major order [X, P, H, N] has (sg, sh) = (H, 1), head-major [X, P, N, H]
// (1, M)).  Dequantization is value(code) * scale as one fp32
// multiply, the same value the persistent codec defines.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "codec_device.h"
#include "internal.h"

namespace kvs {

// scale element i of an INT8-G64 / FP8-row scale plane: fp32 (SB = 4) or
// binary16 (SB = 2), widened exactly
template <int SB>
__device__ __forceinline__ float scale_at(const void* scale, size_t i) {
    if constexpr (SB == 4) return static_cast<const float*>(scale)[i];
    else return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<const uint16_t*>(scale)[i]));
}

template <int CODEC, int D, int SB = 4>
struct KVRow {
    // element d of row `slot`
    static __device__ __forceinline__ float load1(const void* code, const void* scale, size_t slot, int d) {
        if constexpr (CODEC == CODEC_BF16) {
            return bf16_bits_to_f32(static_cast<const uint16_t*>(code)[slot * D + d]);
        } else if constexpr (CODEC == CODEC_INT8_G64) {
            const float s = scale_at<SB>(scale, slot * (D / 64) + d / 64);
            return float(static_cast<const int8_t*>(code)[slot * D + d]) * s;
        } else if constexpr (CODEC == CODEC_FP8_ROW) {
            const float s = scale_at<SB>(scale, slot);
            return e4m3fn_to_f32(static_cast<const uint8_t*>(code)[slot * D + d]) * s;
        } else {
            const float vs = e4m3fn_to_f32(static_cast<const uint8_t*>(scale)[slot * (D / 16) + d / 16]);
            const uint32_t byte = static_cast<const uint8_t*>(code)[slot * (D / 2) + d / 2];
            return e2m1_to_f32((d & 1) ? (byte >> 4) : (byte & 15u)) * vs;
        }
    }

    // elements [d0, d0 + 8), d0 a multiple of 8
    static __device__ __forceinline__ void load8(const void* code, const void* scale, size_t slot, int d0,
                                                 float (&out)[8]) {
        if constexpr (CODEC == CODEC_BF16) {
            const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(code) + slot * D + d0);
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                out[2 * i] = __uint_as_float(w[i] << 16);
                out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
            }
        } else if constexpr (CODEC == CODEC_INT8_G64) {
            const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const int8_t*>(code) + slot * D + d0);
            const float s = scale_at<SB>(scale, slot * (D / 64) + d0 / 64);
            const uint32_t w[2] = {u.x, u.y};
#pragma unroll
            for (int i = 0; i < 8; ++i) out[i] = float(int8_t((w[i / 4] >> (8 * (i % 4))) & 0xFFu)) * s;
        } else if constexpr (CODEC == CODEC_FP8_ROW) {
            const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(code) + slot * D + d0);
            const float s = scale_at<SB>(scale, slot);
            const uint32_t w[2] = {u.x, u.y};
#pragma unroll
            for (int i = 0; i < 8; ++i) out[i] = e4m3fn_to_f32((w[i / 4] >> (8 * (i % 4))) & 0xFFu) * s;
        } else {
            const uint32_t u = *reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(code) + slot * (D / 2) +
                                                                  d0 / 2);
            const float vs = e4m3fn_to_f32(static_cast<const uint8_t*>(scale)[slot * (D / 16) + d0 / 16]);
#pragma unroll
            for (int i = 0; i < 8; ++i) out[i] = e2m1_to_f32((u >> (4 * i)) & 15u) * vs;
        }
    }
};

}  // namespace kvs
