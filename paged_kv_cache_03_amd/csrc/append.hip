// append.hip -- persistent KV codec: quantize new K/V rows into their pages.
//
// NInfer "Paged KV Context Store" page: closed profiles (BF16 stored without
// FP16 conversion; INT8-G64; FP8-E4M3FN-row256; NVFP4-G16; K8V4 = FP8 K +
// NVFP4 V), X-extent list, P=64 translation (block = position >> 6, offset =
// position & 63, page = block_table[row][block]).  The codec header itself is
// not on the pages; rounding follows this library's reading: fp32 arithmetic,
// correctly rounded division, round half to even, saturating FP8/FP4, a zero
// scale gives zero codes.
//
// Mapping: one 64-lane wave per (token, KV head) row writes both the K and V
// row; lane l owns elements [l*EPL, (l+1)*EPL) with EPL = D/64, so the code
// stores of a wave are contiguous.  Group maxima (64, 16 or D elements) are
// butterfly reductions over the lanes holding the group.  Append is tiny next
// to attention (a few rows per sequence per step), so it favours exactness
// and simplicity over throughput.

#include <hip/hip_runtime.h>

#include "codec_device.h"
#include "internal.h"

namespace kvs {
namespace {

struct AppendArgs {
    PoolView pv;
    const int32_t* table_rows;
    const int32_t* pos0;
    const int32_t* cu;
    const uint16_t* k;
    const uint16_t* v;
    int32_t B;
    int32_t total;
};

template <int W>
__device__ __forceinline__ float group_max(float x) {
#pragma unroll
    for (int off = W / 2; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
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

// A scale as stored: fp32 (SB = 4) or binary16 (SB = 2: the quotient saturated
// at 65504, then rounded half to even).  Returns the value the codes are taken
// against and writes it to scale element `idx`.
template <int SB>
__device__ __forceinline__ float store_scale(void* scale, size_t idx, float s32) {
    if constexpr (SB == 4) {
        static_cast<float*>(scale)[idx] = s32;
        return s32;
    } else {
        const _Float16 h = static_cast<_Float16>(fminf(s32, 65504.0f));
        static_cast<uint16_t*>(scale)[idx] = __builtin_bit_cast(uint16_t, h);
        return static_cast<float>(h);
    }
}

template <int SB>
__device__ __forceinline__ float rounded_scale(float s32) {
    if constexpr (SB == 4) return s32;
    else return static_cast<float>(static_cast<_Float16>(fminf(s32, 65504.0f)));
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
    } else if constexpr (CODEC == CODEC_INT8_G64) {
        constexpr int GL = 64 / EPL;                      // lanes per 64-element group
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) a = fmaxf(a, __builtin_fabsf(x[e]));
        a = group_max<GL>(a);
        const float s32 = a / 127.0f;
        const float s = lane % GL == 0 ? store_scale<SB>(scale, slot * (D / 64) + lane / GL, s32)
                                       : rounded_scale<SB>(s32);
        int8_t* c = static_cast<int8_t*>(code) + slot * D + lane * EPL;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            float q = 0.f;
            if (s != 0.f) q = fminf(fmaxf(__builtin_rintf(x[e] / s), -127.f), 127.f);
            c[e] = int8_t(int(q));
        }
    } else if constexpr (CODEC == CODEC_FP8_ROW) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) a = fmaxf(a, __builtin_fabsf(x[e]));
        a = group_max<64>(a);
        const float s32 = a / 448.0f;
        const float s = lane == 0 ? store_scale<SB>(scale, slot, s32) : rounded_scale<SB>(s32);
        uint8_t* c = static_cast<uint8_t*>(code) + slot * D + lane * EPL;
#pragma unroll
        for (int e = 0; e < EPL; ++e) c[e] = uint8_t(s != 0.f ? f32_to_e4m3fn(x[e] / s) : 0u);
    } else {  // CODEC_NVFP4_G16
        constexpr int GL = 16 / EPL;                      // lanes per 16-element group
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) a = fmaxf(a, __builtin_fabsf(x[e]));
        a = group_max<GL>(a);
        const uint32_t sc = f32_to_e4m3fn(a / 6.0f);
        const float vs = e4m3fn_to_f32(sc);
        uint32_t nib[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) nib[e] = vs != 0.f ? f32_to_e2m1(x[e] / vs) : 0u;
        uint8_t* c = static_cast<uint8_t*>(code) + slot * (D / 2);
        if constexpr (EPL == 1) {
            const uint32_t other = uint32_t(__shfl_xor(int(nib[0]), 1, 64));
            if ((lane & 1) == 0) c[lane / 2] = uint8_t(nib[0] | (other << 4));
        } else {
#pragma unroll
            for (int e = 0; e < EPL; e += 2) c[(lane * EPL + e) / 2] = uint8_t(nib[e] | (nib[e + 1] << 4));
        }
        if (lane % GL == 0) static_cast<uint8_t*>(scale)[slot * (D / 16) + lane / GL] = uint8_t(sc);
    }
}

template <int D, int KC, int VC, int SB>
__global__ void __launch_bounds__(256) append_kernel(AppendArgs a) {
    constexpr int EPL = D / 64;
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + int(threadIdx.x >> 6);
    const int H = a.pv.H;
    if (r >= a.total * H) return;
    const int t = r / H, h = r - (r / H) * H;
    // the row's values first (they depend on nothing else), then the entry of
    // token t: the entries k in [1, B) whose rows start at or before t (the
    // starts do not decrease), one load per lane and a ballot for B <= 64
    float kx[EPL], vx[EPL];
    uint32_t kb[EPL], vb[EPL];
    load_row<EPL>(a.k + size_t(r) * D, lane, kx, kb);
    load_row<EPL>(a.v + size_t(r) * D, lane, vx, vb);
    int b = 0;
    if (a.B <= 64) {
        const int start = lane < a.B ? a.cu[lane] : 0;     // cu[k]: first row of entry k
        b = __builtin_popcountll(__builtin_amdgcn_ballot_w64(lane >= 1 && lane < a.B && start <= t));
    } else {
        while (b + 1 < a.B && t >= a.cu[b + 1]) ++b;
    }
    const int c0 = a.cu[b], c1 = a.cu[b + 1];
    const int p0 = a.pos0[b], row = a.table_rows[b];
    if (t < c0 || t >= c1) return;
    const int p = p0 + (t - c0);
    if (p < 0 || row < 0 || row >= a.pv.C) return;
    const int blk = p >> kPageShift, o = p & (kPage - 1);
    if (blk >= a.pv.L) return;
    const int g = a.pv.table[size_t(row) * a.pv.L + blk];
    if (g < 0 || g >= a.pv.M) return;                      // unmapped: caller guarantee broken, skip
    const size_t slot = (size_t(g) * a.pv.sg + size_t(h) * a.pv.sh) * kPage + o;   // row of (g, h, o) in every plane
    write_side<D, KC, SB>(a.pv.lv.k_code, a.pv.lv.k_scale, slot, kx, kb, lane);
    write_side<D, VC, SB>(a.pv.lv.v_code, a.pv.lv.v_scale, slot, vx, vb, lane);
}

template <int D>
hipError_t launch_d(const AppendArgs& a, dim3 grid, hipStream_t s) {
    const int kc = a.pv.k_codec, vc = a.pv.v_codec;
    const bool s16 = a.pv.scale16 != 0;
#define KVS_APPEND_CASE(K, V, SB)                                                                  \
    if (kc == K && vc == V && s16 == (SB == 2)) {                                                  \
        append_kernel<D, K, V, SB><<<grid, 256, 0, s>>>(a);                                       \
        return hipGetLastError();                                                                  \
    }
    KVS_APPEND_CASE(CODEC_BF16, CODEC_BF16, 4)
    KVS_APPEND_CASE(CODEC_INT8_G64, CODEC_INT8_G64, 4)
    KVS_APPEND_CASE(CODEC_FP8_ROW, CODEC_FP8_ROW, 4)
    KVS_APPEND_CASE(CODEC_NVFP4_G16, CODEC_NVFP4_G16, 4)
    KVS_APPEND_CASE(CODEC_FP8_ROW, CODEC_NVFP4_G16, 4)
    KVS_APPEND_CASE(CODEC_INT8_G64, CODEC_INT8_G64, 2)
    KVS_APPEND_CASE(CODEC_FP8_ROW, CODEC_FP8_ROW, 2)
    KVS_APPEND_CASE(CODEC_FP8_ROW, CODEC_NVFP4_G16, 2)
#undef KVS_APPEND_CASE
    return hipErrorNotSupported;
}

}  // namespace

hipError_t launch_append(const PoolView& pv, int B, const int32_t* table_rows, const int32_t* pos0,
                         const int32_t* cu_tokens, int total_tokens, const void* k, const void* v, hipStream_t s) {
    AppendArgs a{pv, table_rows, pos0, cu_tokens, static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                 B, total_tokens};
    const long rows = long(total_tokens) * pv.H;
    const dim3 grid(unsigned((rows + 3) / 4));
    switch (pv.D) {
        case 64: return launch_d<64>(a, grid, s);
        case 128: return launch_d<128>(a, grid, s);
        case 256: return launch_d<256>(a, grid, s);
    }
    return hipErrorNotSupported;
}

}  // namespace kvs
