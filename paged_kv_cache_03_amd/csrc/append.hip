// append.hip -- persistent KV codec: quantize new K/V rows into their pages.
//
// NInfer "Paged KV Context Store" page: closed profiles (BF16 stored without
// FP16 conversion; INT8-G64; FP8-E4M3FN-row256; NVFP4-G16; K8V4 = FP8 K +
// NVFP4 V), X-extent list, P=64 translation (block = position >> 6, offset =
// position & 63, page = block_table[row][block]).  The row quantizer and its
// rounding are codec_write.h's.
//
// Mapping: one 64-lane wave per (token, KV head) row writes both the K and V
// row.  Append is tiny next to attention (a few rows per sequence per step),
// so it favours exactness and simplicity over throughput.

#include <hip/hip_runtime.h>

#include "codec_write.h"
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

template <int D, int KC, int VC, int SB>
__global__ void __launch_bounds__(256) append_kernel(AppendArgs a) {
    constexpr int EPL = D / 64;
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + int(threadIdx.x >> 6);
    const int H = a.pv.H;
    if (r >= a.total * H) return;
    const int t = r / H, h = r - (r / H) * H;
    // the row's values and every entry's row start, position and table row
    // in one round trip (lane k holds entry k's; they depend on nothing
    // else), then the entry of token t: the entries k in [1, B) whose rows
    // start at or before t (the starts do not decrease), by a ballot
    float kx[EPL], vx[EPL];
    uint32_t kb[EPL], vb[EPL];
    load_row<EPL>(a.k + size_t(r) * D, lane, kx, kb);
    load_row<EPL>(a.v + size_t(r) * D, lane, vx, vb);
    int b = 0, c0, c1, p0, row;
    if (a.B < 64) {
        const int start = lane <= a.B ? a.cu[lane] : 0;    // cu[k]: first row of entry k (cu[B]: the total)
        const int pz = lane < a.B ? a.pos0[lane] : 0;
        const int rw = lane < a.B ? a.table_rows[lane] : 0;
        b = __builtin_popcountll(__builtin_amdgcn_ballot_w64(lane >= 1 && lane < a.B && start <= t));
        c0 = __builtin_amdgcn_readlane(start, b);
        c1 = __builtin_amdgcn_readlane(start, b + 1);
        p0 = __builtin_amdgcn_readlane(pz, b);
        row = __builtin_amdgcn_readlane(rw, b);
    } else {
        while (b + 1 < a.B && t >= a.cu[b + 1]) ++b;
        c0 = a.cu[b];
        c1 = a.cu[b + 1];
        p0 = a.pos0[b];
        row = a.table_rows[b];
    }
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
