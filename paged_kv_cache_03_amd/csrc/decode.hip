// decode.hip -- paged decode: split-K over pages, then a cross-split combine.
//
// NInfer "Paged KV Context Store" page: PagedKVBatchLayerView (table_rows[b]
// selects the block-table row of compact entry b), P=64 translation
// (block = position >> 6, offset = position & 63), consumer rules (page
// translation at page granularity, no gather-to-contiguous, free choice of
// tile/split/wave/LDS scheme), wrapper validation and caller guarantees.
//
// Split policy: entry b's pages [0, ceil(ctx/64)) are cut into chunks of
// `chunk_pages` consecutive logical pages.  Chunk boundaries depend only on
// logical positions and the host-side bounds, never on physical page ids,
// and the combine runs in a fixed order, so outputs are bitwise identical
// under any permutation of page ids and for shared versus private pages.

#include <hip/hip_runtime.h>

#include <cmath>

#include "attn_common.h"
#include "internal.h"
#include "kv_read.h"

namespace kvs {
namespace {

struct DecodeArgs {
    PoolView pv;
    const int32_t* table_rows;
    const int32_t* seq_lens;
    const uint16_t* q;
    float* out;
    float* part_ml;     // [items][GQ][2]  (running max in log2 units, sum)
    float* part_acc;    // [items][GQ][D]  (unnormalized)
    float scale_log2;   // sm_scale * log2(e)
    int32_t B;
    int32_t Hq;
    int32_t chunk_pages;
    int32_t max_chunks;
    int32_t max_ctx;    // host bound on seq_lens (<= max_context); larger values are clipped
};

// One 64-lane wave per work item (entry b, KV head h, chunk c).  QK: lane t
// owns token t of the page; PV: lane owns EPL = D/64 head_dim elements.
template <int D, int GQ, int KC, int VC>
__global__ void __launch_bounds__(256) decode_split_kernel(DecodeArgs a) {
    constexpr int EPL = D / 64;
    __shared__ float q_s[4][GQ][D];
    __shared__ float p_s[4][64][GQ];
    const int wave = int(threadIdx.x >> 6), lane = int(threadIdx.x & 63);
    const int H = a.pv.H;
    const int item = int(blockIdx.x) * 4 + wave;
    if (item >= a.B * H * a.max_chunks) return;
    const int c = item % a.max_chunks;
    const int bh = item / a.max_chunks;
    const int h = bh % H, b = bh / H;
    const int row = a.table_rows[b];
    const int ctx = (row >= 0 && row < a.pv.C) ? min(a.seq_lens[b], a.max_ctx) : 0;
    const int n_pages = (ctx + kPage - 1) >> kPageShift;
    const int p0 = c * a.chunk_pages;
    const int p1 = min(p0 + a.chunk_pages, n_pages);
    if (p0 >= p1) return;
    const int32_t* trow = a.pv.table + size_t(row) * a.pv.L;

    const uint16_t* qb = a.q + (size_t(b) * a.Hq + size_t(h) * GQ) * D;
    for (int i = lane; i < GQ * D; i += 64) q_s[wave][i / D][i % D] = bf16_bits_to_f32(qb[i]);
    wave_lds_sync();

    float m[GQ], l[GQ], acc[GQ][EPL];
#pragma unroll
    for (int j = 0; j < GQ; ++j) {
        m[j] = -INFINITY;
        l[j] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[j][e] = 0.f;
    }

    for (int pg = p0; pg < p1; ++pg) {
        const int g = trow[pg];
        if (g < 0 || g >= a.pv.M) continue;       // unmapped block: caller guarantee broken, read nothing
        const size_t slab = (size_t(g) * H + h) * kPage;
        const int tok = pg * kPage + lane;
        const bool valid = tok < ctx;
        float s[GQ];
#pragma unroll
        for (int j = 0; j < GQ; ++j) s[j] = 0.f;
        if (valid) {
            for (int d0 = 0; d0 < D; d0 += 8) {
                float kv[8];
                KVRow<KC, D>::load8(a.pv.lv.k_code, a.pv.lv.k_scale, slab + lane, d0, kv);
#pragma unroll
                for (int j = 0; j < GQ; ++j)
#pragma unroll
                    for (int i = 0; i < 8; ++i) s[j] += kv[i] * q_s[wave][j][d0 + i];
            }
        }
#pragma unroll
        for (int j = 0; j < GQ; ++j) {
            const float sj = valid ? s[j] * a.scale_log2 : -INFINITY;
            const float mn = fmaxf(m[j], wave_max(sj));
            const float alpha = mn == -INFINITY ? 1.f : exp2f(m[j] - mn);
            const float pj = valid ? exp2f(sj - mn) : 0.f;
            l[j] = l[j] * alpha + wave_sum(pj);
            m[j] = mn;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[j][e] *= alpha;
            p_s[wave][lane][j] = pj;
        }
        wave_lds_sync();
        const int nvalid = min(kPage, ctx - pg * kPage);
        for (int t = 0; t < nvalid; ++t) {
            float v[EPL];
#pragma unroll
            for (int e = 0; e < EPL; ++e) v[e] = KVRow<VC, D>::load1(a.pv.lv.v_code, a.pv.lv.v_scale, slab + t,
                                                                      lane * EPL + e);
#pragma unroll
            for (int j = 0; j < GQ; ++j) {
                const float pj = p_s[wave][t][j];
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[j][e] += pj * v[e];
            }
        }
        wave_lds_sync();
    }

    const size_t it = size_t(item);
#pragma unroll
    for (int j = 0; j < GQ; ++j) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) a.part_acc[(it * GQ + j) * D + lane * EPL + e] = acc[j][e];
        if (lane == 0) {
            a.part_ml[(it * GQ + j) * 2] = m[j];
            a.part_ml[(it * GQ + j) * 2 + 1] = l[j];
        }
    }
}

// Combine the chunks of each (entry, query head) in chunk order.
template <int D, int GQ>
__global__ void __launch_bounds__(64) decode_combine_kernel(DecodeArgs a) {
    constexpr int EPL = D / 64;
    const int lane = int(threadIdx.x);
    const int b = int(blockIdx.x) / a.Hq, j = int(blockIdx.x) % a.Hq;
    const int h = j / GQ, jj = j % GQ;
    const int row = a.table_rows[b];
    const int ctx = (row >= 0 && row < a.pv.C) ? min(a.seq_lens[b], a.max_ctx) : 0;
    const int n_pages = (ctx + kPage - 1) >> kPageShift;
    const int n_chunks = (n_pages + a.chunk_pages - 1) / a.chunk_pages;
    float* o = a.out + (size_t(b) * a.Hq + j) * D + lane * EPL;
    if (n_chunks <= 0) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] = 0.f;
        return;
    }
    const size_t base = (size_t(b) * a.pv.H + h) * a.max_chunks;
    float mx = -INFINITY;
    for (int c = 0; c < n_chunks; ++c) mx = fmaxf(mx, a.part_ml[((base + c) * GQ + jj) * 2]);
    float l = 0.f, acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
    for (int c = 0; c < n_chunks; ++c) {
        const size_t it = (base + c) * GQ + jj;
        const float w = exp2f(a.part_ml[it * 2] - mx);
        l += a.part_ml[it * 2 + 1] * w;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] += a.part_acc[it * D + lane * EPL + e] * w;
    }
    const float inv = 1.f / l;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = acc[e] * inv;
}

constexpr int kChunkPages = 8;

int max_chunks_for(int max_seq_len) {
    const int pages = (max_seq_len + kPage - 1) / kPage;
    return (pages + kChunkPages - 1) / kChunkPages;
}

template <int D, int GQ>
hipError_t launch_gq(const DecodeArgs& a, hipStream_t s) {
    const int items = a.B * a.pv.H * a.max_chunks;
    const dim3 grid(unsigned((items + 3) / 4));
    const int kc = a.pv.k_codec, vc = a.pv.v_codec;
    bool launched = false;
#define KVS_DEC_CASE(K, V)                                                       \
    if (!launched && kc == K && vc == V) {                                      \
        if (items > 0) decode_split_kernel<D, GQ, K, V><<<grid, 256, 0, s>>>(a); \
        launched = true;                                                         \
    }
    KVS_DEC_CASE(CODEC_BF16, CODEC_BF16)
    KVS_DEC_CASE(CODEC_INT8_G64, CODEC_INT8_G64)
    KVS_DEC_CASE(CODEC_FP8_ROW, CODEC_FP8_ROW)
    KVS_DEC_CASE(CODEC_NVFP4_G16, CODEC_NVFP4_G16)
    KVS_DEC_CASE(CODEC_FP8_ROW, CODEC_NVFP4_G16)
#undef KVS_DEC_CASE
    if (!launched) return hipErrorNotSupported;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    decode_combine_kernel<D, GQ><<<dim3(unsigned(a.B * a.Hq)), 64, 0, s>>>(a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, int gq, hipStream_t s) {
    switch (gq) {
        case 1: return launch_gq<D, 1>(a, s);
        case 2: return launch_gq<D, 2>(a, s);
        case 4: return launch_gq<D, 4>(a, s);
        case 8: return launch_gq<D, 8>(a, s);
    }
    return hipErrorNotSupported;
}

}  // namespace

bool decode_supported(const PoolView& pv, int Hq) {
    if (pv.H <= 0 || Hq % pv.H) return false;
    const int gq = Hq / pv.H;
    return (pv.D == 64 || pv.D == 128 || pv.D == 256) && (gq == 1 || gq == 2 || gq == 4 || gq == 8);
}

size_t decode_workspace_bytes(const PoolView& pv, int B, int Hq, int max_seq_len) {
    const size_t items = size_t(B) * pv.H * max_chunks_for(max_seq_len);
    const size_t gq = pv.H ? size_t(Hq / pv.H) : 0;
    return items * gq * (size_t(pv.D) + 2) * sizeof(float);
}

hipError_t launch_decode(const PoolView& pv, int B, int Hq, const int32_t* table_rows, const int32_t* seq_lens,
                         int max_seq_len, const void* q, float sm_scale, float* out, void* ws, size_t /*ws_bytes*/,
                         hipStream_t s) {
    DecodeArgs a{};
    a.pv = pv;
    a.table_rows = table_rows;
    a.seq_lens = seq_lens;
    a.q = static_cast<const uint16_t*>(q);
    a.out = out;
    a.B = B;
    a.Hq = Hq;
    a.chunk_pages = kChunkPages;
    a.max_chunks = max_chunks_for(max_seq_len);
    a.max_ctx = max_seq_len;
    const int gq = Hq / pv.H;
    const size_t items = size_t(B) * pv.H * a.max_chunks;
    a.part_ml = static_cast<float*>(ws);
    a.part_acc = a.part_ml + items * gq * 2;
    a.scale_log2 = sm_scale * kLog2e;
    switch (pv.D) {
        case 64: return launch_d<64>(a, gq, s);
        case 128: return launch_d<128>(a, gq, s);
        case 256: return launch_d<256>(a, gq, s);
    }
    return hipErrorNotSupported;
}

}  // namespace kvs
