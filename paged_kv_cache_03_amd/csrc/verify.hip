// verify.hip -- multi-token verify / chunked prefill on paged KV (causal).
//
// NInfer "Paged KV Context Store" page: P=64 translation, consumer rules
// (the valid frontier may end at any in-page offset; a page boundary is not a
// mask boundary -- granularity table), PagedKVBatchLayerView.  Chunk token i
// of entry b sits at position n0[b] + i and attends [0, n0[b] + i]; the chunk's
// own K/V are appended before the call.  Work per KV head is
// AttentionPairs = n0*T + T(T+1)/2 ("Resource Scheduling and Context Cache"
// page, prefill-work equation).
//
// Two paths: chunks of at most 32 query columns (tokens x GQ; BF16, D in
// {64, 128}) go through the matrix-core page stream in chunk mode (decode.hip),
// which reads each page once for all of the entry's query tokens; other
// entries take the per-token kernel below: one wave per (chunk token, KV head)
// streams the causal range page by page with an online softmax.

#include <hip/hip_runtime.h>

#include <cmath>

#include "attn_common.h"
#include "internal.h"
#include "kv_read.h"

namespace kvs {
namespace {

struct VerifyArgs {
    PoolView pv;
    const int32_t* table_rows;
    const int32_t* q_pos0;
    const int32_t* cu_q;
    const uint16_t* q;
    float* out;
    float scale_log2;
    int32_t B;
    int32_t Hq;
    int32_t total_q;
    int32_t max_ctx;
    int32_t min_cols;   // entries with at most this many query columns (tokens x GQ) are left to the page stream
};

template <int D, int GQ>
__global__ void __launch_bounds__(256) verify_scalar_kernel(VerifyArgs a) {
    constexpr int EPL = D / 64;
    __shared__ float q_s[4][GQ][D];
    __shared__ float p_s[4][64][GQ];
    const int wave = int(threadIdx.x >> 6), lane = int(threadIdx.x & 63);
    const int H = a.pv.H;
    const int item = int(blockIdx.x) * 4 + wave;
    if (item >= a.total_q * H) return;
    const int r = item / H, h = item % H;
    int b = 0;
    while (b + 1 < a.B && r >= a.cu_q[b + 1]) ++b;
    if ((a.cu_q[b + 1] - a.cu_q[b]) * GQ <= a.min_cols) return;
    const int row = a.table_rows[b];
    float* o = a.out + (size_t(r) * a.Hq + size_t(h) * GQ) * D;
    const int pos = a.q_pos0[b] + (r - a.cu_q[b]);
    const int ctx = (row >= 0 && row < a.pv.C && r >= a.cu_q[b] && r < a.cu_q[b + 1]) ? min(pos + 1, a.max_ctx) : 0;
    const int32_t* trow = a.pv.table + size_t(row) * a.pv.L;

    const uint16_t* qb = a.q + (size_t(r) * a.Hq + size_t(h) * GQ) * D;
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
    const int n_pages = ctx > 0 ? (ctx + kPage - 1) >> kPageShift : 0;
    for (int pg = 0; pg < n_pages; ++pg) {
        const int g = trow[pg];
        if (g < 0 || g >= a.pv.M) continue;
        const size_t slab = (size_t(g) * H + h) * kPage;
        const bool valid = pg * kPage + lane < ctx;
        float s[GQ];
#pragma unroll
        for (int j = 0; j < GQ; ++j) s[j] = 0.f;
        if (valid) {
            for (int d0 = 0; d0 < D; d0 += 8) {
                float kv[8];
                KVRow<CODEC_BF16, D>::load8(a.pv.lv.k_code, nullptr, slab + lane, d0, kv);
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
            for (int e = 0; e < EPL; ++e)
                v[e] = KVRow<CODEC_BF16, D>::load1(a.pv.lv.v_code, nullptr, slab + t, lane * EPL + e);
#pragma unroll
            for (int j = 0; j < GQ; ++j) {
                const float pj = p_s[wave][t][j];
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[j][e] += pj * v[e];
            }
        }
        wave_lds_sync();
    }
#pragma unroll
    for (int j = 0; j < GQ; ++j) {
        const float inv = l[j] > 0.f ? 1.f / l[j] : 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[size_t(j) * D + lane * EPL + e] = acc[j][e] * inv;
    }
}

template <int D>
hipError_t launch_d(const VerifyArgs& a, int gq, hipStream_t s) {
    const dim3 grid(unsigned((a.total_q * a.pv.H + 3) / 4));
    switch (gq) {
        case 1: verify_scalar_kernel<D, 1><<<grid, 256, 0, s>>>(a); break;
        case 2: verify_scalar_kernel<D, 2><<<grid, 256, 0, s>>>(a); break;
        case 4: verify_scalar_kernel<D, 4><<<grid, 256, 0, s>>>(a); break;
        case 8: verify_scalar_kernel<D, 8><<<grid, 256, 0, s>>>(a); break;
        default: return hipErrorNotSupported;
    }
    return hipGetLastError();
}

}  // namespace

bool verify_supported(const PoolView& pv, int Hq) {
    if (pv.H <= 0 || Hq % pv.H) return false;
    const int gq = Hq / pv.H;
    return pv.k_codec == CODEC_BF16 && pv.v_codec == CODEC_BF16 && (pv.D == 64 || pv.D == 128 || pv.D == 256) &&
           (gq == 1 || gq == 2 || gq == 4 || gq == 8);
}

// Entries with at most kStreamCols query columns (tokens x GQ, e.g. a short
// verify chunk) go through the page stream, which reads each page once for all
// of the entry's query tokens; longer chunks take the per-token kernel.
constexpr int kStreamCols = 32;

size_t verify_workspace_bytes(const PoolView& pv, int B, int Hq, int max_seq_len, int) {
    const int gq = pv.H ? Hq / pv.H : 0;
    return stream_chunk_supported(pv, B, gq) ? stream_chunk_workspace_bytes(pv, B, max_seq_len) : 0;
}

hipError_t launch_verify(const PoolView& pv, int B, int Hq, const int32_t* table_rows, const int32_t* q_pos0,
                         const int32_t* cu_q, int total_q, int /*max_q_len*/, int max_seq_len, const void* q,
                         float sm_scale, float* out, void* ws, size_t /*ws_bytes*/, hipStream_t s) {
    const int gq0 = Hq / pv.H;
    const bool stream = stream_chunk_supported(pv, B, gq0);
    if (stream) {
        hipError_t e = launch_stream_chunk(pv, B, Hq, table_rows, q_pos0, cu_q, max_seq_len, q, sm_scale, out, ws,
                                           kStreamCols, s);
        if (e != hipSuccess) return e;
    }
    VerifyArgs a{};
    a.pv = pv;
    a.table_rows = table_rows;
    a.q_pos0 = q_pos0;
    a.cu_q = cu_q;
    a.q = static_cast<const uint16_t*>(q);
    a.out = out;
    a.scale_log2 = sm_scale * kLog2e;
    a.B = B;
    a.Hq = Hq;
    a.total_q = total_q;
    a.max_ctx = max_seq_len;
    a.min_cols = stream ? kStreamCols : 0;
    const int gq = gq0;
    switch (pv.D) {
        case 64: return launch_d<64>(a, gq, s);
        case 128: return launch_d<128>(a, gq, s);
        case 256: return launch_d<256>(a, gq, s);
    }
    return hipErrorNotSupported;
}

}  // namespace kvs
