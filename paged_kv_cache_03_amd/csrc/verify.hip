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
// BF16 pages with D in {64, 128}: chunks of at most 32 query columns (tokens
// x GQ, e.g. a short verify) go through the matrix-core page stream in chunk
// mode (decode.hip), which reads each page once for all of the entry's query
// tokens; longer chunks (prefill) go to 128-column tiles on the matrix cores
// (verify_tile_kernel).  Quantized pools and BF16 pools at D = 256 take the
// tiles of verify_gtile.hip for every chunk.  The per-token kernel (one wave
// per (chunk token, KV head) streams the causal range with an online softmax)
// covers whatever else a pool and Hq allow.

#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>

#include "attn_common.h"
#include "internal.h"
#include "launch.h"
#include "kv_read.h"
#include "stream_common.h"

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

template <int D, int GQ, int KC, int VC, int SB>
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
        const size_t slab = (size_t(g) * a.pv.sg + size_t(h) * a.pv.sh) * kPage;
        const bool valid = pg * kPage + lane < ctx;
        float s[GQ];
#pragma unroll
        for (int j = 0; j < GQ; ++j) s[j] = 0.f;
        if (valid) {
            for (int d0 = 0; d0 < D; d0 += 8) {
                float kv[8];
                KVRow<KC, D, SB>::load8(a.pv.lv.k_code, a.pv.lv.k_scale, slab + lane, d0, kv);
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
                v[e] = KVRow<VC, D, SB>::load1(a.pv.lv.v_code, a.pv.lv.v_scale, slab + t, lane * EPL + e);
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

// ---------------------------------------------------------------------------
// Long chunks (chunked prefill): a block of 512 threads owns a tile of 128
// query columns -- consecutive chunk tokens x the GQ query heads of one KV
// head -- and streams the tile's causal key range through an LDS ring of
// direct-to-LDS page loads (issued by waves 0-3), NS-1 pages ahead.
// Wave w owns columns [32(w%4), 32(w%4) + 32) (two 16-column tiles) and keys
// [32(w/4), 32(w/4) + 32) of every page, so each wave reads half of a page
// from LDS and two waves per SIMD overlap one's softmax with the other's
// products:
//  * S^T[32 keys x 32] = K . Q^T on v_mfma_f32_16x16x32_bf16;
//  * PV on the same double-rate product with k = 32 keys: the A operand is
//    V^T of two 16-key tiles (two transposing reads, concatenated) and the
//    B operand the P^T registers of the same two tiles in the same order --
//    the key order inside a product is free as long as A and B agree;
//  * P as the bf16 pair p_hi + p_lo; lazy rescale; the causal mask only on
//    the pages that reach a column's limit;
//  * the two waves of a column range merge once, through LDS, at the end.
// Tiles of one (entry, KV head) read the same pages: blocks are mapped so
// that consecutive tiles run on one die (XCD) and share its L2.
template <int D, int GQ>
__global__ void __launch_bounds__(512) verify_tile_kernel(VerifyArgs a) {
    constexpr int NCH = D / 8;                     // 16-byte chunks per row
    constexpr int NT = 256;                        // threads that issue the page loads (waves 0-3)
    constexpr int NB = 512;                        // threads of the block
    constexpr int SLOTS = 64 * NCH;
    constexpr int SLICE_BYTES = SLOTS * 16;
    constexpr int PER_T = SLOTS / NT;
    constexpr int NS = D == 128 ? 4 : 8;
    constexpr int LOADS_PER_PAGE = 2 * PER_T;
    constexpr int NC = D / 32;                     // QK products per key tile, k = 32 each
    constexpr int NDT = D / 16;                    // PV tiles of 16 dims
    constexpr int TCOL = 128;                      // query columns per tile
    constexpr int WCT = 2;                         // 16-column tiles per wave
    constexpr float kHiOnly = 1.f / 256.f;         // largest weight of a page that takes p as one bf16 term
    constexpr int TTOK = TCOL / GQ;                // chunk tokens per tile
    static_assert((D == 64 || D == 128) && TCOL % GQ == 0, "shape");
    static_assert(NS * SLICE_BYTES == 0x10000, "V stages sit 64 KiB above the K stages");
    static_assert(LOADS_PER_PAGE * (NS - 1) < 64, "vmcnt range");
    static_assert(4 * WCT * NDT * 4 * 64 * 4 <= 2 * NS * SLICE_BYTES, "the end merge fits the ring");

    __shared__ u32x4 ring[2][NS][SLOTS];           // [K | V][stage][slot]
    __shared__ float mlx[4][WCT][16][2];           // (m, l) of the key-half-1 waves at the end

    const int tid = int(threadIdx.x);
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, li = lane & 15, lg = lane >> 4;
    const int cw = w & 3, kh = w >> 2;             // column range, key half
    const int H = a.pv.H, M = a.pv.M;

    // items are (entry, KV head, tile) in that order; die x takes items
    // [x*per, (x+1)*per) so that the tiles of one (entry, head) share an L2
    int n_items = 0;
    for (int b = 0; b < a.B; ++b) {
        const int T = ld_uniform(a.cu_q, b + 1) - ld_uniform(a.cu_q, b);
        if (T * GQ > a.min_cols) n_items += H * ((T * GQ + TCOL - 1) / TCOL);
    }
    const int per = (n_items + 7) / 8;
    const int i_blk = int(blockIdx.x);
    if (i_blk / 8 >= per) return;
    int item = (i_blk % 8) * per + i_blk / 8;
    if (item >= n_items) return;
    int b = 0, nt = 0;
    for (; b < a.B; ++b) {
        const int T = ld_uniform(a.cu_q, b + 1) - ld_uniform(a.cu_q, b);
        nt = T * GQ > a.min_cols ? (T * GQ + TCOL - 1) / TCOL : 0;
        if (item < H * nt) break;
        item -= H * nt;
    }
    const int h = item / nt, t = item % nt;
    const int row = ld_uniform(a.table_rows, b);
    const int c0 = ld_uniform(a.cu_q, b), T = ld_uniform(a.cu_q, b + 1) - c0;
    const int n0 = ld_uniform(a.q_pos0, b);
    const int keys = (row >= 0 && row < a.pv.C) ? max(0, min(n0 + T, a.max_ctx)) : 0;
    const int i0 = t * TTOK;                       // first chunk token of the tile
    const int ncol = min(TCOL, (T - i0) * GQ);     // real columns of the tile
    const int kmax = min(n0 + i0 + ncol / GQ, keys);   // largest key limit of the tile
    const int kmin = min(n0 + i0 + 1, keys);           // smallest key limit of a real column
    const int npages = kmax > 0 ? (kmax + kPage - 1) >> kPageShift : 0;

    auto out_ptr = [&](int c) __attribute__((always_inline)) {
        return a.out + (size_t(c0 + i0 + c / GQ) * a.Hq + size_t(h) * GQ + c % GQ) * D;
    };
    if (npages == 0) {                             // nothing to attend: zeros
        for (int x = tid; x < ncol * D; x += NB) out_ptr(x / D)[x % D] = 0.f;
        return;
    }

    // this lane's columns: c = 32cw + 16ct + li; key limits and Q^T operands
    int klim[WCT];
    bf16x8_t qb[WCT][NC];
#pragma unroll
    for (int ct = 0; ct < WCT; ++ct) {
        const int c = 32 * cw + 16 * ct + li;
        const bool real = c < ncol;
        klim[ct] = real ? min(n0 + i0 + c / GQ + 1, keys) : 0;
        const u32x4* qg = reinterpret_cast<const u32x4*>(
            a.q + (size_t(c0 + i0 + (real ? c : 0) / GQ) * a.Hq + size_t(h) * GQ + (real ? c : 0) % GQ) * D);
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            const u32x4 v = qg[4 * k + lg];
            qb[ct][k] = __builtin_bit_cast(bf16x8_t, real ? v : u32x4{0u, 0u, 0u, 0u});
        }
    }
    wait_vmcnt<0>();

    // stage layout and DMA sources as in the page stream (XOR-swizzled rows)
    auto kswz = [](int r) __attribute__((always_inline)) { return NCH == 16 ? (r & 15) : ((r >> 1) & 7); };
    auto vswz = [](int r) __attribute__((always_inline)) { return NCH == 16 ? ((r & 7) << 1) : (((r >> 1) & 3) << 1); };
    const char* kplane = static_cast<const char*>(a.pv.lv.k_code);
    const char* vplane = static_cast<const char*>(a.pv.lv.v_code);
    uint32_t k_src[PER_T], v_src[PER_T];
#pragma unroll
    for (int k = 0; k < PER_T; ++k) {
        const int sl = k * NT + (tid & (NT - 1));
        const int r = sl / NCH, x = sl % NCH;
        k_src[k] = uint32_t(r * NCH + (x ^ kswz(r))) * 16u;
        v_src[k] = uint32_t(r * NCH + (x ^ vswz(r))) * 16u;
    }
    const uint32_t ring_lds = uint32_t(reinterpret_cast<uintptr_t>((lds_byte_ptr)(&ring[0][0][0])));
    const int32_t* trow = a.pv.table + size_t(row) * a.pv.L;
    auto slice_of = [&](int p) __attribute__((always_inline)) {
        const int g0 = ld_uniform(trow, p);
        return (g0 >= 0 && g0 < M) ? g0 * a.pv.sg + h * a.pv.sh : -1;
    };
    auto fetch = [&](int sl, int fs) __attribute__((always_inline)) {
        if (w >= 4) return;                        // waves 0-3 load the pages
        const uint32_t dst = ring_lds + uint32_t(fs * SLICE_BYTES + w * 1024);
        const size_t off = size_t(sl < 0 ? 0 : sl) * SLICE_BYTES;
        if constexpr (PER_T == 4) fetch_page4(dst, kplane + off, vplane + off, k_src, v_src);
        else fetch_page2(dst, kplane + off, vplane + off, k_src, v_src);
    };

    // per-lane LDS offsets of this wave's first key tile in stage 0 (its
    // second tile adds 16 rows, the stage an immediate): K A operand row li,
    // chunk 4c + lg; V^T through the transposing read, rows 4lg + li/4,
    // dims 16dt + 4(li%4)
    const int kr0 = 32 * kh;                       // first key row of this wave
    int koff[NC], voff[NDT];
    {
#pragma unroll
        for (int c = 0; c < NC; ++c) koff[c] = (kr0 + li) * NCH + ((4 * c + lg) ^ kswz(li));
        const int tv = 4 * lg + (li >> 2), qd = li & 3;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
            voff[dt] = 0x10000 + (kr0 + tv) * NCH * 16 + (((2 * dt + (qd >> 1)) ^ vswz(tv)) * 16) + 8 * (qd & 1);
    }

    f32x4_t acc[WCT][NDT];
    // lsum[ct]: the column's sum of probabilities over this wave's keys, on
    // the matrix cores (an all-ones A operand against P^T: every row of the
    // result is the column sum of exactly the bf16 values PV uses)
    f32x4_t lsum[WCT];
    float m_ref[WCT];
    const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
#pragma unroll
    for (int ct = 0; ct < WCT; ++ct) {
        m_ref[ct] = -INFINITY;
        lsum[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[ct][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    int slices[NS];                                // slice of the page in each stage
#pragma unroll
    for (int k = 0; k < NS; ++k) slices[k] = 0;
#pragma unroll
    for (int k = 0; k < NS - 1; ++k) {
        if (k < npages) {
            slices[k] = slice_of(k);
            fetch(slices[k], k);
        }
    }
    int next_slice = NS - 1 < npages ? slice_of(NS - 1) : 0;   // one page of lookahead on the table

    auto step = [&](auto jc, int i) __attribute__((always_inline)) {
        constexpr int J = decltype(jc)::value;
        constexpr int FS = (J + NS - 1) % NS;
        if (i + NS - 1 < npages) {
            wait_vmcnt<LOADS_PER_PAGE * (NS - 2)>();
            block_lds_barrier();
            slices[FS] = next_slice;
            fetch(next_slice, FS);
            if (i + NS < npages) next_slice = slice_of(i + NS);
        } else {
            wait_vmcnt<0>();
            block_lds_barrier();
        }
        const int tok0 = i * kPage;
        const int lim = slices[J] >= 0 ? min(kPage, kmax - tok0) : 0;   // rows any column may see
        if (lim <= 0) return;                      // unmapped page: nothing to read
        if (lim < kPage) {
            // rows past the last limit hold stale bytes (possibly NaN): clear
            // them before any wave reads the stage
            u32x4* vrows = &ring[1][J][lim * NCH];
            for (int x = tid; x < (kPage - lim) * NCH; x += NB) vrows[x] = u32x4{0u, 0u, 0u, 0u};
            block_lds_barrier();
        }
        if (lim <= kr0) return;                    // none of this wave's keys is visible
        const u32x4* kst = &ring[0][J][0];
        const lds_byte_ptr vst = (lds_byte_ptr)(&ring[0][J][0]);   // voff includes the K-to-V distance
        f32x4_t s[2][WCT];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int ct = 0; ct < WCT; ++ct) s[kt][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        // the products issue at raised wave priority, the vector phase at the
        // default (the tile kernel measured 0.8% faster over five runs on one
        // box; raising the vector phase instead gained less, the PV products
        // alone nothing)
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const bf16x8_t kk = __builtin_bit_cast(bf16x8_t, kst[koff[c] + kt * 16 * NCH]);
#pragma unroll
                for (int ct = 0; ct < WCT; ++ct)
                    s[kt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk, qb[ct][c], s[kt][ct], 0, 0, 0);
            }
        }
        __builtin_amdgcn_s_setprio(0);
        // V^T of the wave's 32 keys (two transposing reads per 16 dims),
        // read while the score products run.  k order of the PV product:
        // element e of lane group g is key 16*(e/4) + 4g + e%4 of this wave's
        // 32, the order of the score rows below
        bf16x8_t va[NDT];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(vst + voff[dt]));
            const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4_ptr)(vst + voff[dt] + 16 * NCH * 16));
            va[dt] = __builtin_bit_cast(
                bf16x8_t, u32x4{__builtin_bit_cast(u32x2, v0)[0], __builtin_bit_cast(u32x2, v0)[1],
                                __builtin_bit_cast(u32x2, v1)[0], __builtin_bit_cast(u32x2, v1)[1]});
        }
        // the causal mask, only on the pages that reach some column's limit
        // (every partly written page is one: its key limit lies inside it)
        if (tok0 + kPage > kmin) {
#pragma unroll
            for (int ct = 0; ct < WCT; ++ct)
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (tok0 + kr0 + 16 * kt + 4 * lg + r >= klim[ct]) s[kt][ct][r] = -INFINITY;
        }
        // raw scores; the scale (> 0) is applied in the exponent's fma.  One
        // lazy-rescale decision for both column tiles (a tile that does not
        // need it keeps its reference: factor 1)
        float pm[WCT];
        bool grow = false;
#pragma unroll
        for (int ct = 0; ct < WCT; ++ct) {
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kt][ct][r]);
            pm[ct] = rows_max(mx) * a.scale_log2;
            grow |= pm[ct] > m_ref[ct] + kRescaleLog2;
        }
        if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
            for (int ct = 0; ct < WCT; ++ct) {
                const float mn = pm[ct] > m_ref[ct] + kRescaleLog2 ? pm[ct] : m_ref[ct];
                const float alpha = m_ref[ct] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref[ct] - mn);
                lsum[ct] *= alpha;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) acc[ct][dt] *= alpha;
                m_ref[ct] = mn;
            }
        }
        // P enters the PV product as one bf16 term once no key of the page
        // can weigh much in its column: every column's largest probability
        // on the page is at most kHiOnly of its running sum over this wave's
        // keys (a lower bound of the column's sum).  The sum adds exactly the
        // rounded values the product uses, so the output is the softmax of
        // the rounded weights: a key's rounding (at most 2^-9 of its
        // probability) moves the output by at most 2^-9 w |v - o|, w <= 2^-8
        // its weight, i.e. at most 2^-17 |v - o| per key; the roundings of
        // different keys are independent and add like a random walk.  Pages
        // where some column fails the test (the first pages of every
        // column, peaked distributions) add the second term p_lo.
        bool need_lo = false;
#pragma unroll
        for (int ct = 0; ct < WCT; ++ct)
            need_lo |= !(__builtin_amdgcn_exp2f(pm[ct] - m_ref[ct]) <= kHiOnly * lsum[ct][0]);
        // probabilities; a column whose keys in this half are all masked so
        // far has no reference yet: offset 0 keeps its p at exp2(-inf) = 0,
        // not NaN
        float p[WCT][8];
        bf16x8_t phi[WCT];
#pragma unroll
        for (int ct = 0; ct < WCT; ++ct) {
            const float moff = m_ref[ct] == -INFINITY ? 0.f : -m_ref[ct];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                p[ct][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e >> 2][ct][e & 3], a.scale_log2, moff));
            uint32_t hv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                hv[e] = __builtin_bit_cast(uint32_t,
                                           __builtin_convertvector(f32x2_t{p[ct][2 * e], p[ct][2 * e + 1]}, bf16x2v_t));
            phi[ct] = __builtin_bit_cast(bf16x8_t, u32x4{hv[0], hv[1], hv[2], hv[3]});
        }
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int ct = 0; ct < WCT; ++ct) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
                acc[ct][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[dt], phi[ct], acc[ct][dt], 0, 0, 0);
            lsum[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, phi[ct], lsum[ct], 0, 0, 0);
        }
        if (__builtin_amdgcn_ballot_w64(need_lo)) {
            // p_lo = rne(p - p_hi), the same products on it
#pragma unroll
            for (int ct = 0; ct < WCT; ++ct) {
                const u32x4 hu = __builtin_bit_cast(u32x4, phi[ct]);
                uint32_t lv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float r0 = p[ct][2 * e] - __uint_as_float(hu[e] << 16);
                    const float r1 = p[ct][2 * e + 1] - __uint_as_float(hu[e] & 0xFFFF0000u);
                    lv[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{r0, r1}, bf16x2v_t));
                }
                const bf16x8_t plo = __builtin_bit_cast(bf16x8_t, u32x4{lv[0], lv[1], lv[2], lv[3]});
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
                    acc[ct][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[dt], plo, acc[ct][dt], 0, 0, 0);
                lsum[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, plo, lsum[ct], 0, 0, 0);
            }
        }
    __builtin_amdgcn_s_setprio(0);
    };

    for (int i0p = 0; i0p < npages; i0p += NS) {
        step(std::integral_constant<int, 0>{}, i0p);
        if (i0p + 1 < npages) step(std::integral_constant<int, 1>{}, i0p + 1);
        if (i0p + 2 < npages) step(std::integral_constant<int, 2>{}, i0p + 2);
        if (i0p + 3 < npages) step(std::integral_constant<int, 3>{}, i0p + 3);
        if constexpr (NS == 8) {
            if (i0p + 4 < npages) step(std::integral_constant<int, 4>{}, i0p + 4);
            if (i0p + 5 < npages) step(std::integral_constant<int, 5>{}, i0p + 5);
            if (i0p + 6 < npages) step(std::integral_constant<int, 6>{}, i0p + 6);
            if (i0p + 7 < npages) step(std::integral_constant<int, 7>{}, i0p + 7);
        }
    }

    // merge the two key halves of each column range (through the ring, free
    // now), then wave cw writes its columns
    float lw[WCT];
#pragma unroll
    for (int ct = 0; ct < WCT; ++ct) lw[ct] = lsum[ct][0];
    block_lds_barrier();                           // every wave is done with the ring
    float* xb = reinterpret_cast<float*>(&ring[0][0][0]) + cw * (WCT * NDT * 4 * 64);
    if (kh == 1) {
#pragma unroll
        for (int ct = 0; ct < WCT; ++ct) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int r = 0; r < 4; ++r) xb[((ct * NDT + dt) * 4 + r) * 64 + lane] = acc[ct][dt][r];
            if (lg == 0) {
                mlx[cw][ct][li][0] = m_ref[ct];
                mlx[cw][ct][li][1] = lw[ct];
            }
        }
    }
    block_lds_barrier();
    if (kh == 1) return;
#pragma unroll
    for (int ct = 0; ct < WCT; ++ct) {
        const float m1 = mlx[cw][ct][li][0], l1 = mlx[cw][ct][li][1];
        const float mx = fmaxf(m_ref[ct], m1);
        const float w0 = m_ref[ct] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref[ct] - mx);
        const float w1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mx);
        const float l = lw[ct] * w0 + l1 * w1;
        const int c = 32 * cw + 16 * ct + li;
        if (c >= ncol) continue;
        const float inv = l > 0.f ? 1.f / l : 0.f;
        float* o = out_ptr(c) + 4 * lg;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            f32x4_t v;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                v[r] = (acc[ct][dt][r] * w0 + xb[((ct * NDT + dt) * 4 + r) * 64 + lane] * w1) * inv;
            *reinterpret_cast<float4*>(o + 16 * dt) = make_float4(v[0], v[1], v[2], v[3]);
        }
    }
}

template <int D, int KC, int VC, int SB>
hipError_t launch_scalar(const VerifyArgs& a, int gq, hipStream_t s) {
    const dim3 grid(unsigned((a.total_q * a.pv.H + 3) / 4));
    switch (gq) {
        case 1: return launch_kernel(true, verify_scalar_kernel<D, 1, KC, VC, SB>, grid, dim3(256), s, a);
        case 2: return launch_kernel(true, verify_scalar_kernel<D, 2, KC, VC, SB>, grid, dim3(256), s, a);
        case 4: return launch_kernel(true, verify_scalar_kernel<D, 4, KC, VC, SB>, grid, dim3(256), s, a);
        case 8: return launch_kernel(true, verify_scalar_kernel<D, 8, KC, VC, SB>, grid, dim3(256), s, a);
        default: return hipErrorNotSupported;
    }
}

// the per-token kernel for the pool's closed profile
template <int D>
hipError_t launch_d(const VerifyArgs& a, int gq, hipStream_t s) {
    const int kc = a.pv.k_codec, vc = a.pv.v_codec;
    const bool s16 = a.pv.scale16 != 0;
#define KVS_VSC_CASE(K, V, SB) \
    if (kc == K && vc == V && s16 == (SB == 2)) return launch_scalar<D, K, V, SB>(a, gq, s);
    KVS_VSC_CASE(CODEC_BF16, CODEC_BF16, 4)
    KVS_VSC_CASE(CODEC_INT8_G64, CODEC_INT8_G64, 4)
    KVS_VSC_CASE(CODEC_FP8_ROW, CODEC_FP8_ROW, 4)
    KVS_VSC_CASE(CODEC_NVFP4_G16, CODEC_NVFP4_G16, 4)
    KVS_VSC_CASE(CODEC_FP8_ROW, CODEC_NVFP4_G16, 4)
    KVS_VSC_CASE(CODEC_INT8_G64, CODEC_INT8_G64, 2)
    KVS_VSC_CASE(CODEC_FP8_ROW, CODEC_FP8_ROW, 2)
    KVS_VSC_CASE(CODEC_FP8_ROW, CODEC_NVFP4_G16, 2)
#undef KVS_VSC_CASE
    return hipErrorNotSupported;
}

}  // namespace

bool verify_supported(const PoolView& pv, int Hq) {
    if (pv.H <= 0 || Hq % pv.H) return false;
    const int gq = Hq / pv.H;
    return (pv.D == 64 || pv.D == 128 || pv.D == 256) && (gq == 1 || gq == 2 || gq == 4 || gq == 8);
}

// Entries with at most kStreamCols query columns (tokens x GQ, e.g. a short
// verify chunk) go through the page stream, which reads each page once for all
// of the entry's query tokens; longer chunks take the per-token kernel.
constexpr int kStreamCols = 32;

size_t verify_workspace_bytes(const PoolView& pv, int B, int Hq, int max_seq_len, int max_q_len) {
    const int gq = pv.H ? Hq / pv.H : 0;
    if (stream_chunk_supported(pv, B, gq)) return stream_chunk_workspace_bytes(pv, B, Hq, max_seq_len);
    if (gtile_supported(pv, gq)) return gtile_workspace_bytes(pv, B, Hq, max_seq_len, max_q_len);
    return 0;
}

hipError_t launch_verify(const PoolView& pv, int B, int Hq, const int32_t* table_rows, const int32_t* q_pos0,
                         const int32_t* cu_q, int total_q, int max_q_len, int max_seq_len, const void* q,
                         float sm_scale, float* out, void* ws, size_t /*ws_bytes*/, hipStream_t s) {
    const int gq = Hq / pv.H;
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
    if (stream_chunk_supported(pv, B, gq)) {
        // short chunks: the page stream; long chunks: 128-column tiles
        const bool tiles_follow = max_q_len * gq > kStreamCols;
        hipError_t e = launch_stream_chunk(pv, B, Hq, table_rows, q_pos0, cu_q, max_seq_len, q, sm_scale, out, ws,
                                           kStreamCols, !tiles_follow, s);
        if (e != hipSuccess) return e;
        a.min_cols = kStreamCols;
        if (!tiles_follow) return hipSuccess;
        const long long tiles = (long long)B * pv.H * ((max_q_len * gq + 127) / 128);
        const dim3 grid(unsigned((tiles + 7) / 8 * 8));   // 512 threads each
        e = hipErrorNotSupported;
        switch (pv.D * 16 + gq) {
            case 64 * 16 + 1: e = launch_kernel(true, verify_tile_kernel<64, 1>, grid, dim3(512), s, a); break;
            case 64 * 16 + 2: e = launch_kernel(true, verify_tile_kernel<64, 2>, grid, dim3(512), s, a); break;
            case 64 * 16 + 4: e = launch_kernel(true, verify_tile_kernel<64, 4>, grid, dim3(512), s, a); break;
            case 64 * 16 + 8: e = launch_kernel(true, verify_tile_kernel<64, 8>, grid, dim3(512), s, a); break;
            case 128 * 16 + 1: e = launch_kernel(true, verify_tile_kernel<128, 1>, grid, dim3(512), s, a); break;
            case 128 * 16 + 2: e = launch_kernel(true, verify_tile_kernel<128, 2>, grid, dim3(512), s, a); break;
            case 128 * 16 + 4: e = launch_kernel(true, verify_tile_kernel<128, 4>, grid, dim3(512), s, a); break;
            case 128 * 16 + 8: e = launch_kernel(true, verify_tile_kernel<128, 8>, grid, dim3(512), s, a); break;
            default: return hipErrorNotSupported;
        }
        return e;
    }
    if (gtile_supported(pv, gq))   // quantized pools, BF16 at D = 256: tiles for every entry
        return launch_gtile(pv, B, Hq, table_rows, q_pos0, cu_q, max_q_len, max_seq_len, q, sm_scale, out, ws, s);
    a.min_cols = 0;
    switch (pv.D) {
        case 64: return launch_d<64>(a, gq, s);
        case 128: return launch_d<128>(a, gq, s);
        case 256: return launch_d<256>(a, gq, s);
    }
    return hipErrorNotSupported;
}

}  // namespace kvs
