// decode.hip -- paged decode (one query token per entry) on the page pool.
//
// NInfer "Paged KV Context Store" page: PagedKVBatchLayerView (table_rows[b]
// selects the block-table row of compact entry b), P=64 translation
// (block = position >> 6, offset = position & 63), consumer rules (page
// translation at page granularity, no gather-to-contiguous, free choice of
// tile/split/wave/LDS scheme), wrapper validation and caller guarantees.
//
// Two kernels:
//  * the matrix-core page stream (BF16 pages, D in {64, 128}): every page of
//    the call in one flat list, cut into equal ranges, one 256-thread block
//    per compute unit, with the cross-range combine in the same launch;
//  * the split kernel (every other profile and shape): entry b's pages are
//    cut into chunks of `chunk_pages` consecutive logical pages, one wave per
//    (entry, KV head, chunk), then a combine launch.
// In both, the split depends only on logical positions and the host-side
// bounds, never on physical page ids, and the combine runs in a fixed order,
// so outputs are bitwise identical under any permutation of page ids and for
// shared versus private pages.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <type_traits>

#include "attn_common.h"
#include "internal.h"
#include "kv_read.h"
#include "stream_common.h"

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
    uint32_t* arrive;   // [C*H] partials delivered per segment (page stream)
    float scale_log2;   // sm_scale * log2(e)
    int32_t B;
    int32_t Hq;
    int32_t chunk_pages;
    int32_t max_chunks;
    int32_t max_ctx;    // host bound on seq_lens (<= max_context); larger values are clipped
    // chunk mode (verify / chunked prefill through the page stream): entry b's
    // query tokens are rows cu_q[b] .. cu_q[b+1]-1 at positions q_pos0[b] + i;
    // entries with more than max_cols query columns (tokens x GQ) are left to
    // another kernel
    const int32_t* q_pos0;
    const int32_t* cu_q;
    int32_t max_cols;
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



// ---------------------------------------------------------------------------
// Flat page stream (BF16).  The work of one decode call is the ordered list of
// (entry b, KV head h, page p) for b < B, h < H, p < ceil(ctx_b / 64): segment
// s = b*H + h holds ceil(ctx_b/64) consecutive pages.  Block i of G takes the
// contiguous range [i*Q, min((i+1)*Q, total)), Q = ceil(total / G), so every
// block streams the same number of pages whatever the length mix.  A block
// writes one partial (m, l, acc) per segment it touches, in slot i + s: both
// the block and the segment index only grow along the stream, so no two
// touched (block, segment) pairs share a slot, and G + B*H slots suffice.
// Segment s is covered by the blocks first(s)..last(s) and owns the slots
// first(s)+s .. last(s)+s.  Ranges depend only on the context lengths, never
// on page ids, and the combine adds the slots in block order: deterministic.
struct Seg {
    int b, h, n;       // entry, KV head, pages in the segment
    int start;         // first global page index of the segment
};


__device__ __forceinline__ int ctx_of(const DecodeArgs& a, int b) {
    const int row = ld_uniform(a.table_rows, b);
    return (row >= 0 && row < a.pv.C) ? min(ld_uniform(a.seq_lens, b), a.max_ctx) : 0;
}

// Pages of every entry (B <= 8), read once: independent scalar loads instead
// of a dependent chain per segment step.
struct EntryPages {
    int n[8];
    __device__ __forceinline__ int operator()(int b) const {
        int r = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) r = (b == i) ? n[i] : r;
        return r;
    }
};

__device__ __forceinline__ EntryPages entry_pages(const DecodeArgs& a) {
    EntryPages e;
#pragma unroll
    for (int i = 0; i < 8; ++i) e.n[i] = i < a.B ? (ctx_of(a, i) + kPage - 1) >> kPageShift : 0;
    return e;
}

// floor(x / Q) for 0 <= x < 2^24 through the fp32 reciprocal, corrected to
// the exact quotient (an integer division is a long instruction sequence; the
// segment walks below do many of them).
struct Divider {
    int Q;
    float rq;
    __device__ __forceinline__ explicit Divider(int q) : Q(q), rq(1.0f / float(q)) {}
    __device__ __forceinline__ int operator()(int x) const {
        int d = int(float(x) * rq);
        d -= (d * Q > x) ? 1 : 0;
        d += ((d + 1) * Q <= x) ? 1 : 0;
        return d;
    }
};

// partial slots owned by a segment of n pages starting at `start`
__device__ __forceinline__ int seg_slots(int start, int n, const Divider& dq) {
    return n > 0 ? dq(start + n - 1) - dq(start) + 1 : 0;
}

// Walker over the flat page list: (segment, page within it).
struct PageCursor {
    Seg seg;
    int p;
};

__device__ __forceinline__ void cursor_next(const DecodeArgs& a, const EntryPages& np, PageCursor& c) {
    if (++c.p < c.seg.n) return;
    int b = c.seg.b, h = c.seg.h + 1;
    const int start = c.seg.start + c.seg.n;
    c.p = 0;
    for (;;) {
        if (h == a.pv.H) { h = 0; ++b; }
        if (b >= a.B) { c.seg = Seg{b, 0, 0, start}; return; }
        const int n = np(b);
        if (n > 0) { c.seg = Seg{b, h, n, start}; return; }
        h = a.pv.H;                                  // empty entry: skip its heads
    }
}

// ---------------------------------------------------------------------------
// Matrix-core page stream (BF16 pages, D in {64, 128}, 1..8 entries).
//
// One 256-thread block per compute unit streams its range of the flat page
// list through an LDS ring of NS page stages filled by direct-to-LDS loads,
// so NS-1 pages are in flight while one is computed.  Wave w owns tokens
// [16w, 16w+16) of every page and keeps its own online-softmax state.
//  * QK^T on the matrix cores: S^T[16 tokens x 16] = K . Q^T with
//    v_mfma_f32_16x16x32_bf16; the GQ query heads of the page's KV head are
//    the columns (the other columns are padding: a column of the product
//    only ever depends on its own column of Q^T, and no padding column is
//    read back).
//  * The accumulator layout of S^T (lane l: column l%16, tokens 4(l/16)+r)
//    is the B-operand layout of v_mfma_f32_16x16x16_bf16, so P^T feeds PV
//    in place.
//  * PV on the matrix cores: O^T[16 dims x 16] += V^T . P^T per 16-dim tile,
//    V^T read from LDS with the transposing 64-bit read (ds_read_b64_tr_b16:
//    within a 16-lane row, lane i receives element i%4 of the 8-byte chunks
//    addressed by lanes 4e + i/4).  P enters as two bf16 terms p_hi + p_lo
//    (two products), about 2^-16 relative error instead of bf16's 2^-9.
//  * Lazy rescaling: the exponent reference of a column moves only when a
//    page's maximum exceeds it by more than 2^8, so the accumulators are
//    rescaled a few times per segment instead of on every new maximum.
//  * K rows are XOR-swizzled in 16-byte chunks, V rows in 32-byte units, so
//    both reads are free of LDS bank conflicts.
// Each page's slice, valid rows and segment-end flag are listed in LDS before
// the ring starts.  When a segment ends, the four waves' states are merged
// through the stage just consumed, and the merged partial waits in registers
// until the stream ends (loads and stores share the vector-memory counter
// that the ring waits on).  Then a segment that lies inside one block is
// normalized and written out; the others are stored as partials, and the
// block that brings the last partial of a segment (per-segment arrival
// counter in the workspace) combines them in block order: one launch,
// deterministic output.

// Query columns of one entry for the page stream: keys [0, keys) exist; query
// token i (row cu + i of q and out) sees keys [0, min(n0 + i + 1, keys)).
// One query token per entry (decode) is n0 = ctx - 1, T = 1.  `owned` is false
// for an entry a chunk-mode launch leaves to another kernel.
struct EntryQ {
    int n0, T, cu, keys;
    bool owned;
};

template <bool CHUNK, int GQ>
__device__ __forceinline__ EntryQ entry_q(const DecodeArgs& a, int b) {
    const int row = ld_uniform(a.table_rows, b);
    const bool ok = row >= 0 && row < a.pv.C;
    if constexpr (!CHUNK) {
        const int ctx = ok ? min(ld_uniform(a.seq_lens, b), a.max_ctx) : 0;
        return EntryQ{ctx - 1, 1, b, ctx, true};
    } else {
        const int c0 = ld_uniform(a.cu_q, b), T = ld_uniform(a.cu_q, b + 1) - c0;
        const int n0 = ld_uniform(a.q_pos0, b);
        const int keys = ok ? max(0, min(n0 + T, a.max_ctx)) : 0;
        return EntryQ{n0, T, c0, keys, T * GQ <= a.max_cols};
    }
}

template <bool CHUNK, int GQ>
__device__ __forceinline__ EntryPages stream_pages(const DecodeArgs& a) {
    EntryPages e;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int n = 0;
        if (i < a.B) {
            const EntryQ q = entry_q<CHUNK, GQ>(a, i);
            n = (q.owned && q.T > 0) ? (q.keys + kPage - 1) >> kPageShift : 0;
        }
        e.n[i] = n;
    }
    return e;
}

// NCT column tiles of 16 query columns; column c = 16*ct + lane%16 holds query
// token c / GQ and head c % GQ of the segment's KV head.  CHUNK: several query
// tokens per entry (verify / chunked prefill) with a causal limit per column.
template <int D, int GQ, int NCT, bool CHUNK>
__global__ void __launch_bounds__(256) paged_stream_kernel(DecodeArgs a) {
    constexpr int NCH = D / 8;                     // 16-byte chunks per row
    constexpr int NT = 256;
    constexpr int SLOTS = 64 * NCH;                // chunks per page slice of one plane
    constexpr int SLICE_BYTES = SLOTS * 16;
    constexpr int PER_T = SLOTS / NT;              // direct-to-LDS loads per thread and plane
    constexpr int NS = D == 128 ? 4 : 8;           // ring stages
    constexpr int LOADS_PER_PAGE = 2 * PER_T;
    constexpr int NC = D / 32;                     // QK products, k = 32 each
    constexpr int NDT = D / 16;                    // PV tiles of 16 dims
    constexpr int DPW = NDT / 4;                   // tiles each wave merges and writes
    constexpr int WBUF = NDT * 4 * 64;             // floats of one wave's state in the merge area
    constexpr int NCOL = 16 * NCT;                 // query columns (partial slot width)
    constexpr int QCOL = CHUNK ? NCOL : GQ;        // query rows cached per segment
    constexpr int QSEG_RAW = (CHUNK ? 16384 : 8192) / (QCOL * D * 2);
    constexpr int QSEG = QSEG_RAW < 1 ? 1 : (QSEG_RAW > 8 ? 8 : QSEG_RAW);   // segments with cached queries
    constexpr int PMAX = NCT == 1 ? 3 : 2;         // merged partials held in registers
    static_assert((D == 64 || D == 128) && GQ >= 1 && GQ <= 16 && GQ <= NCOL, "shape");
    static_assert(PER_T == 2 || PER_T == 4, "page fetch shapes");
    static_assert(NS * SLICE_BYTES == 0x10000, "V stages sit 64 KiB above the K stages");
    static_assert(LOADS_PER_PAGE * (NS - 1) < 64, "vmcnt range");
    static_assert(2 * WBUF * 4 <= SLICE_BYTES, "two waves' merge state fit one slice");

    __shared__ u32x4 ring[2][NS][SLOTS];           // [K | V][stage][slot]
    __shared__ int2 pinfo[kStreamPages];           // per page of the range: (slice g*H + h or -1, meta)
    __shared__ u32x4 qcache[QSEG][QCOL * NCH];     // query rows of the first QSEG segments
    __shared__ float mlbuf[4][16][2];              // per-wave (m, l) of every column at a segment end
    __shared__ int4 ctask[PMAX];                   // segments the flushing block completes: (b, h, first slot, slots)
    __shared__ int ctask_n;

    const int tid = int(threadIdx.x);
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, li = lane & 15, lg = lane >> 4;
    const int H = a.pv.H, M = a.pv.M, G = int(gridDim.x), i_blk = int(blockIdx.x);

    const EntryPages np = stream_pages<CHUNK, GQ>(a);
    if (i_blk == 0) {                              // entries with nothing to attend produce zeros
        for (int b = 0; b < a.B; ++b) {
            if (np(b) != 0) continue;
            const EntryQ e = entry_q<CHUNK, GQ>(a, b);
            if (!e.owned) continue;
            for (int x = tid; x < e.T * a.Hq * D; x += NT) a.out[size_t(e.cu) * a.Hq * D + x] = 0.f;
        }
    }
    int total = 0;
    for (int b = 0; b < a.B; ++b) total += np(b) * H;
    if (total == 0) return;
    const int Q = (total + G - 1) / G;             // the host sizes G so that Q <= kStreamPages
    const Divider dq(Q);
    const int u0 = i_blk * Q;
    const int npg = min(u0 + Q, total) - u0;       // pages of this block
    if (npg <= 0) return;

    PageCursor cc{Seg{0, 0, 0, 0}, 0};             // the segment being computed
    {
        int st = 0;                                // first stream page of entry b
        for (int b = 0; b < a.B; ++b) {
            const int n = np(b);
            if (n > 0 && u0 < st + n * H) {
                const int h = (u0 - st) / n;
                cc = PageCursor{Seg{b, h, n, st + h * n}, u0 - st - h * n};
                break;
            }
            st += n * H;
        }
    }

    // query row of column c of entry e (head h*GQ + c%GQ of token c/GQ)
    auto q_row = [&](const EntryQ& e, int h, int c) __attribute__((always_inline)) {
        return a.q + (size_t(e.cu + c / GQ) * a.Hq + size_t(h) * GQ + c % GQ) * D;
    };

    // Before the ring starts: every page's slice, valid rows, segment-end flag
    // and page index (meta = valid rows | 256 at a segment end | page << 9),
    // and the query rows of the first QSEG segments (later ones load theirs
    // when they start).
    {
        PageCursor c = cc;
        int off = 0, k = 0;
        while (off < npg) {
            const int cnt = min(c.seg.n - c.p, npg - off);
            const int row = ld_uniform(a.table_rows, c.seg.b);
            const EntryQ e = entry_q<CHUNK, GQ>(a, c.seg.b);
            const int32_t* trow = a.pv.table + size_t(row) * a.pv.L;
            for (int i = tid; i < cnt; i += NT) {
                const int p = c.p + i;
                const int g0 = trow[p];
                const bool mapped = g0 >= 0 && g0 < M;
                const int lim = mapped ? min(kPage, e.keys - p * kPage) : 0;
                const bool end = (p == c.seg.n - 1) || (off + i == npg - 1);
                pinfo[off + i] = make_int2(mapped ? g0 * H + c.seg.h : -1, lim | (end ? 256 : 0) | (p << 9));
            }
            if (k < QSEG) {
                const int ncol = min(e.T * GQ, QCOL);
                for (int i = tid; i < ncol * NCH; i += NT)
                    qcache[k][i] = reinterpret_cast<const u32x4*>(q_row(e, c.seg.h, i / NCH))[i % NCH];
            }
            ++k;
            off += cnt;
            c.p += cnt - 1;
            cursor_next(a, np, c);
        }
        wait_vmcnt<0>();
        block_lds_barrier();
    }

    // Stage layout: K slot s (row t = s / NCH, position x = s % NCH) holds
    // chunk x ^ kswz(t) of row t; V slot s holds chunk x ^ vswz(t).
    auto kswz = [](int t) __attribute__((always_inline)) { return NCH == 16 ? (t & 15) : ((t >> 1) & 7); };
    auto vswz = [](int t) __attribute__((always_inline)) { return NCH == 16 ? ((t & 7) << 1) : (((t >> 1) & 3) << 1); };
    const char* kplane = static_cast<const char*>(a.pv.lv.k_code);
    const char* vplane = static_cast<const char*>(a.pv.lv.v_code);
    uint32_t k_src[PER_T], v_src[PER_T];           // source byte offsets within a page slice
#pragma unroll
    for (int k = 0; k < PER_T; ++k) {
        const int s = k * NT + tid;
        const int t = s / NCH, x = s % NCH;
        k_src[k] = uint32_t(t * NCH + (x ^ kswz(t))) * 16u;
        v_src[k] = uint32_t(t * NCH + (x ^ vswz(t))) * 16u;
    }
    const uint32_t ring_lds = uint32_t(reinterpret_cast<uintptr_t>((lds_byte_ptr)(&ring[0][0][0])));
    // page fi of the range into stage fs
    auto fetch = [&](int fi, int fs) __attribute__((always_inline)) {
        const uint32_t dst = ring_lds + uint32_t(fs * SLICE_BYTES + w * 1024);
        const int sl = __builtin_amdgcn_readfirstlane(pinfo[fi].x);
        const size_t off = size_t(sl < 0 ? 0 : sl) * SLICE_BYTES;
        if constexpr (PER_T == 4) fetch_page4(dst, kplane + off, vplane + off, k_src, v_src);
        else fetch_page2(dst, kplane + off, vplane + off, k_src, v_src);
    };

    // Per-lane LDS offsets into stage 0, fixed for the whole stream (the
    // stage adds an immediate below 64 KiB).
    //  QK A operand (K): row 16w + li, chunk 4c + lg (u32x4 index)
    //  PV A operand (V^T, transposing read): lane li of row group lg points at
    //  token 16w + 4lg + li/4, dims 16dt + 4(li%4) .. +3 (byte offset from the
    //  K stage 0, i.e. including the 64 KiB to the V stages)
    int koff[NC], voff[NDT];
    {
        const int t = 16 * w + li;
#pragma unroll
        for (int c = 0; c < NC; ++c) koff[c] = t * NCH + ((4 * c + lg) ^ kswz(t));
        const int tv = 16 * w + 4 * lg + (li >> 2), qd = li & 3;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
            voff[dt] = 0x10000 + tv * NCH * 16 + (((2 * dt + (qd >> 1)) ^ vswz(tv)) * 16) + 8 * (qd & 1);
    }

    bf16x8_t qb[NCT][NC];                          // Q^T B operand: column 16ct + li, chunk 4c + lg
    int klim[NCT];                                 // keys this lane's column sees (0: padding column)
    int kmin = 0;                                  // smallest limit of a real column of the segment
    auto start_segment = [&](int k_seg, int b, int h) __attribute__((always_inline)) {
        const EntryQ e = entry_q<CHUNK, GQ>(a, b);
        const int ncol = e.T * GQ;
        kmin = min(e.n0 + 1, e.keys);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const int col = 16 * ct + li;
            klim[ct] = col < ncol ? min(e.n0 + col / GQ + 1, e.keys) : 0;
        }
        if (k_seg < QSEG) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const int col = 16 * ct + li;
                const int cq = min(col, QCOL - 1);
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const u32x4 v = qcache[k_seg][cq * NCH + 4 * c + lg];
                    qb[ct][c] = __builtin_bit_cast(bf16x8_t, col < ncol ? v : u32x4{0u, 0u, 0u, 0u});
                }
            }
        } else {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const int col = 16 * ct + li;
                const u32x4* qg = reinterpret_cast<const u32x4*>(q_row(e, h, col < ncol ? col : 0));
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const u32x4 v = qg[4 * c + lg];
                    qb[ct][c] = __builtin_bit_cast(bf16x8_t, col < ncol ? v : u32x4{0u, 0u, 0u, 0u});
                }
            }
            wait_vmcnt<0>();                       // drains the ring: only past the cached segments
        }
    };

    f32x4_t acc[NCT][NDT];
    float m_ref[NCT], l_part[NCT];
    auto reset = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            m_ref[ct] = -INFINITY;
            l_part[ct] = 0.f;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) acc[ct][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    };

    // merged partials waiting for the end of the stream
    f32x4_t pend_acc[PMAX][NCT][DPW];
    float pend_m[PMAX][NCT], pend_l[PMAX][NCT];
    int pend_b[PMAX], pend_h[PMAX], pend_first[PMAX], pend_nsl[PMAX];   // pend_first: first slot of the segment
    int npend = 0;

    // Partials cross blocks (and the L2s of different dies) as device-scope
    // relaxed atomic stores and loads, which are coherent without cache
    // write-back or invalidation (device-scope fences are L2-wide maintenance
    // operations here, costly for every block on the die).  A block counts
    // its arrival only after its partial stores completed (vmcnt 0), and the
    // last block loads the partials only after its increment returned.
    auto st_dev = [](float* p, float v) __attribute__((always_inline)) {
        __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    auto ld_dev = [](const float* p) __attribute__((always_inline)) {
        return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    // The combine issues the loads of four outputs of a thread before it uses
    // any (one memory round trip for up to four partials per output).
    auto combine = [&](int b, int h, int first, int nsl) __attribute__((always_inline)) {
        constexpr int CMAX = 4, XB = 4;
        const EntryQ e = entry_q<CHUNK, GQ>(a, b);
        const int ncol = min(e.T * GQ, QCOL);
#pragma unroll 1
        for (int x0 = tid; x0 < ncol * D; x0 += XB * NT) {
            float fm[XB], fl[XB], fa[XB];         // running fold of the earlier rounds
#pragma unroll 1
            for (int k0 = 0; k0 < nsl; k0 += CMAX) {   // more than CMAX partials: folded in rounds
                const int kn = min(CMAX, nsl - k0);
                float mk[XB][CMAX], lk[XB][CMAX], ak[XB][CMAX];
#pragma unroll
                for (int xb = 0; xb < XB; ++xb) {
                    const int x = x0 + xb * NT;
                    const int c = x / D, d = x % D;
#pragma unroll
                    for (int k = 0; k < CMAX; ++k) {
                        if (x < ncol * D && k < kn) {
                            const size_t it = size_t(first + k0 + k) * NCOL + c;
                            mk[xb][k] = ld_dev(a.part_ml + it * 2);
                            lk[xb][k] = ld_dev(a.part_ml + it * 2 + 1);
                            ak[xb][k] = ld_dev(a.part_acc + it * D + d);
                        }
                    }
                }
#pragma unroll
                for (int xb = 0; xb < XB; ++xb) {
                    const int x = x0 + xb * NT;
                    if (x >= ncol * D) continue;
                    float mx = k0 > 0 ? fm[xb] : -INFINITY;
#pragma unroll
                    for (int k = 0; k < CMAX; ++k)
                        if (k < kn) mx = fmaxf(mx, mk[xb][k]);
                    float l = 0.f, acc_x = 0.f;
#pragma unroll
                    for (int k = 0; k < CMAX; ++k) {
                        if (k < kn) {
                            const float wgt = mk[xb][k] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mk[xb][k] - mx);
                            l += lk[xb][k] * wgt;
                            acc_x += ak[xb][k] * wgt;
                        }
                    }
                    if (k0 > 0) {
                        const float wp = fm[xb] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(fm[xb] - mx);
                        l += fl[xb] * wp;
                        acc_x += fa[xb] * wp;
                    }
                    fm[xb] = mx;
                    fl[xb] = l;
                    fa[xb] = acc_x;
                }
            }
#pragma unroll
            for (int xb = 0; xb < XB; ++xb) {
                const int x = x0 + xb * NT;
                if (x >= ncol * D) continue;
                const int c = x / D, d = x % D;
                float* o = a.out + (size_t(e.cu + c / GQ) * a.Hq + size_t(h) * GQ + c % GQ) * D + d;
                *o = fl[xb] > 0.f ? fa[xb] * (1.f / fl[xb]) : 0.f;
            }
        }
    };

    // Write out or store every pending partial, count arrivals, combine the
    // segments this block completes.  Block-uniform; waits for all memory
    // traffic of the block.
    auto flush = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < PMAX; ++k) {
            if (k >= npend) break;
            const EntryQ e = entry_q<CHUNK, GQ>(a, pend_b[k]);
            const int ncol = e.T * GQ;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const int c = 16 * ct + li;
                if (c >= ncol) continue;
                if (pend_nsl[k] == 1) {
                    const float inv = pend_l[k][ct] > 0.f ? 1.f / pend_l[k][ct] : 0.f;
                    float* o = a.out + (size_t(e.cu + c / GQ) * a.Hq + size_t(pend_h[k]) * GQ + c % GQ) * D + 4 * lg;
#pragma unroll
                    for (int kk = 0; kk < DPW; ++kk) {
                        const f32x4_t v = pend_acc[k][ct][kk] * inv;
                        *reinterpret_cast<float4*>(o + 16 * (w * DPW + kk)) = make_float4(v[0], v[1], v[2], v[3]);
                    }
                } else {
                    const size_t it = size_t(i_blk + pend_b[k] * H + pend_h[k]) * NCOL + c;
                    float* o = a.part_acc + it * D + 4 * lg;
#pragma unroll
                    for (int kk = 0; kk < DPW; ++kk)
#pragma unroll
                        for (int r = 0; r < 4; ++r) st_dev(o + 16 * (w * DPW + kk) + r, pend_acc[k][ct][kk][r]);
                    if (w == 0 && lg == 0) {
                        st_dev(a.part_ml + it * 2, pend_m[k][ct]);
                        st_dev(a.part_ml + it * 2 + 1, pend_l[k][ct]);
                    }
                }
            }
        }
        wait_vmcnt<0>();                           // this block's partials are complete
        __syncthreads();
        if (tid == 0) {                            // arrive; list the segments this block completes
            int nt = 0;
#pragma unroll
            for (int k = 0; k < PMAX; ++k) {
                if (k >= npend) break;
                if (pend_nsl[k] > 1) {
                    const unsigned old = atomicAdd(a.arrive + pend_b[k] * H + pend_h[k], 1u);
                    if (int(old) + 1 == pend_nsl[k]) {
                        ctask[nt] = make_int4(pend_b[k], pend_h[k], pend_first[k], pend_nsl[k]);
                        ++nt;
                    }
                }
            }
            ctask_n = nt;
        }
        __syncthreads();
        const int nt = __builtin_amdgcn_readfirstlane(ctask_n);
#pragma unroll 1
        for (int t = 0; t < nt; ++t) {
            const int4 c = ctask[t];
            const int cb = __builtin_amdgcn_readfirstlane(c.x), ch = __builtin_amdgcn_readfirstlane(c.y);
            combine(cb, ch, __builtin_amdgcn_readfirstlane(c.z), __builtin_amdgcn_readfirstlane(c.w));
            if (tid == 0)                          // ready for the next call
                __hip_atomic_store(a.arrive + cb * H + ch, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        wait_vmcnt<0>();
        __syncthreads();
        npend = 0;
    };

    // segment end: merge the four waves' states through stage st (waves 0-1
    // use its K slice, waves 2-3 its V slice), one column tile at a time
    auto finish_segment = [&](int st) __attribute__((always_inline)) {
        auto wbuf = [&](int v) __attribute__((always_inline)) {
            return reinterpret_cast<float*>(&ring[v >> 1][st][0]) + (v & 1) * WBUF;
        };
        f32x4_t merged[NCT][DPW];
        float mxs[NCT], lts[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const float lw = rows_sum(l_part[ct]);
            block_lds_barrier();                   // every wave is done with stage st (or the last round)
            float* mine = wbuf(w);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int r = 0; r < 4; ++r) mine[(dt * 4 + r) * 64 + lane] = acc[ct][dt][r];
            if (lg == 0) {
                mlbuf[w][li][0] = m_ref[ct];
                mlbuf[w][li][1] = lw;
            }
            block_lds_barrier();
            float mw[4], cw[4], mx = -INFINITY, lt = 0.f;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                mw[v] = mlbuf[v][li][0];
                mx = fmaxf(mx, mw[v]);
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                cw[v] = mw[v] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw[v] - mx);
                lt += mlbuf[v][li][1] * cw[v];
            }
#pragma unroll
            for (int kk = 0; kk < DPW; ++kk) {
                const int dt = w * DPW + kk;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float x = 0.f;
#pragma unroll
                    for (int v = 0; v < 4; ++v) x += wbuf(v)[(dt * 4 + r) * 64 + lane] * cw[v];
                    merged[ct][kk][r] = x;
                }
            }
            mxs[ct] = mx;
            lts[ct] = lt;
        }
        if (npend == PMAX) flush();                // rare: many segments in one range
#pragma unroll
        for (int k = 0; k < PMAX; ++k) {
            if (k == npend) {
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
                    for (int kk = 0; kk < DPW; ++kk) pend_acc[k][ct][kk] = merged[ct][kk];
                    pend_m[k][ct] = mxs[ct];
                    pend_l[k][ct] = lts[ct];
                }
                pend_b[k] = cc.seg.b;
                pend_h[k] = cc.seg.h;
                pend_first[k] = dq(cc.seg.start) + cc.seg.b * H + cc.seg.h;
                pend_nsl[k] = seg_slots(cc.seg.start, cc.seg.n, dq);
            }
        }
        ++npend;
        reset();
    };

    int seg_k = 0;
    start_segment(seg_k, cc.seg.b, cc.seg.h);
    reset();
    const int tb = 16 * w + 4 * lg;                 // token of accumulator register r: tb + r
    int meta_ring[NS];                              // meta of the pages in the ring, by stage
#pragma unroll
    for (int k = 0; k < NS - 1; ++k) {
        if (k < npg) {
            fetch(k, k);
            meta_ring[k] = __builtin_amdgcn_readfirstlane(pinfo[k].y);
        } else {
            meta_ring[k] = 0;
        }
    }
    meta_ring[NS - 1] = 0;

    // one page in stage J (compile time, so every LDS offset is an immediate)
    auto step = [&](auto jc, int i) __attribute__((always_inline)) {
        constexpr int J = decltype(jc)::value;
        constexpr int FS = (J + NS - 1) % NS;
        // page i is in stage J for every wave, and every wave is done with
        // page i-1, whose stage takes page i+NS-1; the last NS-1 pages of
        // the range wait for everything in flight (nothing is left to issue)
        if (i + NS - 1 < npg) {
            wait_vmcnt<LOADS_PER_PAGE * (NS - 2)>();
            block_lds_barrier();
            fetch(i + NS - 1, FS);
            meta_ring[FS] = __builtin_amdgcn_readfirstlane(pinfo[i + NS - 1].y);
        } else {
            wait_vmcnt<0>();
            block_lds_barrier();
        }

        const int meta = meta_ring[J];
        const int lim = meta & 255;                 // valid rows of the page
        if (lim > 16 * w) {                         // this wave has valid rows in the page
            const int tok0 = (meta >> 9) * kPage;   // first key of the page
            const u32x4* kst = &ring[0][J][0];
            f32x4_t s[NCT];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) s[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const bf16x8_t kk = __builtin_bit_cast(bf16x8_t, kst[koff[c]]);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
                    s[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk, qb[ct][c], s[ct], 0, 0, 0);
            }
            const bool masked = tok0 + kPage > kmin;   // a real column's limit falls inside the page
            s16x4_t phi[NCT], plo[NCT];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                float sj[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) sj[r] = s[ct][r] * a.scale_log2;
                if (masked) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (tok0 + tb + r >= klim[ct]) sj[r] = -INFINITY;
                }
                const float pm = rows_max(fmaxf(fmaxf(sj[0], sj[1]), fmaxf(sj[2], sj[3])));
                if (__builtin_amdgcn_ballot_w64(pm > m_ref[ct] + kRescaleLog2)) {
                    const float mn = pm > m_ref[ct] + kRescaleLog2 ? pm : m_ref[ct];
                    const float alpha = m_ref[ct] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref[ct] - mn);
                    l_part[ct] *= alpha;
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) acc[ct][dt] *= alpha;
                    m_ref[ct] = mn;
                }
                float p[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    p[r] = __builtin_amdgcn_exp2f(sj[r] - m_ref[ct]);
                    // a column with no visible key yet (chunk mode) has no reference
                    if constexpr (CHUNK) p[r] = m_ref[ct] == -INFINITY ? 0.f : p[r];
                }
                l_part[ct] += (p[0] + p[1]) + (p[2] + p[3]);
                uint32_t h01, l01, h23, l23;
                split_bf16(p[0], p[1], h01, l01);
                split_bf16(p[2], p[3], h23, l23);
                phi[ct] = __builtin_bit_cast(s16x4_t, u32x2{h01, h23});
                plo[ct] = __builtin_bit_cast(s16x4_t, u32x2{l01, l23});
            }
            if (lim < kPage) {
                // rows past the frontier hold stale bytes (possibly NaN): this
                // wave clears its own rows of the V slice, which only it reads
                const int r0 = max(lim, 16 * w), rows = 16 * w + 16 - r0;
                u32x4* vrows = &ring[1][J][r0 * NCH];
                for (int x = lane; x < rows * NCH; x += 64) vrows[x] = u32x4{0u, 0u, 0u, 0u};
                wave_lds_sync();
            }
            const lds_byte_ptr vst = (lds_byte_ptr)(&ring[0][J][0]);   // voff includes the K-to-V distance
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const s16x4_t va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(vst + voff[dt]));
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    acc[ct][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, phi[ct], acc[ct][dt], 0, 0, 0);
                    acc[ct][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, plo[ct], acc[ct][dt], 0, 0, 0);
                }
            }
        }

        if (meta & 256) {
            finish_segment(J);
            if (i + 1 < npg) {
                cc.p = cc.seg.n - 1;
                cursor_next(a, np, cc);
                ++seg_k;
                start_segment(seg_k, cc.seg.b, cc.seg.h);
            }
        }
    };

    for (int i0 = 0; i0 < npg; i0 += NS) {
        step(std::integral_constant<int, 0>{}, i0);
        if (i0 + 1 < npg) step(std::integral_constant<int, 1>{}, i0 + 1);
        if (i0 + 2 < npg) step(std::integral_constant<int, 2>{}, i0 + 2);
        if (i0 + 3 < npg) step(std::integral_constant<int, 3>{}, i0 + 3);
        if constexpr (NS == 8) {
            if (i0 + 4 < npg) step(std::integral_constant<int, 4>{}, i0 + 4);
            if (i0 + 5 < npg) step(std::integral_constant<int, 5>{}, i0 + 5);
            if (i0 + 6 < npg) step(std::integral_constant<int, 6>{}, i0 + 6);
            if (i0 + 7 < npg) step(std::integral_constant<int, 7>{}, i0 + 7);
        }
    }
    flush();
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

// Pages per split.  KVS_DECODE_CHUNK_PAGES overrides the default (a tuning
// knob read once per process); the split only depends on logical positions.
int chunk_pages() {
    static const int cp = [] {
        const char* e = std::getenv("KVS_DECODE_CHUNK_PAGES");
        const int v = e ? std::atoi(e) : 0;
        return (v >= 1 && v <= 1024) ? v : 8;
    }();
    return cp;
}

// Blocks of the page-stream kernel: one per compute unit (its LDS ring takes
// most of the 160 KiB), every one streaming the same share of pages; more
// when a share would exceed the kStreamPages a block lists in LDS.
int stream_grid(const PoolView& pv, int B, int max_seq_len) {
    static const int cus = [] {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        const char* e = std::getenv("KVS_DECODE_STREAM_BLOCKS");
        const int v = e ? std::atoi(e) : 0;
        return (v >= 1 && v <= 4096) ? v : n;
    }();
    const long long bound = (long long)B * pv.H * ((max_seq_len + kPage - 1) / kPage);
    const long long need = (bound + kStreamPages - 1) / kStreamPages;
    return int(need > cus ? need : cus);
}

// The matrix-core page stream covers BF16 pages with D in {64, 128} and up to
// eight entries per call; everything else takes the chunked split kernel.
bool stream_path(const PoolView& pv, int B, int gq) {
    return pv.k_codec == CODEC_BF16 && pv.v_codec == CODEC_BF16 && (pv.D == 64 || pv.D == 128) && B <= 8 &&
           (gq == 1 || gq == 2 || gq == 4 || gq == 8);
}

int max_chunks_for(int max_seq_len) {
    const int pages = (max_seq_len + kPage - 1) / kPage;
    return (pages + chunk_pages() - 1) / chunk_pages();
}

template <int D, int GQ>
hipError_t launch_gq(const DecodeArgs& a, hipStream_t s) {
    if constexpr (D == 64 || D == 128) {
        if (stream_path(a.pv, a.B, GQ)) {
            paged_stream_kernel<D, GQ, 1, false><<<dim3(unsigned(stream_grid(a.pv, a.B, a.max_ctx))), 256, 0, s>>>(a);
            return hipGetLastError();
        }
    }
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

// Workspace: [arrival counters][partial (m, l) pairs][partial accumulators],
// each from a 256-byte boundary.  The counters (one per (table row, KV head),
// sized by the pool so the layout does not move with B) must be zero before
// the first call; every call leaves them zero.
size_t arrive_bytes(const PoolView& pv) { return (size_t(pv.C) * pv.H * sizeof(uint32_t) + 255) / 256 * 256; }

size_t ml_floats(size_t items, size_t gq) { return (items * gq * 2 + 63) / 64 * 64; }

// partial slots: one per split (chunk path) or one per (block, touched
// segment) of the page stream, at most G + B*H
size_t partial_slots(const PoolView& pv, int B, int gq, int max_seq_len) {
    if (stream_path(pv, B, gq)) return size_t(stream_grid(pv, B, max_seq_len)) + size_t(B) * pv.H;
    return size_t(B) * pv.H * max_chunks_for(max_seq_len);
}

// partial slot width: the page stream keeps one 16-column tile per slot
size_t slot_cols(const PoolView& pv, int B, int gq) { return stream_path(pv, B, gq) ? 16 : size_t(gq); }

size_t decode_workspace_bytes(const PoolView& pv, int B, int Hq, int max_seq_len) {
    const size_t gq = pv.H ? size_t(Hq / pv.H) : 0;
    const size_t items = partial_slots(pv, B, int(gq), max_seq_len);
    const size_t cols = slot_cols(pv, B, int(gq));
    return arrive_bytes(pv) + (ml_floats(items, cols) + items * cols * size_t(pv.D)) * sizeof(float);
}

bool stream_chunk_supported(const PoolView& pv, int B, int gq) { return stream_path(pv, B, gq); }

size_t stream_chunk_workspace_bytes(const PoolView& pv, int B, int max_seq_len) {
    const size_t items = size_t(stream_grid(pv, B, max_seq_len)) + size_t(B) * pv.H;
    return arrive_bytes(pv) + (ml_floats(items, 32) + items * 32 * size_t(pv.D)) * sizeof(float);
}

template <int D>
hipError_t launch_chunk_d(const DecodeArgs& a, int gq, hipStream_t s) {
    const dim3 grid(unsigned(stream_grid(a.pv, a.B, a.max_ctx)));
    switch (gq) {
        case 1: paged_stream_kernel<D, 1, 2, true><<<grid, 256, 0, s>>>(a); break;
        case 2: paged_stream_kernel<D, 2, 2, true><<<grid, 256, 0, s>>>(a); break;
        case 4: paged_stream_kernel<D, 4, 2, true><<<grid, 256, 0, s>>>(a); break;
        case 8: paged_stream_kernel<D, 8, 2, true><<<grid, 256, 0, s>>>(a); break;
        default: return hipErrorNotSupported;
    }
    return hipGetLastError();
}

hipError_t launch_stream_chunk(const PoolView& pv, int B, int Hq, const int32_t* table_rows, const int32_t* q_pos0,
                               const int32_t* cu_q, int max_seq_len, const void* q, float sm_scale, float* out,
                               void* ws, int max_cols, hipStream_t s) {
    DecodeArgs a{};
    a.pv = pv;
    a.table_rows = table_rows;
    a.q_pos0 = q_pos0;
    a.cu_q = cu_q;
    a.max_cols = max_cols;
    a.q = static_cast<const uint16_t*>(q);
    a.out = out;
    a.B = B;
    a.Hq = Hq;
    a.max_ctx = max_seq_len;
    const int gq = Hq / pv.H;
    const size_t items = size_t(stream_grid(pv, B, max_seq_len)) + size_t(B) * pv.H;
    a.arrive = static_cast<uint32_t*>(ws);
    a.part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + arrive_bytes(pv));
    a.part_acc = a.part_ml + ml_floats(items, 32);
    a.scale_log2 = sm_scale * kLog2e;
    switch (pv.D) {
        case 64: return launch_chunk_d<64>(a, gq, s);
        case 128: return launch_chunk_d<128>(a, gq, s);
    }
    return hipErrorNotSupported;
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
    a.chunk_pages = chunk_pages();
    a.max_chunks = max_chunks_for(max_seq_len);
    a.max_ctx = max_seq_len;
    const int gq = Hq / pv.H;
    const size_t items = partial_slots(pv, B, gq, max_seq_len);
    a.arrive = static_cast<uint32_t*>(ws);
    a.part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + arrive_bytes(pv));
    a.part_acc = a.part_ml + ml_floats(items, slot_cols(pv, B, gq));
    a.scale_log2 = sm_scale * kLog2e;
    switch (pv.D) {
        case 64: return launch_d<64>(a, gq, s);
        case 128: return launch_d<128>(a, gq, s);
        case 256: return launch_d<256>(a, gq, s);
    }
    return hipErrorNotSupported;
}

}  // namespace kvs
