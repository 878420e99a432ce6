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
#include <cstdlib>
#include <type_traits>

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

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
}

// An LDS pointer the optimizer cannot see through: reads through it stay in
// the page loop instead of being hoisted into a query-sized register file.
typedef const u32x4 __attribute__((address_space(3)))* lds_cu4;

__device__ __forceinline__ lds_cu4 opaque_lds(lds_cu4 p) {
    asm volatile("" : "+v"(p));
    return p;
}

// Same, but only once `dep` is available: bounds how many chunks of query
// reads the scheduler may issue ahead of the dot products.
__device__ __forceinline__ lds_cu4 opaque_lds_after(lds_cu4 p, float dep) {
    asm volatile("" : "+v"(p) : "v"(dep));
    return p;
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

typedef const u32x4 __attribute__((address_space(4)))* const_u4;   // read-only: scalar loads

// ---------------------------------------------------------------------------
// Flat page stream (BF16).  The work of one decode call is the ordered list of
// (entry b, KV head h, page p) for b < B, h < H, p < ceil(ctx_b / 64): segment
// s = b*H + h holds ceil(ctx_b/64) consecutive pages.  Block i of G takes the
// contiguous range [i*Q, min((i+1)*Q, total)), Q = ceil(total / G), so every
// block streams the same number of pages whatever the length mix.  A block
// writes one partial (m, l, acc) per segment it touches; segment s owns the
// partial slots base(s) + (i - first(s)) for the blocks first(s)..last(s)
// that cover it.  Ranges depend only on the context lengths, never on page
// ids, and the combine adds the slots in block order: deterministic.
struct Seg {
    int b, h, n;       // entry, KV head, pages in the segment
    int start;         // first global page index of the segment
};

// Wave-uniform metadata reads (block table, rows, lengths) as scalar loads:
// they are read-only for the kernel, and they must not join the vector-memory
// counter that the page ring waits on.
typedef const int32_t __attribute__((address_space(4)))* const_i32;

__device__ __forceinline__ int ld_uniform(const int32_t* p, size_t idx) {
    const const_i32 cp = (const_i32)(const void*)p;
    return cp[__builtin_amdgcn_readfirstlane(int(idx))];
}

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

__device__ __forceinline__ int page_id(const DecodeArgs& a, int b, int p) {
    const int row = ld_uniform(a.table_rows, b);
    return ld_uniform(a.pv.table, size_t(row) * a.pv.L + p);
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

// Ring-pipelined page stream (BF16): one 512-thread block per compute unit,
// the same flat page partition as above.  The block's LDS holds a ring of NS
// page stages (K slice + V slice each), so NS-1 pages are in flight while one
// is computed -- enough outstanding bytes to cover HBM latency under load.
// Eight waves: wave w works on query heads (w & 3) + 4r (r < HPW) for the
// tokens [32*grp, 32*grp + 32) of each page, grp = w >> 2, so two waves share
// every SIMD and each does half of a page's math.  The two token groups keep
// their own online-softmax state and are merged through LDS when a segment
// ends (same lane layout in both).
//  * QK^T: lane l holds token l % 32 of its group and head_dim half l / 32;
//    the two halves' dot products are added across lanes l, l ^ 32
//    (v_permlane32_swap).
//  * one workgroup barrier per page: after it, page u is complete in its
//    stage for every wave and every wave is done with page u-1, whose stage
//    is refilled with page u+NS-1;
//  * the block's page slices are listed into LDS once before the ring
//    starts, so issuing a page needs no dependent table loads.
//  * query: scalar loads (outside the vector-memory counter the ring waits
//    on), then held in vector registers: half a head per lane;
//  * probabilities move from the QK lanes to the PV lanes with ds_bpermute;
//  * finished segments' partials wait in registers (up to PMAX) and are
//    written after the stream, so no store is ever pending while the ring's
//    load counter is waited on; beyond PMAX they are stored at once and the
//    ring is drained before its next wait.
template <int D, int GQ>
__global__ void __launch_bounds__(512) decode_bf16_ring_kernel(DecodeArgs a) {
    constexpr int NCH = D / 8;                     // 16-byte chunks per row
    constexpr int HCH = NCH / 2;                   // chunks per head_dim half
    constexpr int TPI = 64 / NCH;                  // rows per 1 KiB
    constexpr int NT = 512;
    constexpr int SLOTS = 64 * NCH;                // 16-byte chunks per page slice
    static_assert(NCH >= 8 && NCH <= 16 && GQ >= 4, "shape");
    constexpr int PER_T = SLOTS / NT;              // DMA instructions per thread and plane
    constexpr int STAGE_U4 = 2 * SLOTS;
    constexpr int HPW = GQ / 4;                    // heads per wave
    constexpr int NS = 4;                          // ring stages
    constexpr int PMAX = HPW > 1 ? 1 : 2;          // partials held in registers
    constexpr int LOADS_PER_PAGE = 2 * PER_T;
    constexpr int RPG = NCH / 2;                   // PV row groups per token half
    static_assert(LOADS_PER_PAGE * (NS - 1) < 64, "vmcnt range");
    constexpr int PLIST = HPW > 1 ? 2048 : 4096;   // page slices listed per block
    __shared__ u32x4 ring[NS][STAGE_U4];           // [stage][K slots | V slots]
    __shared__ float merge[4][HPW][10][64];        // group-1 state handed to group 0
    __shared__ int plist[PLIST];                   // slice (g*H + h) of each page of the range

    const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
    const int lane = int(threadIdx.x) & 63;
    const int tid = int(threadIdx.x);
    const int wh = w & 3, grp = w >> 2;
    const int H = a.pv.H, M = a.pv.M, G = int(gridDim.x), i_blk = int(blockIdx.x);

    const EntryPages np = entry_pages(a);
    int total = 0;
    for (int b = 0; b < a.B; ++b) total += np(b) * H;
    if (total == 0) return;
    const int Q = (total + G - 1) / G;
    const Divider dq(Q);
    const int u0 = i_blk * Q;
    const int u1 = min(u0 + Q, total);
    if (u0 >= u1) return;

    PageCursor start_c{Seg{0, 0, 0, 0}, 0};
    int base = 0;
    {
        int st = 0;
        for (int b = 0; b < a.B && start_c.seg.n == 0; ++b) {
            const int n = np(b);
            for (int h = 0; h < H; ++h) {
                if (n > 0 && u0 < st + n) { start_c = PageCursor{Seg{b, h, n, st}, u0 - st}; break; }
                base += seg_slots(st, n, dq);
                st += n;
            }
        }
    }

    const u32x4* kbase = static_cast<const u32x4*>(a.pv.lv.k_code);
    const u32x4* vbase = static_cast<const u32x4*>(a.pv.lv.v_code);
    // K row t keeps chunk x in slot x ^ swz(t); swz spreads 16 consecutive
    // rows over all 64 LDS banks for 16-byte reads
    auto swz = [](int t) { return NCH == 16 ? (t & 15) : ((t >> 1) & 7); };
    int k_src[PER_T];
#pragma unroll
    for (int k = 0; k < PER_T; ++k) {
        const int slot = k * NT + tid;
        const int t = slot / NCH, x = slot % NCH;
        k_src[k] = t * NCH + (x ^ swz(t));
    }
    // The range's page slices, listed once into LDS (vector loads of the
    // block table, before the ring starts); ranges longer than the list read
    // the table through scalar loads instead.
    const bool listed = (u1 - u0) <= PLIST;
    if (listed) {
        PageCursor c = start_c;
        int off = 0;
        while (off < u1 - u0) {
            const int cnt = min(c.seg.n - c.p, (u1 - u0) - off);
            const int row = ld_uniform(a.table_rows, c.seg.b);
            const int32_t* trow = a.pv.table + size_t(row) * a.pv.L + c.p;
            for (int i = tid; i < cnt; i += NT) {
                const int g0 = trow[i];
                plist[off + i] = (g0 >= 0 && g0 < M) ? g0 * H + c.seg.h : -1;
            }
            off += cnt;
            c.p += cnt - 1;
            cursor_next(a, np, c);
        }
        wait_vmcnt<0>();
        block_lds_barrier();
    }
    auto slice_of = [&](const PageCursor& c, int u) {
        if (listed) return __builtin_amdgcn_readfirstlane(plist[u - u0]);
        const int g0 = page_id(a, c.seg.b, c.p);
        return (g0 >= 0 && g0 < M) ? g0 * H + c.seg.h : -1;
    };
    auto fetch = [&](const PageCursor& c, int u, int st) {
        const int sl = slice_of(c, u);
        const size_t off = size_t(sl < 0 ? 0 : sl) * SLOTS;
#pragma unroll
        for (int k = 0; k < PER_T; ++k) {
            auto* kd = (void __attribute__((address_space(3)))*)(&ring[st][k * NT + w * 64]);
            auto* vd = (void __attribute__((address_space(3)))*)(&ring[st][SLOTS + k * NT + w * 64]);
            __builtin_amdgcn_global_load_lds((const void*)(kbase + off + k_src[k]), kd, 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const void*)(vbase + off + k * NT + tid), vd, 16, 0, 0);
        }
    };
    auto wait_pages = [&](int n) {
        switch (n) {
            case 0: wait_vmcnt<0>(); break;
            case 1: wait_vmcnt<LOADS_PER_PAGE * 1>(); break;
            case 2: wait_vmcnt<LOADS_PER_PAGE * 2>(); break;
            default: wait_vmcnt<LOADS_PER_PAGE * 3>(); break;
        }
    };

    // lane roles
    const int qt = lane & 31;                      // QK: token within the group's half page
    const int hd = lane >> 5;                      // QK: head_dim half
    const int cpv = lane % NCH, tg = lane / NCH;   // PV: chunk and row group

    u32x4 qr[HPW][HCH];
    auto load_q = [&](int b, int h) {
#pragma unroll
        for (int r = 0; r < HPW; ++r) {
            const int j = wh + 4 * r;
            const const_u4 qg = (const_u4)(const void*)(a.q + (size_t(b) * a.Hq + size_t(h) * GQ + j) * D);
#pragma unroll
            for (int c = 0; c < HCH; ++c) {
                // lanes of both halves issue the same scalar loads; select the half
                const u32x4 lo = qg[c], hi = qg[HCH + c];
                qr[r][c] = hd ? hi : lo;
                asm volatile("" : "+v"(qr[r][c]));
            }
        }
    };
    float m_run[HPW], l_part[HPW], acc[HPW][8];
    auto reset = [&]() {
#pragma unroll
        for (int r = 0; r < HPW; ++r) {
            m_run[r] = -INFINITY;
            l_part[r] = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;
        }
    };
    reset();

    float pend_acc[PMAX][HPW][8], pend_m[PMAX][HPW], pend_l[PMAX][HPW];
    int pend_slot[PMAX];
    int npend = 0;
    auto store_partial = [&](int slot, const float (&ac)[HPW][8], const float (&mm)[HPW], const float (&ll)[HPW]) {
#pragma unroll
        for (int r = 0; r < HPW; ++r) {
            const size_t it = size_t(slot) * GQ + (wh + 4 * r);
            if (tg == 0) {
                float4* dst = reinterpret_cast<float4*>(a.part_acc + it * D + cpv * 8);
                dst[0] = make_float4(ac[r][0], ac[r][1], ac[r][2], ac[r][3]);
                dst[1] = make_float4(ac[r][4], ac[r][5], ac[r][6], ac[r][7]);
            }
            if (lane == 0) {
                a.part_ml[it * 2] = mm[r];
                a.part_ml[it * 2 + 1] = ll[r];
            }
        }
    };
    bool stores_pending = false;
    // segment end: sum row groups, merge the two token groups, keep or store
    auto finish_segment = [&](int slot) {
        float ac[HPW][8], ll[HPW], mm[HPW];
#pragma unroll
        for (int r = 0; r < HPW; ++r) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float x = acc[r][e];
#pragma unroll
                for (int o = NCH; o < 64; o <<= 1) x += __shfl_xor(x, o, 64);
                ac[r][e] = x;
            }
            ll[r] = wave_sum(l_part[r]) * 0.5f;     // both head_dim halves counted each p
            mm[r] = m_run[r];
        }
        if (grp == 1) {
#pragma unroll
            for (int r = 0; r < HPW; ++r) {
#pragma unroll
                for (int e = 0; e < 8; ++e) merge[wh][r][e][lane] = ac[r][e];
                merge[wh][r][8][lane] = mm[r];
                merge[wh][r][9][lane] = ll[r];
            }
        }
        block_lds_barrier();
        if (grp == 0) {
#pragma unroll
            for (int r = 0; r < HPW; ++r) {
                const float m1 = merge[wh][r][8][lane], l1 = merge[wh][r][9][lane];
                const float mx = fmaxf(mm[r], m1);
                const float w0 = mx == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mm[r] - mx);
                const float w1 = mx == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mx);
#pragma unroll
                for (int e = 0; e < 8; ++e) ac[r][e] = ac[r][e] * w0 + merge[wh][r][e][lane] * w1;
                ll[r] = ll[r] * w0 + l1 * w1;
                mm[r] = mx;
            }
            if (npend < PMAX) {
#pragma unroll
                for (int k = 0; k < PMAX; ++k) {
                    if (k == npend) {
#pragma unroll
                        for (int r = 0; r < HPW; ++r) {
#pragma unroll
                            for (int e = 0; e < 8; ++e) pend_acc[k][r][e] = ac[r][e];
                            pend_m[k][r] = mm[r];
                            pend_l[k][r] = ll[r];
                        }
                        pend_slot[k] = slot;
                    }
                }
            } else {
                store_partial(slot, ac, mm, ll);
            }
        }
        if (npend < PMAX) ++npend;
        else stores_pending = true;
        reset();
    };

    PageCursor ic = start_c;                        // next page to issue
    int issued = u0;
    for (int k = 0; k < NS - 1 && issued < u1; ++k) {
        fetch(ic, issued, (issued - u0) % NS);
        cursor_next(a, np, ic);
        ++issued;
    }
    PageCursor cc = start_c;                        // page being computed
    int slot = base + (i_blk - dq(cc.seg.start));
    int cur_ctx = ctx_of(a, cc.seg.b);
    load_q(cc.seg.b, cc.seg.h);

    for (int u = u0; u < u1; ++u) {
        const int st = (u - u0) % NS;
        if (stores_pending) { wait_vmcnt<0>(); stores_pending = false; }
        else wait_pages(issued - u - 1);
        // page u is in stage st for every wave, and every wave is done with page
        // u-1, whose stage takes page u+NS-1
        block_lds_barrier();
        if (issued < u1) {
            fetch(ic, issued, (issued - u0) % NS);
            cursor_next(a, np, ic);
            ++issued;
        }

        const int sl = slice_of(cc, u);
        const int lim = sl >= 0 ? min(kPage, cur_ctx - cc.p * kPage) : 0;
        const int glim = lim - 32 * grp;            // valid rows of this group's half page
        const u32x4* kst = &ring[st][0];
        const u32x4* vst = &ring[st][SLOTS];
        {
            // QK^T: token 32*grp + qt, head_dim half hd
            const int t = 32 * grp + qt;
            u32x4 krow[HCH];
#pragma unroll
            for (int c = 0; c < HCH; ++c) krow[c] = kst[t * NCH + ((hd * HCH + c) ^ swz(t))];
            const bool valid = qt < glim;
            float pj[HPW];
#pragma unroll
            for (int r = 0; r < HPW; ++r) {
                float sc4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < HCH; ++c) {
                    sc4[0] = dot2_bf16(krow[c].x, qr[r][c].x, sc4[0]);
                    sc4[1] = dot2_bf16(krow[c].y, qr[r][c].y, sc4[1]);
                    sc4[2] = dot2_bf16(krow[c].z, qr[r][c].z, sc4[2]);
                    sc4[3] = dot2_bf16(krow[c].w, qr[r][c].w, sc4[3]);
                }
                float sc = (sc4[0] + sc4[1]) + (sc4[2] + sc4[3]);
                {                                   // add the other head_dim half (lane ^ 32)
                    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(sc), __float_as_uint(sc),
                                                                     false, false);
                    sc = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
                }
                const float sj = valid ? sc * a.scale_log2 : -INFINITY;
                const float mn = fmaxf(m_run[r], wave_max_uniform(sj));
                if (mn > m_run[r]) {                // wave-uniform
                    const float alpha = __builtin_amdgcn_exp2f(m_run[r] - mn);
                    l_part[r] *= alpha;
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[r][e] *= alpha;
                    m_run[r] = mn;
                }
                pj[r] = valid ? __builtin_amdgcn_exp2f(sj - m_run[r]) : 0.f;
                l_part[r] += pj[r];
            }
            // PV: rows 32*grp + i*TPI + tg (i < RPG), chunk cpv
            auto pv_rows = [&](auto masked) {
                u32x4 vrow[RPG];
                float pt[HPW][RPG];
#pragma unroll
                for (int i = 0; i < RPG; ++i) vrow[i] = vst[(32 * grp + i * TPI + tg) * NCH + cpv];
#pragma unroll
                for (int r = 0; r < HPW; ++r)
#pragma unroll
                    for (int i = 0; i < RPG; ++i)
                        pt[r][i] = __int_as_float(
                            __builtin_amdgcn_ds_bpermute((i * TPI + tg) << 2, __float_as_int(pj[r])));
#pragma unroll
                for (int i = 0; i < RPG; ++i) {
                    u32x4 vv = vrow[i];
                    if constexpr (decltype(masked)::value) {
                        // rows past the frontier hold stale bytes: never let them reach acc
                        if (i * TPI + tg >= glim) vv = u32x4{0u, 0u, 0u, 0u};
                    }
                    float v[8];
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2) {
                        v[2 * e2] = __uint_as_float(vv[e2] << 16);
                        v[2 * e2 + 1] = __uint_as_float(vv[e2] & 0xFFFF0000u);
                    }
#pragma unroll
                    for (int r = 0; r < HPW; ++r)
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[r][e] += pt[r][i] * v[e];
                }
            };
            if (glim < 32) pv_rows(std::true_type{});
            else pv_rows(std::false_type{});
        }

        const bool more = u + 1 < u1;
        if (cc.p + 1 == cc.seg.n || !more) {
            finish_segment(slot);
            if (more) {
                base += seg_slots(cc.seg.start, cc.seg.n, dq);
                cursor_next(a, np, cc);
                slot = base + (i_blk - dq(cc.seg.start));
                cur_ctx = ctx_of(a, cc.seg.b);
                load_q(cc.seg.b, cc.seg.h);
            }
        } else {
            cursor_next(a, np, cc);
        }
    }

    if (grp == 0) {
#pragma unroll
        for (int k = 0; k < PMAX; ++k)
            if (k < npend) store_partial(pend_slot[k], pend_acc[k], pend_m[k], pend_l[k]);
    }
}

// Combine the stream partials of each (entry, query head), in block order.
template <int D, int GQ>
__global__ void __launch_bounds__(64) decode_stream_combine_kernel(DecodeArgs a, int G) {
    constexpr int EPL = D / 64;
    const int lane = int(threadIdx.x);
    const int b = int(blockIdx.x) / a.Hq, j = int(blockIdx.x) % a.Hq;
    const int h = j / GQ, jj = j % GQ;
    const int H = a.pv.H;
    const EntryPages np = entry_pages(a);
    int total = 0;
    for (int bb = 0; bb < a.B; ++bb) total += np(bb) * H;
    float* o = a.out + (size_t(b) * a.Hq + j) * D + lane * EPL;
    const int n = np(b);
    if (n == 0) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] = 0.f;
        return;
    }
    const int Q = (total + G - 1) / G;
    const Divider dq(Q);
    int base = 0, start = 0;
    for (int bb = 0; bb <= b; ++bb) {
        const int ns = np(bb);
        const int hh_end = bb < b ? H : h;
        for (int hh = 0; hh < hh_end; ++hh) {
            base += seg_slots(start, ns, dq);
            start += ns;
        }
    }
    const int cnt = seg_slots(start, n, dq);
    float mx = -INFINITY;
    for (int k = 0; k < cnt; ++k) mx = fmaxf(mx, a.part_ml[(size_t(base + k) * GQ + jj) * 2]);
    float l = 0.f, acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
    for (int k = 0; k < cnt; ++k) {
        const size_t it = size_t(base + k) * GQ + jj;
        const float wgt = exp2f(a.part_ml[it * 2] - mx);
        l += a.part_ml[it * 2 + 1] * wgt;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] += a.part_acc[it * D + lane * EPL + e] * wgt;
    }
    const float inv = 1.f / l;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = acc[e] * inv;
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
// the whole 160 KiB), every one streaming the same share of pages.
int stream_grid() {
    static const int g = [] {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        const char* e = std::getenv("KVS_DECODE_STREAM_BLOCKS");
        const int v = e ? std::atoi(e) : 0;
        return (v >= 1 && v <= 65536) ? v : cus;
    }();
    return g;
}

bool stream_path(const PoolView& pv, int gq) {
    return pv.k_codec == CODEC_BF16 && pv.v_codec == CODEC_BF16 && (pv.D == 64 || pv.D == 128) &&
           (gq == 4 || gq == 8);
}

int max_chunks_for(int max_seq_len) {
    const int pages = (max_seq_len + kPage - 1) / kPage;
    return (pages + chunk_pages() - 1) / chunk_pages();
}

template <int D, int GQ>
hipError_t launch_gq(const DecodeArgs& a, hipStream_t s) {
    const int items = a.B * a.pv.H * a.max_chunks;
    const dim3 grid(unsigned((items + 3) / 4));
    const int kc = a.pv.k_codec, vc = a.pv.v_codec;
    bool launched = false;
    if constexpr ((D == 64 || D == 128) && (GQ == 4 || GQ == 8)) {
        if (kc == CODEC_BF16 && vc == CODEC_BF16) {
            const int G = stream_grid();
            decode_bf16_ring_kernel<D, GQ><<<dim3(unsigned(G)), 512, 0, s>>>(a);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            decode_stream_combine_kernel<D, GQ><<<dim3(unsigned(a.B * a.Hq)), 64, 0, s>>>(a, G);
            return hipGetLastError();
        }
    }
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

// partial (m, l) pairs first, then the accumulators from a 256-byte boundary
size_t ml_floats(size_t items, size_t gq) { return (items * gq * 2 + 63) / 64 * 64; }

// partial slots: one per split (chunk path) or one per (block, touched
// segment) of the page stream, at most G + B*H
size_t partial_slots(const PoolView& pv, int B, int gq, int max_seq_len) {
    if (stream_path(pv, gq)) return size_t(stream_grid()) + size_t(B) * pv.H;
    return size_t(B) * pv.H * max_chunks_for(max_seq_len);
}

size_t decode_workspace_bytes(const PoolView& pv, int B, int Hq, int max_seq_len) {
    const size_t gq = pv.H ? size_t(Hq / pv.H) : 0;
    const size_t items = partial_slots(pv, B, int(gq), max_seq_len);
    return (ml_floats(items, gq) + items * gq * size_t(pv.D)) * sizeof(float);
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
    a.part_ml = static_cast<float*>(ws);
    a.part_acc = a.part_ml + ml_floats(items, size_t(gq));
    a.scale_log2 = sm_scale * kLog2e;
    switch (pv.D) {
        case 64: return launch_d<64>(a, gq, s);
        case 128: return launch_d<128>(a, gq, s);
        case 256: return launch_d<256>(a, gq, s);
    }
    return hipErrorNotSupported;
}

}  // namespace kvs
