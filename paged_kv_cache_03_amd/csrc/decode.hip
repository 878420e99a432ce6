// decode.hip -- paged decode (one query token per entry) on the page pool.
//
// NInfer "Paged KV Context Store" page: PagedKVBatchLayerView (table_rows[b]
// selects the block-table row of compact entry b), P=64 translation
// (block = position >> 6, offset = position & 63), consumer rules (page
// translation at page granularity, no gather-to-contiguous, free choice of
// tile/split/wave/LDS scheme), wrapper validation and caller guarantees.
//
// A decode is a plan of the batch state (stream_plan.hip; one per step, it
// serves every layer) and a run:
//  * the matrix-core page stream (BF16 pages, D in {64, 128}; quantized
//    pages in qstream.hip): every page of the plan in one flat list, cut
//    into equal ranges, two 256-thread blocks per compute unit; leading
//    pages that entries share are read once for all of them; then a combine
//    launch for outputs with several pieces;
//  * the split kernel (every other profile and shape): entry b's pages are
//    cut into chunks of `chunk_pages` consecutive logical pages, one wave per
//    (entry, KV head, chunk), then a combine launch.
// In both, the split depends only on logical positions, the host-side
// bounds and which logical pages are shared, never on physical page ids, and
// the combine runs in a fixed order, so outputs are bitwise identical under
// any permutation of page ids.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <type_traits>

#include "attn_common.h"
#include "internal.h"
#include "launch.h"
#include "kv_read.h"
#include "stream_common.h"
#include "stream_plan.h"
#include "decode_common.h"

namespace kvs {
namespace {

// One 64-lane wave per work item (entry b, KV head h, chunk c).  QK: lane t
// owns token t of the page; PV: lane owns EPL = D/64 head_dim elements.
template <int D, int GQ, int KC, int VC, int SB>
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
    const int row = plan_ent(a, b, plan::E_ROW);
    const int ctx = plan_ent(a, b, plan::E_KEYS);
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
        const size_t slab = (size_t(g) * a.pv.sg + size_t(h) * a.pv.sh) * kPage;
        const int tok = pg * kPage + lane;
        const bool valid = tok < ctx;
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
            for (int e = 0; e < EPL; ++e) v[e] = KVRow<VC, D, SB>::load1(a.pv.lv.v_code, a.pv.lv.v_scale, slab + t,
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
// Matrix-core page stream, register-fed (BF16 pages, D in {64, 128}, 1..8
// entries): runs a page-stream plan (stream_plan.h).  Block i of two per
// compute unit streams the pages of stream positions [i*Q, (i+1)*Q).  A unit
// (segment s, KV head h) carries the query columns of every entry in the
// segment's mask: GQ heads per entry in decode (shared pages carry the heads
// of all entries that share them), T x GQ (token, head) columns of one entry
// in chunk mode; each column has its own causal key limit.  Wave w owns keys
// [16w, 16w+16) of every page, loads them itself straight into the registers
// the matrix cores read, one page ahead (buffer loads whose range ends at
// the page's last visible row, so stale rows read as zeros; non-temporal: a
// page is read once per call), and keeps its own online-softmax state; the
// waves meet only at unit ends.  Per page and wave:
//  * QK^T: S^T[16 keys x 16 columns] = K . Q^T with v_mfma_f32_16x16x32_bf16;
//    lane (li, lg) loads key 16w + li, dims 8(4c + lg) .. +7 for product c,
//    a 16-byte row load each (padding columns are zero, never read back);
//  * the accumulator layout of S^T (lane l: column l%16, keys 4(l/16) + r)
//    is the operand layout of P^T, which enters as two bf16 terms
//    p_hi + p_lo (about 2^-16 relative error instead of bf16's 2^-9);
//  * PV: O^T[16 dims x 16 columns] += V^T . [P_hi; P_lo] as one k=32 product
//    per tile (the lane's keys listed twice, against P_hi then P_lo).  Lane
//    (li, lg) loads the D/16 dims starting at (D/16) li of keys 16w + 4lg + r,
//    r = 0..3 -- the keys whose probabilities it holds -- and pairs the bf16
//    values of two keys per dim with one byte permute each: the transpose.
//    Row m of tile j holds head dim (D/16) m + j;
//  * lazy rescaling: a column's exponent reference moves only when a page's
//    maximum exceeds it by more than 2^8.
// Before the first page, one round trip brings the plan's tables and the
// block's page list into LDS, with the query rows of the block's first units
// and its new-token rows (decode with the step's rows: the wave owning a new
// row's key takes it from there instead of the loaded one, and the block
// writes the rows into their pages at the end).  When a unit ends, the four
// waves' states are merged through a 16 KiB LDS buffer, four tiles at a time;
// a column whose (entry, KV head) has no other piece is normalized and
// written out, the others are stored as partials in slot i + sigma for the
// combine launch, which folds each (entry, KV head)'s pieces in unit and
// block order: deterministic output.  Both the block index and sigma only
// grow along the stream, so no two (block, unit) pieces share a slot.
template <int D, int GQ, int NCT, bool CHUNK>
__global__ void __launch_bounds__(256, vstream_bpc(D)) paged_vstream_kernel(DecodeArgs a) {
    using namespace plan;
    constexpr int BPC = vstream_bpc(D);            // blocks per compute unit
    constexpr int NCH = D / 8;                     // 16-byte chunks per bf16 row
    constexpr int NT = 256;
    constexpr int NC = D / 32;                     // QK products, k = 32 each
    constexpr int NDT = D / 16;                    // PV tiles of 16 dims
    constexpr int NP = NDT / 4;                    // merge passes, four tiles each
    constexpr int VW = D / 32;                     // 32-bit V words per key and lane (D/16 bf16 dims)
    constexpr int NCOL = 16 * NCT;                 // query columns (partial slot width)
    constexpr int QCHUNKS = 1024 / BPC;            // query cache: 16-byte chunks
    constexpr int QSEG = QCHUNKS / (NCOL * NCH);   // units with cached queries
    constexpr int PAGES = kStreamPages / BPC;      // most pages a block takes
    constexpr int PF = vstream_buffers(D);         // page buffers per wave: PF - 1 pages in flight
    constexpr size_t SLICE = size_t(64) * D * 2;   // bytes of one plane's page slice
    static_assert((D == 64 || D == 128 || (D == 256 && !CHUNK)) && GQ >= 1 && GQ <= 16 && GQ <= NCOL, "shape");
    static_assert(QSEG >= 1 && QSEG * NCOL * NCH == QCHUNKS && QCHUNKS % NT == 0, "query cache shape");
    static_assert(PAGES % NT == 0, "page list");
    typedef unsigned int vrow_t __attribute__((ext_vector_type(VW)));

    __shared__ int2 pinfo[PAGES];                  // the block's pages: (slice number of (g, h) or -1, meta)
    __shared__ u32x4 qcache[QCHUNKS];              // query rows of the first QSEG units: [unit][column][chunk]
    __shared__ float mbuf[4 * 16 * 64];            // unit merge: four waves x four tiles x 4 registers
    __shared__ float mlbuf[4][16][2];              // per-wave (m, l) of every column at a unit's end
    __shared__ int ent_s[kMaxEnt][kEntWords];
    __shared__ int seg_s[kMaxSeg][kSegWords];
    __shared__ int exp_s[kMaxEnt * kMaxH];         // pieces per (entry, KV head)
    __shared__ int patch_s[kMaxPatch];             // the block's new-token rows: page | entry | head | row
    __shared__ u32x4 pstage[NT];                   // their K and V chunks

    const int tid = int(threadIdx.x);
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, li = lane & 15, lg = lane >> 4;
    const int H = a.pv.H, i_blk = int(blockIdx.x), G = int(gridDim.x);
    const int32_t* P = a.plan;

    // one round trip: the plan's header and tables, this block's page list
    const int magic = ld_uniform(P, H_MAGIC), pb = ld_uniform(P, H_B), ph = ld_uniform(P, H_H);
    const int pgq = ld_uniform(P, H_GQ), pg = ld_uniform(P, H_G), pq = ld_uniform(P, H_QCAP);
    const int pchunk = ld_uniform(P, H_CHUNK);
    const bool plan_ok = (magic == kMagic) & (pb == a.B) & (ph == H) & (pgq == GQ) & (pg == G) & (pq == a.qcap) &
                         (pchunk == int(CHUNK));
    const int nseg = ld_uniform(P, H_NSEG), zero = ld_uniform(P, H_ZERO);
    const int npg = ld_uniform(P, off_blk(H) + 4 * size_t(i_blk));
    int sig = ld_uniform(P, off_blk(H) + 4 * size_t(i_blk) + 1);   // unit being computed
    const bool append = !CHUNK && a.k_new != nullptr;
    const int npatch = append ? ld_uniform(P, off_blk(H) + 4 * size_t(i_blk) + 2) : 0;
    {
        static_assert(kMaxEnt * kEntWords <= NT && kMaxSeg * kSegWords <= NT && kMaxPatch <= NT, "tables");
        static_assert(kMaxEnt * kMaxH <= 2 * NT, "tables");
        const int2* pl = reinterpret_cast<const int2*>(P + off_pages(H, G)) + size_t(i_blk) * a.qcap;
        const int ne = kMaxEnt * H;
        const int v_ent = P[kOffEnt + min(tid, kMaxEnt * kEntWords - 1)];
        const int v_seg = P[kOffSeg + min(tid, kMaxSeg * kSegWords - 1)];
        const int v_patch = P[off_patch(H, G) + size_t(i_blk) * kMaxPatch + min(tid, kMaxPatch - 1)];
        const int v_exp0 = P[kOffExp + min(tid, ne - 1)];
        const int v_exp1 = P[kOffExp + min(tid + NT, ne - 1)];
        int2 v_pg[PAGES / NT];
#pragma unroll
        for (int k = 0; k < PAGES / NT; ++k) v_pg[k] = pl[min(tid + k * NT, a.qcap - 1)];
        if (tid < kMaxEnt * kEntWords) ent_s[tid / kEntWords][tid % kEntWords] = v_ent;
        if (tid < kMaxSeg * kSegWords) seg_s[tid / kSegWords][tid % kSegWords] = v_seg;
        if (tid < kMaxPatch) patch_s[tid] = v_patch;
        if (tid < ne) exp_s[tid] = v_exp0;
        if (tid + NT < ne) exp_s[tid + NT] = v_exp1;
#pragma unroll
        for (int k = 0; k < PAGES / NT; ++k)
            if (tid + k * NT < a.qcap) pinfo[tid + k * NT] = v_pg[k];
    }
    block_lds_barrier();
    if (!plan_ok) {                                // a plan of another batch shape: make it visible
        if (!CHUNK && i_blk == 0)
            for (int x = tid; x < a.B * a.Hq * D; x += NT) a.out[x] = __builtin_nanf("");
        return;
    }
    if (i_blk == 0) {                              // entries with nothing to attend produce zeros
        for (int b = 0; b < a.B; ++b) {
            if (!((zero >> b) & 1)) continue;
            const size_t r0 = size_t(ent_s[b][E_CU]) * a.Hq * D;
            for (int x = tid; x < ent_s[b][E_T] * a.Hq * D; x += NT) a.out[r0 + x] = 0.f;
        }
    }
    if (npg <= 0) return;

    // column c of a unit of segment s: entry, query token, head within the group
    struct Col {
        int b, tok, j;
    };
    auto col_of = [&](int s, int c) __attribute__((always_inline)) {
        if constexpr (CHUNK) {
            return Col{seg_s[s][S_OWNER], c / GQ, c % GQ};
        } else {
            int m = seg_s[s][S_MASK];
            for (int k = c / GQ; k > 0; --k) m &= m - 1;
            return Col{__builtin_ctz(unsigned(m | 0x100)), 0, c % GQ};
        }
    };
    auto ncol_of = [&](int s) __attribute__((always_inline)) {
        return __builtin_popcount(unsigned(seg_s[s][S_MASK])) * seg_s[s][S_W];
    };
    auto q_row = [&](const Col& cl, int h) __attribute__((always_inline)) {
        return a.q + (size_t(ent_s[cl.b][E_CU] + cl.tok) * a.Hq + size_t(h) * GQ + cl.j) * D;
    };
    auto unit_seg = [&](int sg) __attribute__((always_inline)) { return sg / H; };

    const char* kplane = static_cast<const char*>(a.pv.lv.k_code);
    const char* vplane = static_cast<const char*>(a.pv.lv.v_code);
    char* kplane_w = static_cast<char*>(a.pv.lv.k_code);
    char* vplane_w = static_cast<char*>(a.pv.lv.v_code);

    // page buffers: K operand chunks and V rows of this wave's keys.  Buffer
    // loads whose range ends at the page's last visible row: rows past it
    // (stale bytes, possibly NaN) come back as zeros.
    u32x4 kbuf[PF][NC];
    vrow_t vbuf[PF][4];
    int pmeta[PF];                                 // meta of the page in each buffer
    const int krow = (16 * w + li) * (2 * D) + 16 * lg;           // byte offset of chunk lg of key 16w + li
    const int vrow = (16 * w + 4 * lg) * (2 * D) + (D / 8) * li;  // byte offset of the lane's dims of key 16w + 4lg
    // Every step issues the same loads: past the block's last page they
    // have an empty range (zeros, no memory access), so the compiler's
    // vector-memory wait counts stay exact across the unrolled loop.
    auto load_page = [&](int fi, u32x4 (&kb)[NC], vrow_t (&vb)[4], int& meta) __attribute__((always_inline)) {
        const bool live = fi < npg;
        const int2 pi = pinfo[live ? fi : 0];
        const int sl = live ? __builtin_amdgcn_readfirstlane(pi.x) : -1;
        meta = live ? __builtin_amdgcn_readfirstlane(pi.y) | (fi == npg - 1 ? 256 : 0) : 0;
        const int bytes = sl < 0 ? 0 : (meta & 255) * (2 * D);   // an unmapped block reads nothing
        const size_t off = size_t(sl < 0 ? 0 : sl) * SLICE;
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kplane) + off, 0, bytes, kBufferWord3);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vplane) + off, 0, bytes, kBufferWord3);
#pragma unroll
        for (int c = 0; c < NC; ++c)
            kb[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, krow + 64 * c, 0, kNonTemporal));
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if constexpr (VW == 8) {
                const u32x4 v0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, vrow + r * 2 * D, 0, kNonTemporal));
                const u32x4 v1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, vrow + r * 2 * D + 16, 0, kNonTemporal));
                vb[r] = vrow_t{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
            } else if constexpr (VW == 4) {
                vb[r] = __builtin_bit_cast(vrow_t, __builtin_amdgcn_raw_buffer_load_b128(rv, vrow + r * 2 * D, 0, kNonTemporal));
            } else {
                vb[r] = __builtin_bit_cast(vrow_t, __builtin_amdgcn_raw_buffer_load_b64(rv, vrow + r * 2 * D, 0, kNonTemporal));
            }
        }
    };

    // the step's new-token rows (staged chunk x of plane pl of row q at
    // pstage[q * PCH + pl * NCH + x]) and the query rows of the first QSEG
    // units (columns past a unit's last read row 0 of the call; never used):
    // loads first, then the first pages, then the LDS writes
    constexpr int PCH = 2 * NCH;                   // chunks of one staged row pair
    u32x4 prow = u32x4{0u, 0u, 0u, 0u};
    if (npatch > 0) {
        const int q = tid / PCH, pl = (tid / NCH) & 1, x = tid % NCH;
        if (q < npatch) {
            const int pe = patch_s[q];
            const int b = (pe >> 12) & 7, h = (pe >> 15) & 63;
            prow = reinterpret_cast<const u32x4*>((pl ? a.v_new : a.k_new) + (size_t(b) * H + h) * D)[x];
        }
    }
    u32x4 qv[QCHUNKS / NT];
#pragma unroll
    for (int k = 0; k < QCHUNKS / NT; ++k) {
        const int x = k * NT + tid;
        const int u = x / (NCOL * NCH), c = (x / NCH) % NCOL, ch = x % NCH;
        const int sg = sig + u, s = unit_seg(sg);
        const u32x4* src = reinterpret_cast<const u32x4*>(a.q);
        if (s < nseg && c < ncol_of(s)) src = reinterpret_cast<const u32x4*>(q_row(col_of(s, c), sg - s * H)) + ch;
        qv[k] = *src;
    }
#pragma unroll
    for (int k = 0; k < PF - 1; ++k) load_page(k, kbuf[k], vbuf[k], pmeta[k]);
    pstage[tid] = prow;
#pragma unroll
    for (int k = 0; k < QCHUNKS / NT; ++k) qcache[k * NT + tid] = qv[k];
    block_lds_barrier();

    typedef const u32x4 __attribute__((address_space(1)))* glb_q_cptr;
    bf16x8_t qb[NCT][NC];                          // Q^T B operand: column 16ct + li, chunk 4c + lg
    int klim[NCT];                                 // keys this lane's column sees (0: padding column)
    int kmin = 0;                                  // smallest limit of a real column of the unit
    auto start_unit = [&](int k_unit, int sg) __attribute__((always_inline)) {
        const int s = unit_seg(sg), h = sg - s * H;
        const int ncol = ncol_of(s);
        kmin = seg_s[s][S_KMIN];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const int c = 16 * ct + li;
            const Col cl = col_of(s, c < ncol ? c : 0);
            klim[ct] = c < ncol ? min(ent_s[cl.b][E_N0] + cl.tok + 1, ent_s[cl.b][E_KEYS]) : 0;
        }
        if (k_unit < QSEG) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const int c = 16 * ct + li;
#pragma unroll
                for (int k = 0; k < NC; ++k) {
                    const u32x4 v = qcache[(k_unit * NCOL + c) * NCH + 4 * k + lg];
                    qb[ct][k] = __builtin_bit_cast(bf16x8_t, c < ncol ? v : u32x4{0u, 0u, 0u, 0u});
                }
            }
        } else {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const int c = 16 * ct + li;
                const glb_q_cptr qg = (glb_q_cptr)(q_row(col_of(s, c < ncol ? c : 0), h));
#pragma unroll
                for (int k = 0; k < NC; ++k) {
                    const u32x4 v = qg[4 * k + lg];
                    qb[ct][k] = __builtin_bit_cast(bf16x8_t, c < ncol ? v : u32x4{0u, 0u, 0u, 0u});
                }
            }
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

    // the staged new-token rows into their pages (nothing in this launch reads
    // them from memory: the waves patched them into their registers)
    auto store_rows = [&]() __attribute__((always_inline)) {
        const int q = tid / PCH, pl = (tid / NCH) & 1, x = tid % NCH;
        if (q < npatch) {
            const int pe = patch_s[q];
            const int sl = pinfo[pe & 0xfff].x, r = (pe >> 21) & 63;
            if (sl >= 0)
                *reinterpret_cast<u32x4*>((pl ? vplane_w : kplane_w) + size_t(sl) * SLICE + r * NCH * 16 + x * 16) =
                    pstage[tid];
        }
    };

    // unit end: merge the four waves' states through mbuf, four tiles per
    // pass; wave w folds accumulator register w, so each lane ends with four
    // consecutive head dims of row 4lg + w of each pass
    auto finish_unit = [&]() __attribute__((always_inline)) {
        f32x4_t merged[NCT][NP];
        float mxs[NCT], lts[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const float lw = rows_sum(l_part[ct]);
            float cw[4], lt = 0.f, mx = -INFINITY;
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                block_lds_barrier();               // every wave read the previous pass
                float* mine = mbuf + w * 1024;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                    for (int r = 0; r < 4; ++r) mine[(jj * 4 + r) * 64 + lane] = acc[ct][4 * p + jj][r];
                if (p == 0 && lg == 0) {
                    mlbuf[w][li][0] = m_ref[ct];
                    mlbuf[w][li][1] = lw;
                }
                block_lds_barrier();
                if (p == 0) {
                    float mw[4];
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
                }
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    float x = 0.f;
#pragma unroll
                    for (int v = 0; v < 4; ++v) x += mbuf[v * 1024 + (jj * 4 + w) * 64 + lane] * cw[v];
                    merged[ct][p][jj] = x;
                }
            }
            mxs[ct] = mx;
            lts[ct] = lt;
        }
        // write: a column whose (entry, KV head) has no other piece is
        // normalized into out; the others go to slot i + sigma for the
        // combine launch (stores are not waited for: the combine is a later
        // launch)
        const int s = unit_seg(sig), h = sig - s * H;
        const int ncol = ncol_of(s);
        const int m = 4 * lg + w;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const int c = 16 * ct + li;
            if (c >= ncol) continue;
            const Col cl = col_of(s, c);
            if (exp_s[cl.b * H + h] == 1) {
                const float inv = lts[ct] > 0.f ? 1.f / lts[ct] : 0.f;
                float* o = a.out + (size_t(ent_s[cl.b][E_CU] + cl.tok) * a.Hq + size_t(h) * GQ + cl.j) * D;
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                    const f32x4_t v = merged[ct][p] * inv;
                    *reinterpret_cast<float4*>(o + NDT * m + 4 * p) = make_float4(v[0], v[1], v[2], v[3]);
                }
            } else {
                const size_t it = size_t(i_blk + sig) * NCOL + c;
                float* o = a.part_acc + it * D;
#pragma unroll
                for (int p = 0; p < NP; ++p)
                    *reinterpret_cast<float4*>(o + NDT * m + 4 * p) =
                        make_float4(merged[ct][p][0], merged[ct][p][1], merged[ct][p][2], merged[ct][p][3]);
                if (w == 0 && lg == 0) *reinterpret_cast<float2*>(a.part_ml + it * 2) = make_float2(mxs[ct], lts[ct]);
            }
        }
        reset();
    };

    reset();
    int unit_k = 0;
    start_unit(unit_k, sig);
    const int tb = 16 * w + 4 * lg;                 // key of accumulator register r: tb + r

    // one page of this wave's keys: K operand chunks kb, V rows vb
    auto compute = [&](const u32x4 (&kb)[NC], const vrow_t (&vb)[4], int meta) __attribute__((always_inline)) {
        const int lim = meta & 255;                 // rows any column of the unit may see
        if (lim <= 16 * w) return;                  // none of them among this wave's keys
        const int tok0 = ((meta >> 9) & 0x7fff) * kPage;   // first key of the page
        f32x4_t s[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) s[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        // the score products at raised wave priority (config 2: kernel 0.2%,
        // step 0.25% faster in three A/B pairs on one box; the same in the
        // quantized streams, around their dequantizing score loop, was slower)
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const bf16x8_t kk = __builtin_bit_cast(bf16x8_t, kb[c]);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) s[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk, qb[ct][c], s[ct], 0, 0, 0);
        }
        __builtin_amdgcn_s_setprio(0);
        const bool masked = tok0 + kPage > kmin;   // a real column's limit falls inside the page
        bf16x8_t bop[NCT];
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
                // a column with no visible key in this wave yet has no reference
                p[r] = m_ref[ct] == -INFINITY ? 0.f : p[r];
            }
            l_part[ct] += (p[0] + p[1]) + (p[2] + p[3]);
            uint32_t h01, l01, h23, l23;
            split_bf16(p[0], p[1], h01, l01);
            split_bf16(p[2], p[3], h23, l23);
            bop[ct] = __builtin_bit_cast(bf16x8_t, u32x4{h01, h23, l01, l23});
        }
        // V^T tiles: dims 2e and 2e + 1 of the lane's run from word e of the
        // four keys, two keys per 32-bit pair
#pragma unroll
        for (int e = 0; e < VW; ++e) {
            const uint32_t lo01 = __builtin_amdgcn_perm(vb[1][e], vb[0][e], 0x05040100u);
            const uint32_t lo23 = __builtin_amdgcn_perm(vb[3][e], vb[2][e], 0x05040100u);
            const uint32_t hi01 = __builtin_amdgcn_perm(vb[1][e], vb[0][e], 0x07060302u);
            const uint32_t hi23 = __builtin_amdgcn_perm(vb[3][e], vb[2][e], 0x07060302u);
            const bf16x8_t alo = __builtin_bit_cast(bf16x8_t, u32x4{lo01, lo23, lo01, lo23});
            const bf16x8_t ahi = __builtin_bit_cast(bf16x8_t, u32x4{hi01, hi23, hi01, hi23});
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                acc[ct][2 * e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bop[ct], acc[ct][2 * e], 0, 0, 0);
                acc[ct][2 * e + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bop[ct], acc[ct][2 * e + 1], 0, 0, 0);
            }
        }
    };

    typedef const u32x4 __attribute__((address_space(3)))* lds_u32x4_cptr;
    typedef const u32x4 __attribute__((address_space(1)))* glb_u32x4_cptr;
    typedef const vrow_t __attribute__((address_space(3)))* lds_vrow_cptr;
    typedef const vrow_t __attribute__((address_space(1)))* glb_vrow_cptr;
    const lds_u32x4_cptr pst = (lds_u32x4_cptr)(&pstage[0]);

    // page i from buffer set J (compile time, so the buffers stay registers)
    auto step = [&](auto jc, int i) __attribute__((always_inline)) {
        constexpr int J = decltype(jc)::value;
        constexpr int FB = (J + PF - 1) % PF;
        const int meta = pmeta[J];
        load_page(i + PF - 1, kbuf[FB], vbuf[FB], pmeta[FB]);
        if (append && (meta & kPatchBit)) {
            // an entry's new token lies in this page: its row replaces the
            // loaded one in the wave that owns the key (from the staged copy;
            // past the staged ones from memory, and then that wave also
            // writes it into the page)
            const int s = unit_seg(sig), h = sig - s * H, pg_idx = (meta >> 9) & 0x7fff;
            const int mask = seg_s[s][S_MASK];
#pragma unroll 1
            for (int b = 0; b < kMaxEnt; ++b) {
                const int keys = ent_s[b][E_KEYS];
                if (!((mask >> b) & 1) || keys <= 0 || ((keys - 1) >> kPageShift) != pg_idx) continue;
                const int r = (keys - 1) & 63;
                if ((r >> 4) != w) continue;
                int q = -1;
                for (int k = 0; k < npatch; ++k) {
                    const int pe = patch_s[k];
                    if ((pe & 0xfff) == i && ((pe >> 12) & 7) == b) q = k;
                }
                const int vx = (D / 8) * li;       // byte offset of the lane's dims within the row
                u32x4 kr[NC];
                vrow_t vr;
                if (q >= 0) {
#pragma unroll
                    for (int c = 0; c < NC; ++c) kr[c] = pst[q * PCH + 4 * c + lg];
                    vr = *(lds_vrow_cptr)((const char __attribute__((address_space(3)))*)(pst + q * PCH + NCH) + vx);
                } else {
                    const glb_u32x4_cptr kn = (glb_u32x4_cptr)(a.k_new + (size_t(b) * H + h) * D);
                    const glb_u32x4_cptr vn = (glb_u32x4_cptr)(a.v_new + (size_t(b) * H + h) * D);
#pragma unroll
                    for (int c = 0; c < NC; ++c) kr[c] = kn[4 * c + lg];
                    vr = *(glb_vrow_cptr)((const char __attribute__((address_space(1)))*)vn + vx);
                    const int sl = pinfo[i].x;
                    if (sl >= 0 && lane < PCH) {
                        const int pl = lane / NCH, x = lane % NCH;
                        const u32x4 v = pl ? vn[x] : kn[x];
                        *reinterpret_cast<u32x4*>((pl ? vplane_w : kplane_w) + size_t(sl) * SLICE + r * NCH * 16 + x * 16) = v;
                    }
                }
                const bool kl = li == (r & 15), vl = lg == ((r & 15) >> 2);
#pragma unroll
                for (int c = 0; c < NC; ++c) kbuf[J][c] = kl ? kr[c] : kbuf[J][c];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) vbuf[J][rr] = (vl && rr == (r & 3)) ? vr : vbuf[J][rr];
            }
        }
        compute(kbuf[J], vbuf[J], meta);

        if (meta & 256) {
            finish_unit();
            if (i + 1 < npg) {
                ++sig;
                ++unit_k;
                start_unit(unit_k, sig);
            }
        }
    };

    for (int i0 = 0; i0 < npg; i0 += PF) ring_round<0, PF>(step, i0, npg);
    if (npatch > 0) store_rows();
}


// Combine the chunks of each (entry, query head) in chunk order.
template <int D, int GQ>
__global__ void __launch_bounds__(64) decode_combine_kernel(DecodeArgs a) {
    constexpr int EPL = D / 64;
    const int lane = int(threadIdx.x);
    const int b = int(blockIdx.x) / a.Hq, j = int(blockIdx.x) % a.Hq;
    const int h = j / GQ, jj = j % GQ;
    const int ctx = plan_ent(a, b, plan::E_KEYS);
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

// Pages per split of the chunked split kernel (the shapes the page stream
// does not take); the split depends only on logical positions.
constexpr int kChunkPages = 8;
int chunk_pages() { return kChunkPages; }

// Blocks of the page stream: bpc per compute unit (two for the BF16 stream,
// whose pages go straight into registers; the quantized stream runs one or
// two by its register needs), every one streaming the same share of pages;
// more when a share would exceed the kStreamPages / bpc pages a block lists.
int stream_grid(const PoolView& pv, int B, int max_seq_len, int bpc = 1) {
    static const int cus = [] {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        return n;
    }();
    const int per_block = kStreamPages / bpc;
    const long long need = (stream_bound(pv, B, max_seq_len) + per_block - 1) / per_block;
    return int(need > cus * bpc ? need : cus * bpc);
}

// blocks per compute unit of the page stream for these pages
int stream_bpc(const PoolView& pv) {
    return pv.k_codec != CODEC_BF16 ? qstream_blocks_per_cu(pv) : vstream_bpc(pv.D);
}

// The matrix-core page stream covers BF16 pages with D in {64, 128}, up to
// eight entries per call, 64 KV heads and 32768 logical pages per row (the
// page index shares a word with the page's flags), and at most 4096 blocks;
// everything else takes the chunked split kernel.
bool stream_path(const PoolView& pv, int B, int gq) {
    return pv.k_codec == CODEC_BF16 && pv.v_codec == CODEC_BF16 && (pv.D == 64 || pv.D == 128 || pv.D == 256) &&
           B <= 8 && pv.H <= plan::kMaxH && pv.L <= 32768 &&
           (long long)B * pv.H * pv.L <= 4096LL * (kStreamPages / vstream_bpc(pv.D)) &&
           (gq == 1 || gq == 2 || gq == 4 || gq == 8);
}

// chunk mode (several query tokens per entry) on the BF16 stream: D in {64, 128}
bool chunk_path(const PoolView& pv, int B, int gq) { return stream_path(pv, B, gq) && pv.D <= 128; }

int max_chunks_for(int max_seq_len) {
    const int pages = (max_seq_len + kPage - 1) / kPage;
    return (pages + chunk_pages() - 1) / chunk_pages();
}

// Workspace: [plan][partial (m, l) pairs][partial accumulators], each from a
// 256-byte boundary.  Every call writes what it reads: no initialization.
struct WsLayout {
    bool stream;
    int G, qcap;        // page stream: blocks, page slots per block
    int share;          // per mille of the stream the first half of the blocks takes
    size_t plan, ml, acc, total;
    size_t cols;        // partial slot width
};

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Share (per mille) of the stream positions blocks [0, G/2) take.  The
// streams run two blocks on every compute unit (one at D = 256 for BF16 and
// INT8-G64), and the block dispatched first (blocks [0, G/2) of the grid: one
// per compute unit before the second) gets the SIMDs' issue slots first.
// With an even split it streamed about 30% faster (per-block timestamps of
// the BF16 stream: 40 against 52 us), and the second block then ran alone
// with half the loads in flight for the last part of the launch.  57%
// measured best for the quantized streams (INT8-G64 and K8V4 kernels 2.9%
// faster; 60% and more slower), 53% for the BF16 stream (config 2 step
// 0.8-1.0% faster in two sweeps of 52-56% on two boxes; 56% no different).
// The split fixes which block reads which pages, so results stay independent
// of timing.
int stream_share(const PoolView& pv) {
    if (stream_bpc(pv) != 2) return 500;
    return pv.k_codec != CODEC_BF16 ? 570 : 530;
}

// page slots a block needs under that split for at most `bound` positions
int split_qcap(long long bound, int G, int share) {
    if (bound <= 0 || G <= 0) return 1;
    const long long na = (share != 500 && G >= 2) ? G / 2 : 0;
    const long long qa = na > 0 ? (bound * share + 1000LL * na - 1) / (1000LL * na) : 0;
    const long long qb = (bound * (1000 - (na > 0 ? share : 0)) + 1000LL * (G - na) - 1) / (1000LL * (G - na));
    return int(qa > qb ? qa : qb);
}

WsLayout ws_layout(const PoolView& pv, int B, int gq, int max_seq_len, bool chunk) {
    WsLayout l{};
    l.stream = chunk || stream_path(pv, B, gq) || qstream_path(pv, B, gq);
    size_t slots;
    if (l.stream) {
        l.G = stream_grid(pv, B, max_seq_len, stream_bpc(pv));
        const long long bound = stream_bound(pv, B, max_seq_len);
        l.share = chunk ? 500 : stream_share(pv);
        l.qcap = split_qcap(bound, l.G, l.share);
        if (l.qcap > kStreamPages / stream_bpc(pv)) {   // the first half's lists would not fit: an even split
            l.share = 500;
            l.qcap = split_qcap(bound, l.G, l.share);
        }
        slots = size_t(l.G) + size_t(plan::kMaxSeg) * pv.H;     // (block, unit) pieces
        l.cols = chunk ? 32 : 16;
    } else {
        slots = size_t(B) * pv.H * max_chunks_for(max_seq_len);  // one per split
        l.cols = size_t(gq);
    }
    l.plan = 0;
    l.ml = l.plan + plan::plan_bytes(pv.H, l.G, l.qcap);
    l.acc = l.ml + align256(slots * l.cols * 2 * sizeof(float));
    l.total = l.acc + slots * l.cols * size_t(pv.D) * sizeof(float);
    return l;
}

DecodeArgs run_args(const PoolView& pv, const WsLayout& l, int B, int Hq, int max_seq_len, const void* q,
                    float sm_scale, float* out, void* ws, const void* k_new = nullptr, const void* v_new = nullptr) {
    DecodeArgs a{};
    char* base = static_cast<char*>(ws);
    a.pv = pv;
    a.plan = reinterpret_cast<const int32_t*>(base + l.plan);
    a.qcap = l.qcap;
    a.G = l.G;
    a.q = static_cast<const uint16_t*>(q);
    a.k_new = static_cast<const uint16_t*>(k_new);
    a.v_new = static_cast<const uint16_t*>(v_new);
    a.out = out;
    a.B = B;
    a.Hq = Hq;
    a.chunk_pages = chunk_pages();
    a.max_chunks = max_chunks_for(max_seq_len);
    a.max_ctx = max_seq_len;
    a.part_ml = reinterpret_cast<float*>(base + l.ml);
    a.part_acc = reinterpret_cast<float*>(base + l.acc);
    a.scale_log2 = sm_scale * kLog2e;
    return a;
}

template <int D, int GQ>
hipError_t launch_gq(const DecodeArgs& a, bool stream, hipStream_t s) {
    if (stream && a.pv.k_codec != CODEC_BF16) return launch_qstream(a, GQ, s);
    {
        if (stream) {
            const hipError_t e =
                launch_kernel(true, paged_vstream_kernel<D, GQ, 1, false>, dim3(unsigned(a.G)), dim3(256), s, a);
            if (e != hipSuccess) return e;
            DecodeArgs c = a;
            c.cgroups = combine_groups(GQ, D);
            stream_combine_kernel<D, GQ, 16><<<dim3(unsigned(a.B * a.pv.H * c.cgroups)), 64, 0, s>>>(c);
            return hipGetLastError();
        }
    }
    const int items = a.B * a.pv.H * a.max_chunks;
    const dim3 grid(unsigned((items + 3) / 4));
    const int kc = a.pv.k_codec, vc = a.pv.v_codec;
    bool launched = false;
    const bool s16 = a.pv.scale16 != 0;
#define KVS_DEC_CASE(K, V, SB)                                                                       \
    if (!launched && kc == K && vc == V && s16 == (SB == 2)) {                                      \
        if (items > 0) (void)launch_kernel(true, decode_split_kernel<D, GQ, K, V, SB>, grid, dim3(256), s, a); \
        launched = true;                                                                             \
    }
    KVS_DEC_CASE(CODEC_BF16, CODEC_BF16, 4)
    KVS_DEC_CASE(CODEC_INT8_G64, CODEC_INT8_G64, 4)
    KVS_DEC_CASE(CODEC_FP8_ROW, CODEC_FP8_ROW, 4)
    KVS_DEC_CASE(CODEC_NVFP4_G16, CODEC_NVFP4_G16, 4)
    KVS_DEC_CASE(CODEC_FP8_ROW, CODEC_NVFP4_G16, 4)
    KVS_DEC_CASE(CODEC_INT8_G64, CODEC_INT8_G64, 2)
    KVS_DEC_CASE(CODEC_FP8_ROW, CODEC_FP8_ROW, 2)
    KVS_DEC_CASE(CODEC_FP8_ROW, CODEC_NVFP4_G16, 2)
#undef KVS_DEC_CASE
    if (!launched) return hipErrorNotSupported;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    decode_combine_kernel<D, GQ><<<dim3(unsigned(a.B * a.Hq)), 64, 0, s>>>(a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, int gq, bool stream, hipStream_t s) {
    switch (gq) {
        case 1: return launch_gq<D, 1>(a, stream, s);
        case 2: return launch_gq<D, 2>(a, stream, s);
        case 4: return launch_gq<D, 4>(a, stream, s);
        case 8: return launch_gq<D, 8>(a, stream, s);
    }
    return hipErrorNotSupported;
}

template <int D>
hipError_t launch_chunk_d(const DecodeArgs& a, int gq, int G, bool trace, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(G));
    DecodeArgs c = a;
    c.cgroups = combine_groups(32, D);
    const dim3 cgrid(static_cast<unsigned>(a.B * a.pv.H * c.cgroups));
    switch (gq) {
#define KVS_CHUNK_CASE(GQ)                                                  \
    case GQ:                                                                \
        (void)launch_kernel(trace, paged_vstream_kernel<D, GQ, 2, true>, grid, dim3(256), s, a); \
        if (hipPeekAtLastError() == hipSuccess)                             \
            stream_combine_kernel<D, GQ, 32><<<cgrid, 64, 0, s>>>(c);       \
        break;
        KVS_CHUNK_CASE(1)
        KVS_CHUNK_CASE(2)
        KVS_CHUNK_CASE(4)
        KVS_CHUNK_CASE(8)
#undef KVS_CHUNK_CASE
        default: return hipErrorNotSupported;
    }
    return hipGetLastError();
}

}  // namespace

long long stream_bound(const PoolView& pv, int B, int max_seq_len) {
    return (long long)B * pv.H * ((max_seq_len + kPage - 1) / kPage);
}

bool decode_supported(const PoolView& pv, int Hq) {
    if (pv.H <= 0 || Hq % pv.H) return false;
    const int gq = Hq / pv.H;
    return (pv.D == 64 || pv.D == 128 || pv.D == 256) && (gq == 1 || gq == 2 || gq == 4 || gq == 8);
}

size_t decode_workspace_bytes(const PoolView& pv, int B, int Hq, int max_seq_len) {
    const int gq = pv.H ? Hq / pv.H : 0;
    return ws_layout(pv, B, gq, max_seq_len, false).total;
}

hipError_t launch_decode_plan(const PoolView& pv, int B, int Hq, const int32_t* table_rows, const int32_t* seq_lens,
                              int max_seq_len, void* ws, hipStream_t s) {
    const int gq = Hq / pv.H;
    const WsLayout l = ws_layout(pv, B, gq, max_seq_len, false);
    int32_t* planp = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + l.plan);
    return launch_stream_plan(pv, B, gq, table_rows, seq_lens, nullptr, nullptr, max_seq_len, 0, false, l.stream,
                              l.stream, l.G, l.qcap, l.share, planp, s);
}

bool decode_append_supported(const PoolView& pv, int B, int Hq) {
    return pv.H > 0 && Hq % pv.H == 0 && (stream_path(pv, B, Hq / pv.H) || qstream_path(pv, B, Hq / pv.H));
}

hipError_t launch_decode_run(const PoolView& pv, int B, int Hq, int max_seq_len, const void* q, float sm_scale,
                             float* out, void* ws, hipStream_t s, const void* k_new, const void* v_new) {
    const int gq = Hq / pv.H;
    const WsLayout l = ws_layout(pv, B, gq, max_seq_len, false);
    if (k_new && !l.stream) return hipErrorNotSupported;
    const DecodeArgs a = run_args(pv, l, B, Hq, max_seq_len, q, sm_scale, out, ws, k_new, v_new);
    switch (pv.D) {
        case 64: return launch_d<64>(a, gq, l.stream, s);
        case 128: return launch_d<128>(a, gq, l.stream, s);
        case 256: return launch_d<256>(a, gq, l.stream, s);
    }
    return hipErrorNotSupported;
}

hipError_t launch_decode(const PoolView& pv, int B, int Hq, const int32_t* table_rows, const int32_t* seq_lens,
                         int max_seq_len, const void* q, float sm_scale, float* out, void* ws, hipStream_t s) {
    hipError_t e = launch_decode_plan(pv, B, Hq, table_rows, seq_lens, max_seq_len, ws, s);
    if (e != hipSuccess) return e;
    return launch_decode_run(pv, B, Hq, max_seq_len, q, sm_scale, out, ws, s);
}

bool stream_chunk_supported(const PoolView& pv, int B, int gq) { return chunk_path(pv, B, gq); }

size_t stream_chunk_workspace_bytes(const PoolView& pv, int B, int Hq, int max_seq_len) {
    return ws_layout(pv, B, Hq / pv.H, max_seq_len, true).total;
}

hipError_t launch_stream_chunk(const PoolView& pv, int B, int Hq, const int32_t* table_rows, const int32_t* q_pos0,
                               const int32_t* cu_q, int max_seq_len, const void* q, float sm_scale, float* out,
                               void* ws, int max_cols, bool trace, hipStream_t s) {
    const int gq = Hq / pv.H;
    const WsLayout l = ws_layout(pv, B, gq, max_seq_len, true);
    int32_t* planp = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + l.plan);
    hipError_t e = launch_stream_plan(pv, B, gq, table_rows, nullptr, q_pos0, cu_q, max_seq_len, max_cols, true,
                                      false, true, l.G, l.qcap, l.share, planp, s);
    if (e != hipSuccess) return e;
    const DecodeArgs a = run_args(pv, l, B, Hq, max_seq_len, q, sm_scale, out, ws);
    switch (pv.D) {
        case 64: return launch_chunk_d<64>(a, gq, l.G, trace, s);
        case 128: return launch_chunk_d<128>(a, gq, l.G, trace, s);
    }
    return hipErrorNotSupported;
}

}  // namespace kvs
