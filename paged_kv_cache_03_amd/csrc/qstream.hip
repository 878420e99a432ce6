// qstream.hip -- the matrix-core page stream for quantized pages.
//
// NInfer "Paged KV Context Store" page: the closed KV profiles (code and
// scale planes per side: INT8-G64, FP8-E4M3FN-row256, NVFP4-G16, and K8V4 =
// FP8 K with NVFP4 V), P=64 translation, consumer rules (page-granular reads
// through the block table, no gather-to-contiguous, free choice of
// tile/split/wave/LDS scheme).
//
// It runs the same plan (stream_plan.hip), work split, online softmax, unit
// merge and combine as the BF16 page stream of decode.hip; what differs is
// how a page reaches the matrix cores.  A ring stage holds one page's raw
// planes -- K codes, V codes, K scales, V scales -- brought in by
// direct-to-LDS loads, and the codes become bf16 operands in registers:
//  * every code value is exact in bf16 (int8 in [-127, 127]; e4m3 has 4
//    significant bits; e2m1 2), and so is an e2m1 value times its e4m3 group
//    scale (at most 6 significant bits, inside bf16's exponent range), so
//    NVFP4 pages are dequantized in full before the products;
//  * INT8-G64 and FP8-row scales are fp32 and do not fold into a bf16
//    operand exactly, so they act on fp32 values: K scales multiply each
//    key's per-group partial scores, V scales multiply the key's probability
//    (p * s, split into two bf16 terms like p itself), one copy of P per
//    64-dim scale group;
//  * PV runs V^T . [P_hi; P_lo] as one k=32 product per 16-dim tile: the
//    lane's four keys appear twice in the V^T operand, once against P_hi,
//    once against P_lo;
//  * a V^T operand comes from four row reads per lane (the four keys whose
//    probabilities the lane holds); packing the fp32 values of two keys into
//    one bf16 pair is the transpose.  Row m of tile j then holds head dim
//    64(j/4) + 4m + j%4 for INT8-G64 V (a tile stays in one scale group) and
//    (D/16) m + j for the others.
// Keys of a wave's 16-row band enter the score tile in the order
// 4(m%4) + m/4 (row m), so that the four keys a V read touches at once are
// consecutive rows, which the stage layout puts in different LDS banks.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "attn_common.h"
#include "decode_common.h"
#include "internal.h"
#include "stream_common.h"
#include "stream_plan.h"

namespace kvs {

namespace {

// bytes per page row (one key of one KV head) of a side's code and scale planes
template <int C, int D>
struct QRow {
    static constexpr int code = C == CODEC_NVFP4_G16 ? D / 2 : D;
    static constexpr int scale = C == CODEC_INT8_G64 ? 4 * (D / 64) : (C == CODEC_FP8_ROW ? 4 : D / 16);
};

// Blocks per compute unit: two for D <= 128 (two waves per SIMD hide each
// other's LDS and matrix-core latencies; each block gets half of the LDS and
// at most 256 registers per lane), one for D = 256 (its registers do not fit
// twice).
template <int D>
constexpr int qstream_bpc() { return D <= 128 ? 2 : 1; }

// LDS ring of the quantized stream: stage = [K codes | V codes | K scales |
// V scales], at least 16 KiB (the unit merge passes through one stage)
template <int KC, int VC, int D, int BPC>
struct QRing {
    static constexpr int KCB = 64 * QRow<KC, D>::code;
    static constexpr int VCB = 64 * QRow<VC, D>::code;
    static constexpr int KSB = 64 * QRow<KC, D>::scale;
    static constexpr int VSB = 64 * QRow<VC, D>::scale;
    static constexpr int OFF_V = KCB, OFF_KS = KCB + VCB, OFF_VS = OFF_KS + KSB;
    static constexpr int DATA = OFF_VS + VSB;
    static constexpr int MERGE = 4 * 16 * 64 * 4;          // four waves x four tiles of accumulators
    static constexpr int STRIDE = DATA > MERGE ? DATA : MERGE;
    static constexpr int KL = KCB / 4096, VL = VCB / 4096; // 16-byte loads per thread and page
    static constexpr int SCW = (KSB + VSB) / 64;           // scale chunks per wave and page
    static constexpr int LPP = KL + VL + 1;                // loads per wave and page
    static constexpr int LDS = 163840 / BPC;                // the block's share of the compute unit's LDS
    static constexpr int FIXED = (8192 + 16384) / BPC + 4096;   // page list, query cache, tables (upper bound)
    static constexpr int NS_LDS = (LDS - FIXED) / STRIDE;
    static constexpr int NS = NS_LDS > 8 ? 8 : NS_LDS;     // ring stages
};

typedef const uint8_t __attribute__((address_space(3)))* lds_cu8;
typedef const uint32_t __attribute__((address_space(3)))* lds_cu32;
typedef const u32x2 __attribute__((address_space(3)))* lds_cu32x2;
typedef const u32x4 __attribute__((address_space(3)))* lds_cu32x4;
typedef const float __attribute__((address_space(3)))* lds_cf32;

__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2v_t));
}

// signed byte k of w as fp32 (one sub-dword convert)
template <int K>
__device__ __forceinline__ float i8f(uint32_t w) {
    return float(int8_t((w >> (8 * K)) & 0xFFu));
}

// E4M3FN byte (bits 7:0 of w) as fp32
__device__ __forceinline__ float e4m3_f32(uint32_t w) { return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false)[0]; }

// the two e2m1 values of byte b of w / the two e4m3 values of half h of w,
// as fp32 (b and h are constants once the callers' loops are unrolled)
__device__ __forceinline__ f32x2_t fp4_pair(uint32_t w, int b) {
    switch (b & 3) {
        case 0: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
        case 1: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
        case 2: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
        default: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    }
}
__device__ __forceinline__ f32x2_t fp8_pair(uint32_t w, int h) {
    return h ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, true) : __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
}

template <int D, int KC, int VC>
__global__ void __launch_bounds__(256, qstream_bpc<D>()) paged_qstream_kernel(DecodeArgs a) {
    using namespace plan;
    constexpr int BPC = qstream_bpc<D>();
    using R = QRing<KC, VC, D, BPC>;
    constexpr int NT = 256;
    constexpr int NS = R::NS;
    constexpr int STRIDE = R::STRIDE;
    constexpr int LPP = R::LPP;
    constexpr int NCH = D / 8;                     // 16-byte chunks of a bf16 query row
    constexpr int NU = D / 64;                     // 64-dim groups: K reads of 16 dims per lane
    constexpr int NDT = D / 16;                    // PV tiles
    constexpr int NP = NDT / 4;                    // merge passes, four tiles each
    constexpr int NCOL = 16;
    constexpr int QCHUNKS = 1024 / BPC;            // query cache: 16 KiB / BPC of 16-byte chunks
    constexpr int PAGES = kStreamPages / BPC;      // most pages a block takes
    constexpr int QSEG = QCHUNKS / (NCOL * NCH);   // units with cached queries
    constexpr int KROW = QRow<KC, D>::code, VROW = QRow<VC, D>::code;
    constexpr int KSROW = QRow<KC, D>::scale, VSROW = QRow<VC, D>::scale;
    constexpr int KCHR = KROW / 16;                // 16-byte chunks per K code row
    constexpr bool KI8 = KC == CODEC_INT8_G64, KF8 = KC == CODEC_FP8_ROW;
    constexpr bool VI8 = VC == CODEC_INT8_G64, VF8 = VC == CODEC_FP8_ROW;
    constexpr int NGK = KI8 ? NU : 1;              // score accumulators: one per K scale group
    constexpr int NPV = VI8 ? NU : 1;              // copies of P: one per V scale group
    static_assert(KC != CODEC_BF16 && VC != CODEC_BF16, "quantized sides only");
    static_assert((D == 64 || D == 128 || D == 256) && R::KL >= 1 && R::VL >= 1, "shape");
    static_assert(R::SCW >= 1 && R::SCW <= 64 && NS >= 3, "ring shape");
    static_assert(LPP * (NS - 2) + QCHUNKS / NT < 64, "vmcnt range");
    static_assert(QSEG >= 1 && QSEG * NCOL * NCH == QCHUNKS, "query cache shape");

    __shared__ u32x4 ring[NS * STRIDE / 16];
    __shared__ int2 pinfo[PAGES];                  // the block's pages: (slice g*H + h or -1, meta)
    __shared__ u32x4 qcache[QCHUNKS];              // query rows of the first QSEG units: [unit][column][chunk]
    __shared__ float mlbuf[4][16][2];              // per-wave (m, l) of every column at a unit's end
    __shared__ int ent_s[kMaxEnt][kEntWords];
    __shared__ int seg_s[kMaxSeg][kSegWords];
    __shared__ int exp_s[kMaxEnt * kMaxH];         // pieces per (entry, KV head)
    static_assert(NS * STRIDE + sizeof(pinfo) + sizeof(qcache) + sizeof(mlbuf) + sizeof(ent_s) + sizeof(seg_s) +
                          sizeof(exp_s) <= R::LDS, "LDS");

    const int tid = int(threadIdx.x);
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, li = lane & 15, lg = lane >> 4;
    const int H = a.pv.H, i_blk = int(blockIdx.x), G = int(gridDim.x);
    const int GQ = a.Hq / H;
    const int gq_sh = __builtin_ctz(unsigned(GQ));
    const int32_t* P = a.plan;

    // one round trip: the plan's header and tables, this block's page list
    const int magic = ld_uniform(P, H_MAGIC), pb = ld_uniform(P, H_B), ph = ld_uniform(P, H_H);
    const int pgq = ld_uniform(P, H_GQ), pg = ld_uniform(P, H_G), pq = ld_uniform(P, H_QCAP);
    const int pchunk = ld_uniform(P, H_CHUNK);
    const bool plan_ok = (magic == kMagic) & (pb == a.B) & (ph == H) & (pgq == GQ) & (pg == G) & (pq == a.qcap) &
                         (pchunk == 0);
    const int nseg = ld_uniform(P, H_NSEG), zero = ld_uniform(P, H_ZERO);
    const int npg = ld_uniform(P, off_blk(H) + 4 * size_t(i_blk));
    int sig = ld_uniform(P, off_blk(H) + 4 * size_t(i_blk) + 1);   // unit being computed
    {
        static_assert(kMaxEnt * kEntWords <= NT && kMaxSeg * kSegWords <= NT, "tables");
        static_assert(kMaxEnt * kMaxH <= 2 * NT && PAGES % NT == 0, "tables");
        const int2* pl = reinterpret_cast<const int2*>(P + off_pages(H, G)) + size_t(i_blk) * a.qcap;
        const int ne = kMaxEnt * H;
        const int v_ent = P[kOffEnt + min(tid, kMaxEnt * kEntWords - 1)];
        const int v_seg = P[kOffSeg + min(tid, kMaxSeg * kSegWords - 1)];
        const int v_exp0 = P[kOffExp + min(tid, ne - 1)];
        const int v_exp1 = P[kOffExp + min(tid + NT, ne - 1)];
        int2 v_pg[PAGES / NT];
#pragma unroll
        for (int k = 0; k < PAGES / NT; ++k) v_pg[k] = pl[min(tid + k * NT, a.qcap - 1)];
        if (tid < kMaxEnt * kEntWords) ent_s[tid / kEntWords][tid % kEntWords] = v_ent;
        if (tid < kMaxSeg * kSegWords) seg_s[tid / kSegWords][tid % kSegWords] = v_seg;
        if (tid < ne) exp_s[tid] = v_exp0;
        if (tid + NT < ne) exp_s[tid + NT] = v_exp1;
#pragma unroll
        for (int k = 0; k < PAGES / NT; ++k)
            if (tid + k * NT < a.qcap) pinfo[tid + k * NT] = v_pg[k];
    }
    block_lds_barrier();
    if (!plan_ok) {                                // a plan of another batch shape: make it visible
        if (i_blk == 0)
            for (int x = tid; x < a.B * a.Hq * D; x += NT) a.out[x] = __builtin_nanf("");
        return;
    }
    if (i_blk == 0) {                              // entries with nothing to attend produce zeros
        for (int b = 0; b < a.B; ++b) {
            if (!((zero >> b) & 1)) continue;
            const size_t r0 = size_t(ent_s[b][E_CU]) * a.Hq * D;
            for (int x = tid; x < a.Hq * D; x += NT) a.out[r0 + x] = 0.f;
        }
    }
    if (npg <= 0) return;

    // column c of a unit of segment s: entry, head within the group
    struct Col {
        int b, j;
    };
    auto col_of = [&](int s, int c) __attribute__((always_inline)) {
        int m = seg_s[s][S_MASK];
        for (int k = c >> gq_sh; k > 0; --k) m &= m - 1;
        return Col{__builtin_ctz(unsigned(m | 0x100)), c & (GQ - 1)};
    };
    auto ncol_of = [&](int s) __attribute__((always_inline)) {
        return __builtin_popcount(unsigned(seg_s[s][S_MASK])) * seg_s[s][S_W];
    };
    auto q_row = [&](const Col& cl, int h) __attribute__((always_inline)) {
        return a.q + (size_t(ent_s[cl.b][E_CU]) * a.Hq + size_t(h) * GQ + cl.j) * D;
    };
    auto unit_seg = [&](int sg) __attribute__((always_inline)) { return sg / H; };

    // query rows of the first QSEG units, straight into LDS (columns past a
    // unit's last read row 0 of the call; they are never used)
    const uint32_t qcache_lds = uint32_t(reinterpret_cast<uintptr_t>((lds_byte_ptr)(&qcache[0])));
#pragma unroll
    for (int k = 0; k < QCHUNKS / NT; ++k) {
        const int x = k * NT + tid;
        const int u = x / (NCOL * NCH), c = (x / NCH) % NCOL, ch = x % NCH;
        const int sg = sig + u, s = unit_seg(sg);
        const u32x4* src = reinterpret_cast<const u32x4*>(a.q);
        if (s < nseg && c < ncol_of(s)) src = reinterpret_cast<const u32x4*>(q_row(col_of(s, c), sg - s * H)) + ch;
        fetch_chunk(qcache_lds + uint32_t((k * NT + w * 64) * 16), src);
    }

    // Stage layout: K code row t keeps its 16-byte chunk x at position
    // x ^ kswz(t), so the 16 rows one K read touches spread over the banks;
    // INT8 V rows move their 64-byte quarters by vswz(t) for the same reason.
    auto kswz = [](int t) __attribute__((always_inline)) {
        return (KROW >= 256 ? t : t / (256 / KROW)) & (KCHR - 1);
    };
    auto vswz = [](int t) __attribute__((always_inline)) {
        if constexpr (VI8 && D == 128) return 4 * ((t >> 1) & 1);
        else if constexpr (VI8 && D == 256) return 4 * (t & 3);
        else return 0 * t;
    };
    constexpr int VCHR = VROW / 16;
    uint32_t k_src[R::KL], v_src[R::VL];           // source byte offsets within a page slice
#pragma unroll
    for (int k = 0; k < R::KL; ++k) {
        const int s = k * NT + tid, t = s / KCHR, x = s % KCHR;
        k_src[k] = uint32_t(t * KCHR + (x ^ kswz(t))) * 16u;
    }
#pragma unroll
    for (int k = 0; k < R::VL; ++k) {
        const int s = k * NT + tid, t = s / VCHR, x = s % VCHR;
        v_src[k] = uint32_t(t * VCHR + (x ^ vswz(t))) * 16u;
    }
    // this lane's scale chunk (lanes below SCW): chunk x of [K scales | V scales]
    const int sc_x = w * R::SCW + lane;
    const bool sc_k = sc_x < R::KSB / 16;
    const uint32_t sc_off = uint32_t(sc_k ? sc_x : sc_x - R::KSB / 16) * 16u;
    const char* kplane = static_cast<const char*>(a.pv.lv.k_code);
    const char* vplane = static_cast<const char*>(a.pv.lv.v_code);
    const char* ksplane = static_cast<const char*>(a.pv.lv.k_scale);
    const char* vsplane = static_cast<const char*>(a.pv.lv.v_scale);
    const uint32_t ring_lds = uint32_t(reinterpret_cast<uintptr_t>((lds_byte_ptr)(&ring[0])));
    // page fi of the range into stage fs
    auto fetch = [&](int fi, int fs) __attribute__((always_inline)) {
        const int sl = __builtin_amdgcn_readfirstlane(pinfo[fi].x);
        const size_t slc = size_t(sl < 0 ? 0 : sl);
        const uint32_t dst = ring_lds + uint32_t(fs * STRIDE + w * 1024);
#pragma unroll
        for (int k = 0; k < R::KL; ++k) fetch_lds16(dst + k * 4096, kplane + slc * R::KCB, k_src[k]);
#pragma unroll
        for (int k = 0; k < R::VL; ++k) fetch_lds16(dst + R::OFF_V + k * 4096, vplane + slc * R::VCB, v_src[k]);
        const char* src = sc_k ? ksplane + slc * R::KSB + sc_off : vsplane + slc * R::VSB + sc_off;
        if (lane < R::SCW) fetch_chunk(ring_lds + uint32_t(fs * STRIDE + R::OFF_KS + w * R::SCW * 16), src);
    };
    // meta of page fi: the last page of the block also ends its unit here
    auto meta_of = [&](int fi) __attribute__((always_inline)) {
        return __builtin_amdgcn_readfirstlane(pinfo[fi].y) | (fi == npg - 1 ? 256 : 0);
    };

    // Per-lane LDS byte offsets within a stage, fixed for the whole stream.
    //  K operand, group g: key tq = 16w + 4(li%4) + li/4, dims 64g + 16lg .. +15
    //  accumulator register r: key tk(r) = 16w + 4r + lg (score row 4lg + r)
    const int tq = 16 * w + 4 * (li & 3) + (li >> 2);
    int koff[NU];
#pragma unroll
    for (int g = 0; g < NU; ++g) {
        if constexpr (KC == CODEC_NVFP4_G16)
            koff[g] = tq * KROW + 16 * ((2 * g + (lg >> 1)) ^ kswz(tq)) + 8 * (lg & 1);
        else
            koff[g] = tq * KROW + 16 * ((4 * g + lg) ^ kswz(tq));
    }
    int tk[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) tk[r] = 16 * w + 4 * r + lg;

    bf16x8_t qb[D / 32];                           // Q^T operand: column li, dims 64(c/2) + 16lg + 8(c%2) .. +7
    int klim = 0;                                  // keys this lane's column sees (0: padding column)
    int kmin = 0;                                  // smallest limit of a real column of the unit
    auto start_unit = [&](int k_unit, int sg) __attribute__((always_inline)) {
        const int s = unit_seg(sg), h = sg - s * H;
        const int ncol = ncol_of(s);
        kmin = seg_s[s][S_KMIN];
        const Col cl = col_of(s, li < ncol ? li : 0);
        klim = li < ncol ? ent_s[cl.b][E_KEYS] : 0;
        if (k_unit < QSEG) {
#pragma unroll
            for (int c = 0; c < D / 32; ++c) {
                const u32x4 v = qcache[(k_unit * NCOL + li) * NCH + 8 * (c >> 1) + 2 * lg + (c & 1)];
                qb[c] = __builtin_bit_cast(bf16x8_t, li < ncol ? v : u32x4{0u, 0u, 0u, 0u});
            }
        } else {
            const u32x4* qg = reinterpret_cast<const u32x4*>(q_row(cl, h));
#pragma unroll
            for (int c = 0; c < D / 32; ++c) {
                const u32x4 v = qg[8 * (c >> 1) + 2 * lg + (c & 1)];
                qb[c] = __builtin_bit_cast(bf16x8_t, li < ncol ? v : u32x4{0u, 0u, 0u, 0u});
            }
            wait_vmcnt<0>();                       // drains the ring: only past the cached units
        }
    };

    f32x4_t acc[NDT];
    float m_ref, l_part;
    auto reset = [&]() __attribute__((always_inline)) {
        m_ref = -INFINITY;
        l_part = 0.f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    };

    // unit end: merge the four waves' states through stage st, four tiles
    // per pass; wave w folds accumulator register w of the pass's tiles, so
    // each lane ends with four consecutive head dims of row 4lg + w
    auto finish_unit = [&](int st) __attribute__((always_inline)) {
        float* buf = reinterpret_cast<float*>(reinterpret_cast<char*>(&ring[0]) + st * STRIDE);
        const float lw = rows_sum(l_part);
        f32x4_t merged[NP];
        float cw[4], lt = 0.f, mx = -INFINITY;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            block_lds_barrier();                   // stage st is free, or every wave read the last pass
            float* mine = buf + w * 1024;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                for (int r = 0; r < 4; ++r) mine[(jj * 4 + r) * 64 + lane] = acc[4 * p + jj][r];
            if (p == 0 && lg == 0) {
                mlbuf[w][li][0] = m_ref;
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
                for (int v = 0; v < 4; ++v) x += buf[v * 1024 + (jj * 4 + w) * 64 + lane] * cw[v];
                merged[p][jj] = x;
            }
        }
        // write (stores are not waited for: the ring's waits cover them and
        // the combine is a later launch); a column whose (entry, KV head) has
        // no other piece is normalized into out, the others go to slot i + sigma
        const int s = unit_seg(sig), h = sig - s * H;
        if (li < ncol_of(s)) {
            const Col cl = col_of(s, li);
            const int m = 4 * lg + w;
            if (exp_s[cl.b * H + h] == 1) {
                const float inv = lt > 0.f ? 1.f / lt : 0.f;
                float* o = a.out + (size_t(ent_s[cl.b][E_CU]) * a.Hq + size_t(h) * GQ + cl.j) * D;
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                    const int d0 = VI8 ? 64 * p + 4 * m : NDT * m + 4 * p;
                    const f32x4_t v = merged[p] * inv;
                    *reinterpret_cast<float4*>(o + d0) = make_float4(v[0], v[1], v[2], v[3]);
                }
            } else {
                const size_t it = size_t(i_blk + sig) * NCOL + li;
                float* o = a.part_acc + it * D;
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                    const int d0 = VI8 ? 64 * p + 4 * m : NDT * m + 4 * p;
                    *reinterpret_cast<float4*>(o + d0) = make_float4(merged[p][0], merged[p][1], merged[p][2], merged[p][3]);
                }
                if (w == 0 && lg == 0) *reinterpret_cast<float2*>(a.part_ml + it * 2) = make_float2(mx, lt);
            }
        }
        reset();
    };

    reset();
    int meta_ring[NS];                             // meta of the pages in the ring, by stage
#pragma unroll
    for (int k = 0; k < NS - 1; ++k) {
        if (k < npg) {
            fetch(k, k);
            meta_ring[k] = meta_of(k);
        } else {
            meta_ring[k] = 0;
        }
    }
    meta_ring[NS - 1] = 0;
    // the query cache and the first page have landed (loads complete in order)
    if (npg >= NS - 1) wait_vmcnt<LPP * (NS - 2)>();
    else wait_vmcnt<0>();
    block_lds_barrier();
    int unit_k = 0;
    start_unit(unit_k, sig);

    // one page in stage J (compile time: stage offsets fold into the reads)
    auto step = [&](auto jc, int i) __attribute__((always_inline)) {
        constexpr int J = decltype(jc)::value;
        constexpr int FS = (J + NS - 1) % NS;
        if (i + NS - 1 < npg) {
            wait_vmcnt<LPP * (NS - 2)>();
            block_lds_barrier();
            fetch(i + NS - 1, FS);
            meta_ring[FS] = meta_of(i + NS - 1);
        } else {
            wait_vmcnt<0>();
            block_lds_barrier();
        }
        const int meta = meta_ring[J];
        const int lim = meta & 255;                // rows any column of the unit may see
        if (lim > 16 * w) {
            const int tok0 = ((meta >> 9) & 0x7fff) * kPage;
            const lds_byte_ptr sb = (lds_byte_ptr)(&ring[0]) + J * STRIDE;

            // every LDS read of the page first, unconditionally (all inside
            // the stage): one wait instead of one per dependent use
            constexpr int NKW = KC == CODEC_NVFP4_G16 ? 2 : 4;    // K words per group and lane
            constexpr int NVW = VI8 ? NU : (VF8 ? NDT / 4 : NDT / 8);   // V words per key and lane
            constexpr int NKS = KI8 ? NU : (KF8 ? 1 : NU);        // K scales per lane
            constexpr int NVS = VI8 ? NU : 1;                     // V scales per key
            uint32_t kx[NU][NKW];
#pragma unroll
            for (int g = 0; g < NU; ++g) {
                if constexpr (NKW == 2) {
                    const u32x2 v = *reinterpret_cast<lds_cu32x2>(sb + koff[g]);
                    kx[g][0] = v[0];
                    kx[g][1] = v[1];
                } else {
                    const u32x4 v = *reinterpret_cast<lds_cu32x4>(sb + koff[g]);
                    kx[g][0] = v[0];
                    kx[g][1] = v[1];
                    kx[g][2] = v[2];
                    kx[g][3] = v[3];
                }
            }
            float ksc[4][NKS];                     // INT8 / FP8: scales of key tk(r); NVFP4: of the lane's 16 dims
            if constexpr (KC == CODEC_NVFP4_G16) {
#pragma unroll
                for (int g = 0; g < NU; ++g)
                    ksc[0][g] = e4m3_f32(uint32_t(reinterpret_cast<lds_cu8>(sb)[R::OFF_KS + tq * KSROW + 4 * g + lg]));
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int g = 0; g < NKS; ++g)
                        ksc[r][g] = reinterpret_cast<lds_cf32>(sb + R::OFF_KS + tk[r] * KSROW)[g];
            }
            float vsc[4][NVS];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if constexpr (VC == CODEC_NVFP4_G16) {
                    vsc[r][0] = e4m3_f32(uint32_t(reinterpret_cast<lds_cu8>(sb)[R::OFF_VS + tk[r] * VSROW + (NDT * li) / 16]));
                } else {
#pragma unroll
                    for (int g = 0; g < NVS; ++g) vsc[r][g] = reinterpret_cast<lds_cf32>(sb + R::OFF_VS + tk[r] * VSROW)[g];
                }
            }
            uint32_t vx[4][NVW];                   // INT8: word g = dims 64g + 4li .. +3; else the lane's NDT dims
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = tk[r];
                if constexpr (VI8) {
#pragma unroll
                    for (int g = 0; g < NU; ++g)
                        vx[r][g] = *reinterpret_cast<lds_cu32>(sb + R::OFF_V + t * VROW +
                                                               16 * ((4 * g + (li >> 2)) ^ vswz(t)) + 4 * (li & 3));
                } else {
                    const int off = R::OFF_V + t * VROW + 4 * NVW * li;
                    if constexpr (NVW == 4) {
                        const u32x4 v = *reinterpret_cast<lds_cu32x4>(sb + off);
                        vx[r][0] = v[0];
                        vx[r][1] = v[1];
                        vx[r][2] = v[2];
                        vx[r][3] = v[3];
                    } else if constexpr (NVW == 2) {
                        const u32x2 v = *reinterpret_cast<lds_cu32x2>(sb + off);
                        vx[r][0] = v[0];
                        vx[r][1] = v[1];
                    } else {
                        vx[r][0] = *reinterpret_cast<lds_cu32>(sb + off);
                    }
                }
            }

            // QK^T: S^T[16 keys x 16 columns], per K scale group for INT8
            f32x4_t sacc[NGK];
#pragma unroll
            for (int g = 0; g < NGK; ++g) sacc[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int g = 0; g < NU; ++g) {
                u32x4 op0, op1;
                if constexpr (KC == CODEC_NVFP4_G16) {
                    const float sc = ksc[0][g];
                    uint32_t o[8];
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const f32x2_t f0 = fp4_pair(kx[g][0], b);
                        const f32x2_t f1 = fp4_pair(kx[g][1], b);
                        o[b] = pk_bf16(f0[0] * sc, f0[1] * sc);
                        o[4 + b] = pk_bf16(f1[0] * sc, f1[1] * sc);
                    }
                    op0 = u32x4{o[0], o[1], o[2], o[3]};
                    op1 = u32x4{o[4], o[5], o[6], o[7]};
                } else if constexpr (KI8) {
                    const uint32_t* x = kx[g];
                    op0 = u32x4{pk_bf16(i8f<0>(x[0]), i8f<1>(x[0])), pk_bf16(i8f<2>(x[0]), i8f<3>(x[0])),
                                pk_bf16(i8f<0>(x[1]), i8f<1>(x[1])), pk_bf16(i8f<2>(x[1]), i8f<3>(x[1]))};
                    op1 = u32x4{pk_bf16(i8f<0>(x[2]), i8f<1>(x[2])), pk_bf16(i8f<2>(x[2]), i8f<3>(x[2])),
                                pk_bf16(i8f<0>(x[3]), i8f<1>(x[3])), pk_bf16(i8f<2>(x[3]), i8f<3>(x[3]))};
                } else {
                    uint32_t o[8];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        o[2 * e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kx[g][e], 1.0f, false));
                        o[2 * e + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kx[g][e], 1.0f, true));
                    }
                    op0 = u32x4{o[0], o[1], o[2], o[3]};
                    op1 = u32x4{o[4], o[5], o[6], o[7]};
                }
                const int ga = KI8 ? g : 0;
                sacc[ga] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, op0), qb[2 * g],
                                                                   sacc[ga], 0, 0, 0);
                sacc[ga] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, op1), qb[2 * g + 1],
                                                                   sacc[ga], 0, 0, 0);
            }
            float sj[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if constexpr (KI8) {
                    float x = 0.f;
#pragma unroll
                    for (int g = 0; g < NU; ++g) x += sacc[g][r] * ksc[r][g];
                    sj[r] = x * a.scale_log2;
                } else if constexpr (KF8) {
                    sj[r] = sacc[0][r] * ksc[r][0] * a.scale_log2;
                } else {
                    sj[r] = sacc[0][r] * a.scale_log2;
                }
            }
            if (tok0 + kPage > kmin) {             // a real column's limit falls inside the page
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (tok0 + tk[r] >= klim) sj[r] = -INFINITY;
            }
            const float pm = rows_max(fmaxf(fmaxf(sj[0], sj[1]), fmaxf(sj[2], sj[3])));
            if (__builtin_amdgcn_ballot_w64(pm > m_ref + kRescaleLog2)) {
                const float mn = pm > m_ref + kRescaleLog2 ? pm : m_ref;
                const float alpha = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - mn);
                l_part *= alpha;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) acc[dt] *= alpha;
                m_ref = mn;
            }
            float p[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                p[r] = __builtin_amdgcn_exp2f(sj[r] - m_ref);
                // a column with no visible key in this wave yet has no reference
                p[r] = m_ref == -INFINITY ? 0.f : p[r];
            }
            l_part += (p[0] + p[1]) + (p[2] + p[3]);

            // keys past the last limit hold stale bytes (possibly NaN codes or
            // scales): their V codes and scales count as zero
            if (lim < kPage) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool live = tk[r] < lim;
#pragma unroll
                    for (int e = 0; e < NVW; ++e) vx[r][e] = live ? vx[r][e] : 0u;
#pragma unroll
                    for (int g = 0; g < NVS; ++g) vsc[r][g] = live ? vsc[r][g] : 0.f;
                }
            }

            // P^T operands [P_hi; P_lo], one per V scale group
            bf16x8_t bop[NPV];
#pragma unroll
            for (int g = 0; g < NPV; ++g) {
                float pv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) pv[r] = (VC == CODEC_NVFP4_G16) ? p[r] : p[r] * vsc[r][g];
                uint32_t h01, l01, h23, l23;
                split_bf16(pv[0], pv[1], h01, l01);
                split_bf16(pv[2], pv[3], h23, l23);
                bop[g] = __builtin_bit_cast(bf16x8_t, u32x4{h01, h23, l01, l23});
            }

            // PV: O^T[16 dims x 16 columns] += V^T . P^T per tile
            auto pv_tile = [&](int dt, uint32_t x01, uint32_t x23, int g) __attribute__((always_inline)) {
                acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, u32x4{x01, x23, x01, x23}), bop[g], acc[dt], 0, 0, 0);
            };
            if constexpr (VI8) {
#pragma unroll
                for (int g = 0; g < NU; ++g) {
                    const uint32_t x0 = vx[0][g], x1 = vx[1][g], x2 = vx[2][g], x3 = vx[3][g];
                    pv_tile(4 * g + 0, pk_bf16(i8f<0>(x0), i8f<0>(x1)), pk_bf16(i8f<0>(x2), i8f<0>(x3)), g);
                    pv_tile(4 * g + 1, pk_bf16(i8f<1>(x0), i8f<1>(x1)), pk_bf16(i8f<1>(x2), i8f<1>(x3)), g);
                    pv_tile(4 * g + 2, pk_bf16(i8f<2>(x0), i8f<2>(x1)), pk_bf16(i8f<2>(x2), i8f<2>(x3)), g);
                    pv_tile(4 * g + 3, pk_bf16(i8f<3>(x0), i8f<3>(x1)), pk_bf16(i8f<3>(x2), i8f<3>(x3)), g);
                }
            } else {
                // two tiles per step: dims 2q and 2q + 1 of the lane's run
#pragma unroll
                for (int q = 0; q < NDT / 2; ++q) {
                    f32x2_t f[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if constexpr (VF8) {
                            f[r] = fp8_pair(vx[r][q / 2], q & 1);
                        } else {
                            f[r] = fp4_pair(vx[r][q / 4], q & 3);
                            f[r] = f[r] * vsc[r][0];
                        }
                    }
                    pv_tile(2 * q, pk_bf16(f[0][0], f[1][0]), pk_bf16(f[2][0], f[3][0]), 0);
                    pv_tile(2 * q + 1, pk_bf16(f[0][1], f[1][1]), pk_bf16(f[2][1], f[3][1]), 0);
                }
            }
        }

        if (meta & 256) {
            finish_unit(J);
            if (i + 1 < npg) {
                ++sig;
                ++unit_k;
                start_unit(unit_k, sig);
            }
        }
    };

    for (int i0 = 0; i0 < npg; i0 += NS) ring_round<0, NS>(step, i0, npg);
}

template <int D, int KC, int VC>
hipError_t launch_one(const DecodeArgs& a, int gq, hipStream_t s) {
    paged_qstream_kernel<D, KC, VC><<<dim3(static_cast<unsigned>(a.G)), 256, 0, s>>>(a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    DecodeArgs c = a;
    c.cgroups = combine_groups(gq, D);
    const dim3 cgrid(static_cast<unsigned>(a.B * a.pv.H * c.cgroups));
    switch (gq) {
        case 1: stream_combine_kernel<D, 1, 16><<<cgrid, 64, 0, s>>>(c); break;
        case 2: stream_combine_kernel<D, 2, 16><<<cgrid, 64, 0, s>>>(c); break;
        case 4: stream_combine_kernel<D, 4, 16><<<cgrid, 64, 0, s>>>(c); break;
        case 8: stream_combine_kernel<D, 8, 16><<<cgrid, 64, 0, s>>>(c); break;
        default: return hipErrorNotSupported;
    }
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, int gq, hipStream_t s) {
    const int kc = a.pv.k_codec, vc = a.pv.v_codec;
    if (kc == CODEC_INT8_G64 && vc == CODEC_INT8_G64) return launch_one<D, CODEC_INT8_G64, CODEC_INT8_G64>(a, gq, s);
    if (kc == CODEC_FP8_ROW && vc == CODEC_FP8_ROW) return launch_one<D, CODEC_FP8_ROW, CODEC_FP8_ROW>(a, gq, s);
    if constexpr (D >= 128) {
        if (kc == CODEC_NVFP4_G16 && vc == CODEC_NVFP4_G16)
            return launch_one<D, CODEC_NVFP4_G16, CODEC_NVFP4_G16>(a, gq, s);
        if (kc == CODEC_FP8_ROW && vc == CODEC_NVFP4_G16) return launch_one<D, CODEC_FP8_ROW, CODEC_NVFP4_G16>(a, gq, s);
    }
    return hipErrorNotSupported;
}

}  // namespace

// Profiles (the four quantized ones), D in {64, 128, 256} (NVFP4 sides: 128
// and 256), and the plan's limits: eight entries, 64 KV heads, 32768 logical
// pages per row, 4096 blocks of at most kStreamPages / (blocks per CU) pages.
bool qstream_path(const PoolView& pv, int B, int gq) {
    const int kc = pv.k_codec, vc = pv.v_codec;
    const bool combo = (kc == CODEC_INT8_G64 && vc == CODEC_INT8_G64) || (kc == CODEC_FP8_ROW && vc == CODEC_FP8_ROW) ||
                       (kc == CODEC_NVFP4_G16 && vc == CODEC_NVFP4_G16) ||
                       (kc == CODEC_FP8_ROW && vc == CODEC_NVFP4_G16);
    const bool fp4 = kc == CODEC_NVFP4_G16 || vc == CODEC_NVFP4_G16;
    const bool dims = pv.D == 128 || pv.D == 256 || (pv.D == 64 && !fp4);
    return combo && dims && B <= plan::kMaxEnt && pv.H <= plan::kMaxH && pv.L <= 32768 &&
           (long long)B * pv.H * pv.L <= 4096LL * (kStreamPages / qstream_blocks_per_cu(pv)) &&
           (gq == 1 || gq == 2 || gq == 4 || gq == 8);
}

int qstream_blocks_per_cu(const PoolView& pv) { return pv.D <= 128 ? qstream_bpc<128>() : qstream_bpc<256>(); }

hipError_t launch_qstream(const DecodeArgs& a, int gq, hipStream_t s) {
    switch (a.pv.D) {
        case 64: return launch_d<64>(a, gq, s);
        case 128: return launch_d<128>(a, gq, s);
        case 256: return launch_d<256>(a, gq, s);
    }
    return hipErrorNotSupported;
}

}  // namespace kvs
