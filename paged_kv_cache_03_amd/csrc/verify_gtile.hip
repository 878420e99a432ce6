// verify_gtile.hip -- verify / chunked prefill on matrix-core tiles for the
// pools the BF16 tile kernel of verify.hip does not take: the quantized closed
// profiles (INT8-G64, FP8-row, NVFP4-G16 and K8V4; Paged KV Context Store
// page, closed-profile paragraph and X-extent list) at D in {64, 128, 256},
// and BF16 pages at D = 256 (the size the page's D256 payload table is
// written for).
//
// Chunk token i of entry b sits at position n0[b] + i and attends
// [0, n0[b] + i]; the chunk's K/V are appended before the call.  A tile is
// TCOL query columns (consecutive chunk tokens x the GQ heads of one KV head):
// 128 at D <= 128, 64 at D = 256.  A block of eight waves streams the tile's
// causal key range, optionally a 1/S share of it (below), one page at a time:
//  * every thread loads the codes and scales of a few 8-dim chunks of the
//    next page into registers (buffer loads: an unmapped page reads zeros),
//    while the waves compute the current page;
//  * it then dequantizes them exactly as the codec defines -- value(code) *
//    scale in fp32 -- and writes each value as a bf16 pair hi + lo, hi =
//    rne(v), lo = rne(v - hi) (about 2^-17 relative error left), into LDS
//    tiles laid out as the BF16 tile kernel's stages.  NVFP4 values (an e2m1
//    code times an e4m3 scale: at most 6 significant bits) and BF16 values
//    are exact in bf16: those sides have no lo tile.  Rows past the page's
//    last visible key are written as zeros, so stale bytes never reach a
//    product;
//  * wave w owns columns [16 WCT (w%4), 16 WCT (w%4 + 1)) and keys
//    [32(w/4), 32(w/4) + 32) of the page: S^T = (K_hi + K_lo) . Q^T and
//    O^T += (V_hi + V_lo)^T . P^T on v_mfma_f32_16x16x32_bf16, P as one bf16
//    term on pages where no key weighs more than 1/64 of its column's running
//    sum and as p_hi + p_lo elsewhere (as in the BF16 tiles), column sums of
//    exactly the P values used on the matrix cores, lazy rescaling, the
//    causal mask on the pages that reach a column's limit;
//  * the two key halves of each column range merge once at the end.
// Split: a launch whose tiles alone cannot fill the chip (short chunks, few
// entries) cuts every tile's page range into S equal parts; each part writes
// its columns' (m, l, acc) and gtile_combine_kernel folds the parts in part
// order, so the result does not depend on timing.  Blocks are mapped so that
// the parts of consecutive tiles run on one die (XCD) and share its L2.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "attn_common.h"
#include "codec_device.h"
#include "internal.h"
#include "launch.h"
#include "stream_common.h"

namespace kvs {
namespace {

struct GTileArgs {
    PoolView pv;
    const int32_t* table_rows;
    const int32_t* q_pos0;
    const int32_t* cu_q;
    const uint16_t* q;
    float* out;
    float* part_ml;      // [tile * S + part][TCOL][2]: (running max in log2 units, sum)
    float* part_acc;     // [tile * S + part][TCOL][D] (unnormalized)
    float scale_log2;    // sm_scale * log2(e)
    int32_t B;
    int32_t Hq;
    int32_t max_ctx;
    int32_t S;           // page parts per tile (1: outputs written directly)
    int32_t nblk;        // blocks of the tile launch (a multiple of 8)
};

// bytes per page row (one key of one KV head) of a side's code and scale
// planes
template <int C, int D, int SB>
struct GRow {
    static constexpr int code = C == CODEC_BF16 ? 2 * D : (C == CODEC_NVFP4_G16 ? D / 2 : D);
    static constexpr int chunk = code / (D / 8);   // code bytes of one 8-dim chunk: 16, 8 or 4
    static constexpr int scale = C == CODEC_BF16 ? 0 : C == CODEC_INT8_G64 ? SB * (D / 64)
                                                    : C == CODEC_FP8_ROW  ? SB : D / 16;
};

template <int D>
constexpr int gtile_cols() { return D == 256 ? 64 : 128; }

// one page's codes and scales of a thread's J chunks of one side
template <int J>
struct RawSide {
    u32x4 code[J];
    uint32_t scale[J];
};

// chunk j of the page (rows of NCH chunks): its row and chunk index
template <int NCH>
__device__ __forceinline__ void job_of(int j, int& r, int& x) {
    r = j / NCH;
    x = j % NCH;
}

// loads of one side's chunks of a page slice (base: the plane's slice start;
// mapped: the page has a group)
template <int C, int D, int SB, int J, int NT>
__device__ __forceinline__ void load_side(RawSide<J>& rs, const char* code_base, const char* scale_base, bool mapped,
                                          int tid) {
    using R = GRow<C, D, SB>;
    constexpr int NCH = D / 8;
    const __amdgpu_buffer_rsrc_t rc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(code_base), 0, mapped ? 64 * R::code : 0, kBufferWord3);
    __amdgpu_buffer_rsrc_t rsc = rc;
    if constexpr (R::scale > 0)
        rsc = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(scale_base), 0, mapped ? 64 * R::scale : 0,
                                                kBufferWord3);
#pragma unroll
    for (int k = 0; k < J; ++k) {
        int r, x;
        job_of<NCH>(tid + NT * k, r, x);
        const int co = r * R::code + x * R::chunk;
        if constexpr (R::chunk == 16) {
            rs.code[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, co, 0, kNonTemporal));
        } else if constexpr (R::chunk == 8) {
            const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rc, co, 0, kNonTemporal));
            rs.code[k] = u32x4{v[0], v[1], 0u, 0u};
        } else {
            rs.code[k] = u32x4{__builtin_amdgcn_raw_buffer_load_b32(rc, co, 0, kNonTemporal), 0u, 0u, 0u};
        }
        if constexpr (C == CODEC_INT8_G64) {
            const int so = r * R::scale + (8 * x / 64) * SB;
            rs.scale[k] = SB == 4 ? __builtin_amdgcn_raw_buffer_load_b32(rsc, so, 0, kNonTemporal)
                                  : uint32_t(__builtin_amdgcn_raw_buffer_load_b16(rsc, so, 0, kNonTemporal));
        } else if constexpr (C == CODEC_FP8_ROW) {
            const int so = r * R::scale;
            rs.scale[k] = SB == 4 ? __builtin_amdgcn_raw_buffer_load_b32(rsc, so, 0, kNonTemporal)
                                  : uint32_t(__builtin_amdgcn_raw_buffer_load_b16(rsc, so, 0, kNonTemporal));
        } else if constexpr (C == CODEC_NVFP4_G16) {
            rs.scale[k] = uint32_t(__builtin_amdgcn_raw_buffer_load_b8(rsc, r * R::scale + (8 * x) / 16, 0,
                                                                       kNonTemporal));
        } else {
            rs.scale[k] = 0u;
        }
    }
}

template <int SB>
__device__ __forceinline__ float wide_scale(uint32_t w) {
    if constexpr (SB == 4) return __uint_as_float(w);
    else return static_cast<float>(__builtin_bit_cast(_Float16, uint16_t(w & 0xFFFFu)));
}

// the 8 values of a chunk, dequantized (value(code) * scale, one fp32 multiply)
template <int C, int SB>
__device__ __forceinline__ void dequant8(const u32x4& code, uint32_t sw, float (&v)[8]) {
    if constexpr (C == CODEC_INT8_G64) {
        const float s = wide_scale<SB>(sw);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = float(int8_t((code[i / 4] >> (8 * (i % 4))) & 0xFFu)) * s;
    } else if constexpr (C == CODEC_FP8_ROW) {
        const float s = wide_scale<SB>(sw);
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const f32x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(code[w], 1.0f, false);
            const f32x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(code[w], 1.0f, true);
            v[4 * w] = a[0] * s;
            v[4 * w + 1] = a[1] * s;
            v[4 * w + 2] = b[0] * s;
            v[4 * w + 3] = b[1] * s;
        }
    } else {   // NVFP4-G16: e2m1 codes, element 2k in the low nibble of byte k
        const float s = e4m3fn_to_f32(sw & 0xFFu);
        const f32x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code[0], 1.0f, 0);
        const f32x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code[0], 1.0f, 1);
        const f32x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code[0], 1.0f, 2);
        const f32x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code[0], 1.0f, 3);
        v[0] = p0[0] * s; v[1] = p0[1] * s; v[2] = p1[0] * s; v[3] = p1[1] * s;
        v[4] = p2[0] * s; v[5] = p2[1] * s; v[6] = p3[0] * s; v[7] = p3[1] * s;
    }
}

template <int D, int GQ, int KC, int VC, int SB>
__global__ void __launch_bounds__(512) verify_gtile_kernel(GTileArgs a) {
    constexpr int NT = 512;
    constexpr int NCH = D / 8;                     // 16-byte bf16 chunks per row
    constexpr int J = 64 * NCH / NT;               // chunks of a page plane per thread
    constexpr int NC = D / 32;                     // QK products per key tile, k = 32 each
    constexpr int NDT = D / 16;                    // PV tiles of 16 dims
    constexpr int TCOL = gtile_cols<D>();          // query columns per tile
    constexpr int WCT = TCOL / 64;                 // 16-column tiles per wave
    constexpr int TTOK = TCOL / GQ;                // chunk tokens per tile
    constexpr float kHiOnly = 1.f / 256.f;         // largest weight of a page that takes p as one bf16 term
    // INT8-G64 and FP8-row sides: the tile holds the codes (exact in bf16);
    // the K scales act on each key's per-group partial scores, the V scales on
    // the key's probability (one copy of P per V scale group, as p * s rounded
    // to bf16 like p itself).  NVFP4 and BF16 sides hold their values (exact in
    // bf16).
    constexpr bool KSC = KC == CODEC_INT8_G64 || KC == CODEC_FP8_ROW;
    constexpr int NGK = KC == CODEC_INT8_G64 ? D / 64 : 1;   // score accumulators: one per K scale group
    constexpr bool VSC = VC == CODEC_INT8_G64 || VC == CODEC_FP8_ROW;
    constexpr int NGV = VC == CODEC_INT8_G64 ? D / 64 : 1;   // copies of P: one per V scale group
    // the products at raised wave priority for INT8-G64 pages (the prefill
    // mix on them 2.5% faster over two A/B pairs on one box; K8V4 1% and BF16
    // at D = 256 4.5% slower, so those keep the default)
    constexpr bool PRIO = KC == CODEC_INT8_G64;
    constexpr int PLANE = 64 * NCH;                // u32x4 slots of one bf16 page tile
    constexpr int OFF_VH = PLANE;
    constexpr int NPL = 2;
    constexpr int OFF_KS = NPL * PLANE;            // K scales [group][64 keys] as fp32
    constexpr int KS_SLOTS = KSC ? NGK * 64 / 4 : 0;
    constexpr int OFF_VS = OFF_KS + KS_SLOTS;      // V scales [group][64 keys] as fp32
    constexpr int VS_SLOTS = VSC ? NGV * 64 / 4 : 0;
    constexpr int MERGE = WCT * NDT * 4 * 64 * 4 / 16 * 4;   // u32x4 slots of the end merge (4 column ranges)
    // two stages of tiles where they fit in LDS (the next page is converted
    // while the current one is computed), else one
    constexpr int STAGE = NPL * PLANE + KS_SLOTS + VS_SLOTS;
    constexpr int NSTG = 2 * STAGE * 16 <= 144 * 1024 ? 2 : 1;
    constexpr int SLOTS = NSTG * STAGE > MERGE ? NSTG * STAGE : MERGE;
    static_assert(J >= 1 && 64 * NCH % NT == 0 && TCOL % GQ == 0, "shape");

    __shared__ u32x4 lds[SLOTS];
    __shared__ float mlx[4][WCT][16][2];

    const int tid = int(threadIdx.x);
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, li = lane & 15, lg = lane >> 4;
    const int cw = w & 3, kh = w >> 2;             // column range, key half
    const int H = a.pv.H, M = a.pv.M;

    // (tile, part) units in (entry, KV head, tile, part) order; die x takes
    // units [x*per, (x+1)*per)
    int n_tiles = 0;
    for (int b = 0; b < a.B; ++b) {
        const int T = ld_uniform(a.cu_q, b + 1) - ld_uniform(a.cu_q, b);
        n_tiles += H * ((T * GQ + TCOL - 1) / TCOL);
    }
    const int per = a.nblk / 8;
    const int unit = (int(blockIdx.x) % 8) * per + int(blockIdx.x) / 8;
    const int tile = unit / a.S, part = unit % a.S;
    if (tile >= n_tiles) return;
    int item = tile, b = 0, nt = 0;
    for (; b < a.B; ++b) {
        const int T = ld_uniform(a.cu_q, b + 1) - ld_uniform(a.cu_q, b);
        nt = (T * GQ + TCOL - 1) / TCOL;
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
    const int per_part = (npages + a.S - 1) / a.S;
    const int p0 = min(npages, part * per_part), p1 = min(npages, p0 + per_part);

    // this lane's columns: c = 16 (WCT cw + ct) + li; key limits and Q^T operands
    int klim[WCT];
    bf16x8_t qb[WCT][NC];
#pragma unroll
    for (int ct = 0; ct < WCT; ++ct) {
        const int c = 16 * (WCT * cw + ct) + li;
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

    // LDS tile layouts (XOR-swizzled 16-byte chunks, as the BF16 tile kernel)
    auto kswz = [](int r) __attribute__((always_inline)) { return NCH >= 16 ? (r & 15) : ((r >> 1) & 7); };
    auto vswz = [](int r) __attribute__((always_inline)) { return NCH >= 16 ? ((r & 7) << 1) : (((r >> 1) & 3) << 1); };
    const int kr0 = 32 * kh;                       // first key row of this wave
    int koff[NC], voff[NDT];
    {
#pragma unroll
        for (int c = 0; c < NC; ++c) koff[c] = (kr0 + li) * NCH + ((4 * c + lg) ^ kswz(li));
        const int tv = 4 * lg + (li >> 2), qd = li & 3;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
            voff[dt] = (kr0 + tv) * NCH * 16 + (((2 * dt + (qd >> 1)) ^ vswz(tv)) * 16) + 8 * (qd & 1);
    }

    const char* kcp = static_cast<const char*>(a.pv.lv.k_code);
    const char* ksp = static_cast<const char*>(a.pv.lv.k_scale);
    const char* vcp = static_cast<const char*>(a.pv.lv.v_code);
    const char* vsp = static_cast<const char*>(a.pv.lv.v_scale);
    using RK = GRow<KC, D, SB>;
    using RV = GRow<VC, D, SB>;
    const int32_t* trow = a.pv.table + size_t(row) * a.pv.L;
    auto slice_of = [&](int p) __attribute__((always_inline)) {
        const int g0 = ld_uniform(trow, p);
        return (g0 >= 0 && g0 < M) ? g0 * a.pv.sg + h * a.pv.sh : -1;
    };

    RawSide<J> rk, rv;
    auto load_page = [&](int p) __attribute__((always_inline)) {
        const int sl = slice_of(p);
        const size_t s = size_t(sl < 0 ? 0 : sl) * 64;
        load_side<KC, D, SB, J, NT>(rk, kcp + s * RK::code, ksp + s * RK::scale, sl >= 0, tid);
        load_side<VC, D, SB, J, NT>(rv, vcp + s * RV::code, vsp + s * RV::scale, sl >= 0, tid);
        return sl;
    };
    // the loaded page into the LDS tiles of stage st; rows at or past lim become zeros
    auto convert = [&](int lim, int st) __attribute__((always_inline)) {
        u32x4* const tl = &lds[st * STAGE];
#pragma unroll
        for (int k = 0; k < J; ++k) {
            int r, x;
            job_of<NCH>(tid + NT * k, r, x);
            const bool vis = r < lim;
            u32x4 khi, vhi;
            if constexpr (KC == CODEC_BF16) {
                khi = vis ? rk.code[k] : u32x4{0u, 0u, 0u, 0u};
            } else if constexpr (KC == CODEC_INT8_G64) {
                const u32x4 c = rk.code[k];
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t src = c[e >> 1] >> (16 * (e & 1));
                    w[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(
                        f32x2_t{float(int8_t(src & 0xFFu)), float(int8_t((src >> 8) & 0xFFu))}, bf16x2v_t));
                }
                khi = vis ? u32x4{w[0], w[1], w[2], w[3]} : u32x4{0u, 0u, 0u, 0u};
            } else if constexpr (KC == CODEC_FP8_ROW) {
                const u32x4 c = rk.code[k];
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    w[2 * e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[e], 1.0f, false));
                    w[2 * e + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[e], 1.0f, true));
                }
                khi = vis ? u32x4{w[0], w[1], w[2], w[3]} : u32x4{0u, 0u, 0u, 0u};
            } else {   // NVFP4 K: dequantized values, exact in bf16
                float v[8];
                dequant8<KC, SB>(rk.code[k], rk.scale[k], v);
                uint32_t hw[4], lw[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) split_bf16(v[2 * e], v[2 * e + 1], hw[e], lw[e]);
                khi = vis ? u32x4{hw[0], hw[1], hw[2], hw[3]} : u32x4{0u, 0u, 0u, 0u};
            }
            if constexpr (KSC) {                   // the chunk that starts a scale group writes its scale
                constexpr int GCH = KC == CODEC_INT8_G64 ? 8 : NCH;    // chunks per scale group
                if (x % GCH == 0)
                    reinterpret_cast<float*>(&tl[OFF_KS])[(x / GCH) * 64 + r] = vis ? wide_scale<SB>(rk.scale[k]) : 0.f;
            }
            if constexpr (VC == CODEC_BF16) {
                vhi = vis ? rv.code[k] : u32x4{0u, 0u, 0u, 0u};
            } else if constexpr (VC == CODEC_INT8_G64) {
                const u32x4 c = rv.code[k];
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t src = c[e >> 1] >> (16 * (e & 1));
                    w[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(
                        f32x2_t{float(int8_t(src & 0xFFu)), float(int8_t((src >> 8) & 0xFFu))}, bf16x2v_t));
                }
                vhi = vis ? u32x4{w[0], w[1], w[2], w[3]} : u32x4{0u, 0u, 0u, 0u};
            } else if constexpr (VC == CODEC_FP8_ROW) {
                const u32x4 c = rv.code[k];
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    w[2 * e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[e], 1.0f, false));
                    w[2 * e + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[e], 1.0f, true));
                }
                vhi = vis ? u32x4{w[0], w[1], w[2], w[3]} : u32x4{0u, 0u, 0u, 0u};
            } else {   // NVFP4 V: dequantized values, exact in bf16
                float v[8];
                dequant8<VC, SB>(rv.code[k], rv.scale[k], v);
                uint32_t hw[4], lw[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) split_bf16(v[2 * e], v[2 * e + 1], hw[e], lw[e]);
                vhi = vis ? u32x4{hw[0], hw[1], hw[2], hw[3]} : u32x4{0u, 0u, 0u, 0u};
            }
            if constexpr (VSC) {                   // the chunk that starts a V scale group writes its scale
                constexpr int GCH = VC == CODEC_INT8_G64 ? 8 : NCH;    // chunks per scale group
                if (x % GCH == 0)
                    reinterpret_cast<float*>(&tl[OFF_VS])[(x / GCH) * 64 + r] = vis ? wide_scale<SB>(rv.scale[k]) : 0.f;
            }
            const int ks = r * NCH + (x ^ kswz(r)), vs = r * NCH + (x ^ vswz(r));
            tl[ks] = khi;
            tl[OFF_VH + vs] = vhi;
        }
    };

    f32x4_t acc[WCT][NDT];
    f32x4_t lsum[WCT];                              // column sums of the P values used, on the matrix cores
    float m_ref[WCT];
    const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
#pragma unroll
    for (int ct = 0; ct < WCT; ++ct) {
        m_ref[ct] = -INFINITY;
        lsum[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[ct][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    const lds_byte_ptr lbase = (lds_byte_ptr)(&lds[0]);
    auto read_vt = [&](int plane, int dt) __attribute__((always_inline)) {
        const lds_byte_ptr vst = lbase + plane * 16;   // plane: slot offset of the tile (stage included)
        const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(vst + voff[dt]));
        const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(vst + voff[dt] + 16 * NCH * 16));
        return __builtin_bit_cast(bf16x8_t, u32x4{__builtin_bit_cast(u32x2, v0)[0], __builtin_bit_cast(u32x2, v0)[1],
                                                  __builtin_bit_cast(u32x2, v1)[0], __builtin_bit_cast(u32x2, v1)[1]});
    };

    // one page from the LDS tiles of stage st
    auto compute = [&](int i, int lim, int st) __attribute__((always_inline)) {
        const int tok0 = i * kPage;
        const int sb = st * STAGE;
        if (lim <= kr0) return;                    // none of this wave's keys is visible
        f32x4_t s[2][WCT];
        {
            // partial scores per K scale group (INT8-G64: 64 dims = two
            // products of k = 32), then each key's scales applied in fp32
            f32x4_t sg[NGK][2][WCT];
#pragma unroll
            for (int g = 0; g < NGK; ++g)
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int ct = 0; ct < WCT; ++ct) sg[g][kt][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    constexpr int CPG = NGK > 1 ? NC / NGK : NC;
                    const int g = NGK > 1 ? c / CPG : 0;
                    const bf16x8_t kk = __builtin_bit_cast(bf16x8_t, lds[sb + koff[c] + kt * 16 * NCH]);
#pragma unroll
                    for (int ct = 0; ct < WCT; ++ct)
                        sg[g][kt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk, qb[ct][c], sg[g][kt][ct], 0, 0, 0);
                }
            }
            if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
            if constexpr (KSC) {
                const float* kst = reinterpret_cast<const float*>(&lds[sb + OFF_KS]);
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                    for (int ct = 0; ct < WCT; ++ct) s[kt][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int g = 0; g < NGK; ++g) {
                        const f32x4_t sc = *reinterpret_cast<const f32x4_t*>(kst + g * 64 + kr0 + 16 * kt + 4 * lg);
#pragma unroll
                        for (int ct = 0; ct < WCT; ++ct) s[kt][ct] += sg[g][kt][ct] * sc;
                    }
                }
            } else {
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int ct = 0; ct < WCT; ++ct) s[kt][ct] = sg[0][kt][ct];
            }
        }
        // the causal mask, only on the pages that reach some column's limit
        if (tok0 + kPage > kmin) {
#pragma unroll
            for (int ct = 0; ct < WCT; ++ct)
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (tok0 + kr0 + 16 * kt + 4 * lg + r >= klim[ct]) s[kt][ct][r] = -INFINITY;
        }
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
        bool need_lo = false;
#pragma unroll
        for (int ct = 0; ct < WCT; ++ct)
            need_lo |= !(__builtin_amdgcn_exp2f(pm[ct] - m_ref[ct]) <= kHiOnly * lsum[ct][0]);
        float p[WCT][8];
        bf16x8_t phi[WCT];                         // rne(p): the column sums, and the PV weights without V scales
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
        // V scales of this lane's keys kr0 + 16 kt + 4 lg + r, per group
        f32x4_t vsc[NGV][2];
        if constexpr (VSC) {
            const float* vst = reinterpret_cast<const float*>(&lds[sb + OFF_VS]);
#pragma unroll
            for (int g = 0; g < NGV; ++g)
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
                    vsc[g][kt] = *reinterpret_cast<const f32x4_t*>(vst + g * 64 + kr0 + 16 * kt + 4 * lg);
        }
        // the PV weights of V scale group g (term 0: rne(p * s); term 1: the remainder)
        auto weights = [&](int g, int ct, bool lo_term) __attribute__((always_inline)) {
            uint32_t hv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float x0 = p[ct][2 * e], x1 = p[ct][2 * e + 1];
                if constexpr (VSC) {
                    x0 *= vsc[g][(2 * e) >> 2][(2 * e) & 3];
                    x1 *= vsc[g][(2 * e + 1) >> 2][(2 * e + 1) & 3];
                }
                uint32_t h, l;
                split_bf16(x0, x1, h, l);
                hv[e] = lo_term ? l : h;
            }
            return __builtin_bit_cast(bf16x8_t, u32x4{hv[0], hv[1], hv[2], hv[3]});
        };
        constexpr int DPG = NDT / NGV;             // PV tiles per V scale group
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int g = 0; g < NGV; ++g) {
            bf16x8_t pw[WCT];
#pragma unroll
            for (int ct = 0; ct < WCT; ++ct) pw[ct] = VSC ? weights(g, ct, false) : phi[ct];
#pragma unroll
            for (int d = 0; d < DPG; ++d) {
                const int dt = g * DPG + d;
                const bf16x8_t va = read_vt(sb + OFF_VH, dt);
#pragma unroll
                for (int ct = 0; ct < WCT; ++ct)
                    acc[ct][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pw[ct], acc[ct][dt], 0, 0, 0);
            }
        }
#pragma unroll
        for (int ct = 0; ct < WCT; ++ct) lsum[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, phi[ct], lsum[ct], 0, 0, 0);
        if (__builtin_amdgcn_ballot_w64(need_lo)) {
            // the remainders rne(w - rne(w)) of the weights, the same products on them
#pragma unroll
            for (int g = 0; g < NGV; ++g) {
                bf16x8_t pw[WCT];
#pragma unroll
                for (int ct = 0; ct < WCT; ++ct) pw[ct] = weights(g, ct, true);
#pragma unroll
                for (int d = 0; d < DPG; ++d) {
                    const int dt = g * DPG + d;
                    const bf16x8_t va = read_vt(sb + OFF_VH, dt);
#pragma unroll
                    for (int ct = 0; ct < WCT; ++ct)
                        acc[ct][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pw[ct], acc[ct][dt], 0, 0, 0);
                }
            }
            bf16x8_t plo[WCT];
#pragma unroll
            for (int ct = 0; ct < WCT; ++ct) plo[ct] = weights(0, ct, true);
            if constexpr (VSC) {
#pragma unroll
                for (int ct = 0; ct < WCT; ++ct) {   // the column sums take the remainder of p itself
                    const u32x4 hu = __builtin_bit_cast(u32x4, phi[ct]);
                    uint32_t lv[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float r0 = p[ct][2 * e] - __uint_as_float(hu[e] << 16);
                        const float r1 = p[ct][2 * e + 1] - __uint_as_float(hu[e] & 0xFFFF0000u);
                        lv[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{r0, r1}, bf16x2v_t));
                    }
                    plo[ct] = __builtin_bit_cast(bf16x8_t, u32x4{lv[0], lv[1], lv[2], lv[3]});
                }
            }
#pragma unroll
            for (int ct = 0; ct < WCT; ++ct)
                lsum[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, plo[ct], lsum[ct], 0, 0, 0);
        }
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
    };

    // pages [p0, p1); rows any column may see on page i: lim_of
    auto lim_of = [&](int i, int sl) __attribute__((always_inline)) {
        return sl >= 0 ? min(kPage, kmax - i * kPage) : 0;
    };
    if (p0 < p1) {
        if constexpr (NSTG == 2) {
            // page i+1 is converted into the other stage while page i is
            // computed, page i+2's loads in flight: one barrier per page
            int sl = load_page(p0);
            int lim = lim_of(p0, sl);
            convert(lim, 0);
            if (p0 + 1 < p1) sl = load_page(p0 + 1);
            block_lds_barrier();
            for (int i = p0; i < p1; ++i) {
                const int st = (i - p0) & 1;
                const int lim_next = i + 1 < p1 ? lim_of(i + 1, sl) : 0;
                compute(i, lim, st);
                if (i + 1 < p1) {
                    convert(lim_next, st ^ 1);
                    if (i + 2 < p1) sl = load_page(i + 2);
                }
                block_lds_barrier();               // stage st is free, stage st^1 is written
                lim = lim_next;
            }
        } else {
            // one stage: the next page's loads are in flight while one is computed
            int sl = load_page(p0);
            for (int i = p0; i < p1; ++i) {
                const int lim = lim_of(i, sl);
                convert(lim, 0);
                block_lds_barrier();
                if (i + 1 < p1) sl = load_page(i + 1);
                compute(i, lim, 0);
                block_lds_barrier();               // every wave is done with the tiles
            }
        }
    }

    // merge the two key halves of each column range through the LDS tiles,
    // then wave cw writes its columns (or their part's partials)
    float lw[WCT];
#pragma unroll
    for (int ct = 0; ct < WCT; ++ct) lw[ct] = lsum[ct][0];
    float* xb = reinterpret_cast<float*>(&lds[0]) + cw * (WCT * NDT * 4 * 64);
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
        const int c = 16 * (WCT * cw + ct) + li;
        if (c >= ncol) continue;
        if (a.S == 1) {
            const float inv = l > 0.f ? 1.f / l : 0.f;
            float* o = a.out + (size_t(c0 + i0 + c / GQ) * a.Hq + size_t(h) * GQ + c % GQ) * D + 4 * lg;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                f32x4_t v;
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = (acc[ct][dt][r] * w0 + xb[((ct * NDT + dt) * 4 + r) * 64 + lane] * w1) * inv;
                *reinterpret_cast<float4*>(o + 16 * dt) = make_float4(v[0], v[1], v[2], v[3]);
            }
        } else {
            const size_t u = size_t(tile) * a.S + part;
            float* o = a.part_acc + (u * TCOL + c) * D + 4 * lg;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                f32x4_t v;
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = acc[ct][dt][r] * w0 + xb[((ct * NDT + dt) * 4 + r) * 64 + lane] * w1;
                *reinterpret_cast<float4*>(o + 16 * dt) = make_float4(v[0], v[1], v[2], v[3]);
            }
            if (lg == 0) *reinterpret_cast<float2*>(a.part_ml + (u * TCOL + c) * 2) = make_float2(mx, l);
        }
    }
}

// The parts of every tile, folded in part order: one wave per (tile, column),
// D/64 outputs per lane.
template <int D, int GQ>
__global__ void __launch_bounds__(256) gtile_combine_kernel(GTileArgs a) {
    constexpr int TCOL = gtile_cols<D>();
    constexpr int EPL = D / 64;
    const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6), lane = int(threadIdx.x) & 63;
    const int gidx = int(blockIdx.x) * 4 + w;
    const int tile = gidx / TCOL, c = gidx % TCOL;
    const int H = a.pv.H;
    int item = tile, b = 0, nt = 0;
    for (; b < a.B; ++b) {
        const int T = ld_uniform(a.cu_q, b + 1) - ld_uniform(a.cu_q, b);
        nt = (T * GQ + TCOL - 1) / TCOL;
        if (item < H * nt) break;
        item -= H * nt;
    }
    if (b >= a.B) return;
    const int h = item / nt, t = item % nt;
    const int c0 = ld_uniform(a.cu_q, b), T = ld_uniform(a.cu_q, b + 1) - c0;
    const int i0 = t * (TCOL / GQ);
    if (c >= min(TCOL, (T - i0) * GQ)) return;
    const size_t u0 = size_t(tile) * a.S;
    float mx = -INFINITY;
    for (int p = 0; p < a.S; ++p) mx = fmaxf(mx, a.part_ml[((u0 + p) * TCOL + c) * 2]);
    float l = 0.f, acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
    for (int p = 0; p < a.S; ++p) {
        const size_t it = (u0 + p) * TCOL + c;
        const float mp = a.part_ml[it * 2];
        const float wgt = mp == -INFINITY ? 0.f : exp2f(mp - mx);
        l += a.part_ml[it * 2 + 1] * wgt;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] += a.part_acc[it * D + lane * EPL + e] * wgt;
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* o = a.out + (size_t(c0 + i0 + c / GQ) * a.Hq + size_t(h) * GQ + c % GQ) * D + lane * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = acc[e] * inv;
}

// tiles bound of a launch (every entry at max_q_len tokens)
long long gtile_bound(const PoolView& pv, int B, int gq, int max_q_len) {
    const int tcol = pv.D == 256 ? 64 : 128;
    return (long long)B * pv.H * ((max_q_len * gq + tcol - 1) / tcol);
}

// parts per tile: enough (tile, part) units for two per compute unit, each
// part at least 8 pages, at most 32 parts
int gtile_parts(const PoolView& pv, int B, int gq, int max_q_len, int max_seq_len) {
    static const int cus = [] {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        return n;
    }();
    const long long tiles = gtile_bound(pv, B, gq, max_q_len);
    if (tiles <= 0) return 1;
    long long s = (2LL * cus + tiles - 1) / tiles;
    const long long pages = (max_seq_len + kPage - 1) / kPage;
    s = std::min(s, std::max(1LL, pages / 8));
    return int(std::max(1LL, std::min(s, 32LL)));
}

template <int D, int GQ, int KC, int VC, int SB>
hipError_t launch_gtile_one(const GTileArgs& a, hipStream_t s) {
    const hipError_t e = launch_kernel(true, verify_gtile_kernel<D, GQ, KC, VC, SB>, dim3(unsigned(a.nblk)), dim3(512),
                                       s, a);
    if (e != hipSuccess || a.S == 1) return e;
    const long long tiles = (long long)a.nblk / a.S;   // a bound: blocks past the real tiles return
    const dim3 cgrid(unsigned((tiles * gtile_cols<D>() + 3) / 4));
    gtile_combine_kernel<D, GQ><<<cgrid, 256, 0, s>>>(a);
    return hipGetLastError();
}

template <int D, int KC, int VC, int SB>
hipError_t launch_gtile_gq(const GTileArgs& a, int gq, hipStream_t s) {
    switch (gq) {
        case 1: return launch_gtile_one<D, 1, KC, VC, SB>(a, s);
        case 2: return launch_gtile_one<D, 2, KC, VC, SB>(a, s);
        case 4: return launch_gtile_one<D, 4, KC, VC, SB>(a, s);
        case 8: return launch_gtile_one<D, 8, KC, VC, SB>(a, s);
    }
    return hipErrorNotSupported;
}

template <int D>
hipError_t launch_gtile_d(const GTileArgs& a, int gq, hipStream_t s) {
    const int kc = a.pv.k_codec, vc = a.pv.v_codec;
    const bool s16 = a.pv.scale16 != 0;
#define KVS_GT_CASE(K, V, SB) \
    if (kc == K && vc == V && s16 == (SB == 2)) return launch_gtile_gq<D, K, V, SB>(a, gq, s);
    if constexpr (D == 256) KVS_GT_CASE(CODEC_BF16, CODEC_BF16, 4)
    KVS_GT_CASE(CODEC_INT8_G64, CODEC_INT8_G64, 4)
    KVS_GT_CASE(CODEC_FP8_ROW, CODEC_FP8_ROW, 4)
    KVS_GT_CASE(CODEC_NVFP4_G16, CODEC_NVFP4_G16, 4)
    KVS_GT_CASE(CODEC_FP8_ROW, CODEC_NVFP4_G16, 4)
    KVS_GT_CASE(CODEC_INT8_G64, CODEC_INT8_G64, 2)
    KVS_GT_CASE(CODEC_FP8_ROW, CODEC_FP8_ROW, 2)
    KVS_GT_CASE(CODEC_FP8_ROW, CODEC_NVFP4_G16, 2)
#undef KVS_GT_CASE
    return hipErrorNotSupported;
}

}  // namespace

bool gtile_supported(const PoolView& pv, int gq) {
    const bool quant = pv.k_codec != CODEC_BF16 || pv.v_codec != CODEC_BF16;
    return (quant ? (pv.D == 64 || pv.D == 128 || pv.D == 256) : pv.D == 256) &&
           (gq == 1 || gq == 2 || gq == 4 || gq == 8);
}

size_t gtile_workspace_bytes(const PoolView& pv, int B, int Hq, int max_seq_len, int max_q_len) {
    const int gq = Hq / pv.H;
    const int S = gtile_parts(pv, B, gq, max_q_len, max_seq_len);
    if (S == 1) return 0;
    const size_t units = (size_t(gtile_bound(pv, B, gq, max_q_len)) * S + 7) / 8 * 8;   // every launched block
    const size_t cols = pv.D == 256 ? 64 : 128;
    const size_t ml = (units * cols * 2 * sizeof(float) + 255) / 256 * 256;
    return ml + units * cols * size_t(pv.D) * sizeof(float);
}

hipError_t launch_gtile(const PoolView& pv, int B, int Hq, const int32_t* table_rows, const int32_t* q_pos0,
                        const int32_t* cu_q, int max_q_len, int max_seq_len, const void* q, float sm_scale,
                        float* out, void* ws, hipStream_t s) {
    const int gq = Hq / pv.H;
    GTileArgs a{};
    a.pv = pv;
    a.table_rows = table_rows;
    a.q_pos0 = q_pos0;
    a.cu_q = cu_q;
    a.q = static_cast<const uint16_t*>(q);
    a.out = out;
    a.scale_log2 = sm_scale * kLog2e;
    a.B = B;
    a.Hq = Hq;
    a.max_ctx = max_seq_len;
    a.S = gtile_parts(pv, B, gq, max_q_len, max_seq_len);
    const long long units = gtile_bound(pv, B, gq, max_q_len) * a.S;
    if (units <= 0) return hipSuccess;
    a.nblk = int((units + 7) / 8 * 8);
    if (a.S > 1) {
        const size_t cols = pv.D == 256 ? 64 : 128;
        const size_t ml = (size_t(a.nblk) * cols * 2 * sizeof(float) + 255) / 256 * 256;
        a.part_ml = static_cast<float*>(ws);
        a.part_acc = reinterpret_cast<float*>(static_cast<char*>(ws) + ml);
    }
    switch (pv.D) {
        case 64: return launch_gtile_d<64>(a, gq, s);
        case 128: return launch_gtile_d<128>(a, gq, s);
        case 256: return launch_gtile_d<256>(a, gq, s);
    }
    return hipErrorNotSupported;
}

}  // namespace kvs
