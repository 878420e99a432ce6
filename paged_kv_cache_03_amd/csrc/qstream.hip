// qstream.hip -- the matrix-core page stream for quantized pages.
//
// NInfer "Paged KV Context Store" page: the closed KV profiles (code and
// scale planes per side: INT8-G64, FP8-E4M3FN-row256, NVFP4-G16, and K8V4 =
// FP8 K with NVFP4 V), P=64 translation, consumer rules (page-granular reads
// through the block table, no gather-to-contiguous, free choice of
// tile/split/wave/LDS scheme).
//
// It runs the same plan (stream_plan.hip), work split, online softmax, unit
// merge and combine as the BF16 page stream of decode.hip, register-fed the
// same way: wave w of each of two blocks per compute unit loads the codes and
// scales of its 16 keys of every page straight into registers, one page
// ahead, through buffer loads whose range ends at the page's last visible row
// (codes and scales past it read as zeros, so stale bytes never reach the
// products).  What differs is how the codes become matrix-core operands:
//  * every code value is exact in bf16 (int8 in [-127, 127]; e4m3 has 4
//    significant bits; e2m1 2), and so is an e2m1 value times its e4m3 group
//    scale (at most 6 significant bits, inside bf16's exponent range), so
//    NVFP4 sides are dequantized in full before the products;
//  * INT8-G64 and FP8-row scales are fp32 and do not fold into a bf16
//    operand exactly, so they act on fp32 values: K scales multiply each
//    key's per-group partial scores, V scales multiply the key's probability
//    (p * s, split into two bf16 terms like p itself), one copy of P per
//    64-dim scale group;
//  * PV runs V^T . P_hi and V^T . P_lo as two k=16 products per 16-dim tile
//    on the same V^T operand: lane group lg's four keys are exactly the k
//    slots 4lg .. 4lg+3 of a k=16 product;
//  * a V^T operand holds the lane's four keys at the head dim of its tile
//    row; packing the fp32 values of two keys into one bf16 pair is the
//    transpose.  Row m of tile j holds head dim 64(j/4) + 4m + j%4 for
//    INT8-G64 V (a tile stays in one scale group: four bytes per key, group
//    and lane) and (D/16) m + j for the others (one row load per key);
//  * the page's load instructions, more than its bytes, bound the stream:
//    INT8-G64 V codes come as a few 16-byte loads per lane that the wave
//    writes into its own LDS stage and reads back four bytes at a time, and
//    the INT8-G64 / FP8-row scales of a 16-lane row's four keys come as one
//    4-byte load per lane, each scale then broadcast within the row.
//
// With the step's rows (decode that appends): the wave that will load row r
// of a page quantizes the new row that lands there (codec_write.h, the append
// kernel's arithmetic) and stores it before it issues that page's loads.
// Rows 16w .. 16w + 15 of every plane of a page reach the products only
// through wave w's loads, and the vector memory operations of one wave take
// effect in issue order, so the wave's later loads of the page read the new
// row.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "attn_common.h"
#include "codec_write.h"
#include "decode_common.h"
#include "internal.h"
#include "launch.h"
#include "stream_common.h"
#include "stream_plan.h"

namespace kvs {

namespace {

// bytes per page row (one key of one KV head) of a side's code and scale
// planes; SB: bytes of an INT8-G64 / FP8-row scale (4: fp32, 2: binary16)
template <int C, int D, int SB>
struct QRow {
    static constexpr int code = C == CODEC_NVFP4_G16 ? D / 2 : D;
    static constexpr int scale = C == CODEC_INT8_G64 ? SB * (D / 64) : (C == CODEC_FP8_ROW ? SB : D / 16);
};

// word of lane k of this lane's 16-lane row (a row broadcast: one vector
// move; k is a constant once the callers' loops are unrolled)
__device__ __forceinline__ uint32_t row_word(uint32_t v, int k) {
    switch (k & 15) {
        case 0: return __builtin_amdgcn_mov_dpp(v, 0x150, 0xf, 0xf, false);
        case 1: return __builtin_amdgcn_mov_dpp(v, 0x151, 0xf, 0xf, false);
        case 2: return __builtin_amdgcn_mov_dpp(v, 0x152, 0xf, 0xf, false);
        case 3: return __builtin_amdgcn_mov_dpp(v, 0x153, 0xf, 0xf, false);
        case 4: return __builtin_amdgcn_mov_dpp(v, 0x154, 0xf, 0xf, false);
        case 5: return __builtin_amdgcn_mov_dpp(v, 0x155, 0xf, 0xf, false);
        case 6: return __builtin_amdgcn_mov_dpp(v, 0x156, 0xf, 0xf, false);
        case 7: return __builtin_amdgcn_mov_dpp(v, 0x157, 0xf, 0xf, false);
        case 8: return __builtin_amdgcn_mov_dpp(v, 0x158, 0xf, 0xf, false);
        case 9: return __builtin_amdgcn_mov_dpp(v, 0x159, 0xf, 0xf, false);
        case 10: return __builtin_amdgcn_mov_dpp(v, 0x15a, 0xf, 0xf, false);
        case 11: return __builtin_amdgcn_mov_dpp(v, 0x15b, 0xf, 0xf, false);
        case 12: return __builtin_amdgcn_mov_dpp(v, 0x15c, 0xf, 0xf, false);
        case 13: return __builtin_amdgcn_mov_dpp(v, 0x15d, 0xf, 0xf, false);
        case 14: return __builtin_amdgcn_mov_dpp(v, 0x15e, 0xf, 0xf, false);
        default: return __builtin_amdgcn_mov_dpp(v, 0x15f, 0xf, 0xf, false);
    }
}

// scale f (fp32 word f, or binary16 half f widened exactly) of a run of
// scales spread one dword per lane over a 16-lane row
template <int SB>
__device__ __forceinline__ float row_scale(uint32_t v, int f) {
    if constexpr (SB == 4) {
        return __uint_as_float(row_word(v, f));
    } else {
        const uint32_t w = row_word(v, f >> 1);
        return static_cast<float>(__builtin_bit_cast(_Float16, uint16_t((f & 1) ? (w >> 16) : (w & 0xFFFFu))));
    }
}

// Blocks per compute unit: two (two waves per SIMD hide each other's
// latencies; at most 256 registers per lane; three measured slower at
// D = 128), one for INT8-G64 at D = 256 (its registers do not fit twice).
template <int D, int KC>
constexpr int qstream_bpc() { return (D == 256 && KC == CODEC_INT8_G64) ? 1 : 2; }

// Page buffers per wave (PF - 1 pages in flight while one is computed).  A
// third buffer (two pages in flight) measured no faster once the narrow loads
// were gone: the page's load instructions, not the bytes in flight, bound
// these streams.
template <int D, int KC>
constexpr int qstream_buffers() { return 2; }

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

// INT8-G64 V codes through LDS.  A wave's 16 rows of a page (16 x D bytes)
// arrive as D/64 loads of 16 bytes per lane (a few wide loads in place of
// 4 x D/64 four-byte ones: the narrow loads, not the bytes, bound the
// stream); the wave writes them into its own LDS stage and each lane then
// reads the four bytes of every (key, scale group) its PV tiles take.  Chunk
// (row R, 16-byte column k) of the rows sits at slot R' * D/16 + k' of the
// stage (lane l of load c holds slot 64 c + l), permuted so that every such
// read (64 lanes, 16 rows x 4 chunks) hits 64 distinct banks:
//   D = 64:  R' = 4 (R % 4) + R / 4,        k' = k
//   D = 128: R' = 2 (R % 8) + R / 8,        k' = k ^ 4 ((R / 4) % 2)
//   D = 256: R' = R,                        k' = k ^ 4 ((R / 4) % 4)
template <int D>
__device__ __forceinline__ uint32_t vstage_src(int slot) {   // byte offset within the 16 rows of the chunk at slot
    constexpr int VCH = D / 16;
    const int rp = slot / VCH, kp = slot % VCH;
    int R, k;
    if constexpr (D == 64) {
        R = 4 * (rp % 4) + rp / 4;
        k = kp;
    } else if constexpr (D == 128) {
        R = 8 * (rp % 2) + rp / 2;
        k = kp ^ (4 * ((R / 4) % 2));
    } else {
        R = rp;
        k = kp ^ (4 * ((R / 4) % 4));
    }
    return uint32_t(R * D + 16 * k);
}
// NVFP4 V codes through the same kind of stage (D/2-byte rows, 16-byte chunks;
// the D/32 bytes of key 4 lg + r that lane li takes are read at 256 r + a):
//   D = 128: R' = 4 (R % 4) + R / 4                   (4-byte reads)
//   D = 256: R' = 2 (R % 4) + (R / 4) % 2 + 8 (R / 8)   (8-byte reads)
// and each 16-lane row's run of scale rows (16 x D/16 bytes) after the codes.
template <int D>
__device__ __forceinline__ uint32_t fp4_stage_src(int slot) {   // byte offset within the 16 rows of the chunk at slot
    constexpr int VCH = D / 32;                  // 16-byte chunks of a row
    const int rp = slot / VCH, k = slot % VCH;
    int R;
    if constexpr (D == 128) R = 4 * (rp % 4) + rp / 4;
    else R = (rp % 8) / 2 + 4 * (rp % 2) + 8 * (rp / 8);
    return uint32_t(R * (D / 2) + 16 * k);
}
template <int D>
__device__ __forceinline__ uint32_t fp4_stage_dst(int li, int lg) {
    if constexpr (D == 128) return uint32_t(64 * lg + 4 * li);
    else return uint32_t(128 * (lg % 2) + 1024 * (lg / 2) + 8 * li);
}

// byte offset within the stage of the four bytes of key 4 lg + r (r = 0: add
// 256 r for the others), dims 64 g + 4 li .. +3
template <int D>
__device__ __forceinline__ uint32_t vstage_dst(int li, int lg, int g) {
    if constexpr (D == 64) return uint32_t(64 * lg + 4 * li);
    else if constexpr (D == 128) return uint32_t(1024 * (lg % 2) + 128 * (lg / 2) + 64 * (g ^ (lg % 2)) + 4 * li);
    else return uint32_t(1024 * lg + 64 * (g ^ lg) + 4 * li);
}

template <int D, int KC, int VC, int SB>
__global__ void __launch_bounds__(256, (qstream_bpc<D, KC>())) paged_qstream_kernel(DecodeArgs a) {
    using namespace plan;
    constexpr int BPC = qstream_bpc<D, KC>();
    constexpr int PF = qstream_buffers<D, KC>();
    constexpr int NT = 256;
    constexpr int NCH = D / 8;                     // 16-byte chunks of a bf16 query row
    constexpr int NU = D / 64;                     // 64-dim groups: K operand units of 16 dims per lane
    constexpr int NDT = D / 16;                    // PV tiles
    constexpr int NP = NDT / 4;                    // merge passes, four tiles each
    constexpr int NCOL = 16;
    constexpr int QCHUNKS = 1024 / BPC;            // query cache: 16-byte chunks
    constexpr int QSEG = QCHUNKS / (NCOL * NCH);   // units with cached queries
    constexpr int PAGES = kStreamPages / BPC;      // most pages a block takes
    constexpr int KROW = QRow<KC, D, SB>::code, VROW = QRow<VC, D, SB>::code;
    constexpr int KSROW = QRow<KC, D, SB>::scale, VSROW = QRow<VC, D, SB>::scale;
    constexpr bool KI8 = KC == CODEC_INT8_G64, KF8 = KC == CODEC_FP8_ROW, KF4 = KC == CODEC_NVFP4_G16;
    constexpr bool VI8 = VC == CODEC_INT8_G64, VF8 = VC == CODEC_FP8_ROW;
    constexpr int NGK = KI8 ? NU : 1;              // score accumulators: one per K scale group
    constexpr int NPV = VI8 ? NU : 1;              // copies of P: one per V scale group
    constexpr int NKW = KF4 ? 2 : 4;               // K code words per group and lane
    // K scale loads per lane: 16 bytes each (8 for a shorter run of four keys' scales)
    constexpr int NKS4 = KF4 ? (KSROW + 15) / 16 : 1;
    constexpr int NVW = VI8 ? NU : (VF8 ? NDT / 4 : NDT / 8);         // V code words per key and lane
    constexpr int NVS4 = (VI8 || VF8) ? 1 : 0;    // V scale loads per lane, as for K
    // INT8-G64 / FP8-row scales: the four keys of a 16-lane row have at most
    // 16 dwords of scales per side; lane li loads dword li of its row's run
    // and each scale is broadcast from the lane that holds it
    static_assert(KF4 || 4 * KSROW <= 64, "K scales per row");
    static_assert(!(VI8 || VF8) || 4 * VSROW <= 64, "V scales per row");
    static_assert(KC != CODEC_BF16 && VC != CODEC_BF16, "quantized sides only");
    static_assert(D == 64 || D == 128 || D == 256, "shape");
    static_assert(NVW >= 1 && NKS4 >= 1 && (VI8 || VF8 || NVS4 == 0), "register layout");
    static_assert(QSEG >= 1 && QSEG * NCOL * NCH == QCHUNKS && QCHUNKS % NT == 0 && PAGES % NT == 0, "LDS shapes");
    typedef unsigned int vword_t __attribute__((ext_vector_type(NVW)));
    constexpr bool VF4 = !VI8 && !VF8;             // NVFP4 V
    constexpr bool VST = VI8 || VF4;               // V codes through an LDS stage
    constexpr int NVL = VI8 ? D / 64 : (VF4 ? D / 128 : 1);   // 16-byte V code loads per page and lane (staged V)
    constexpr int VCODES = 16 * VROW;              // code bytes of a wave's stage, then NVFP4 scale rows
    constexpr int VSTAGE = VF4 ? VCODES + 256 : VCODES;

    __shared__ int2 pinfo[PAGES];                  // the block's pages: (slice number of (g, h) or -1, meta)
    __shared__ u32x4 qcache[QCHUNKS];              // query rows of the first QSEG units: [unit][column][chunk]
    __shared__ float mbuf[4 * 16 * 64];            // unit merge: four waves x four tiles x 4 registers
    __shared__ float mlbuf[4][16][2];              // per-wave (m, l) of every column at a unit's end
    __shared__ int ent_s[kMaxEnt][kEntWords];
    __shared__ int seg_s[kMaxSeg][kSegWords];
    __shared__ int exp_s[kMaxEnt * kMaxH];         // pieces per (entry, KV head)
    __shared__ __attribute__((aligned(16))) u32x4 vstage[VST ? 4 * VSTAGE / 16 : 1];   // [wave]

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
    const bool append = a.k_new != nullptr;
    const int npatch = append ? ld_uniform(P, off_blk(H) + 4 * size_t(i_blk) + 2) : 0;   // > 0: new rows here
    {
        static_assert(kMaxEnt * kEntWords <= NT && kMaxSeg * kSegWords <= NT && kMaxEnt * kMaxH <= 2 * NT, "tables");
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

    char* kcp = static_cast<char*>(a.pv.lv.k_code);
    char* vcp = static_cast<char*>(a.pv.lv.v_code);
    char* ksp = static_cast<char*>(a.pv.lv.k_scale);
    char* vsp = static_cast<char*>(a.pv.lv.v_scale);

    // the step's rows: the pages of the block's list that hold an entry's new
    // token (position keys - 1) carry kPatchBit; the unit of page f is the
    // block's first unit plus the unit ends before f.  A row goes in before
    // the loads of its page by the wave that owns the row (see the top of the
    // file).  Every wave scans the whole list in the same order, so all number
    // the block's rows alike.  Row j (kRows of them at most) is quantized while
    // the first page is in flight, its K side by wave 2j % 4 and its V side by
    // wave (2j + 1) % 4, and handed over through mbuf (free until the first
    // unit ends); after the prologue's barrier its owner stores it.  A row
    // whose page is among the first PF - 1 pages, and rows past kRows, are
    // written by their owner during the scan.
    constexpr int EPL = D / 64;
    constexpr int kRows = 8;                       // rows handed over through mbuf: 4 x 64 words each
    constexpr int kHeld = kRows / 2;               // sides one wave quantizes
    static_assert(kRows * 4 * 64 <= 4 * 16 * 64, "hand-over space");
    __shared__ long long row_slot[kRows];          // plane row of hand-over row j
    __shared__ int row_owner[kRows];               // and the wave that stores it
    const bool vside = (w & 1) != 0;               // the side this wave quantizes: K (even waves) or V
    int nrows = 0;                                 // rows handed over (the same in every wave)
    int nheld = 0;                                 // this wave's sides to quantize
    int hrow[kHeld];                               // their (entry, KV head) rows of k_new / v_new
    int hidx[kHeld];                               // and their hand-over numbers
#pragma unroll
    for (int j = 0; j < kHeld; ++j) {
        hrow[j] = 0;
        hidx[j] = 0;
    }
    if (append && npatch > 0) {
        // entry keys and segment masks in registers (lane b: entry b, lane s: segment s)
        const int ekeys = lane < a.B ? ent_s[lane][E_KEYS] : 0;
        const int smask = lane < kMaxSeg ? seg_s[lane][S_MASK] : 0;
        int unit0 = sig;                           // unit of page c0
        for (int c0 = 0; c0 < npg; c0 += 64) {
            const int fi = c0 + lane;
            const int2 pi = fi < npg ? pinfo[fi] : make_int2(-1, 0);
            const uint64_t ends = __builtin_amdgcn_ballot_w64((pi.y & 256) != 0);
            uint64_t todo = __builtin_amdgcn_ballot_w64((pi.y & kPatchBit) != 0);
            const int sg_l = unit0 + int(__builtin_popcountll(ends & ((uint64_t(1) << lane) - 1)));
            while (todo) {
                const int k = int(__builtin_ctzll(todo));
                todo &= todo - 1;
                const int sg = __builtin_amdgcn_readlane(sg_l, k), meta = __builtin_amdgcn_readlane(pi.y, k);
                const int sl = __builtin_amdgcn_readlane(pi.x, k);
                const int s = unit_seg(sg), h = sg - s * H, pgi = (meta >> 9) & 0x7fff;
                const int mask = __builtin_amdgcn_readlane(smask, s);
                uint64_t ents = __builtin_amdgcn_ballot_w64(lane < a.B && ((mask >> lane) & 1) && ekeys > 0 &&
                                                            ((ekeys - 1) >> kPageShift) == pgi && sl >= 0);
                while (ents) {
                    const int b = int(__builtin_ctzll(ents));
                    ents &= ents - 1;
                    const int r = (__builtin_amdgcn_readlane(ekeys, b) - 1) & (kPage - 1);
                    const size_t slot = size_t(sl) * kPage + r;
                    if (c0 + k >= PF - 1 && nrows < kRows) {
                        const int j = nrows++;
                        if (((2 * j) & 3) == w && lane == 0) {   // the K side's wave records it
                            row_slot[j] = (long long)slot;
                            row_owner[j] = r >> 4;
                        }
                        if (((2 * j + (vside ? 1 : 0)) & 3) == w) {
#pragma unroll
                            for (int t = 0; t < kHeld; ++t)
                                if (t == nheld) {
                                    hrow[t] = b * H + h;
                                    hidx[t] = j;
                                }
                            ++nheld;
                        }
                        continue;
                    }
                    if ((r >> 4) != w) continue;   // its owner writes it now
                    float kx[EPL], vx[EPL];
                    row_floats<EPL>(load_row_bits<EPL>(a.k_new + (size_t(b) * H + h) * D, lane), kx);
                    row_floats<EPL>(load_row_bits<EPL>(a.v_new + (size_t(b) * H + h) * D, lane), vx);
                    store_side<D, KC, SB>(kcp, ksp, slot, quantize_side<D, KC, SB>(kx, lane), lane);
                    store_side<D, VC, SB>(vcp, vsp, slot, quantize_side<D, VC, SB>(vx, lane), lane);
                }
            }
            unit0 += int(__builtin_popcountll(ends));
        }
        asm volatile("" ::: "memory");             // the page loads stay after these stores
    }
    uint2 hx[kHeld];                               // the sides' bf16 bits
    const uint16_t* const xnew = vside ? a.v_new : a.k_new;
#pragma unroll
    for (int j = 0; j < kHeld; ++j) {
        hx[j] = make_uint2(0u, 0u);
        if (j < nheld) hx[j] = load_row_bits<EPL>(xnew + size_t(hrow[j]) * D, lane);
    }
    uint32_t* const hand = reinterpret_cast<uint32_t*>(mbuf);   // [row][K code, K scale, V code, V scale][lane]
    auto quantize_held = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < kHeld; ++j) {          // fixed indices: the rows stay in registers
            if (j >= nheld) continue;
            float x[EPL];
            row_floats<EPL>(hx[j], x);
            const RowCode rc = vside ? quantize_side<D, VC, SB>(x, lane) : quantize_side<D, KC, SB>(x, lane);
            uint32_t* const o = hand + hidx[j] * 256 + (vside ? 128 : 0) + lane;
            o[0] = rc.code;
            o[64] = rc.scale;
        }
    };
    auto store_owned = [&]() __attribute__((always_inline)) {
#pragma unroll 1
        for (int j = 0; j < nrows; ++j) {
            if (row_owner[j] != w) continue;
            const uint32_t* const o = hand + j * 256 + lane;
            const size_t slot = size_t(row_slot[j]);
            store_side<D, KC, SB>(kcp, ksp, slot, RowCode{o[0], o[64]}, lane);
            store_side<D, VC, SB>(vcp, vsp, slot, RowCode{o[128], o[192]}, lane);
        }
        asm volatile("" ::: "memory");             // the page loads stay after these stores
    };

    // page buffers: this wave's K code units and scales, V code words and
    // scales.  Buffer loads whose range ends at the page's last visible row:
    // codes and scales past it (stale bytes, possibly NaN) come back as zeros.
    //  K operand, group g: key 16w + li, dims 64g + 16lg .. +15
    //  accumulator register r: key tk(r) = 16w + 4lg + r (score row 4lg + r)
    const int kq = 16 * w + li, tk0 = 16 * w + 4 * lg;
    u32x4 kbuf[PF][NU];                            // K units (NVFP4: words 0-1)
    u32x4 ksbuf[KF4 ? PF : 1][NKS4];               // NVFP4 K scales: key kq's row
    uint32_t ksw[PF], vsw[PF];                     // INT8 / FP8 scales: dword li of the row's run
    vword_t vbuf[VST ? 1 : PF][4];                 // V code words of keys tk(r) (not for V through LDS)
    u32x4 vwide[VST ? PF : 1][NVL];                // V codes for the stage: slots 64 c + lane
    uint32_t vsb[VST ? 1 : PF][4];                 // NVFP4 V: the word holding key tk(r)'s scale byte (unstaged)
    uint32_t vscw[VF4 ? PF : 1];                   // NVFP4 V, staged: dword lane of the wave's scale rows
    int pmeta[PF];
    int vsrc[NVL];                                 // this lane's source offsets of the stage's chunks
#pragma unroll
    for (int c = 0; c < NVL; ++c)
        vsrc[c] = int(16 * w * VROW + (VI8 ? vstage_src<D>(64 * c + lane) : fp4_stage_src<D>(64 * c + lane)));
    auto load_page = [&](int fi, int J) __attribute__((always_inline)) {
        const bool live = fi < npg;
        const int2 pi = pinfo[live ? fi : 0];
        const int sl = live ? __builtin_amdgcn_readfirstlane(pi.x) : -1;
        pmeta[J] = live ? __builtin_amdgcn_readfirstlane(pi.y) | (fi == npg - 1 ? 256 : 0) : 0;
        const int rows = sl < 0 ? 0 : (pmeta[J] & 255);   // an unmapped block reads nothing
        const size_t s0 = size_t(sl < 0 ? 0 : sl) * 64;
        const __amdgpu_buffer_rsrc_t rkc = __builtin_amdgcn_make_buffer_rsrc(kcp + s0 * KROW, 0, rows * KROW, kBufferWord3);
        // the range check of a buffer load works on whole dwords: 2-byte scale
        // rows round their range up to one (the key past the last visible row
        // that this lets through is zeroed where the scales are used)
        const int ksr = SB == 2 && !KF4 ? (rows * KSROW + 3) & ~3 : rows * KSROW;
        const int vsr = SB == 2 && (VI8 || VF8) ? (rows * VSROW + 3) & ~3 : rows * VSROW;
        const __amdgpu_buffer_rsrc_t rks = __builtin_amdgcn_make_buffer_rsrc(ksp + s0 * KSROW, 0, ksr, kBufferWord3);
        const __amdgpu_buffer_rsrc_t rvc = __builtin_amdgcn_make_buffer_rsrc(vcp + s0 * VROW, 0, rows * VROW, kBufferWord3);
        const __amdgpu_buffer_rsrc_t rvs = __builtin_amdgcn_make_buffer_rsrc(vsp + s0 * VSROW, 0, vsr, kBufferWord3);
#pragma unroll
        for (int g = 0; g < NU; ++g) {
            if constexpr (KF4) {
                const u32x2 x = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rkc, kq * KROW + 32 * g + 8 * lg, 0, kNonTemporal));
                kbuf[J][g] = u32x4{x[0], x[1], 0u, 0u};
            } else {
                kbuf[J][g] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rkc, kq * KROW + 64 * g + 16 * lg, 0, kNonTemporal));
            }
        }
#pragma unroll
        for (int k = 0; k < NKS4; ++k) {
            if constexpr (KF4) {
                if constexpr (KSROW == 8) {
                    const u32x2 x = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rks, kq * KSROW, 0, kNonTemporal));
                    ksbuf[J][k] = u32x4{x[0], x[1], 0u, 0u};
                } else {
                    ksbuf[J][k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rks, kq * KSROW + 16 * k, 0, kNonTemporal));
                }
            } else {
                ksw[J] = __builtin_amdgcn_raw_buffer_load_b32(rks, tk0 * KSROW + 4 * li, 0, kNonTemporal);
            }
        }
        if constexpr (VST) {
#pragma unroll
            for (int c = 0; c < NVL; ++c)
                vwide[J][c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rvc, vsrc[c], 0, kNonTemporal));
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = tk0 + r;
            if constexpr (VST) {
                (void)t;
            } else if constexpr (NVW == 4) {
                vbuf[J][r] = __builtin_bit_cast(vword_t, __builtin_amdgcn_raw_buffer_load_b128(rvc, t * VROW + 16 * li, 0, kNonTemporal));
            } else if constexpr (NVW == 2) {
                vbuf[J][r] = __builtin_bit_cast(vword_t, __builtin_amdgcn_raw_buffer_load_b64(rvc, t * VROW + 8 * li, 0, kNonTemporal));
            } else {
                vbuf[J][r] = __builtin_bit_cast(vword_t, __builtin_amdgcn_raw_buffer_load_b32(rvc, t * VROW + 4 * li, 0, kNonTemporal));
            }
            if constexpr (VF4 && !VST)             // NVFP4: the aligned word holding byte (D/16) li / 16 of the row
                vsb[J][r] = __builtin_amdgcn_raw_buffer_load_b32(rvs, t * VSROW + (((NDT * li) / 16) & ~3), 0, kNonTemporal);
        }
        if constexpr (VI8 || VF8) vsw[J] = __builtin_amdgcn_raw_buffer_load_b32(rvs, tk0 * VSROW + 4 * li, 0, kNonTemporal);
        if constexpr (VF4 && VST) vscw[J] = __builtin_amdgcn_raw_buffer_load_b32(rvs, 16 * w * VSROW + 4 * lane, 0, kNonTemporal);
    };

    // query rows of the first QSEG units (columns past a unit's last read
    // row 0 of the call; they are never used): loads first, then the first
    // page, then the LDS writes
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
    for (int k = 0; k < PF - 1; ++k) load_page(k, k);
    if (nheld > 0) quantize_held();
#pragma unroll
    for (int k = 0; k < QCHUNKS / NT; ++k) qcache[k * NT + tid] = qv[k];
    block_lds_barrier();
    if (nrows > 0) store_owned();

    typedef const u32x4 __attribute__((address_space(1)))* glb_q_cptr;
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
            const glb_q_cptr qg = (glb_q_cptr)(q_row(cl, h));
#pragma unroll
            for (int c = 0; c < D / 32; ++c) {
                const u32x4 v = qg[8 * (c >> 1) + 2 * lg + (c & 1)];
                qb[c] = __builtin_bit_cast(bf16x8_t, li < ncol ? v : u32x4{0u, 0u, 0u, 0u});
            }
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

    // unit end: merge the four waves' states through mbuf, four tiles per
    // pass; wave w folds accumulator register w, so each lane ends with four
    // consecutive head dims of row 4lg + w of each pass
    auto finish_unit = [&]() __attribute__((always_inline)) {
        const float lw = rows_sum(l_part);
        f32x4_t merged[NP];
        float cw[4], lt = 0.f, mx = -INFINITY;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            block_lds_barrier();                   // every wave read the previous pass
            float* mine = mbuf + w * 1024;
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
                for (int v = 0; v < 4; ++v) x += mbuf[v * 1024 + (jj * 4 + w) * 64 + lane] * cw[v];
                merged[p][jj] = x;
            }
        }
        // write (not waited for: the combine is a later launch); a column
        // whose (entry, KV head) has no other piece is normalized into out,
        // the others go to slot i + sigma
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

    // one page of this wave's keys from buffer set J
    auto compute = [&](auto jc) __attribute__((always_inline)) {
        constexpr int J = decltype(jc)::value;
        const int meta = pmeta[J];
        // rows any column of the unit may see; a wave whose keys all lie past
        // them still runs the page (its codes read as zeros and its scores are
        // masked, so it adds exact zeros): a skipped page would leave its
        // loads pending on one path into the ring, and the compiler's waits
        // after the merge would then cover the next page's loads as well
        const int lim = meta & 255;
        const int tok0 = ((meta >> 9) & 0x7fff) * kPage;
        if constexpr (VST) {                       // the page's V codes into this wave's stage
            typedef u32x4 __attribute__((address_space(3)))* lds_u32x4_ptr;
            const lds_u32x4_ptr sw = (lds_u32x4_ptr)(&vstage[0]) + w * (VSTAGE / 16);
#pragma unroll
            for (int c = 0; c < NVL; ++c) sw[64 * c + lane] = vwide[J][c];
            if constexpr (VF4) {
                typedef uint32_t __attribute__((address_space(3)))* lds_u32_ptr;
                ((lds_u32_ptr)(sw + VCODES / 16))[lane] = vscw[J];
            }
        }

        // QK^T: S^T[16 keys x 16 columns], per K scale group for INT8
        f32x4_t sacc[NGK];
#pragma unroll
        for (int g = 0; g < NGK; ++g) sacc[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int g = 0; g < NU; ++g) {
            const u32x4 x = kbuf[J][g];
            u32x4 op0, op1;
            if constexpr (KF4) {
                const uint32_t sw = ksbuf[J][0][(4 * g + lg) >> 2];
                const float sc = e4m3_f32(sw >> (8 * ((4 * g + lg) & 3)));
                uint32_t o[8];
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const f32x2_t f0 = fp4_pair(x[0], b);
                    const f32x2_t f1 = fp4_pair(x[1], b);
                    o[b] = pk_bf16(f0[0] * sc, f0[1] * sc);
                    o[4 + b] = pk_bf16(f1[0] * sc, f1[1] * sc);
                }
                op0 = u32x4{o[0], o[1], o[2], o[3]};
                op1 = u32x4{o[4], o[5], o[6], o[7]};
            } else if constexpr (KI8) {
                op0 = u32x4{pk_bf16(i8f<0>(x[0]), i8f<1>(x[0])), pk_bf16(i8f<2>(x[0]), i8f<3>(x[0])),
                            pk_bf16(i8f<0>(x[1]), i8f<1>(x[1])), pk_bf16(i8f<2>(x[1]), i8f<3>(x[1]))};
                op1 = u32x4{pk_bf16(i8f<0>(x[2]), i8f<1>(x[2])), pk_bf16(i8f<2>(x[2]), i8f<3>(x[2])),
                            pk_bf16(i8f<0>(x[3]), i8f<1>(x[3])), pk_bf16(i8f<2>(x[3]), i8f<3>(x[3]))};
            } else {
                uint32_t o[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    o[2 * e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[e], 1.0f, false));
                    o[2 * e + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[e], 1.0f, true));
                }
                op0 = u32x4{o[0], o[1], o[2], o[3]};
                op1 = u32x4{o[4], o[5], o[6], o[7]};
            }
            const int ga = KI8 ? g : 0;
            sacc[ga] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, op0), qb[2 * g], sacc[ga], 0, 0, 0);
            sacc[ga] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, op1), qb[2 * g + 1], sacc[ga], 0, 0, 0);
        }
        // K scales of key tk(r): float r*NU + g (INT8) or r (FP8) of the loaded run
        // (2-byte scales: a key at or past the page's last visible row counts 0)
        auto kscale = [&](int r, int g) __attribute__((always_inline)) {
            const float sc = row_scale<SB>(ksw[J], KI8 ? r * NU + g : r);
            return SB == 2 && tk0 + r >= lim ? 0.f : sc;
        };
        float sj[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if constexpr (KI8) {
                float x = 0.f;
#pragma unroll
                for (int g = 0; g < NU; ++g) x += sacc[g][r] * kscale(r, g);
                sj[r] = x * a.scale_log2;
            } else if constexpr (KF8) {
                sj[r] = sacc[0][r] * kscale(r, 0) * a.scale_log2;
            } else {
                sj[r] = sacc[0][r] * a.scale_log2;
            }
        }
        if (tok0 + kPage > kmin) {                 // a real column's limit falls inside the page
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (tok0 + tk0 + r >= klim) sj[r] = -INFINITY;
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

        // P^T operands [P_hi; P_lo], one per V scale group (keys past the
        // last limit have zero codes and scales from the buffer range)
        auto vscale = [&](int r, int g) __attribute__((always_inline)) {
            const float sc = row_scale<SB>(vsw[J], VI8 ? r * NU + g : r);
            return SB == 2 && tk0 + r >= lim ? 0.f : sc;
        };
        s16x4_t bhi[NPV], blo[NPV];
#pragma unroll
        for (int g = 0; g < NPV; ++g) {
            float pv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) pv[r] = (VI8 || VF8) ? p[r] * vscale(r, g) : p[r];
            uint32_t h01, l01, h23, l23;
            split_bf16(pv[0], pv[1], h01, l01);
            split_bf16(pv[2], pv[3], h23, l23);
            bhi[g] = __builtin_bit_cast(s16x4_t, u32x2{h01, h23});
            blo[g] = __builtin_bit_cast(s16x4_t, u32x2{l01, l23});
        }

        // INT8-G64 V: the value products and their operands at raised wave
        // priority (config 3 kernel 0.8% faster in two A/B pairs on one box;
        // K8V4 0.8% slower, and the score loop at raised priority slower for
        // both, so those keep the default)
        if constexpr (VI8) __builtin_amdgcn_s_setprio(1);
        // PV: O^T[16 dims x 16 columns] += V^T . P_hi^T + V^T . P_lo^T per tile
        auto pv_tile = [&](int dt, uint32_t x01, uint32_t x23, int g) __attribute__((always_inline)) {
            const s16x4_t vt = __builtin_bit_cast(s16x4_t, u32x2{x01, x23});
            acc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, bhi[g], acc[dt], 0, 0, 0);
            acc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, blo[g], acc[dt], 0, 0, 0);
        };
        if constexpr (VI8) {                       // INT8-G64 V: four bytes per key, group and lane from the stage
            typedef const uint32_t __attribute__((address_space(3)))* lds_u32_cptr;
            const lds_u32_cptr st = (lds_u32_cptr)(&vstage[0]) + w * (VSTAGE / 4);
#pragma unroll
            for (int g = 0; g < NU; ++g) {
                const lds_u32_cptr sg = st + vstage_dst<D>(li, lg, g) / 4;
                const uint32_t x0 = sg[0], x1 = sg[64], x2 = sg[128], x3 = sg[192];
                pv_tile(4 * g + 0, pk_bf16(i8f<0>(x0), i8f<0>(x1)), pk_bf16(i8f<0>(x2), i8f<0>(x3)), g);
                pv_tile(4 * g + 1, pk_bf16(i8f<1>(x0), i8f<1>(x1)), pk_bf16(i8f<1>(x2), i8f<1>(x3)), g);
                pv_tile(4 * g + 2, pk_bf16(i8f<2>(x0), i8f<2>(x1)), pk_bf16(i8f<2>(x2), i8f<2>(x3)), g);
                pv_tile(4 * g + 3, pk_bf16(i8f<3>(x0), i8f<3>(x1)), pk_bf16(i8f<3>(x2), i8f<3>(x3)), g);
            }
        } else {
            float sc[4];
            vword_t vrow[4];                       // the lane's code words of keys tk(r)
            if constexpr (VF4) {
                typedef const vword_t __attribute__((address_space(3)))* lds_vword_cptr;
                typedef const uint8_t __attribute__((address_space(3)))* lds_u8_cptr;
                typedef const char __attribute__((address_space(3)))* lds_byte_cptr;
                const lds_byte_cptr sb = (lds_byte_cptr)(&vstage[0]) + w * VSTAGE;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    vrow[r] = *(lds_vword_cptr)(sb + fp4_stage_dst<D>(li, lg) + 256 * r);
                    sc[r] = e4m3_f32(*(lds_u8_cptr)(sb + VCODES + (tk0 - 16 * w + r) * VSROW + (NDT * li) / 16));
                }
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) vrow[r] = vbuf[J][r];
            }
            // two tiles per step: dims 2q and 2q + 1 of the lane's run
#pragma unroll
            for (int q = 0; q < NDT / 2; ++q) {
                f32x2_t f[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if constexpr (VF8) {
                        f[r] = fp8_pair(vrow[r][q / 2], q & 1);
                    } else {
                        f[r] = fp4_pair(vrow[r][q / 4], q & 3);
                        f[r] = f[r] * sc[r];
                    }
                }
                pv_tile(2 * q, pk_bf16(f[0][0], f[1][0]), pk_bf16(f[2][0], f[3][0]), 0);
                pv_tile(2 * q + 1, pk_bf16(f[0][1], f[1][1]), pk_bf16(f[2][1], f[3][1]), 0);
            }
        }
        if constexpr (VI8) __builtin_amdgcn_s_setprio(0);
    };

    reset();
    int unit_k = 0;
    start_unit(unit_k, sig);
    // page i from buffer set J, the next PF - 1 pages in flight in the others;
    // every step issues the same loads (empty ranges past the block's last
    // page), so the compiler's vector-memory waits stay exact
    auto step = [&](auto jc, int i) __attribute__((always_inline)) {
        constexpr int J = decltype(jc)::value;
        const int meta = pmeta[J];
        load_page(i + PF - 1, (J + PF - 1) % PF);
        compute(jc);
        if (meta & 256) {
            finish_unit();
            if (i + 1 < npg) {
                ++sig;
                ++unit_k;
                start_unit(unit_k, sig);
            }
        }
    };
    ring_run<PF>(step, npg);
}

template <int D, int KC, int VC>
hipError_t launch_one(const DecodeArgs& a, int gq, hipStream_t s) {
    constexpr bool wide = KC == CODEC_INT8_G64 || KC == CODEC_FP8_ROW || VC == CODEC_INT8_G64 || VC == CODEC_FP8_ROW;
    bool launched = false;
    hipError_t e = hipSuccess;
    if constexpr (wide) {
        if (a.pv.scale16) {
            e = launch_kernel(true, paged_qstream_kernel<D, KC, VC, 2>, dim3(static_cast<unsigned>(a.G)), dim3(256), s,
                              a);
            launched = true;
        }
    }
    if (!launched)
        e = launch_kernel(true, paged_qstream_kernel<D, KC, VC, 4>, dim3(static_cast<unsigned>(a.G)), dim3(256), s, a);
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

int qstream_blocks_per_cu(const PoolView& pv) {
    if (pv.D <= 128) return qstream_bpc<128, CODEC_FP8_ROW>();
    return pv.k_codec == CODEC_INT8_G64 ? qstream_bpc<256, CODEC_INT8_G64>() : qstream_bpc<256, CODEC_FP8_ROW>();
}

hipError_t launch_qstream(const DecodeArgs& a, int gq, hipStream_t s) {
    switch (a.pv.D) {
        case 64: return launch_d<64>(a, gq, s);
        case 128: return launch_d<128>(a, gq, s);
        case 256: return launch_d<256>(a, gq, s);
    }
    return hipErrorNotSupported;
}

}  // namespace kvs
