// decode_common.h -- what the decode kernels of decode.hip and qstream.hip
// share: the launch arguments, the plan's entry table accessor and the
// combine of the page stream.  Private to the library; the kernels sit in an
// unnamed namespace, so every translation unit that launches one has its own
// instance.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "attn_common.h"
#include "internal.h"
#include "stream_common.h"
#include "stream_plan.h"

namespace kvs {

struct DecodeArgs {
    PoolView pv;
    const int32_t* plan;   // the call's plan (stream_plan.h): entry table, page list
    int32_t qcap;          // page slots per block in the plan's page list
    int32_t G;             // blocks of the page stream
    int32_t cgroups;       // combine: waves per task (groups of 512 outputs)
    const uint16_t* q;
    const uint16_t* k_new;  // decode with the step's rows: bf16 [B][H][D] K and V appended at keys - 1
    const uint16_t* v_new;  // (nullptr: the rows are already in the planes)
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

// Entry table of the call's plan (row, keys, ...), read by every kernel of
// the decode launch.
__device__ __forceinline__ int plan_ent(const DecodeArgs& a, int b, int field) {
    return a.plan[plan::kOffEnt + b * plan::kEntWords + field];
}

// pages [i0, i0 + NS) of a ring of NS stages or buffers, stage J for page
// i0 + J, while they exist (J is a compile-time constant in step)
template <int J, int NS, class F>
__device__ __forceinline__ void ring_round(F& step, int i0, int npg) {
    if constexpr (J < NS) {
        if (i0 + J < npg) {
            step(std::integral_constant<int, J>{}, i0 + J);
            ring_round<J + 1, NS>(step, i0, npg);
        }
    }
}

// pages [0, npg) through a ring of NS buffers: whole rounds in a loop, then
// the last npg % NS pages after it.  A loop whose rounds may end early has a
// path from a partial round back into the next one, along which the
// compiler's vector-memory waits must also cover loads issued one stage
// later: they would hold back the ring's deepest prefetch on every round.
template <int NS, class F>
__device__ __forceinline__ void ring_run(F& step, int npg) {
    int i0 = 0;
    for (; i0 + NS <= npg; i0 += NS) ring_round<0, NS>(step, i0, i0 + NS);
    ring_round<0, NS>(step, i0, npg);
}

// The BF16 register-fed page stream: blocks of four waves per compute unit,
// and page buffers per wave (buffers - 1 pages in flight while one is
// computed).  At D = 256 a wave's page is twice the bytes and registers, so
// one block per compute unit keeps two pages in flight per wave instead.
constexpr int vstream_bpc(int D) { return D == 256 ? 1 : 2; }
constexpr int vstream_buffers(int D) { return D == 256 ? 3 : 2; }

// single-wave combine blocks per task: groups of 128 outputs of up to ncol columns
constexpr int combine_groups(int ncol, int D) { return (ncol * D + 127) / 128; }

namespace {


// Combine of the page stream: one single-wave block per task of the plan --
// an (entry, KV head) whose outputs have more than one piece -- and group of
// kCombineOut of its outputs, so the partial reads spread over every compute
// unit.  The task lists its pieces (the (block, unit) partials of the entry's
// units in segment order, each unit's slots in block order): a fixed order,
// so the result does not depend on timing.  Every lane folds two consecutive
// outputs of one column over all pieces in as few memory rounds as the
// record allows: the task record and its first CMAX piece ids are read with
// scalar loads in the same round trip as the header, and the record's other
// inline ids (one per lane) with a vector load beside them.  A task of at
// most CMAX pieces (the longest (entry, head) of a 32K-token batch has about
// 20) takes one round of CMAX; one of up to kTaskInline pieces (a 64K-token
// entry over fewer heads spans 33-40 blocks) one round of kTaskInline; longer
// lists continue from the overflow list.
constexpr int kCombineOut = 128;

template <int D, int GQ, int NCOL>
__global__ void __launch_bounds__(64) stream_combine_kernel(DecodeArgs a) {
    using namespace plan;
    constexpr int CMAX = 32;
    const int lane = int(threadIdx.x) & 63;
    const int H = a.pv.H;
    const int tg = int(blockIdx.x);
    const int t = tg / a.cgroups, grp = tg - t * a.cgroups;   // task, its group of outputs
    const int32_t* P = a.plan;
    const int32_t* rec = P + off_tasks(H, int(a.G)) + size_t(t) * kTaskWords;
    // header and task record together (no branch between the loads)
    const int magic = ld_uniform(P, H_MAGIC), pb = ld_uniform(P, H_B), ph = ld_uniform(P, H_H);
    const int pgq = ld_uniform(P, H_GQ), ntask = ld_uniform(P, H_NTASK);
    const int E = ld_uniform(rec, T_E), ncolb = ld_uniform(rec, T_NCOL), obase = ld_uniform(rec, T_OUT);
    const int poff = ld_uniform(rec, T_POFF);
    int sp[CMAX];                                  // the first CMAX piece ids, in the same round trip
#pragma unroll
    for (int kk = 0; kk < CMAX; ++kk) sp[kk] = ld_uniform(rec, T_PIECE + kk);
    constexpr int CV = kTaskInline - CMAX;         // the record's other inline ids: lane k holds piece CMAX + k
    static_assert(CV > 0 && CV <= 64, "inline piece ids");
    int pid2 = rec[T_PIECE + CMAX + min(lane, CV - 1)];
    const bool run = (magic == kMagic) & (pb == a.B) & (ph == H) & (pgq == GQ) & (t < ntask) &
                     (grp * kCombineOut < ncolb * D);
    // the piece ids and the partial and output pointers are needed only past
    // the return below; the compiler would issue their loads there, one more
    // round trip: these uses keep every scalar load above in one
#pragma unroll
    for (int kk = 0; kk < CMAX; ++kk) asm volatile("" ::"s"(sp[kk]));
    asm volatile("" ::"s"(a.part_ml), "s"(a.part_acc), "s"(a.out));
    asm volatile("" : "+v"(pid2));
    if (!run) return;                              // (a plan of another shape: the stream marked the outputs)
    const int32_t* over_list = P + off_over(H, int(a.G));

    // this wave's group of outputs; uniform trip counts: every lane takes
    // part in the readlane lookups
    const int e0 = grp * kCombineOut + lane * 2;
    const bool act = e0 < ncolb * D;
    const int c = act ? e0 / D : 0, d0 = act ? e0 % D : 0;
    float fm = -INFINITY, fl = 0.f, fa0 = 0.f, fa1 = 0.f;
    // one memory round of N pieces (ids from pid_of; pieces from nvalid on
    // repeat a valid one and get weight 0): every load in flight together,
    // then the fold in piece order
    auto round = [&](auto n_c, auto pid_of, int nvalid) __attribute__((always_inline)) {
        constexpr int N = decltype(n_c)::value;
        float2 ml[N], av[N];
#pragma unroll
        for (int kk = 0; kk < N; ++kk) {
            const size_t it = size_t(pid_of(kk)) + c;
            ml[kk] = *reinterpret_cast<const float2*>(a.part_ml + it * 2);
            av[kk] = *reinterpret_cast<const float2*>(a.part_acc + it * D + d0);
        }
        // keep every load of the round above the fold (the scheduler would
        // otherwise sink each one to its use, one round trip each)
        __builtin_amdgcn_sched_barrier(0);
        float mx = fm;
#pragma unroll
        for (int kk = 0; kk < N; ++kk) mx = fmaxf(mx, ml[kk].x);   // repeats change nothing
        const float wp = fm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(fm - mx);
        fl *= wp;
        fa0 *= wp;
        fa1 *= wp;
#pragma unroll
        for (int kk = 0; kk < N; ++kk) {
            const float wgt = (kk >= nvalid || ml[kk].x == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ml[kk].x - mx);
            fl += ml[kk].y * wgt;
            fa0 += av[kk].x * wgt;
            fa1 += av[kk].y * wgt;
        }
        fm = mx;
    };
    int w_rest;                                    // first piece past the first round
    if (E <= CMAX) {                               // the scalar ids
        round(std::integral_constant<int, CMAX>{},
              [&](int kk) __attribute__((always_inline)) { return kk < E ? sp[kk] : sp[0]; }, E);
        w_rest = CMAX;
    } else {                                       // the scalar ids, then the lanes' inline ids
        const int nv = min(E, kTaskInline);
        round(std::integral_constant<int, kTaskInline>{},
              [&](int kk) __attribute__((always_inline)) {
                  return kk < CMAX ? sp[kk] : __builtin_amdgcn_readlane(pid2, min(kk - CMAX, nv - CMAX - 1));
              }, nv);
        w_rest = kTaskInline;
    }
    // the rest: lane k holds the id of piece w0 + k
#pragma unroll 1
    for (int w0 = w_rest; w0 < E; w0 += 64) {
        const int k = w0 + lane;
        int pid = 0;
        if (k < E) pid = k < kTaskInline ? rec[T_PIECE + k] : over_list[poff + k - kTaskInline];
        const int wn = min(64, E - w0);
#pragma unroll 1
        for (int k0 = 0; k0 < wn; k0 += CMAX)
            round(std::integral_constant<int, CMAX>{}, [&](int kk) __attribute__((always_inline)) {
                return __builtin_amdgcn_readlane(pid, min(k0 + kk, wn - 1));
            }, wn - k0);
    }
    if (act) {
        const float inv = fl > 0.f ? 1.f / fl : 0.f;
        float* o = a.out + obase + size_t(c / GQ) * a.Hq * D + size_t(c % GQ) * D + d0;
        *reinterpret_cast<float2*>(o) = make_float2(fa0 * inv, fa1 * inv);
    }
}

}  // namespace

// The matrix-core page stream for quantized pages (qstream.hip): profiles,
// head sizes and shapes it covers, and its launch (the stream kernel, then
// the combine).
bool qstream_path(const PoolView& pv, int B, int gq);
int qstream_blocks_per_cu(const PoolView& pv);   // its grid: this many blocks per compute unit
hipError_t launch_qstream(const DecodeArgs& a, int gq, hipStream_t s);

}  // namespace kvs
