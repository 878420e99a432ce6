// stream_plan.hip -- builds the page-stream plan of one batch state (layout
// and structure in stream_plan.h).
//
// NInfer "Paged KV Context Store" page: PagedKVBatchLayerView (table_rows[b]
// selects the block-table row of entry b), P=64 translation, fork and tail
// copy-on-write (a fork shares its parent's leading pages), consumer rules
// (the op chooses its own split; pages are read in place through the table).
//
// Every block of the launch derives the same entry, sharing and segment
// tables (one lane per entry of wave 0), then does one job: block k < nspan
// writes its share of the page list (stream positions [k * kPlanSpan,
// (k + 1) * kPlanSpan)); the blocks after them write, in parallel, the
// header, tables and piece counts; the combine tasks with their piece lists
// (kTaskBlocks blocks, every kTaskBlocks-th task each); the new-token lists
// and the per-block ranges.  Shared runs
// are found by comparing table entries, so a plan is exact for any table: two
// entries read a page once only where both rows hold the same mapped page
// group.  The kernel reads only its inputs from global memory and never reads
// back what it writes, so its barriers order LDS traffic only (they do not
// wait for the plan's stores to land).

#include <hip/hip_runtime.h>

#include <climits>

#include "attn_common.h"
#include "internal.h"
#include "stream_plan.h"

namespace kvs {
namespace {

using namespace plan;

constexpr int kPlanSpan = 1024;   // stream positions per plan block
constexpr int kMaxStreamBlocks = 4096;
constexpr int kNT = 256;
constexpr int kTaskBlocks = 4;    // blocks that write the combine tasks

struct PlanArgs {
    const int32_t* table;   // [C][L]
    int32_t L, C, M, H;
    int32_t sg, sh;           // slice number of (g, h): g * sg + h * sh
    const int32_t* table_rows;
    const int32_t* seq_lens;  // decode
    const int32_t* q_pos0;    // chunk mode
    const int32_t* cu_q;      // chunk mode
    int32_t B, gq, max_ctx, max_cols, G, qcap, chunk, emax, pages;
    int32_t D, ncol;          // head dim, partial slot width (columns)
    int32_t nspan;            // blocks that write the page list
    int32_t share;            // per mille of the stream positions blocks [0, G/2) take (500: an even split)
    int32_t* plan;
};

// floor(x / q) for 0 <= x < 2^24 and 0 < q < 2^24 through the fp32
// reciprocal, corrected to the exact quotient (an integer division is a long
// instruction sequence on these parts)
struct Div {
    int q;
    float rq;
    __device__ __forceinline__ explicit Div(int q_) : q(q_ > 0 ? q_ : 1), rq(1.0f / float(q_ > 0 ? q_ : 1)) {}
    __device__ __forceinline__ int operator()(int x) const {
        int d = int(float(x) * rq);
        d -= (d * q > x) ? 1 : 0;
        d += ((d + 1) * q <= x) ? 1 : 0;
        return d;
    }
};

// The stream's positions over the blocks.  An even split gives every block
// ceil(total / G) positions.  Otherwise blocks [0, na), na = G / 2, take qa
// positions each (share per mille of the stream between them) and the others
// qb; paged_attn_workspace_bytes sizes the page list for the larger of the two.
struct Split {
    int na, qa, qb, ua;                            // ua: positions of blocks [0, na)
    Div da, db;
    __device__ __forceinline__ Split(int total, int G, int share) : na(0), qa(0), qb(0), ua(0), da(1), db(1) {
        na = (share != 500 && G >= 2) ? G / 2 : 0;
        qa = na > 0 ? int((static_cast<long long>(total) * share + 1000LL * na - 1) / (1000LL * na)) : 0;
        ua = min(total, na * qa);
        qb = G - na > 0 ? (total - ua + (G - na) - 1) / (G - na) : 0;
        da = Div(qa);
        db = Div(qb);
    }
    __device__ __forceinline__ int block(int u) const { return u < ua ? da(u) : na + db(u - ua); }
    __device__ __forceinline__ int start(int i) const { return i < na ? i * qa : ua + (i - na) * qb; }
    __device__ __forceinline__ int count(int i, int total) const {
        return max(0, min(i < na ? qa : qb, total - start(i)));
    }
};

// Inclusive prefix sum over lanes [0, n) of a wave (NL = 8 or 64; every lane
// of the wave active): shifts within 16-lane rows (data-parallel moves, no
// LDS round trip), then the rows' totals.  Lanes past n hold sums nothing reads.
template <int NL>
__device__ __forceinline__ int wave_scan(int v) {
    static_assert(NL == 8 || NL == 64, "scan width");
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
    if constexpr (NL == 64) {
        v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
        const int lane = int(__lane_id());
        const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31);
        const int r2 = __builtin_amdgcn_readlane(v, 47);
        v += (lane >= 16 ? r0 : 0) + (lane >= 32 ? r1 : 0) + (lane >= 48 ? r2 : 0);
    }
    return v;
}

// blocks that stream positions [start, start + n) touch
__device__ __forceinline__ int pieces(int start, int n, const Split& sp) {
    return n > 0 ? sp.block(start + n - 1) - sp.block(start) + 1 : 0;
}

__global__ void __launch_bounds__(kNT) stream_plan_kernel(PlanArgs a) {
    __shared__ int ent[kMaxEnt][kEntWords];
    __shared__ int lcp[kMaxEnt][kMaxEnt];          // [i][j], j < i: leading pages rows i and j share
    __shared__ int cand[kMaxEnt * kMaxEnt];        // pairs still to scan (i << 3 | j)
    __shared__ int cpre[kMaxEnt * kMaxEnt + 1];    // scan positions before each pair
    __shared__ int ncand_s;
    __shared__ int clo[kMaxEnt][kMaxEnt], chi[kMaxEnt][kMaxEnt];   // [b][o]: pages of owner o carrying b
    __shared__ int seg[kMaxSeg][kSegWords];
    __shared__ int res_s[3];                       // segments, zero mask, total
    __shared__ int ex[kMaxEnt * kMaxH];            // pieces per (entry, KV head)
    __shared__ int pcnt[kMaxStreamBlocks];         // new-token pages per block

    const int tid = int(threadIdx.x);
    const int H = a.H;

    if (tid < kMaxEnt) {
        const int b = tid;
        int row = -1, keys = 0, n0 = 0, cu = 0, T = 0, owned = 0;
        if (b < a.B) {
            row = a.table_rows[b];
            const bool ok = row >= 0 && row < a.C;
            if (!a.chunk) {
                keys = ok ? max(0, min(a.seq_lens[b], a.max_ctx)) : 0;
                n0 = keys - 1;
                cu = b;
                T = 1;
                owned = 1;
            } else {
                cu = a.cu_q[b];
                T = a.cu_q[b + 1] - cu;
                n0 = a.q_pos0[b];
                keys = ok ? max(0, min(n0 + T, a.max_ctx)) : 0;
                owned = T * a.gq <= a.max_cols ? 1 : 0;
            }
        }
        ent[b][E_ROW] = row;
        ent[b][E_KEYS] = keys;
        ent[b][E_N0] = n0;
        ent[b][E_CU] = cu;
        ent[b][E_T] = T;
        ent[b][E_NPAGES] = (owned && T > 0) ? (keys + kPage - 1) >> kPageShift : 0;
        ent[b][E_OWNED] = owned;
        ent[b][7] = 0;
    }
    block_lds_barrier();

    // shared leading runs: pairs whose first pages agree are compared page by
    // page; the first mismatch (or unmapped page) ends the run
    if (a.emax > 1) {
        if (tid < kMaxEnt * kMaxEnt) {
            const int i = tid >> 3, j = tid & 7;
            int v = 0;
            if (j < i && ent[i][E_NPAGES] > 0 && ent[j][E_NPAGES] > 0) {
                const int gi = a.table[size_t(ent[i][E_ROW]) * a.L], gj = a.table[size_t(ent[j][E_ROW]) * a.L];
                if (gi == gj && gi >= 0 && gi < a.M) v = min(ent[i][E_NPAGES], ent[j][E_NPAGES]);
            }
            lcp[i][j] = v;
        }
        block_lds_barrier();
        if (tid < 64) {                            // wave 0, lane i*8 + j: pair (i, j), j < i, in that order
            const int i = tid >> 3, j = tid & 7;
            const int c = (j < i && lcp[i][j] > 1) ? 1 : 0;
            const int len = c ? lcp[i][j] - 1 : 0;
            const int pc = wave_scan<64>(c), pl = wave_scan<64>(len);   // inclusive prefix sums over the lanes
            if (c) {
                cand[pc - 1] = i << 3 | j;
                cpre[pc - 1] = pl - len;
            }
            if (tid == 63) {
                cpre[pc] = pl;
                ncand_s = pc;
            }
        }
        block_lds_barrier();
        const int n = __builtin_amdgcn_readfirstlane(ncand_s);
        const int tot = __builtin_amdgcn_readfirstlane(cpre[n]);
        // every position's lookups run without branches (a position past tot
        // repeats the last one and is not applied), so the eight of a thread
        // overlap their LDS and table round trips
        for (int base0 = 0; base0 < tot; base0 += kNT * 8) {
            const int base = base0 + tid;
            const int kn = min(8, (tot - base0 + kNT - 1) / kNT);   // positions per thread this round (uniform)
            int gi[8], gj[8], pr[8], pp[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                pr[k] = 0;
                pp[k] = 0;
                gi[k] = gj[k] = 0;
                if (k >= kn) continue;
                const int idx = min(base + kNT * k, tot - 1);
                // the pair whose range holds idx: last c with cpre[c] <= idx
                // (cpre increases strictly; n <= 28 pairs; steps past n skipped
                // as a whole, the others select)
                int c = 0;
#pragma unroll
                for (int step = 16; step > 0; step >>= 1) {
                    if (step < n) {
                        const int cs = c + step, v = cpre[min(cs, n - 1)];
                        c = (cs < n && v <= idx) ? cs : c;
                    }
                }
                const int pair = cand[c];
                const int i = pair >> 3, j = pair & 7;
                pp[k] = 1 + idx - cpre[c];
                pr[k] = pair;
                gi[k] = a.table[size_t(ent[i][E_ROW]) * a.L + pp[k]];
                gj[k] = a.table[size_t(ent[j][E_ROW]) * a.L + pp[k]];
            }
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if (k < kn && base + kNT * k < tot && (gi[k] != gj[k] || gi[k] < 0 || gi[k] >= a.M))
                    atomicMin(&lcp[pr[k] >> 3][pr[k] & 7], pp[k]);
        }
        block_lds_barrier();
    }

    // sharing trees and segments: wave 0, lane = entry (B <= 8)
    if (tid < 64) {
        const int lane = tid;
        const bool me = lane < a.B;
        const int np = me ? ent[lane][E_NPAGES] : 0;
        // this lane's entry: parent, shared run, root, size of its tree; the
        // trees grow one entry at a time (entry b joins the tree of its
        // parent), every member lane keeping the tree's size, so each step
        // is register reads (readlane) and lane-local updates
        int par = -1, ell = 0, root = lane, tsz = 1;
        int lrow[kMaxEnt];                         // lcp[b][lane]: run this lane's entry shares with entry b
#pragma unroll
        for (int b = 0; b < kMaxEnt; ++b) lrow[b] = lcp[b][lane & 7];
#pragma unroll
        for (int b = 1; b < kMaxEnt; ++b) {
            if (b >= a.B || __builtin_amdgcn_readlane(np, b) == 0) continue;
            // earlier entry with the longest shared run whose tree has room (ties: lowest index)
            const int key = (a.emax > 1 && lane < b && np > 0 && tsz < a.emax && lrow[b] > 0)
                                ? lrow[b] * 8 + (7 - lane) : -1;
            int best = -1;
#pragma unroll
            for (int j = 0; j < b; ++j) best = max(best, __builtin_amdgcn_readlane(key, j));
            if (best >= 0) {
                const int bp = 7 - (best & 7);
                const int r = __builtin_amdgcn_readlane(root, bp);
                const int size = __builtin_amdgcn_readlane(tsz, bp) + 1;
                if (lane == b) {
                    par = bp;
                    ell = best >> 3;
                    root = r;
                }
                if (root == r) tsz = size;
            }
        }
        // b's columns ride along owner o over pages [clo, chi): o = b for
        // [l_b, n_b); up the chain, the pages below every l passed so far
        if (lane < kMaxEnt * kMaxEnt) clo[lane >> 3][lane & 7] = chi[lane >> 3][lane & 7] = 0;
        wave_lds_sync();
        {
            int o = lane & 7, hi = np;
            bool done = np == 0;
#pragma unroll
            for (int step = 0; step < kMaxEnt; ++step) {
                const int ell_o = __shfl(ell, o), par_o = __shfl(par, o);
                if (!done) {
                    if (ell_o < hi) {
                        clo[lane][o] = ell_o;
                        chi[lane][o] = hi;
                    }
                    if (par_o < 0) {
                        done = true;
                    } else {
                        hi = min(hi, ell_o);
                        o = par_o;
                    }
                }
            }
        }
        wave_lds_sync();
        // owner lane o: its range [l_o, n_o) cut where the carried set changes
        int lo[kMaxEnt], hi[kMaxEnt], cut[kMaxEnt + 2];
#pragma unroll
        for (int b = 0; b < kMaxEnt; ++b) {
            lo[b] = clo[b][lane & 7];
            hi[b] = chi[b][lane & 7];
        }
        const bool owner = me && np > 0 && ell < np;
        cut[0] = ell;
        cut[1] = np;
#pragma unroll
        for (int b = 0; b < kMaxEnt; ++b) cut[2 + b] = hi[b] > lo[b] ? hi[b] : np;
#pragma unroll
        for (int x = 1; x < kMaxEnt + 2; ++x)        // insertion sort, fixed shape
#pragma unroll
            for (int y = x; y > 0; --y) {
                const int u = min(cut[y - 1], cut[y]), v = max(cut[y - 1], cut[y]);
                cut[y - 1] = u;
                cut[y] = v;
            }
        int nown = 0;                                 // segments of this owner
#pragma unroll
        for (int x = 0; x + 1 < kMaxEnt + 2; ++x) nown += (owner && cut[x + 1] > cut[x]) ? 1 : 0;
        const int pages = owner ? np - ell : 0;
        // exclusive prefix sums over the lanes: segment index, pages
        int sbase = wave_scan<8>(nown), pbase = wave_scan<8>(pages);   // lanes 0-7 (owners are entries)
        const int nseg_all = __builtin_amdgcn_readlane(sbase, 7), pages_all = __builtin_amdgcn_readlane(pbase, 7);
        sbase -= nown;
        pbase -= pages;
        int ekeys[kMaxEnt], elim[kMaxEnt];           // keys, and the causal limit of the entry's column
#pragma unroll
        for (int b = 0; b < kMaxEnt; ++b) {
            ekeys[b] = ent[b][E_KEYS];
            elim[b] = min(ent[b][E_N0] + 1, ekeys[b]);
        }
        if (owner) {
            int si = sbase, pre = pbase * H;
#pragma unroll
            for (int x = 0; x + 1 < kMaxEnt + 2; ++x) {
                const int c0 = cut[x], c1 = cut[x + 1];
                if (c1 <= c0) continue;
                int mask = 0, maxk = 0, kmin = INT_MAX;
#pragma unroll
                for (int b = 0; b < kMaxEnt; ++b)
                    if (hi[b] > lo[b] && lo[b] <= c0 && c1 <= hi[b]) {
                        mask |= 1 << b;
                        maxk = max(maxk, ekeys[b]);
                        kmin = min(kmin, elim[b]);
                    }
                seg[si][S_OWNER] = lane;
                seg[si][S_P0] = c0;
                seg[si][S_N] = c1 - c0;
                seg[si][S_MASK] = mask;
                seg[si][S_MAXKEYS] = maxk;
                seg[si][S_KMIN] = kmin;
                seg[si][S_PRE] = pre;
                seg[si][S_W] = (a.chunk ? ent[lane][E_T] : 1) * a.gq;
                pre += H * (c1 - c0);
                ++si;
            }
        }
        const uint64_t zb = __builtin_amdgcn_ballot_w64(me && np == 0 && ent[lane & 7][E_OWNED] && ent[lane & 7][E_T] > 0);
        if (lane == 0) {
            res_s[0] = nseg_all;
            res_s[1] = int(zb & 0xff);
            res_s[2] = pages_all * H;
        }
    }
    block_lds_barrier();

    const int nseg = res_s[0], total = res_s[2];
    const Split dq(total, a.G, a.share);
    const int Q = max(dq.qa, dq.qb);               // most positions of a block
    // unit (segment s, head h) and page within it of stream position u
    auto locate = [&](int u, int& s, int& h, int& pp) __attribute__((always_inline)) {
        s = 0;                                     // binary search: last segment with S_PRE <= u
#pragma unroll
        for (int step = kMaxSeg / 2; step > 0; step >>= 1)
            if (s + step < nseg && seg[s + step][S_PRE] <= u) s += step;
        const int off = u - seg[s][S_PRE], n = seg[s][S_N];
        h = Div(n)(off);
        pp = off - h * n;
    };

    int32_t* P = a.plan;
    // Roles: blocks [0, nspan) write the page list (span blockIdx.x; role < 0);
    // block nspan the header, the entry and segment tables and the piece
    // counts (role 0); the next kTaskBlocks blocks the combine tasks (roles
    // 1 .. kTaskBlocks); the last the new-token lists and the per-block
    // ranges.  Without a page list one block writes the tables.
    constexpr int kRoleBlk = kTaskBlocks + 1;
    const int role = a.pages ? int(blockIdx.x) - a.nspan : 0;
    // roles 0 .. kTaskBlocks: pieces (block, unit) of every unit (s, h), its
    // first block, then the pieces carrying each (entry, KV head) x into ex
    __shared__ int upc[kMaxSeg * kMaxH], ufirst[kMaxSeg * kMaxH];
    if (a.pages && role >= 0 && role < kRoleBlk) {
        for (int y = tid; y < nseg * H; y += kNT) {
            const int s = y / H, h = y - s * H;
            const int n = seg[s][S_N], start = seg[s][S_PRE] + h * n;
            upc[y] = pieces(start, n, dq);
            ufirst[y] = dq.block(start);
        }
        block_lds_barrier();
        int smask[kMaxSeg];
#pragma unroll
        for (int s = 0; s < kMaxSeg; ++s) {
            const int m = seg[s][S_MASK];
            smask[s] = s < nseg ? m : 0;
        }
        for (int x = tid; x < kMaxEnt * H; x += kNT) {
            const int b = x / H, h = x - b * H;
            int e = 0;                             // (every load issued, then selected: one LDS wait)
#pragma unroll
            for (int s = 0; s < kMaxSeg; ++s) {
                const int v = upc[min(s, max(nseg - 1, 0)) * H + h];
                e += ((smask[s] >> b) & 1) ? v : 0;
            }
            ex[x] = x < a.B * H ? e : 0;
        }
        block_lds_barrier();
    }
    if (role == 0) {
        if (tid < H_WORDS) {
            int v = 0;
            switch (tid) {
                case H_MAGIC: v = kMagic; break;
                case H_B: v = a.B; break;
                case H_H: v = H; break;
                case H_GQ: v = a.gq; break;
                case H_G: v = a.G; break;
                case H_QCAP: v = a.qcap; break;
                case H_TOTAL: v = total; break;
                case H_Q: v = Q; break;
                case H_NSEG: v = nseg; break;
                case H_ZERO: v = res_s[1]; break;
                case H_CHUNK: v = a.chunk; break;
                default: break;
            }
            if (tid != H_NTASK) P[tid] = v;      // written with the task list
        }
        if (tid < kMaxEnt * kEntWords) P[kOffEnt + tid] = ent[tid / kEntWords][tid % kEntWords];
        if (tid < kMaxSeg * kSegWords)
            P[kOffSeg + tid] = tid / kSegWords < nseg ? seg[tid / kSegWords][tid % kSegWords] : 0;
        if (a.pages)
            for (int x = tid; x < kMaxEnt * H; x += kNT) P[kOffExp + x] = ex[x];
        if (!a.pages && tid == 0) P[H_NTASK] = 0;
        return;
    }
    if (role >= 1 && role < kRoleBlk) {
        // combine tasks: (entry, KV head) pairs with more than one piece, in
        // pair order; a task lists its pieces in unit order, each unit's
        // slots in block order.  Every task block numbers all tasks alike and
        // writes tasks r, r + kTaskBlocks, ... (r = role - 1)
        const int r = role - 1;
        __shared__ int tpair[kMaxEnt * kMaxH], tpoff[kMaxEnt * kMaxH], tpre[kMaxEnt * kMaxH + 1], ntask_s;
        if (tid < 64) {                            // wave 0: task numbers, piece and overflow offsets
            const int lane = tid;
            const int n = a.B * H, per = (n + 63) / 64;
            int cnt = 0, over = 0, all = 0;
            for (int i = 0; i < per; ++i) {
                const int x = lane * per + i;
                if (x < n && ex[x] > 1) {
                    ++cnt;
                    over += max(0, ex[x] - kTaskInline);
                    all += ex[x];
                }
            }
            int tb = wave_scan<64>(cnt), ob = wave_scan<64>(over), ab = wave_scan<64>(all);   // then exclusive:
            const int ntask = __builtin_amdgcn_readlane(tb, 63);
            const int npiece = __builtin_amdgcn_readlane(ab, 63);
            tb -= cnt;
            ob -= over;
            ab -= all;
            for (int i = 0; i < per; ++i) {
                const int x = lane * per + i;
                if (x >= n || ex[x] <= 1) continue;
                const int b = x / H, h = x - b * H;
                if (tb % kTaskBlocks == r) {
                    int* rec = P + off_tasks(H, a.G) + size_t(tb) * kTaskWords;
                    rec[T_B] = b;
                    rec[T_H] = h;
                    rec[T_E] = ex[x];
                    rec[T_OUT] = (ent[b][E_CU] * H * a.gq + h * a.gq) * a.D;
                    rec[T_NCOL] = ent[b][E_T] * a.gq;
                    rec[T_POFF] = ob;
                }
                tpair[tb] = x;
                tpoff[tb] = ob;
                tpre[tb] = ab;
                ++tb;
                ob += max(0, ex[x] - kTaskInline);
                ab += ex[x];
            }
            if (lane == 0) {
                if (r == 0) P[H_NTASK] = ntask;
                ntask_s = ntask;
                tpre[ntask] = npiece;
            }
        }
        block_lds_barrier();
        // piece lists: a group of nt threads per task (no search for the
        // task); piece k of task t is slot j of the unit (s, h) that holds it,
        // s the segment carrying the task's entry whose pieces cover k
        const int ntask = ntask_s;
        int* over_list = P + off_over(H, a.G);
        int smask[kMaxSeg];
#pragma unroll
        for (int s = 0; s < kMaxSeg; ++s) {
            const int m = seg[s][S_MASK];
            smask[s] = s < nseg ? m : 0;
        }
        const int mine = (ntask - r + kTaskBlocks - 1) / kTaskBlocks;   // tasks r, r + kTaskBlocks, ...
        const int nt = mine > 0 ? max(1, kNT / mine) : 1, ngroups = kNT / nt;
        if (tid / nt < ngroups) {
            for (int t = r + kTaskBlocks * (tid / nt); t < ntask; t += kTaskBlocks * ngroups) {
                const int x = tpair[t], b = x / H, h = x - b * H;
                const int E = tpre[t + 1] - tpre[t];
                int c[kMaxSeg];                    // pieces of each segment's unit carrying b
#pragma unroll
                for (int s2 = 0; s2 < kMaxSeg; ++s2) {
                    const int v = upc[min(s2, max(nseg - 1, 0)) * H + h];
                    c[s2] = (smask[s2] >> b) & 1 ? v : 0;
                }
                int* rec = P + off_tasks(H, a.G) + size_t(t) * kTaskWords;
                for (int k = tid % nt; k < E; k += nt) {
                    int s = 0, j = k;
                    bool found = false;
#pragma unroll
                    for (int s2 = 0; s2 < kMaxSeg; ++s2) {
                        if (found || c[s2] == 0) continue;
                        s = s2;
                        if (j < c[s2]) found = true;
                        else j -= c[s2];
                    }
                    const int colb = __builtin_popcount(unsigned(seg[s][S_MASK]) & ((1u << b) - 1u)) * seg[s][S_W];
                    const int v = (ufirst[s * H + h] + j + s * H + h) * a.ncol + colb;
                    if (k < kTaskInline) rec[T_PIECE + k] = v;
                    else over_list[tpoff[t] + k - kTaskInline] = v;
                }
            }
        }
        return;
    }
    if (role == kRoleBlk) {
        // decode: the block that streams the page with an entry's new token
        // (position keys - 1) at head h lists (page, entry, head, row)
        const int maxp = min(kMaxPatch, 1024 / a.D);
        for (int i = tid; i < a.G; i += kNT) pcnt[i] = 0;
        block_lds_barrier();
        if (!a.chunk) {
            int* plist = P + off_patch(H, a.G);
            for (int x = tid; x < a.B * H; x += kNT) {
                const int b = x / H, h = x - b * H, keys = ent[b][E_KEYS];
                if (ent[b][E_NPAGES] == 0) continue;
                const int p = (keys - 1) >> kPageShift;
                for (int s = 0; s < nseg; ++s) {
                    if (!((seg[s][S_MASK] >> b) & 1) || p < seg[s][S_P0] || p >= seg[s][S_P0] + seg[s][S_N])
                        continue;
                    const int u = seg[s][S_PRE] + h * seg[s][S_N] + (p - seg[s][S_P0]);
                    const int i = dq.block(u), o = u - dq.start(i);
                    const int k = atomicAdd(&pcnt[i], 1);
                    if (k < maxp) plist[size_t(i) * kMaxPatch + k] = o | (b << 12) | (h << 15) | (((keys - 1) & 63) << 21);
                    break;
                }
            }
            block_lds_barrier();
        }
        int4* blk = reinterpret_cast<int4*>(P + off_blk(H));
        for (int i = tid; i < a.G; i += kNT) {
            const int u0 = dq.start(i);
            const int npg = dq.count(i, total);
            int s = 0, h = 0, pp = 0;
            if (npg > 0) locate(u0, s, h, pp);
            blk[i] = make_int4(npg, s * H + h, min(pcnt[i], maxp), 0);
        }
        return;
    }

    // page list: this block's span of stream positions, four per thread with
    // the table reads issued together; the segment starts, the entries' rows
    // and their new-token pages in registers
    int2* pages = reinterpret_cast<int2*>(P + off_pages(H, a.G));
    const int u_end = min(total, (int(blockIdx.x) + 1) * kPlanSpan);
    int pre[kMaxSeg], erow[kMaxEnt], enew[kMaxEnt];
#pragma unroll
    for (int t = 0; t < kMaxSeg; ++t) pre[t] = t < nseg ? seg[t][S_PRE] : INT_MAX;
#pragma unroll
    for (int b = 0; b < kMaxEnt; ++b) {
        erow[b] = ent[b][E_ROW];
        enew[b] = (!a.chunk && ent[b][E_KEYS] > 0) ? (ent[b][E_KEYS] - 1) >> kPageShift : -1;
    }
    for (int u0 = int(blockIdx.x) * kPlanSpan + tid; u0 < u_end; u0 += 4 * kNT) {
        int g[4], sl[4], meta[4], dst[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int u = u0 + k * kNT;
            dst[k] = -1;
            if (u < u_end) {
                int s = 0;                         // last segment with S_PRE <= u (the starts increase)
#pragma unroll
                for (int t = 1; t < kMaxSeg; ++t) s += pre[t] <= u ? 1 : 0;
                const int n = seg[s][S_N], p0 = seg[s][S_P0], owner = seg[s][S_OWNER];
                const int mask = seg[s][S_MASK], maxk = seg[s][S_MAXKEYS];
                const int off = u - seg[s][S_PRE];
                const int h = Div(n)(off), pp = off - h * n;
                const int p = p0 + pp;
                int row = erow[0], patch = 0;      // patch: an entry's new token lies in this page (decode)
#pragma unroll
                for (int b = 0; b < kMaxEnt; ++b) {
                    row = owner == b ? erow[b] : row;
                    patch |= (((mask >> b) & 1) && enew[b] == p) ? kPatchBit : 0;
                }
                g[k] = a.table[size_t(row) * a.L + p];
                sl[k] = h;
                const int lim = min(kPage, maxk - p * kPage);
                meta[k] = lim | (pp == n - 1 ? 256 : 0) | (p << 9) | patch;
                const int i = dq.block(u);
                dst[k] = i * a.qcap + (u - dq.start(i));
            }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (dst[k] >= 0) {
                const bool mapped = g[k] >= 0 && g[k] < a.M;
                pages[dst[k]] = make_int2(mapped ? g[k] * a.sg + sl[k] * a.sh : -1, meta[k]);
            }
    }
}

}  // namespace

int stream_plan_blocks(int bound) { return bound > 0 ? (bound + kPlanSpan - 1) / kPlanSpan : 1; }

hipError_t launch_stream_plan(const PoolView& pv, int B, int gq, const int32_t* table_rows, const int32_t* seq_lens,
                              const int32_t* q_pos0, const int32_t* cu_q, int max_seq_len, int max_cols, bool chunk,
                              bool dedup, bool pages, int G, int qcap, int share, int32_t* plan, hipStream_t s) {
    PlanArgs a{};
    a.table = pv.table;
    a.L = pv.L;
    a.C = pv.C;
    a.M = pv.M;
    a.H = pv.H;
    a.sg = pv.sg;
    a.sh = pv.sh;
    a.table_rows = table_rows;
    a.seq_lens = seq_lens;
    a.q_pos0 = q_pos0;
    a.cu_q = cu_q;
    a.B = B;
    a.gq = gq;
    a.max_ctx = max_seq_len;
    a.max_cols = max_cols;
    a.G = G;
    a.qcap = qcap;
    a.chunk = chunk ? 1 : 0;
    // a sharing tree stays within the 16 columns of one tile
    a.emax = (dedup && !chunk) ? (16 / gq < kMaxEnt ? 16 / gq : kMaxEnt) : 1;
    a.pages = pages ? 1 : 0;
    a.D = pv.D;
    a.ncol = chunk ? 32 : 16;
    a.share = share;
    a.plan = plan;
    const long long bound = (long long)B * pv.H * ((max_seq_len + kPage - 1) / kPage);
    a.nspan = pages ? stream_plan_blocks(int(bound)) : 0;
    stream_plan_kernel<<<dim3(unsigned(pages ? a.nspan + kTaskBlocks + 2 : 1)), kNT, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace kvs
