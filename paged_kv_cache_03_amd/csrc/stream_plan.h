// stream_plan.h -- layout of a page-stream plan in the attention workspace.
//
// A plan is the work list of one batch state (table rows, lengths, chunk
// shapes): which pages each block of the page stream reads, for which query
// columns.  It depends only on the block table and the lengths, so one plan
// serves every layer of a step.  Entries whose table rows map the same page
// groups over a leading range of logical blocks (forks share a prefix of
// their parent's pages: Paged KV Context Store page, fork and tail
// copy-on-write) read that range once: the pages go through the matrix cores
// with the query columns of every sharing entry, instead of once per entry.
//
// Structure.  Entry b has n_b = ceil(keys_b / 64) pages.  Entries form
// sharing trees: entry b's parent is the earlier entry with which it shares
// the longest leading run of mapped page groups, l_b pages (ties: the lowest
// index), as long as the tree stays within the columns of one tile.  Entry b
// reads pages [l_b, n_b) itself; a page p < l_b is read by the nearest
// ancestor a on b's chain with p >= l_a.  Each entry's own range, cut where
// the set of entries reading along changes, gives the segments: (owner
// entry, first page, page count, mask of entries whose columns it carries).
// There are at most 2B - 1 of them.  Stream unit sigma = s * H + h is
// segment s at KV head h; the flat stream lists every unit's pages in sigma
// order, and block i of G takes stream positions [i*Q, min((i+1)*Q, total)).
// The work split depends only on which logical pages are shared, never on
// physical page ids.
//
// Word offsets (int32) from the plan base; every array starts on a 256-byte
// boundary.
#pragma once

#include <cstddef>
#include <cstdint>

namespace kvs {
namespace plan {

constexpr int kMagic = 0x4e414c50;    // marks a page-stream plan
constexpr int kMaxEnt = 8;            // entries per call (B <= C <= 8)
constexpr int kMaxSeg = 16;           // segments per call (at most 2B - 1)
constexpr int kMaxH = 64;             // KV heads the page stream handles
constexpr int kEntWords = 8;
constexpr int kSegWords = 8;

// header
enum : int {
    H_MAGIC = 0,
    H_B,        // entries of the call
    H_H,        // KV heads
    H_GQ,       // query heads per KV head
    H_G,        // blocks of the run
    H_QCAP,     // page slots per block in the page list
    H_TOTAL,    // stream positions
    H_Q,        // positions per block
    H_NSEG,     // segments
    H_ZERO,     // mask of entries with query rows and nothing to attend
    H_CHUNK,    // 1: several query tokens per entry (verify / chunked prefill)
    H_NTASK,    // (entry, KV head) pairs with more than one piece: combine tasks
    H_WORDS = 64
};

// entry table [kMaxEnt][kEntWords]
enum : int {
    E_ROW = 0,  // block-table row
    E_KEYS,     // keys that exist: positions [0, keys)
    E_N0,       // position of the entry's first query token
    E_CU,       // first query row of the entry in q / out
    E_T,        // query tokens
    E_NPAGES,   // pages the entry attends (0: none)
    E_OWNED,    // 1 if this run computes the entry
};

// segment table [kMaxSeg][kSegWords]
enum : int {
    S_OWNER = 0,  // entry whose table row addresses the pages
    S_P0,         // first logical page
    S_N,          // pages
    S_MASK,       // entries whose query columns the segment carries
    S_MAXKEYS,    // largest key count among them (rows any column may see)
    S_KMIN,       // smallest causal limit among their columns
    S_PRE,        // stream position of unit (s, 0): H x pages of earlier segments
    S_W,          // query columns per entry (tokens x GQ)
};

constexpr int kOffEnt = H_WORDS;
constexpr int kOffSeg = kOffEnt + kMaxEnt * kEntWords;
constexpr int kOffExp = kOffSeg + kMaxSeg * kSegWords;     // [kMaxEnt][H] pieces per (entry, KV head)

// combine task record [kMaxEnt * H][kTaskWords]: the pieces of one (entry,
// KV head) -- partial index slot * NCOL + the entry's first column, in unit
// order, each unit's slots in block order; pieces past kTaskInline continue
// in the overflow list at T_POFF
constexpr int kTaskWords = 64;
constexpr int kTaskInline = kTaskWords - 8;
enum : int {
    T_B = 0,    // entry
    T_H,        // KV head
    T_E,        // pieces
    T_OUT,      // float offset of the entry's first output of this head: (cu * Hq + h * GQ) * D
    T_NCOL,     // the entry's columns (tokens x GQ)
    T_POFF,     // overflow list offset (pieces kTaskInline ..)
    T_PIECE = 8
};

constexpr size_t align64w(size_t w) { return (w + 63) / 64 * 64; }

// Decode with the step's rows: the page that holds an entry's new token
// (position keys - 1) carries bit kPatchBit in its meta, and its block finds
// the row in its patch list: (page within the block | entry << 12 | KV head
// << 15 | row << 21), at most kMaxPatch per block (more: the block loads the
// row when it reaches the page).
constexpr int kPatchBit = 1 << 24;
constexpr int kMaxPatch = 16;

// per block: int4 (pages, first unit, staged patches, 0)
constexpr size_t off_blk(int H) { return align64w(size_t(kOffExp) + size_t(kMaxEnt) * H); }
constexpr size_t off_patch(int H, int G) { return off_blk(H) + align64w(4 * size_t(G)); }
constexpr size_t off_tasks(int H, int G) { return off_patch(H, G) + align64w(size_t(kMaxPatch) * G); }
// overflow pieces: every (block, unit) piece carries at most kMaxEnt entries
constexpr size_t max_pieces(int H, int G) { return (size_t(G) + size_t(kMaxSeg) * H) * kMaxEnt; }
constexpr size_t off_over(int H, int G) { return off_tasks(H, G) + size_t(kTaskWords) * kMaxEnt * H; }
// per block: qcap int2 (slice number g*sg + h*sh or -1, valid rows | 256 at a unit's end | page << 9 | kPatchBit)
constexpr size_t off_pages(int H, int G) { return off_over(H, G) + align64w(max_pieces(H, G)); }
constexpr size_t plan_words(int H, int G, int qcap) { return off_pages(H, G) + 2 * size_t(G) * size_t(qcap); }
constexpr size_t plan_bytes(int H, int G, int qcap) { return (plan_words(H, G, qcap) * 4 + 255) / 256 * 256; }

}  // namespace plan
}  // namespace kvs
