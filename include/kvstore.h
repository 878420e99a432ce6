/*
 * kvstore.h -- C ABI of the paged KV context store hot path for MI355X (gfx950).
 *
 * What it implements is defined by the NInfer maintainer pages
 * ("Paged KV Context Store", "Engine Architecture", "Resource Scheduling and
 * Context Cache").  Their headings were lost in extraction, so each entry point
 * names the passage it follows by what that passage holds.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every call returns kv_status.  KV_OK is success.  No C++ exception crosses
 *   this boundary; kv_last_error_message() gives a human-readable detail for
 *   the last failure on the calling thread.
 * - A capacity shortfall is a status plus a deficit out-parameter, never an
 *   exception (Paged KV Context Store page, invariant list: a shortfall does
 *   not leave a step through an exception).
 * - Device memory is caller-owned: plane tensors, the block-table matrix,
 *   inputs, outputs and workspaces.  Their base addresses must stay valid and
 *   stable for the pool's lifetime (graph-stable bases passage).  The pool owns
 *   only host metadata (free list, references, generations, address spaces and
 *   a host mirror of the block table).
 * - All device work is enqueued on the caller's hipStream_t, in call order.
 *   Nothing here synchronizes the device except kv_pool_destroy.
 * - Pointers named d_* are device pointers; all others are host pointers.
 * - Errors KV_E_DEVICE mean a HIP runtime call failed: treat it as an
 *   engine-wide failure (Engine Architecture page, error classes).
 */
#ifndef KVSTORE_H
#define KVSTORE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------ status codes */
typedef int32_t kv_status;
#define KV_OK             0  /* success */
#define KV_E_INVALID      1  /* bad argument, null pointer, unknown handle use */
#define KV_E_GEOMETRY     2  /* geometry rejected: P != 64, C not in [1,8], M outside
                                [max(L,C), C*L], head_dim/group mismatch, B > C, Hq % H != 0 */
#define KV_E_CAPACITY     3  /* not enough free page groups; the deficit is reported */
#define KV_E_STALE        4  /* sequence handle generation does not match (released) */
#define KV_E_SHARED_WRITE 5  /* write domain touches a page with several references:
                                copy the tail first (kv_cow_tail_page) */
#define KV_E_UNMAPPED     6  /* commit beyond the mapped pages */
#define KV_E_DEVICE       7  /* a HIP runtime call failed */
#define KV_E_UNSUPPORTED  8  /* valid request this library has no kernel for */

/* ------------------------------------------------ closed profiles / planes */
/* Closed KV profiles (Paged KV Context Store page, closed-profile paragraph).
 * K8V4 is closed and asymmetric: K = FP8-E4M3FN-row256, V = NVFP4-G16. */
#define KV_PROFILE_BF16              0
#define KV_PROFILE_INT8_G64          1
#define KV_PROFILE_FP8_E4M3FN_ROW256 2
#define KV_PROFILE_NVFP4_G16         3
#define KV_PROFILE_K8V4              4

/* Plane element types. */
#define KV_DT_BF16     0  /* 2 bytes, stored unchanged from the bf16 input */
#define KV_DT_I8       1  /* INT8-G64 codes */
#define KV_DT_E4M3FN   2  /* FP8 E4M3FN codes (OCP, bias 7, saturating at +-448) */
#define KV_DT_E2M1X2   3  /* two FP4 E2M1 codes per byte, element 2k in the low nibble */
#define KV_DT_F32      4  /* fp32 scales (INT8-G64 per 64 elements, FP8-row per row) */
#define KV_DT_U8_E4M3  5  /* NVFP4-G16 scales: one E4M3FN byte per 16 elements */
#define KV_DT_F16      6  /* binary16 scales (INT8-G64, FP8-row): the 2-byte scale planes of the D256 payload
                             table; scale = binary16(fp32 quotient), rounded half to even, saturated at 65504 */

/* Plane roles; the K and V code planes and scale planes of one layer share a
 * page-group id (plane-grouping rule). */
#define KV_ROLE_K_CODE  0
#define KV_ROLE_K_SCALE 1
#define KV_ROLE_V_CODE  2
#define KV_ROLE_V_SCALE 3

/* Plane orders (PagedKVStorageLayout passage: the closed physical orders and
 * the address-translation equations; head-major swaps the head and
 * page-group terms).  Every plane of one pool takes the same order. */
#define KV_LAYOUT_PAGE_MAJOR 0   /* [X, P, H, N]: C-order [M][H][64][X] */
#define KV_LAYOUT_HEAD_MAJOR 1   /* [X, P, N, H]: C-order [H][M][64][X] (the Draft Full order) */

/* Expanded pool geometry (capacity-geometry equations):
 *   L = ceil(max_context / page_size), valid M in [max(L, C), C * L]. */
typedef struct KVPageGeometry {
    uint32_t page_size;        /* P; must be 64 */
    uint32_t num_kv_heads;     /* H */
    uint32_t head_dim;         /* D; 64, 128 or 256 */
    uint32_t num_layers;       /* layers whose planes share the page-group id */
    uint32_t max_context;      /* S */
    uint32_t max_concurrency;  /* C, 1..8: block-table rows */
    uint32_t num_page_groups;  /* M */
} KVPageGeometry;

/* One plane in a closed order (first extent fastest) with contiguous
 * strides (address-translation equations); element (x, o, h, g) lives at
 *   page-major [X, P, H, N], C-order [M][H][64][X]:
 *     base + elem_bytes * (x + X * (o + 64 * (h + H * g)))
 *   head-major [X, P, N, H], C-order [H][M][64][X]:
 *     base + elem_bytes * (x + X * (o + 64 * (g + M * h)))
 * base is caller-owned device memory of M * H * 64 * X * elem_bytes bytes,
 * 256-byte aligned.  layout is KV_LAYOUT_PAGE_MAJOR (0, what
 * kv_profile_planes writes) or KV_LAYOUT_HEAD_MAJOR; every plane of a pool
 * takes the same one (KV_E_INVALID otherwise).  Results of every call are
 * the same in either order; only the addresses differ. */
typedef struct KVPlaneDesc {
    uint32_t layer;
    uint32_t role;       /* KV_ROLE_* */
    uint32_t dtype;      /* KV_DT_* */
    uint32_t x_extent;   /* X: D for codes, D/2 packed FP4, D/64 INT8 scales, 1 FP8 row
                            scale, D/16 NVFP4 scales (X-extent list) */
    uint32_t elem_bytes; /* bytes per element of dtype */
    uint32_t layout;     /* KV_LAYOUT_* */
    void*    base;       /* device pointer, caller-owned */
} KVPlaneDesc;

typedef struct kv_pool kv_pool;   /* opaque host object */
typedef uint64_t kv_seq;          /* generation-tagged address-space handle; 0 is never valid */

/* Schema of one layer of a closed profile (PagedKVStorageLayout passage: a
 * closed profile resolves to K/V data/scale planes).  Writes up to *n_inout
 * descriptors (layer 0, base NULL) and sets *n_inout to the count (2 or 4).
 * KV_E_INVALID if the buffer is too small; KV_E_GEOMETRY if head_dim is not a
 * multiple of the profile's groups. */
kv_status kv_profile_planes(uint32_t profile, uint32_t head_dim, KVPlaneDesc* out, uint32_t* n_inout);

/* kv_profile_planes with the dtype of the INT8-G64 / FP8-row scale planes:
 * KV_DT_F32 (as kv_profile_planes) or KV_DT_F16 (2-byte scales: bytes per
 * token and KV head at D=256 are those of the page's D256 payload table,
 * 1024 / 528 / 516 / 288 / 402).  NVFP4-G16 scales are E4M3 bytes either
 * way.  A pool takes one scale dtype for all its planes.  KV_E_INVALID for
 * another dtype. */
kv_status kv_profile_planes_ex(uint32_t profile, uint32_t head_dim, uint32_t scale_dtype, KVPlaneDesc* out,
                               uint32_t* n_inout);

/* Bytes of one plane slab for a geometry: M * H * 64 * X * elem_bytes. */
kv_status kv_plane_bytes(const KVPageGeometry* geo, const KVPlaneDesc* plane, uint64_t* bytes);

/* Create a homogeneous pool (Paged KV Context Store page: homogeneous pools,
 * capacity geometry, device block-table matrix).
 *   planes / n_planes : num_layers copies of one profile's schema, bases set.
 *   d_block_tables    : caller-owned int32 [C][L] device matrix; set to -1
 *                       (unmapped) on `stream`.  NULL makes a host-only pool:
 *                       metadata and host mirror only, no device work at all,
 *                       kernels refuse it (used to test the allocator on CPU).
 *   free_order        : optional permutation of [0, M): page groups are taken
 *                       from the front of a FIFO in this order and freed ones
 *                       are appended at the back in logical-block order.  NULL
 *                       means 0, 1, ..., M-1.  Correctness never depends on it.
 * KV_E_GEOMETRY / KV_E_INVALID on rejected input; *out is NULL then. */
kv_status kv_pool_create(const KVPageGeometry* geo, const KVPlaneDesc* planes, uint32_t n_planes,
                         int32_t* d_block_tables, const int32_t* free_order, hipStream_t stream,
                         kv_pool** out);

/* Synchronize the device and free the host object.  Device memory is the
 * caller's to free afterwards.  NULL is ignored. */
void kv_pool_destroy(kv_pool* pool);

/* Lease accounting: allocated + reserved + available == M.  allocated:
 * page groups with references; reserved: groups held in address spaces'
 * active reservations (kv_seq_reserve, kv_seq_trim); available: the free
 * list. */
kv_status kv_pool_stats(const kv_pool* pool, uint32_t* allocated, uint32_t* reserved, uint32_t* available);

/* Copy the host mirror of the block-table matrix, int32 [C][L], into out. */
kv_status kv_pool_table_host(const kv_pool* pool, int32_t* out, size_t n_entries);

/* References held on page group g by address spaces (0 when free). */
kv_status kv_pool_page_refs(const kv_pool* pool, uint32_t page_group, uint32_t* refs);

/* New empty address space leasing block-table row `table_row`
 * (KVAddressSpace descriptor, execution-row lease).  The row is set to -1 on
 * `stream`.  KV_E_INVALID if the row is out of range or already leased. */
kv_status kv_seq_open(kv_pool* pool, uint32_t table_row, hipStream_t stream, kv_seq* out);

/* Fork (Paged KV Context Store page, Fork passage and worked example): a new
 * address space on `table_row` sharing src's pages covering [0, frontier),
 * frontier <= src's committed frontier.  Full pages gain a reference; a
 * partial tail is shared too and must be copied with kv_cow_tail_page before
 * any write.  The frontier is kept exactly (not rounded down to a page).  The
 * row's mapping is published on `stream`. */
kv_status kv_seq_fork(kv_pool* pool, kv_seq src, uint32_t frontier, uint32_t table_row,
                      hipStream_t stream, kv_seq* out);

/* ensure_mapped_to_tokens: map page groups so that positions [0, tokens) are
 * covered.  A lower bound: never trims, never moves the frontier.  Allocates
 * only the missing pages (ordinary decode: one page at a page crossing) and
 * publishes the new contiguous slice of the row on `stream` before any later
 * kernel on that stream (mapping publication order).
 *   *deficit : set to the missing page count on KV_E_CAPACITY, else 0.
 * KV_E_CAPACITY: nothing is allocated.  KV_E_SHARED_WRITE: the write domain
 * [frontier, tokens) starts inside a shared partial tail (writer-cardinality
 * rules).  KV_E_INVALID: tokens > max_context. */
kv_status kv_seq_ensure_mapped(kv_pool* pool, kv_seq seq, uint32_t tokens, uint32_t* deficit,
                               hipStream_t stream);

/* Advance the committed frontier after the unit that wrote [old, frontier)
 * has been enqueued (frontier commit happens at the GPU boundary).
 * KV_E_INVALID if frontier < current; KV_E_UNMAPPED if beyond the mapping. */
kv_status kv_seq_commit(kv_pool* pool, kv_seq seq, uint32_t frontier);

/* Finish / release: drop this address space's page references (a page is
 * freed on its last one), release its table row (set to -1 on `stream`) and
 * retire the handle (later use returns KV_E_STALE). */
kv_status kv_seq_release(kv_pool* pool, kv_seq seq, hipStream_t stream);

/* Active reservation (Paged KV Context Store page, lease accounting and
 * active-reservation rules): move `pages` page groups from the front of the
 * free list to the back of this address space's reservation, a FIFO of
 * concrete groups that only this space maps from.  kv_seq_ensure_mapped and
 * kv_cow_tail_page take from the reservation's front before the free list;
 * kv_seq_release returns the reservation to the back of the free list, in
 * its order.  Host metadata only.
 *   *deficit : the missing count on KV_E_CAPACITY (nothing moves), else 0. */
kv_status kv_seq_reserve(kv_pool* pool, kv_seq seq, uint32_t pages, uint32_t* deficit);

/* Trim the membership of a speculative unit (Paged KV Context Store page,
 * retained-membership equation and speculative termination): keep
 * NeededPages = ceil(max(committed frontier, provisional) / 64) mappings;
 * the trailing ones are removed from the row (-1, published on `stream`) and
 * each group whose last reference this was goes to the back of this space's
 * reservation, in logical-block order -- not to the free list, so no other
 * address space can map it.  The last partial page stays mapped; its bytes
 * past the frontier are outside the valid domain and the next append at the
 * frontier overwrites them.  The publication is ordered after every kernel
 * enqueued earlier on `stream` (a verify still reading the removed pages);
 * work on other streams must be ordered by the caller.  A no-op when nothing
 * trails.  KV_E_INVALID: provisional > max_context. */
kv_status kv_seq_trim(kv_pool* pool, kv_seq seq, uint32_t provisional, hipStream_t stream);

/* Close a speculative unit that wrote `produced` rows from the committed
 * frontier (accepted-prefix commit, Engine Architecture page: a row that is
 * not cancelled accepts 1 <= accepted <= produced, a cancelled row 0): the
 * frontier advances by `accepted`, then kv_seq_trim(seq, new frontier).
 * KV_E_INVALID on the bounds; KV_E_UNMAPPED if frontier + produced is past
 * the mapping (nothing changes then). */
kv_status kv_seq_commit_accepted(kv_pool* pool, kv_seq seq, uint32_t produced, uint32_t accepted, int cancelled,
                                 hipStream_t stream);

/* Page groups held in this address space's reservation. */
kv_status kv_seq_reservation(const kv_pool* pool, kv_seq seq, uint32_t* pages);

/* Physical pages of an MTP draft pool with draft window K >= 1 next to a Main
 * pool of `main_pages` (Paged KV Context Store page, backend capacity list):
 * main_pages + max_concurrency * ceil((K - 1) / 64), one provisional lead of
 * K - 1 tokens per active row.  KV_E_INVALID if K == 0. */
kv_status kv_draft_pool_pages(uint32_t main_pages, uint32_t max_concurrency, uint32_t draft_window,
                              uint32_t* pages);

/* Host replica (Paged KV Context Store page, host replica passage): the
 * logical-order packed HostKVPageLayout.  Page i of a replica is logical
 * block i of the address space; it holds, for every layer in ascending order
 * and every plane of the layer in the order K code, K scale, V code, V scale,
 * that plane's [H][64][X] slice of the page group (all 64 rows: the full
 * page payload).  No device page id or table hole is stored; a replica of n
 * pages takes n * page_bytes bytes. */
kv_status kv_replica_page_bytes(const kv_pool* pool, uint64_t* bytes);

/* Copy the committed pages [0, ceil(frontier / 64)) of `seq` into `host` in
 * the replica layout (device to host, a kernel on `stream`).  host: pinned
 * host memory (hipHostMalloc or a pinned tensor), 16-byte aligned,
 * host_bytes >= pages * page_bytes.  *pages and *frontier receive the page
 * count and the committed frontier the replica covers.  The copy completes
 * in `stream` order: the caller keeps the address space unchanged (no
 * append, trim, COW or release) and reads `host` only after it.
 * KV_E_INVALID for memory that is not pinned or too small. */
kv_status kv_seq_offload(kv_pool* pool, kv_seq seq, void* host, size_t host_bytes, uint32_t* pages,
                         uint32_t* frontier, hipStream_t stream);

/* A new address space on `table_row` from a replica: maps ceil(frontier /
 * 64) page groups, copies each replica page into its group (host to device,
 * a kernel on `stream`), then publishes the row on `stream` -- the row names
 * the pages only after their payload has landed (replica publication order)
 * -- and commits `frontier`.  `host` stays unchanged until the copy has
 * completed.  KV_E_CAPACITY with *deficit when too few groups are free
 * (nothing changes); KV_E_INVALID for a leased row or unpinned memory. */
kv_status kv_seq_restore(kv_pool* pool, uint32_t table_row, const void* host, size_t host_bytes, uint32_t frontier,
                         uint32_t* deficit, hipStream_t stream, kv_seq* out);

/* Row, committed frontier and mapped page count of a live address space. */
kv_status kv_seq_info(const kv_pool* pool, kv_seq seq, uint32_t* table_row, uint32_t* frontier,
                      uint32_t* mapped_pages);

/* Partial-tail COW (Fork passage: copy the tail's committed columns into a
 * private page; Engine Architecture page: restore, tail COW and mapping
 * upload go in order on one stream).  If the committed frontier F is not
 * page-aligned and its tail page is shared: allocate g', copy columns
 * [0, F mod 64) of every plane of every layer from g to g', rebind the row's
 * entry to g' and drop the reference on g -- copy and rebind on `stream`.
 * A no-op (KV_OK) when F is aligned or the tail is already private.
 * KV_E_CAPACITY (deficit 1) when no page group is free. */
kv_status kv_cow_tail_page(kv_pool* pool, kv_seq seq, hipStream_t stream);

/* Persistent KV codec: quantize and write new K/V rows at their positions
 * (Paged KV Context Store page: closed profiles, X-extent list, P=64
 * translation; the codec header itself is not on the pages -- rounding rules:
 * fp32 arithmetic, round half to even, saturating FP8/FP4, zero scale gives
 * zero codes).
 *   B                : compact batch entries; entry b uses table row
 *                      d_table_rows[b] (PagedKVBatchLayerView: batch order,
 *                      lane and table row may all differ).
 *   d_pos0[B]        : position of each entry's first new row.
 *   d_cu_tokens[B+1] : rows of entry b are [cu[b], cu[b+1]) of the inputs.
 *   d_k, d_v         : bf16 [total_tokens][H][D], contiguous.
 * Does not move any frontier.  Caller guarantees (wrapper validation and
 * caller guarantees passage): every written block is mapped in a private
 * page, rows are stable until the unit completes.  Rows whose table entry is
 * -1 are skipped.  KV_E_GEOMETRY if B > C. */
kv_status kv_append(const kv_pool* pool, uint32_t layer, uint32_t B, const int32_t* d_table_rows,
                    const int32_t* d_pos0, const int32_t* d_cu_tokens, uint32_t total_tokens,
                    const void* d_k, const void* d_v, hipStream_t stream);

/* Workspace bytes paged_attn_decode / paged_attn_verify need for these bounds
 * (the batch state's plan and the split-K partials).  max_q_len 0 means
 * decode.  The caller owns the workspace; it needs no initialization (every
 * call writes what it reads).  Calls that overlap in time (other streams)
 * need workspaces of their own. */
size_t paged_attn_workspace_bytes(const kv_pool* pool, uint32_t B, uint32_t Hq, uint32_t max_seq_len,
                                  uint32_t max_q_len);

/* Paged decode for a compact batch of 1..C sequences (Paged KV Context Store
 * page: PagedKVBatchLayerView, P=64 translation, consumer rules).  Entry b's
 * query (the step's last token, already appended) attends positions
 * [0, d_seq_lens[b]) of table row d_table_rows[b]:
 *     out[b][j] = sum_i softmax_i(q[b][j] . k_i * sm_scale) v_i,
 *     KV head of query head j = j / (Hq / H).
 * Pages are read through the block table, a page at a time; split-K over
 * pages with a deterministic cross-split combine, so results do not depend
 * on physical page ids.  Leading pages that several entries' rows share are
 * read once for all of them (the split then differs from that of private
 * copies of the same pages, within rounding).  seq_len 0 yields zeros.
 *   d_q   : bf16 [B][Hq][D];  d_out: fp32 [B][Hq][D].
 *   max_seq_len : host upper bound of d_seq_lens (sizes the split grid).
 *   d_ws / ws_bytes : >= paged_attn_workspace_bytes(pool, B, Hq, max_seq_len, 0).
 * KV_E_GEOMETRY on B > C or Hq % H != 0; KV_E_INVALID unless sm_scale is
 * finite and > 0; KV_E_UNSUPPORTED for shapes with no kernel instance (see
 * paged_attn_supported). */
kv_status paged_attn_decode(const kv_pool* pool, uint32_t layer, uint32_t B, uint32_t Hq,
                            const int32_t* d_table_rows, const int32_t* d_seq_lens, uint32_t max_seq_len,
                            const void* d_q, float sm_scale, float* d_out, void* d_ws, size_t ws_bytes,
                            hipStream_t stream);

/* paged_attn_decode for callers that cannot allocate device memory or bring
 * a workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  The same plan and run as paged_attn_decode, with
 * the library's own static device scratch (KV_DECODE_SCRATCH_BYTES per GPU,
 * a file-scope device array that each GPU the library runs on holds until
 * the process ends) in place of d_ws.  Calls no allocator.  The scratch
 * needs no clearing (every call writes what it reads), but every call on
 * one GPU shares it: calls that overlap in time on one GPU (other streams,
 * other threads, other graphs) race, and the caller serializes them.
 * KV_E_INVALID when paged_attn_workspace_bytes(pool, B, Hq, max_seq_len, 0)
 * exceeds KV_DECODE_SCRATCH_BYTES (use paged_attn_decode then); other errors
 * and results exactly as paged_attn_decode. */
#define KV_DECODE_SCRATCH_BYTES (32u << 20)
kv_status paged_attn_decode_noalloc(const kv_pool* pool, uint32_t layer, uint32_t B, uint32_t Hq,
                                    const int32_t* d_table_rows, const int32_t* d_seq_lens, uint32_t max_seq_len,
                                    const void* d_q, float sm_scale, float* d_out, hipStream_t stream);

/* Decode split in two, for callers that run the same batch state over many
 * layers (consumer rules: the op chooses its own split; the work list depends
 * only on the block table and the lengths, which a step keeps for all
 * layers).
 *
 * paged_attn_decode_plan writes the batch state's work list into d_ws: the
 * entry table, and for the matrix-core page stream the page list of every
 * block.  Entries whose table rows hold the same page groups over a leading
 * run of logical blocks (forks: fork and tail copy-on-write) have that run
 * read once, with the query heads of all of them in the matrix-core columns.
 * Reads d_table_rows, d_seq_lens and the block table on the stream; the plan
 * stays valid until any of them changes for an entry of the batch.
 *
 * paged_attn_decode_run computes layer `layer` from the plan in d_ws, with
 * the same result definition as paged_attn_decode.  B, Hq, max_seq_len and
 * d_ws must be those of the plan (a plan of another B, Hq or grid is
 * detected on the device and turns every output of the call into NaN).  The
 * workspace is as for paged_attn_decode (>= paged_attn_workspace_bytes(pool,
 * B, Hq, max_seq_len, 0)); runs on one workspace must not
 * overlap in time.  paged_attn_decode is exactly a plan followed by a run.
 * Errors as for paged_attn_decode; the plan checks no sm_scale. */
kv_status paged_attn_decode_plan(const kv_pool* pool, uint32_t B, uint32_t Hq, const int32_t* d_table_rows,
                                 const int32_t* d_seq_lens, uint32_t max_seq_len, void* d_ws, size_t ws_bytes,
                                 hipStream_t stream);
kv_status paged_attn_decode_run(const kv_pool* pool, uint32_t layer, uint32_t B, uint32_t Hq, uint32_t max_seq_len,
                                const void* d_q, float sm_scale, float* d_out, void* d_ws, size_t ws_bytes,
                                hipStream_t stream);

/* paged_attn_decode_run with the step's rows appended by the run itself: the
 * K and V row of entry b (bf16 d_k, d_v [B][H][D]) go to position
 * seq_len[b] - 1 of its table row (the lengths of the plan; entries with
 * seq_len 0 append nothing), and the decode attends them, as kv_append
 * (pos0 = seq_len - 1, one token per entry) followed by
 * paged_attn_decode_run would, with the same outputs and planes.  The page
 * that receives a row must not be shared (fork and tail copy-on-write: copy
 * the tail first), as for kv_append.  Pages on the matrix-core streams: every
 * closed profile at D in {64, 128, 256} (NVFP4 sides at 128 and 256) with
 * Hq / H in {1, 2, 4, 8}, at most 8 entries; KV_E_UNSUPPORTED otherwise (use
 * kv_append and paged_attn_decode_run). */
kv_status paged_attn_decode_append_run(const kv_pool* pool, uint32_t layer, uint32_t B, uint32_t Hq,
                                       uint32_t max_seq_len, const void* d_k, const void* d_v, const void* d_q,
                                       float sm_scale, float* d_out, void* d_ws, size_t ws_bytes, hipStream_t stream);

/* Multi-token verify / chunked prefill on paged KV (causal): chunk token i of
 * entry b sits at position d_q_pos0[b] + i and attends [0, d_q_pos0[b] + i]
 * (the chunk's own K/V are appended first; the mask starts at any in-page
 * frontier).  Work is AttentionPairs = n0*T + T(T+1)/2 per head (Resource
 * Scheduling page, prefill-work equation).  QK^T and PV run on MFMA.
 *   d_cu_q[B+1] : rows of entry b are [cu[b], cu[b+1]) of d_q / d_out.
 *   d_q   : bf16 [total_q][Hq][D];  d_out: fp32 [total_q][Hq][D].
 *   max_q_len, max_seq_len : host upper bounds (max T, max n0 + T).
 *   d_ws / ws_bytes : >= paged_attn_workspace_bytes(pool, B, Hq, max_seq_len,
 *   max_q_len).
 * KV_E_INVALID unless sm_scale is finite and > 0.  Every closed profile at
 * D in {64, 128, 256} with Hq / H in {1, 2, 4, 8} (Paged KV Context Store
 * page, pool sets: Main Text and MTP pages take the engine-selected
 * profile); KV_E_UNSUPPORTED for other head groupings. */
kv_status paged_attn_verify(const kv_pool* pool, uint32_t layer, uint32_t B, uint32_t Hq,
                            const int32_t* d_table_rows, const int32_t* d_q_pos0, const int32_t* d_cu_q,
                            uint32_t total_q, uint32_t max_q_len, uint32_t max_seq_len, const void* d_q,
                            float sm_scale, float* d_out, void* d_ws, size_t ws_bytes, hipStream_t stream);

/* One decode step of layers 0 .. n_layers-1 as a HIP graph (Paged KV Context
 * Store page, graph-stable bases: plane and table bases stay fixed while page
 * ids, table rows, lengths and positions are data; one graph per exact B).
 * The graph holds exactly the work of an eager step: paged_attn_decode_plan,
 * then per layer l the append of the step's rows and the decode run.  The
 * caller picks the append's form:
 *   d_pos0 == d_cu_tokens == NULL : paged_attn_decode_append_run(d_k[l],
 *       d_v[l]) -- one row per entry at position seq_len - 1 (total_tokens
 *       == B); the shapes paged_attn_decode_append_run takes,
 *       KV_E_UNSUPPORTED otherwise;
 *   both set : kv_append(d_pos0, d_cu_tokens, total_tokens) then
 *       paged_attn_decode_run, for any rows and positions.
 * d_k == d_v == NULL: runs only, nothing appended.
 *   d_q[l], d_out[l], d_k[l], d_v[l] : host arrays of n_layers device
 *       pointers, as for the eager calls; d_pos0 / d_cu_tokens [B] / [B+1]
 *       device arrays (the kv_append form).
 * Every pointer, B, Hq, max_seq_len, sm_scale and the workspace are fixed at
 * capture; the contents they point to are read at each replay, so a caller
 * updates lengths, rows, queries and step rows in place and maps new pages
 * (kv_seq_ensure_mapped, publication on its stream) before launching.
 * Capture runs on a private stream; nothing is enqueued on any caller stream.
 * Errors of the captured calls are returned as they would be eagerly;
 * KV_E_DEVICE if capture or instantiation fails. */
typedef struct kv_step_graph kv_step_graph;
kv_status kv_decode_step_graph_create(const kv_pool* pool, uint32_t B, uint32_t Hq, uint32_t max_seq_len,
                                      const int32_t* d_table_rows, const int32_t* d_seq_lens, uint32_t n_layers,
                                      const void* const* d_k, const void* const* d_v, const int32_t* d_pos0,
                                      const int32_t* d_cu_tokens, uint32_t total_tokens, const void* const* d_q,
                                      float sm_scale, float* const* d_out, void* d_ws, size_t ws_bytes,
                                      kv_step_graph** out);

/* Replay the step on `stream` (ordered after earlier work on it, like an
 * eager step).  Replays on one graph share its workspace: they must not
 * overlap in time. */
kv_status kv_step_graph_launch(kv_step_graph* graph, hipStream_t stream);

/* Free the graph (no device synchronization; the caller makes sure no replay
 * is still running).  NULL is ignored. */
void kv_step_graph_destroy(kv_step_graph* graph);

/* 1 if decode (max_q_len == 0) or verify has a kernel for this pool and Hq. */
int paged_attn_supported(const kv_pool* pool, uint32_t Hq, uint32_t max_q_len);

/* Measurement hook.  The next paged_attn_decode, paged_attn_decode_run,
 * paged_attn_decode_append_run or paged_attn_verify call made on this thread
 * attaches `before` and `after` to the dispatch of its dominant kernel
 * (hipExtLaunchKernel: the events mark that kernel's start and end on its
 * stream, with no packets of their own), then forgets both.  The dominant kernel is the page stream of a decode (the split kernel
 * where the stream does not apply) and, for a verify, the prefill tile kernel
 * when wide chunks are present, else the page stream in chunk mode (or the
 * per-token kernel).  The events are the caller's (hipEventCreate, timing
 * enabled); hipEventElapsedTime(before, after) is then that kernel's time on
 * the stream.  Not for use under graph capture.  NULL, NULL clears;
 * KV_E_INVALID if only one is NULL. */
kv_status kv_trace_next_kernel(hipEvent_t before, hipEvent_t after);

/* Measurement: the HBM read ceiling of the paged decode's access pattern
 * (Paged KV Context Store page, consumer rules: pages are read in place, one
 * (page group, KV head) slice at a time, in table order).  Reads slices
 * i = 0 .. n_slices-1 of slice_bytes bytes at d_base + d_slice_ids[i] *
 * slice_bytes once each, with 16-byte non-temporal loads, on blocks_per_cu
 * blocks of four waves per compute unit, each block taking a contiguous
 * share of the list as the page stream does, and writes one checksum word
 * per block to d_sink (so no load is dead).  The caller times it.
 *   slice_bytes   : 8192, 16384 (a BF16 D=128 K or V slice) or 32768.
 *   blocks_per_cu : 1..8.
 *   d_sink        : >= compute units * blocks_per_cu uint32.
 * Every d_slice_ids[i] * slice_bytes + slice_bytes must lie inside the
 * caller's buffer (not checked: device data).  KV_E_INVALID on other sizes. */
kv_status kv_read_probe(const void* d_base, const int32_t* d_slice_ids, uint32_t n_slices, uint32_t slice_bytes,
                        uint32_t blocks_per_cu, uint32_t* d_sink, hipStream_t stream);

/* Detail of the last non-OK status on the calling thread ("" if none). */
const char* kv_last_error_message(void);

#ifdef __cplusplus
}
#endif
#endif /* KVSTORE_H */
