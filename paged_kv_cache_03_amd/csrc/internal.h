// internal.h -- structures shared by the host layer (pool.cpp) and the HIP
// kernel launchers.  Not part of the C ABI.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include <hip/hip_runtime_api.h>

#include "../../include/kvstore.h"

namespace kvs {

constexpr int kPage = 64;          // P (granularity table: allocation granularity 64)
constexpr int kPageShift = 6;      // position >> 6 == logical block (P=64 translation)

// Storage kind of one side (K or V) of a closed profile.
enum Codec : int { CODEC_BF16 = 0, CODEC_INT8_G64 = 1, CODEC_FP8_ROW = 2, CODEC_NVFP4_G16 = 3 };

// Device-side view of one layer's planes (PagedKVLayerView without the table row).
struct LayerView {
    void* k_code;
    void* k_scale;   // nullptr for BF16
    void* v_code;
    void* v_scale;   // nullptr for BF16
};

// Everything a kernel needs to address a pool; passed by value.
struct PoolView {
    LayerView lv;
    const int32_t* table;   // [C][L]
    int32_t H;
    int32_t D;
    int32_t L;
    int32_t C;
    int32_t M;
    int32_t k_codec;
    int32_t v_codec;
    int32_t scale16;        // 1: INT8-G64 / FP8-row scale planes hold binary16 (2 bytes), else fp32
    // slice (g, h) of every plane -- its 64 rows of X elements -- is slice
    // number g * sg + h * sh: page-major [X, P, H, N] (sg, sh) = (H, 1),
    // head-major [X, P, N, H] (1, M)
    int32_t sg;
    int32_t sh;
};

// Measurement hook (kv_trace_next_kernel): the events a caller asked to have
// recorded around the dominant kernel of its next attention call on this
// thread.  take_trace hands them out once (false when none are set); the
// launcher attaches them to that kernel's dispatch (launch.h).
bool take_trace(hipEvent_t* before, hipEvent_t* after);

// Launchers (defined in the .hip files).  Each returns hipSuccess or the
// first launch error; argument validation happens in pool.cpp.
hipError_t launch_table_fill(int32_t* d_table, int32_t n, int32_t value, hipStream_t s);
hipError_t launch_table_publish(int32_t* d_dst, const int32_t* host_vals, int32_t n, hipStream_t s);

struct CopyPlane {
    void* base;
    uint32_t row_bytes;   // X * elem_bytes (multiple of 4)
};
hipError_t launch_cow_copy(const CopyPlane* planes, int n_planes, int H, int sg, int sh, int src_g, int dst_g,
                           int cols, hipStream_t s);

// Host replica copy (logical-order packed layout): page i of the replica is
// pages[i], each plane's [H][64][X] image at host + i * page_bytes +
// plane.host_off, whatever the device layout (slice (g, h) of a plane at
// slice number g * sg + h * sh).  to_host: device pages -> host; else host ->
// device pages.  `host` is the device-visible address of pinned host memory.
struct ReplicaPlane {
    void* base;          // device plane
    uint32_t head_bytes; // 64 * X * elem_bytes, a multiple of 16: one (group, head) slice
    uint64_t host_off;   // offset of this plane's image inside a replica page
};
hipError_t launch_replica_copy(const ReplicaPlane* planes, int n_planes, const int32_t* pages, int n_pages,
                               uint64_t page_bytes, int H, int sg, int sh, char* host, bool to_host, hipStream_t s);

hipError_t launch_append(const PoolView& pv, int B, const int32_t* table_rows, const int32_t* pos0,
                         const int32_t* cu_tokens, int total_tokens, const void* k, const void* v,
                         hipStream_t s);

// Page-stream plans (stream_plan.hip): the work list of one batch state in
// the workspace.  chunk: several query tokens per entry (entries with more
// than max_cols columns are left out); dedup: shared leading pages are read
// once; pages: write the page list (the split kernel reads only the entry
// table).
int stream_plan_blocks(int bound);
long long stream_bound(const PoolView& pv, int B, int max_seq_len);   // B x H x ceil(max_seq_len / 64)
hipError_t launch_stream_plan(const PoolView& pv, int B, int gq, const int32_t* table_rows, const int32_t* seq_lens,
                              const int32_t* q_pos0, const int32_t* cu_q, int max_seq_len, int max_cols, bool chunk,
                              bool dedup, bool pages, int G, int qcap, int share, int32_t* plan, hipStream_t s);

// Decode: a plan of the batch state, then the run (the page stream, or split
// partials and a combine).  Returns hipErrorNotSupported for shapes with no
// kernel instance.
bool decode_supported(const PoolView& pv, int Hq);
size_t decode_workspace_bytes(const PoolView& pv, int B, int Hq, int max_seq_len);
hipError_t launch_decode_plan(const PoolView& pv, int B, int Hq, const int32_t* table_rows, const int32_t* seq_lens,
                              int max_seq_len, void* ws, hipStream_t s);
// k_new / v_new (bf16 [B][H][D], or nullptr): the step's rows, appended at
// position keys - 1 of each entry by the run itself (page stream only).
bool decode_append_supported(const PoolView& pv, int B, int Hq);
hipError_t launch_decode_run(const PoolView& pv, int B, int Hq, int max_seq_len, const void* q, float sm_scale,
                             float* out, void* ws, hipStream_t s, const void* k_new = nullptr,
                             const void* v_new = nullptr);
hipError_t launch_decode(const PoolView& pv, int B, int Hq, const int32_t* table_rows, const int32_t* seq_lens,
                         int max_seq_len, const void* q, float sm_scale, float* out, void* ws, hipStream_t s);

// The page stream in chunk mode (several query tokens per entry, causal):
// entries with at most max_cols query columns (tokens x GQ); the workspace
// layout matches decode's (arrival counters first, then the plan).
bool stream_chunk_supported(const PoolView& pv, int B, int gq);
size_t stream_chunk_workspace_bytes(const PoolView& pv, int B, int Hq, int max_seq_len);
// trace: the chunk stream is the call's dominant kernel (no tiles follow it).
hipError_t launch_stream_chunk(const PoolView& pv, int B, int Hq, const int32_t* table_rows, const int32_t* q_pos0,
                               const int32_t* cu_q, int max_seq_len, const void* q, float sm_scale, float* out,
                               void* ws, int max_cols, bool trace, hipStream_t s);

// Matrix-core tiles for verify / prefill on quantized pools (D in {64, 128,
// 256}) and BF16 pools at D = 256 (verify_gtile.hip): every entry of the call,
// each tile's page range cut into parts when the tiles alone cannot fill the
// chip; the workspace holds the parts' partial results.
bool gtile_supported(const PoolView& pv, int gq);
size_t gtile_workspace_bytes(const PoolView& pv, int B, int Hq, int max_seq_len, int max_q_len);
hipError_t launch_gtile(const PoolView& pv, int B, int Hq, const int32_t* table_rows, const int32_t* q_pos0,
                        const int32_t* cu_q, int max_q_len, int max_seq_len, const void* q, float sm_scale,
                        float* out, void* ws, hipStream_t s);

bool verify_supported(const PoolView& pv, int Hq);
size_t verify_workspace_bytes(const PoolView& pv, int B, int Hq, int max_seq_len, int max_q_len);
hipError_t launch_verify(const PoolView& pv, int B, int Hq, const int32_t* table_rows, const int32_t* q_pos0,
                         const int32_t* cu_q, int total_q, int max_q_len, int max_seq_len, const void* q,
                         float sm_scale, float* out, void* ws, size_t ws_bytes, hipStream_t s);

// Read-ceiling probe (read_probe.hip): n slices of slice_bytes at
// base + ids[i] * slice_bytes, read once each by `blocks` blocks.
int read_probe_blocks(int blocks_per_cu);
hipError_t launch_read_probe(const void* base, const int32_t* ids, int n, int slice_bytes, int blocks,
                             uint32_t* sink, hipStream_t s);

}  // namespace kvs
