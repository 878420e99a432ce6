// pool.cpp -- host side of the paged KV context store C ABI.
//
// NInfer "Paged KV Context Store" page:
//   - homogeneous pools with fixed P, plane order and page-group count; one
//     page-group id selects slice g of every grouped plane (page-group diagram);
//   - capacity geometry L = ceil(S/P), M in [max(L, C), C*L];
//   - lease accounting allocated + reserved + available = capacity;
//   - KVAddressSpace: ordered block -> page membership, committed frontier,
//     execution-row lease, active reservation; device block-table matrix
//     [N_logical, C];
//   - ensure_mapped_to_tokens, Fork (+ worked example), writer cardinality,
//     finish/release, mapping publication order;
//   - speculative units: accepted-prefix commit, then the retained membership
//     ceil(max(committed, provisional) / P); removed trailing leases go back
//     to the address space's own reservation.
// Allocator work never runs inside a kernel (GPU-unit stability list): every
// mutation here is host metadata plus an ordered publication on the caller's
// stream.

#include <algorithm>
#include <cmath>
#include <cstring>
#include <deque>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include <hip/hip_runtime.h>

#include "internal.h"

using namespace kvs;

namespace {

thread_local std::string g_last_error;

// events of kv_trace_next_kernel, for the next attention call on this thread
thread_local hipEvent_t g_trace_before = nullptr;
thread_local hipEvent_t g_trace_after = nullptr;

kv_status fail(kv_status st, const std::string& msg) {
    g_last_error = msg;
    return st;
}

kv_status ok() { return KV_OK; }

uint32_t ceil_div(uint32_t a, uint32_t b) { return (a + b - 1) / b; }

uint32_t dtype_bytes(uint32_t dt) {
    switch (dt) {
        case KV_DT_BF16: return 2;
        case KV_DT_I8: case KV_DT_E4M3FN: case KV_DT_E2M1X2: case KV_DT_U8_E4M3: return 1;
        case KV_DT_F32: return 4;
        case KV_DT_F16: return 2;
        default: return 0;
    }
}

// Planes of one side of a closed profile (X-extent list).
struct SideSchema {
    int codec;
    uint32_t code_dt, code_x, scale_dt, scale_x;  // scale_dt == UINT32_MAX: no scale plane
};

bool side_schema(int codec, uint32_t D, SideSchema* s, uint32_t scale_dt = KV_DT_F32) {
    s->codec = codec;
    switch (codec) {
        case CODEC_BF16: *s = {codec, KV_DT_BF16, D, UINT32_MAX, 0}; return true;
        case CODEC_INT8_G64:
            if (D % 64) return false;
            *s = {codec, KV_DT_I8, D, scale_dt, D / 64}; return true;
        case CODEC_FP8_ROW: *s = {codec, KV_DT_E4M3FN, D, scale_dt, 1}; return true;
        case CODEC_NVFP4_G16:
            if (D % 16) return false;
            *s = {codec, KV_DT_E2M1X2, D / 2, KV_DT_U8_E4M3, D / 16}; return true;
    }
    return false;
}

bool profile_codecs(uint32_t profile, int* kc, int* vc) {
    switch (profile) {
        case KV_PROFILE_BF16: *kc = *vc = CODEC_BF16; return true;
        case KV_PROFILE_INT8_G64: *kc = *vc = CODEC_INT8_G64; return true;
        case KV_PROFILE_FP8_E4M3FN_ROW256: *kc = *vc = CODEC_FP8_ROW; return true;
        case KV_PROFILE_NVFP4_G16: *kc = *vc = CODEC_NVFP4_G16; return true;
        case KV_PROFILE_K8V4: *kc = CODEC_FP8_ROW; *vc = CODEC_NVFP4_G16; return true;
    }
    return false;
}

// Which codec a (code dtype, scale dtype, scale X) triple denotes (INT8-G64
// and FP8-row scales may be fp32 or binary16).
int codec_of(uint32_t code_dt, bool has_scale, uint32_t scale_dt, uint32_t scale_x, uint32_t D) {
    const bool wide = scale_dt == KV_DT_F32 || scale_dt == KV_DT_F16;
    if (code_dt == KV_DT_BF16 && !has_scale) return CODEC_BF16;
    if (code_dt == KV_DT_I8 && has_scale && wide && scale_x == D / 64) return CODEC_INT8_G64;
    if (code_dt == KV_DT_E4M3FN && has_scale && wide && scale_x == 1) return CODEC_FP8_ROW;
    if (code_dt == KV_DT_E2M1X2 && has_scale && scale_dt == KV_DT_U8_E4M3 && scale_x == D / 16)
        return CODEC_NVFP4_G16;
    return -1;
}

struct Space {
    bool live = false;
    uint32_t gen = 0;
    uint32_t row = 0;
    uint32_t frontier = 0;
    std::vector<int32_t> pages;   // logical block -> page-group id
    std::deque<int32_t> reserve;  // active reservation: page groups held for this space, FIFO
};

}  // namespace

struct kv_pool {
    KVPageGeometry geo{};
    uint32_t L = 0;
    int k_codec = 0, v_codec = 0;
    int scale16 = 0;                      // INT8-G64 / FP8-row scale planes are binary16
    int32_t sg = 1, sh = 1;               // slice number of (g, h) in every plane: g * sg + h * sh
    std::vector<LayerView> layers;
    std::vector<KVPlaneDesc> planes;
    int32_t* d_table = nullptr;           // null: host-only pool
    std::vector<int32_t> h_table;         // [C][L] host mirror
    std::deque<int32_t> free_q;
    std::vector<uint32_t> refs;
    std::vector<Space> spaces;            // slot-indexed
    std::vector<int32_t> row_owner;       // slot leasing each row, or -1

    bool device() const { return d_table != nullptr; }

    kv_status publish(uint32_t row, uint32_t b0, uint32_t b1, hipStream_t s) {
        if (!device() || b1 <= b0) return KV_OK;
        hipError_t e = launch_table_publish(d_table + size_t(row) * L + b0, h_table.data() + size_t(row) * L + b0,
                                            int32_t(b1 - b0), s);
        if (e != hipSuccess) return fail(KV_E_DEVICE, std::string("table publication: ") + hipGetErrorString(e));
        return KV_OK;
    }

    Space* lookup(kv_seq h) {
        uint32_t slot = uint32_t(h & 0xFFFFFFFFu), gen = uint32_t(h >> 32);
        if (slot >= spaces.size() || gen == 0) return nullptr;
        Space* s = &spaces[slot];
        if (!s->live || s->gen != gen) return nullptr;
        return s;
    }

    kv_status new_space(uint32_t row, kv_seq* out, Space** sp) {
        size_t slot = 0;
        while (slot < spaces.size() && spaces[slot].live) ++slot;
        if (slot == spaces.size()) spaces.emplace_back();
        Space& s = spaces[slot];
        s.live = true;
        s.gen += 1;
        if (s.gen == 0) s.gen = 1;
        s.row = row;
        s.frontier = 0;
        s.pages.clear();
        s.reserve.clear();
        row_owner[row] = int32_t(slot);
        std::fill(h_table.begin() + size_t(row) * L, h_table.begin() + size_t(row + 1) * L, -1);
        *out = (uint64_t(s.gen) << 32) | uint64_t(slot);
        *sp = &s;
        return KV_OK;
    }

    // a page group for space s: from its reservation first, else the free list
    int32_t alloc(Space* s = nullptr) {
        std::deque<int32_t>& q = (s && !s->reserve.empty()) ? s->reserve : free_q;
        int32_t g = q.front();
        q.pop_front();
        refs[g] = 1;
        return g;
    }

    uint32_t reserved_total() const {
        size_t n = 0;
        for (const Space& s : spaces)
            if (s.live) n += s.reserve.size();
        return uint32_t(n);
    }

    void unref(int32_t g) {
        if (--refs[g] == 0) free_q.push_back(g);
    }

    PoolView view(uint32_t layer) const {
        PoolView pv{};
        pv.lv = layers[layer];
        pv.table = d_table;
        pv.H = int32_t(geo.num_kv_heads);
        pv.D = int32_t(geo.head_dim);
        pv.L = int32_t(L);
        pv.C = int32_t(geo.max_concurrency);
        pv.M = int32_t(geo.num_page_groups);
        pv.k_codec = k_codec;
        pv.v_codec = v_codec;
        pv.scale16 = scale16;
        pv.sg = sg;
        pv.sh = sh;
        return pv;
    }
};

namespace kvs {

bool take_trace(hipEvent_t* before, hipEvent_t* after) {
    if (!g_trace_before) return false;
    *before = g_trace_before;
    *after = g_trace_after;
    g_trace_before = g_trace_after = nullptr;
    return true;
}

}  // namespace kvs

extern "C" {

const char* kv_last_error_message(void) { return g_last_error.c_str(); }

kv_status kv_read_probe(const void* d_base, const int32_t* d_slice_ids, uint32_t n_slices, uint32_t slice_bytes,
                        uint32_t blocks_per_cu, uint32_t* d_sink, hipStream_t stream) {
    if (!d_base || !d_slice_ids || !d_sink) return fail(KV_E_INVALID, "null device pointer");
    if (slice_bytes != 8192 && slice_bytes != 16384 && slice_bytes != 32768)
        return fail(KV_E_INVALID, "slice_bytes must be 8192, 16384 or 32768");
    if (blocks_per_cu < 1 || blocks_per_cu > 8) return fail(KV_E_INVALID, "blocks_per_cu must be 1..8");
    if (n_slices == 0) return ok();
    if (n_slices > (1u << 30)) return fail(KV_E_INVALID, "too many slices");
    const hipError_t e = launch_read_probe(d_base, d_slice_ids, int(n_slices), int(slice_bytes),
                                           read_probe_blocks(int(blocks_per_cu)), d_sink, stream);
    if (e != hipSuccess) return fail(KV_E_DEVICE, std::string("read probe: ") + hipGetErrorString(e));
    return ok();
}

kv_status kv_trace_next_kernel(hipEvent_t before, hipEvent_t after) {
    if ((before == nullptr) != (after == nullptr)) return fail(KV_E_INVALID, "before and after go together");
    g_trace_before = before;
    g_trace_after = after;
    return ok();
}

kv_status kv_profile_planes(uint32_t profile, uint32_t head_dim, KVPlaneDesc* out, uint32_t* n_inout) {
    return kv_profile_planes_ex(profile, head_dim, KV_DT_F32, out, n_inout);
}

kv_status kv_profile_planes_ex(uint32_t profile, uint32_t head_dim, uint32_t scale_dtype, KVPlaneDesc* out,
                               uint32_t* n_inout) {
    if (!n_inout) return fail(KV_E_INVALID, "n_inout is null");
    if (scale_dtype != KV_DT_F32 && scale_dtype != KV_DT_F16) return fail(KV_E_INVALID, "scale dtype is F32 or F16");
    int kc, vc;
    if (!profile_codecs(profile, &kc, &vc)) return fail(KV_E_INVALID, "unknown profile");
    SideSchema ks, vs;
    if (head_dim == 0 || !side_schema(kc, head_dim, &ks, scale_dtype) || !side_schema(vc, head_dim, &vs, scale_dtype))
        return fail(KV_E_GEOMETRY, "head_dim not divisible by the profile's groups");
    KVPlaneDesc tmp[4];
    uint32_t n = 0;
    const SideSchema* sides[2] = {&ks, &vs};
    for (int side = 0; side < 2; ++side) {
        const SideSchema* s = sides[side];
        tmp[n++] = KVPlaneDesc{0, uint32_t(side == 0 ? KV_ROLE_K_CODE : KV_ROLE_V_CODE), s->code_dt, s->code_x,
                               dtype_bytes(s->code_dt), 0, nullptr};
        if (s->scale_dt != UINT32_MAX)
            tmp[n++] = KVPlaneDesc{0, uint32_t(side == 0 ? KV_ROLE_K_SCALE : KV_ROLE_V_SCALE), s->scale_dt,
                                   s->scale_x, dtype_bytes(s->scale_dt), 0, nullptr};
    }
    if (!out || *n_inout < n) {
        *n_inout = n;
        return fail(KV_E_INVALID, "output buffer too small");
    }
    std::memcpy(out, tmp, n * sizeof(KVPlaneDesc));
    *n_inout = n;
    return ok();
}

kv_status kv_plane_bytes(const KVPageGeometry* geo, const KVPlaneDesc* plane, uint64_t* bytes) {
    if (!geo || !plane || !bytes) return fail(KV_E_INVALID, "null argument");
    *bytes = uint64_t(geo->num_page_groups) * geo->num_kv_heads * kPage * plane->x_extent * plane->elem_bytes;
    return ok();
}

kv_status kv_pool_create(const KVPageGeometry* geo, const KVPlaneDesc* planes, uint32_t n_planes,
                         int32_t* d_block_tables, const int32_t* free_order, hipStream_t stream, kv_pool** out) {
    if (!out) return fail(KV_E_INVALID, "out is null");
    *out = nullptr;
    if (!geo || (!planes && n_planes)) return fail(KV_E_INVALID, "null geometry or planes");
    const KVPageGeometry& g = *geo;
    if (g.page_size != uint32_t(kPage)) return fail(KV_E_GEOMETRY, "page_size must be 64");
    if (g.max_concurrency < 1 || g.max_concurrency > 8) return fail(KV_E_GEOMETRY, "max_concurrency not in [1, 8]");
    if (g.max_context < 1 || g.num_kv_heads < 1 || g.num_layers < 1) return fail(KV_E_GEOMETRY, "empty geometry");
    if (g.head_dim != 64 && g.head_dim != 128 && g.head_dim != 256)
        return fail(KV_E_GEOMETRY, "head_dim must be 64, 128 or 256");
    uint32_t L = ceil_div(g.max_context, kPage);
    uint64_t m_min = std::max<uint64_t>(L, g.max_concurrency), m_max = uint64_t(g.max_concurrency) * L;
    if (g.num_page_groups < m_min || g.num_page_groups > m_max)
        return fail(KV_E_GEOMETRY, "num_page_groups outside [max(L, C), C*L]");
    if (uint64_t(g.num_page_groups) * g.num_kv_heads * kPage * g.head_dim * 2 >= (uint64_t(1) << 46))
        return fail(KV_E_GEOMETRY, "plane too large");

    // resolve the plane inventory: every layer must carry the same closed profile
    std::vector<LayerView> layers(g.num_layers, LayerView{nullptr, nullptr, nullptr, nullptr});
    std::vector<KVPlaneDesc> seen(size_t(g.num_layers) * 4);
    std::vector<uint8_t> have(size_t(g.num_layers) * 4, 0);
    int layout = -1;
    for (uint32_t i = 0; i < n_planes; ++i) {
        const KVPlaneDesc& p = planes[i];
        if (p.layer >= g.num_layers || p.role > 3) return fail(KV_E_INVALID, "plane layer/role out of range");
        size_t k = size_t(p.layer) * 4 + p.role;
        if (have[k]) return fail(KV_E_INVALID, "duplicate plane");
        if (dtype_bytes(p.dtype) == 0 || p.elem_bytes != dtype_bytes(p.dtype))
            return fail(KV_E_INVALID, "bad plane dtype/elem_bytes");
        if (d_block_tables && (!p.base || (reinterpret_cast<uintptr_t>(p.base) & 255)))
            return fail(KV_E_INVALID, "plane base must be non-null and 256-byte aligned");
        if (p.layout != KV_LAYOUT_PAGE_MAJOR && p.layout != KV_LAYOUT_HEAD_MAJOR)
            return fail(KV_E_INVALID, "plane layout must be KV_LAYOUT_PAGE_MAJOR or KV_LAYOUT_HEAD_MAJOR");
        if (layout >= 0 && int(p.layout) != layout) return fail(KV_E_INVALID, "the planes of one pool share one layout");
        layout = int(p.layout);
        have[k] = 1;
        seen[k] = p;
    }
    int kc = -1, vc = -1;
    int wide_dt = -1;                     // dtype of every INT8-G64 / FP8-row scale plane
    for (uint32_t l = 0; l < g.num_layers; ++l) {
        int codecs[2];
        for (int side = 0; side < 2; ++side) {
            size_t c = size_t(l) * 4 + (side ? KV_ROLE_V_CODE : KV_ROLE_K_CODE);
            size_t s = size_t(l) * 4 + (side ? KV_ROLE_V_SCALE : KV_ROLE_K_SCALE);
            if (!have[c]) return fail(KV_E_INVALID, "missing code plane");
            int codec = codec_of(seen[c].dtype, have[s] != 0, have[s] ? seen[s].dtype : 0,
                                 have[s] ? seen[s].x_extent : 0, g.head_dim);
            SideSchema ss;
            if (codec < 0 || !side_schema(codec, g.head_dim, &ss) || seen[c].x_extent != ss.code_x)
                return fail(KV_E_INVALID, "plane inventory is not a closed profile");
            if (codec == CODEC_INT8_G64 || codec == CODEC_FP8_ROW) {
                if (wide_dt >= 0 && int(seen[s].dtype) != wide_dt)
                    return fail(KV_E_INVALID, "the scale planes of one pool share one dtype");
                wide_dt = int(seen[s].dtype);
            }
            codecs[side] = codec;
        }
        if (l == 0) {
            kc = codecs[0];
            vc = codecs[1];
        } else if (codecs[0] != kc || codecs[1] != vc) {
            return fail(KV_E_INVALID, "layers of one pool must share a profile");
        }
        // the closed profiles: symmetric ones plus K8V4 (FP8 K, NVFP4 V)
        if (kc != vc && !(kc == CODEC_FP8_ROW && vc == CODEC_NVFP4_G16))
            return fail(KV_E_INVALID, "K/V combination is not a closed profile");
        LayerView& lv = layers[l];
        lv.k_code = seen[size_t(l) * 4 + KV_ROLE_K_CODE].base;
        lv.v_code = seen[size_t(l) * 4 + KV_ROLE_V_CODE].base;
        lv.k_scale = have[size_t(l) * 4 + KV_ROLE_K_SCALE] ? seen[size_t(l) * 4 + KV_ROLE_K_SCALE].base : nullptr;
        lv.v_scale = have[size_t(l) * 4 + KV_ROLE_V_SCALE] ? seen[size_t(l) * 4 + KV_ROLE_V_SCALE].base : nullptr;
    }

    std::vector<int32_t> order(g.num_page_groups);
    if (free_order) {
        std::vector<uint8_t> hit(g.num_page_groups, 0);
        for (uint32_t i = 0; i < g.num_page_groups; ++i) {
            int32_t v = free_order[i];
            if (v < 0 || uint32_t(v) >= g.num_page_groups || hit[v])
                return fail(KV_E_INVALID, "free_order is not a permutation of [0, M)");
            hit[v] = 1;
            order[i] = v;
        }
    } else {
        for (uint32_t i = 0; i < g.num_page_groups; ++i) order[i] = int32_t(i);
    }

    kv_pool* p = new (std::nothrow) kv_pool();
    if (!p) return fail(KV_E_INVALID, "out of host memory");
    p->geo = g;
    p->L = L;
    p->k_codec = kc;
    p->v_codec = vc;
    p->scale16 = wide_dt == int(KV_DT_F16) ? 1 : 0;
    const bool head_major = layout == int(KV_LAYOUT_HEAD_MAJOR);
    p->sg = head_major ? 1 : int32_t(g.num_kv_heads);
    p->sh = head_major ? int32_t(g.num_page_groups) : 1;
    p->layers = std::move(layers);
    p->planes.assign(planes, planes + n_planes);
    p->d_table = d_block_tables;
    p->h_table.assign(size_t(g.max_concurrency) * L, -1);
    p->free_q.assign(order.begin(), order.end());
    p->refs.assign(g.num_page_groups, 0);
    p->row_owner.assign(g.max_concurrency, -1);
    if (p->device()) {
        hipError_t e = launch_table_fill(d_block_tables, int32_t(g.max_concurrency * L), -1, stream);
        if (e != hipSuccess) {
            delete p;
            return fail(KV_E_DEVICE, std::string("table init: ") + hipGetErrorString(e));
        }
    }
    *out = p;
    return ok();
}

void kv_pool_destroy(kv_pool* pool) {
    if (!pool) return;
    if (pool->device()) (void)hipDeviceSynchronize();
    delete pool;
}

kv_status kv_pool_stats(const kv_pool* pool, uint32_t* allocated, uint32_t* reserved, uint32_t* available) {
    if (!pool) return fail(KV_E_INVALID, "null pool");
    uint32_t avail = uint32_t(pool->free_q.size()), held = pool->reserved_total();
    if (allocated) *allocated = pool->geo.num_page_groups - avail - held;
    if (reserved) *reserved = held;
    if (available) *available = avail;
    return ok();
}

kv_status kv_pool_table_host(const kv_pool* pool, int32_t* out, size_t n_entries) {
    if (!pool || !out) return fail(KV_E_INVALID, "null argument");
    if (n_entries < pool->h_table.size()) return fail(KV_E_INVALID, "buffer smaller than C*L");
    std::memcpy(out, pool->h_table.data(), pool->h_table.size() * sizeof(int32_t));
    return ok();
}

kv_status kv_pool_page_refs(const kv_pool* pool, uint32_t page_group, uint32_t* refs) {
    if (!pool || !refs) return fail(KV_E_INVALID, "null argument");
    if (page_group >= pool->geo.num_page_groups) return fail(KV_E_INVALID, "page group out of range");
    *refs = pool->refs[page_group];
    return ok();
}

kv_status kv_seq_open(kv_pool* pool, uint32_t table_row, hipStream_t stream, kv_seq* out) {
    if (!pool || !out) return fail(KV_E_INVALID, "null argument");
    if (table_row >= pool->geo.max_concurrency || pool->row_owner[table_row] >= 0)
        return fail(KV_E_INVALID, "table row out of range or leased");
    Space* s;
    kv_status st = pool->new_space(table_row, out, &s);
    if (st != KV_OK) return st;
    return pool->publish(table_row, 0, pool->L, stream);
}

kv_status kv_seq_fork(kv_pool* pool, kv_seq src, uint32_t frontier, uint32_t table_row, hipStream_t stream,
                      kv_seq* out) {
    if (!pool || !out) return fail(KV_E_INVALID, "null argument");
    Space* s = pool->lookup(src);
    if (!s) return fail(KV_E_STALE, "stale or unknown source handle");
    if (frontier > s->frontier) return fail(KV_E_INVALID, "fork frontier beyond the committed frontier");
    if (table_row >= pool->geo.max_concurrency || pool->row_owner[table_row] >= 0)
        return fail(KV_E_INVALID, "table row out of range or leased");
    size_t src_slot = size_t(s - pool->spaces.data());
    Space* d;
    kv_status st = pool->new_space(table_row, out, &d);   // may grow spaces: re-read source
    if (st != KV_OK) return st;
    s = &pool->spaces[src_slot];
    uint32_t n = ceil_div(frontier, kPage);
    d->pages.assign(s->pages.begin(), s->pages.begin() + n);
    for (int32_t g : d->pages) pool->refs[g] += 1;
    d->frontier = frontier;
    std::copy(d->pages.begin(), d->pages.end(), pool->h_table.begin() + size_t(table_row) * pool->L);
    return pool->publish(table_row, 0, pool->L, stream);
}

kv_status kv_seq_ensure_mapped(kv_pool* pool, kv_seq seq, uint32_t tokens, uint32_t* deficit, hipStream_t stream) {
    if (deficit) *deficit = 0;
    if (!pool) return fail(KV_E_INVALID, "null pool");
    Space* s = pool->lookup(seq);
    if (!s) return fail(KV_E_STALE, "stale or unknown handle");
    if (tokens > pool->geo.max_context) return fail(KV_E_INVALID, "tokens beyond max_context");
    if (tokens > s->frontier && (s->frontier % kPage)) {
        uint32_t tail = s->frontier / kPage;
        if (tail < s->pages.size() && pool->refs[s->pages[tail]] > 1)
            return fail(KV_E_SHARED_WRITE, "write into a shared partial tail; copy it first");
    }
    uint32_t need_pages = ceil_div(tokens, kPage);
    uint32_t have = uint32_t(s->pages.size());
    if (need_pages <= have) return ok();
    uint32_t need = need_pages - have;
    uint32_t can = uint32_t(s->reserve.size() + pool->free_q.size());
    if (need > can) {
        if (deficit) *deficit = need - can;
        return fail(KV_E_CAPACITY, "not enough free page groups");
    }
    for (uint32_t i = 0; i < need; ++i) {
        int32_t g = pool->alloc(s);
        s->pages.push_back(g);
        pool->h_table[size_t(s->row) * pool->L + s->pages.size() - 1] = g;
    }
    return pool->publish(s->row, have, need_pages, stream);
}

kv_status kv_seq_commit(kv_pool* pool, kv_seq seq, uint32_t frontier) {
    if (!pool) return fail(KV_E_INVALID, "null pool");
    Space* s = pool->lookup(seq);
    if (!s) return fail(KV_E_STALE, "stale or unknown handle");
    if (frontier < s->frontier) return fail(KV_E_INVALID, "frontier moves backwards");
    if (uint64_t(frontier) > uint64_t(kPage) * s->pages.size()) return fail(KV_E_UNMAPPED, "commit beyond mapping");
    s->frontier = frontier;
    return ok();
}

kv_status kv_seq_release(kv_pool* pool, kv_seq seq, hipStream_t stream) {
    if (!pool) return fail(KV_E_INVALID, "null pool");
    Space* s = pool->lookup(seq);
    if (!s) return fail(KV_E_STALE, "stale or unknown handle");
    for (int32_t g : s->pages) pool->unref(g);
    s->pages.clear();
    pool->free_q.insert(pool->free_q.end(), s->reserve.begin(), s->reserve.end());
    s->reserve.clear();
    s->live = false;
    uint32_t row = s->row;
    pool->row_owner[row] = -1;
    std::fill(pool->h_table.begin() + size_t(row) * pool->L, pool->h_table.begin() + size_t(row + 1) * pool->L, -1);
    return pool->publish(row, 0, pool->L, stream);
}

kv_status kv_seq_reserve(kv_pool* pool, kv_seq seq, uint32_t pages, uint32_t* deficit) {
    if (deficit) *deficit = 0;
    if (!pool) return fail(KV_E_INVALID, "null pool");
    Space* s = pool->lookup(seq);
    if (!s) return fail(KV_E_STALE, "stale or unknown handle");
    if (pages > pool->free_q.size()) {
        if (deficit) *deficit = pages - uint32_t(pool->free_q.size());
        return fail(KV_E_CAPACITY, "not enough free page groups to reserve");
    }
    for (uint32_t i = 0; i < pages; ++i) {
        s->reserve.push_back(pool->free_q.front());
        pool->free_q.pop_front();
    }
    return ok();
}

kv_status kv_seq_trim(kv_pool* pool, kv_seq seq, uint32_t provisional, hipStream_t stream) {
    if (!pool) return fail(KV_E_INVALID, "null pool");
    Space* s = pool->lookup(seq);
    if (!s) return fail(KV_E_STALE, "stale or unknown handle");
    if (provisional > pool->geo.max_context) return fail(KV_E_INVALID, "provisional extent beyond max_context");
    const uint32_t keep = ceil_div(std::max(s->frontier, provisional), kPage);
    const uint32_t have = uint32_t(s->pages.size());
    if (keep >= have) return ok();
    for (uint32_t b = keep; b < have; ++b) {
        const int32_t g = s->pages[b];
        if (--pool->refs[g] == 0) s->reserve.push_back(g);
        pool->h_table[size_t(s->row) * pool->L + b] = -1;
    }
    s->pages.resize(keep);
    return pool->publish(s->row, keep, have, stream);
}

kv_status kv_seq_commit_accepted(kv_pool* pool, kv_seq seq, uint32_t produced, uint32_t accepted, int cancelled,
                                 hipStream_t stream) {
    if (!pool) return fail(KV_E_INVALID, "null pool");
    Space* s = pool->lookup(seq);
    if (!s) return fail(KV_E_STALE, "stale or unknown handle");
    if (produced < 1) return fail(KV_E_INVALID, "a speculative unit produces at least one row");
    if (cancelled ? accepted != 0 : (accepted < 1 || accepted > produced))
        return fail(KV_E_INVALID, "accepted rows outside [1, produced] (0 for a cancelled row)");
    if (uint64_t(s->frontier) + produced > uint64_t(kPage) * s->pages.size())
        return fail(KV_E_UNMAPPED, "produced rows beyond the mapping");
    s->frontier += accepted;
    return kv_seq_trim(pool, seq, s->frontier, stream);
}

kv_status kv_seq_reservation(const kv_pool* pool, kv_seq seq, uint32_t* pages) {
    if (!pool || !pages) return fail(KV_E_INVALID, "null argument");
    Space* s = const_cast<kv_pool*>(pool)->lookup(seq);
    if (!s) return fail(KV_E_STALE, "stale or unknown handle");
    *pages = uint32_t(s->reserve.size());
    return ok();
}

kv_status kv_draft_pool_pages(uint32_t main_pages, uint32_t max_concurrency, uint32_t draft_window,
                              uint32_t* pages) {
    if (!pages) return fail(KV_E_INVALID, "null argument");
    if (draft_window < 1) return fail(KV_E_INVALID, "draft window must be >= 1");
    const uint64_t n = uint64_t(main_pages) + uint64_t(max_concurrency) * ceil_div(draft_window - 1, kPage);
    if (n > UINT32_MAX) return fail(KV_E_GEOMETRY, "draft pool too large");
    *pages = uint32_t(n);
    return ok();
}

// ----------------------------------------------------------- host replica --
// Planes of a replica page in their order (layers ascending, then K code,
// K scale, V code, V scale) with each slice's offset inside the page.
static uint64_t replica_planes(const kv_pool* pool, std::vector<ReplicaPlane>* out) {
    out->clear();
    uint64_t off = 0;
    const uint32_t H = pool->geo.num_kv_heads;
    for (uint32_t l = 0; l < pool->geo.num_layers; ++l) {
        for (uint32_t role = 0; role < 4; ++role) {
            for (const KVPlaneDesc& p : pool->planes) {
                if (p.layer != l || p.role != role) continue;
                const uint32_t head = kPage * p.x_extent * p.elem_bytes;
                out->push_back(ReplicaPlane{p.base, head, off});
                off += uint64_t(H) * head;
            }
        }
    }
    return off;
}

// The device-visible address of pinned host memory, or null.
static char* host_device_ptr(const void* host) {
    void* d = nullptr;
    if (!host || (reinterpret_cast<uintptr_t>(host) & 15)) return nullptr;
    if (hipHostGetDevicePointer(&d, const_cast<void*>(host), 0) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    return static_cast<char*>(d);
}

kv_status kv_replica_page_bytes(const kv_pool* pool, uint64_t* bytes) {
    if (!pool || !bytes) return fail(KV_E_INVALID, "null argument");
    std::vector<ReplicaPlane> planes;
    *bytes = replica_planes(pool, &planes);
    return ok();
}

kv_status kv_seq_offload(kv_pool* pool, kv_seq seq, void* host, size_t host_bytes, uint32_t* pages,
                         uint32_t* frontier, hipStream_t stream) {
    if (!pool) return fail(KV_E_INVALID, "null pool");
    if (!pool->device()) return fail(KV_E_INVALID, "host-only pool has no device planes");
    Space* s = pool->lookup(seq);
    if (!s) return fail(KV_E_STALE, "stale or unknown handle");
    std::vector<ReplicaPlane> planes;
    const uint64_t pb = replica_planes(pool, &planes);
    const uint32_t n = ceil_div(s->frontier, kPage);
    if (uint64_t(host_bytes) < pb * n) return fail(KV_E_INVALID, "host buffer smaller than the replica");
    char* dhost = n ? host_device_ptr(host) : nullptr;
    if (n && !dhost) return fail(KV_E_INVALID, "host buffer must be 16-byte aligned pinned memory (hipHostMalloc)");
    if (pages) *pages = n;
    if (frontier) *frontier = s->frontier;
    if (n == 0) return ok();
    const hipError_t e = launch_replica_copy(planes.data(), int(planes.size()), s->pages.data(), int(n), pb,
                                             int(pool->geo.num_kv_heads), pool->sg, pool->sh, dhost, true, stream);
    if (e != hipSuccess) return fail(KV_E_DEVICE, std::string("replica copy: ") + hipGetErrorString(e));
    return ok();
}

kv_status kv_seq_restore(kv_pool* pool, uint32_t table_row, const void* host, size_t host_bytes, uint32_t frontier,
                         uint32_t* deficit, hipStream_t stream, kv_seq* out) {
    if (deficit) *deficit = 0;
    if (!pool || !out) return fail(KV_E_INVALID, "null argument");
    if (!pool->device()) return fail(KV_E_INVALID, "host-only pool has no device planes");
    if (table_row >= pool->geo.max_concurrency || pool->row_owner[table_row] >= 0)
        return fail(KV_E_INVALID, "table row out of range or leased");
    if (frontier > pool->geo.max_context) return fail(KV_E_INVALID, "frontier beyond max_context");
    std::vector<ReplicaPlane> planes;
    const uint64_t pb = replica_planes(pool, &planes);
    const uint32_t n = ceil_div(frontier, kPage);
    if (uint64_t(host_bytes) < pb * n) return fail(KV_E_INVALID, "host buffer smaller than the replica");
    char* dhost = n ? host_device_ptr(host) : nullptr;
    if (n && !dhost) return fail(KV_E_INVALID, "host buffer must be 16-byte aligned pinned memory (hipHostMalloc)");
    if (n > pool->free_q.size()) {
        if (deficit) *deficit = n - uint32_t(pool->free_q.size());
        return fail(KV_E_CAPACITY, "not enough free page groups for the replica");
    }
    Space* s;
    kv_status st = pool->new_space(table_row, out, &s);
    if (st != KV_OK) return st;
    for (uint32_t i = 0; i < n; ++i) {
        const int32_t g = pool->alloc(s);
        s->pages.push_back(g);
        pool->h_table[size_t(table_row) * pool->L + i] = g;
    }
    s->frontier = frontier;
    // the payload lands before the row names the pages: copy, then publish
    if (n) {
        const hipError_t e = launch_replica_copy(planes.data(), int(planes.size()), s->pages.data(), int(n), pb,
                                                 int(pool->geo.num_kv_heads), pool->sg, pool->sh, dhost, false,
                                                 stream);
        if (e != hipSuccess) {
            (void)kv_seq_release(pool, *out, stream);
            *out = 0;
            return fail(KV_E_DEVICE, std::string("replica copy: ") + hipGetErrorString(e));
        }
    }
    return pool->publish(table_row, 0, pool->L, stream);
}

kv_status kv_seq_info(const kv_pool* pool, kv_seq seq, uint32_t* table_row, uint32_t* frontier,
                      uint32_t* mapped_pages) {
    if (!pool) return fail(KV_E_INVALID, "null pool");
    Space* s = const_cast<kv_pool*>(pool)->lookup(seq);
    if (!s) return fail(KV_E_STALE, "stale or unknown handle");
    if (table_row) *table_row = s->row;
    if (frontier) *frontier = s->frontier;
    if (mapped_pages) *mapped_pages = uint32_t(s->pages.size());
    return ok();
}

kv_status kv_cow_tail_page(kv_pool* pool, kv_seq seq, hipStream_t stream) {
    if (!pool) return fail(KV_E_INVALID, "null pool");
    Space* s = pool->lookup(seq);
    if (!s) return fail(KV_E_STALE, "stale or unknown handle");
    uint32_t cols = s->frontier % kPage;
    if (cols == 0) return ok();
    uint32_t b = s->frontier / kPage;
    int32_t src = s->pages[b];
    if (pool->refs[src] == 1) return ok();
    if (s->reserve.empty() && pool->free_q.empty()) return fail(KV_E_CAPACITY, "no free page group for the tail copy");
    const bool from_reserve = !s->reserve.empty();
    int32_t dst = pool->alloc(s);
    if (pool->device()) {
        std::vector<CopyPlane> cp;
        cp.reserve(pool->planes.size());
        for (const KVPlaneDesc& p : pool->planes) cp.push_back(CopyPlane{p.base, p.x_extent * p.elem_bytes});
        hipError_t e = launch_cow_copy(cp.data(), int(cp.size()), int(pool->geo.num_kv_heads), pool->sg, pool->sh,
                                       src, dst, int(cols), stream);
        if (e != hipSuccess) {
            pool->refs[dst] = 0;   // back to the front of the queue it came from
            (from_reserve ? s->reserve : pool->free_q).push_front(dst);
            return fail(KV_E_DEVICE, std::string("tail copy: ") + hipGetErrorString(e));
        }
    }
    s->pages[b] = dst;
    pool->h_table[size_t(s->row) * pool->L + b] = dst;
    pool->unref(src);
    return pool->publish(s->row, b, b + 1, stream);
}

// ---------------------------------------------------------------- kernels --
static kv_status check_compute(const kv_pool* pool, uint32_t layer, uint32_t B) {
    if (!pool) return fail(KV_E_INVALID, "null pool");
    if (!pool->device()) return fail(KV_E_INVALID, "host-only pool has no device planes");
    if (layer >= pool->geo.num_layers) return fail(KV_E_INVALID, "layer out of range");
    if (B > pool->geo.max_concurrency) return fail(KV_E_GEOMETRY, "batch larger than max_concurrency");
    return KV_OK;
}

kv_status kv_append(const kv_pool* pool, uint32_t layer, uint32_t B, const int32_t* d_table_rows,
                    const int32_t* d_pos0, const int32_t* d_cu_tokens, uint32_t total_tokens, const void* d_k,
                    const void* d_v, hipStream_t stream) {
    kv_status st = check_compute(pool, layer, B);
    if (st != KV_OK) return st;
    if (total_tokens == 0 || B == 0) return ok();
    if (!d_table_rows || !d_pos0 || !d_cu_tokens || !d_k || !d_v) return fail(KV_E_INVALID, "null device pointer");
    if (uint64_t(total_tokens) * pool->geo.num_kv_heads > (uint64_t(1) << 31))
        return fail(KV_E_INVALID, "too many rows for one launch");
    hipError_t e = launch_append(pool->view(layer), int(B), d_table_rows, d_pos0, d_cu_tokens, int(total_tokens),
                                 d_k, d_v, stream);
    if (e != hipSuccess) return fail(KV_E_DEVICE, std::string("append launch: ") + hipGetErrorString(e));
    return ok();
}

size_t paged_attn_workspace_bytes(const kv_pool* pool, uint32_t B, uint32_t Hq, uint32_t max_seq_len,
                                  uint32_t max_q_len) {
    if (!pool || pool->geo.num_layers == 0) return 0;
    PoolView pv = pool->view(0);
    if (max_q_len == 0) return decode_workspace_bytes(pv, int(B), int(Hq), int(max_seq_len));
    return verify_workspace_bytes(pv, int(B), int(Hq), int(max_seq_len), int(max_q_len));
}

int paged_attn_supported(const kv_pool* pool, uint32_t Hq, uint32_t max_q_len) {
    if (!pool || pool->geo.num_layers == 0) return 0;
    PoolView pv = pool->view(0);
    return max_q_len == 0 ? int(decode_supported(pv, int(Hq))) : int(verify_supported(pv, int(Hq)));
}

// Shared checks of the decode entry points; *skip is set when B == 0 (a
// call with nothing to do).
static kv_status check_decode(const kv_pool* pool, uint32_t layer, uint32_t B, uint32_t Hq, uint32_t max_seq_len,
                              void* d_ws, size_t ws_bytes, bool* skip) {
    *skip = false;
    kv_status st = check_compute(pool, layer, B);
    if (st != KV_OK) return st;
    if (Hq == 0 || Hq % pool->geo.num_kv_heads) return fail(KV_E_GEOMETRY, "Hq must be a multiple of H");
    if (B == 0) {
        *skip = true;
        return ok();
    }
    if (max_seq_len > pool->geo.max_context) return fail(KV_E_INVALID, "max_seq_len beyond max_context");
    PoolView pv = pool->view(layer);
    if (!decode_supported(pv, int(Hq))) return fail(KV_E_UNSUPPORTED, "no decode kernel for this shape");
    size_t need = decode_workspace_bytes(pv, int(B), int(Hq), int(max_seq_len));
    if (need && (!d_ws || ws_bytes < need)) return fail(KV_E_INVALID, "workspace too small");
    return ok();
}

kv_status paged_attn_decode(const kv_pool* pool, uint32_t layer, uint32_t B, uint32_t Hq,
                            const int32_t* d_table_rows, const int32_t* d_seq_lens, uint32_t max_seq_len,
                            const void* d_q, float sm_scale, float* d_out, void* d_ws, size_t ws_bytes,
                            hipStream_t stream) {
    bool skip = false;
    kv_status st = check_decode(pool, layer, B, Hq, max_seq_len, d_ws, ws_bytes, &skip);
    if (st != KV_OK) return st;
    if (!(sm_scale > 0.f) || !std::isfinite(sm_scale)) return fail(KV_E_INVALID, "sm_scale must be finite and > 0");
    if (skip) return ok();
    if (!d_table_rows || !d_seq_lens || !d_q || !d_out) return fail(KV_E_INVALID, "null device pointer");
    hipError_t e = launch_decode(pool->view(layer), int(B), int(Hq), d_table_rows, d_seq_lens, int(max_seq_len), d_q,
                                 sm_scale, d_out, d_ws, stream);
    if (e != hipSuccess) return fail(KV_E_DEVICE, std::string("decode launch: ") + hipGetErrorString(e));
    return ok();
}

}  // extern "C"

// ------------------------------------------------- decode without a workspace --
// The scratch of paged_attn_decode_noalloc: a file-scope device array, one
// copy per GPU the library runs on, held until the process ends.  In host
// code `scratch` names a host-side stand-in, never the device memory: host
// code uses only the address hipGetSymbolAddress returns for the current
// device, kept per device.
static __device__ __align__(256) unsigned char scratch[KV_DECODE_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// The current device's copy of `scratch`, looked up once per device.
kv_status scratch_of_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices)
        return fail(KV_E_DEVICE, "no current device for the decode scratch");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(KV_E_DEVICE, std::string("decode scratch address: ") + hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return KV_OK;
}

}  // namespace

extern "C" {

kv_status paged_attn_decode_noalloc(const kv_pool* pool, uint32_t layer, uint32_t B, uint32_t Hq,
                                    const int32_t* d_table_rows, const int32_t* d_seq_lens, uint32_t max_seq_len,
                                    const void* d_q, float sm_scale, float* d_out, hipStream_t stream) {
    kv_status st = check_compute(pool, layer, B);
    if (st != KV_OK) return st;
    if (Hq == 0 || Hq % pool->geo.num_kv_heads) return fail(KV_E_GEOMETRY, "Hq must be a multiple of H");
    if (B == 0) return ok();
    if (max_seq_len > pool->geo.max_context) return fail(KV_E_INVALID, "max_seq_len beyond max_context");
    const size_t need = decode_workspace_bytes(pool->view(layer), int(B), int(Hq), int(max_seq_len));
    if (need > size_t(KV_DECODE_SCRATCH_BYTES))
        return fail(KV_E_INVALID, "this decode needs a workspace of " + std::to_string(need) +
                                      " bytes, more than the static scratch of " +
                                      std::to_string(size_t(KV_DECODE_SCRATCH_BYTES)) +
                                      " bytes: use paged_attn_decode with a workspace");
    void* ws = nullptr;
    st = scratch_of_current_device(&ws);
    if (st != KV_OK) return st;
    return paged_attn_decode(pool, layer, B, Hq, d_table_rows, d_seq_lens, max_seq_len, d_q, sm_scale, d_out, ws,
                             size_t(KV_DECODE_SCRATCH_BYTES), stream);
}

kv_status paged_attn_decode_plan(const kv_pool* pool, uint32_t B, uint32_t Hq, const int32_t* d_table_rows,
                                 const int32_t* d_seq_lens, uint32_t max_seq_len, void* d_ws, size_t ws_bytes,
                                 hipStream_t stream) {
    bool skip = false;
    kv_status st = check_decode(pool, 0, B, Hq, max_seq_len, d_ws, ws_bytes, &skip);
    if (st != KV_OK || skip) return st;
    if (!d_table_rows || !d_seq_lens) return fail(KV_E_INVALID, "null device pointer");
    hipError_t e = launch_decode_plan(pool->view(0), int(B), int(Hq), d_table_rows, d_seq_lens, int(max_seq_len),
                                      d_ws, stream);
    if (e != hipSuccess) return fail(KV_E_DEVICE, std::string("decode plan launch: ") + hipGetErrorString(e));
    return ok();
}

kv_status paged_attn_decode_run(const kv_pool* pool, uint32_t layer, uint32_t B, uint32_t Hq, uint32_t max_seq_len,
                                const void* d_q, float sm_scale, float* d_out, void* d_ws, size_t ws_bytes,
                                hipStream_t stream) {
    bool skip = false;
    kv_status st = check_decode(pool, layer, B, Hq, max_seq_len, d_ws, ws_bytes, &skip);
    if (st != KV_OK) return st;
    if (!(sm_scale > 0.f) || !std::isfinite(sm_scale)) return fail(KV_E_INVALID, "sm_scale must be finite and > 0");
    if (skip) return ok();
    if (!d_q || !d_out) return fail(KV_E_INVALID, "null device pointer");
    hipError_t e = launch_decode_run(pool->view(layer), int(B), int(Hq), int(max_seq_len), d_q, sm_scale, d_out,
                                     d_ws, stream);
    if (e != hipSuccess) return fail(KV_E_DEVICE, std::string("decode run launch: ") + hipGetErrorString(e));
    return ok();
}

kv_status paged_attn_decode_append_run(const kv_pool* pool, uint32_t layer, uint32_t B, uint32_t Hq,
                                       uint32_t max_seq_len, const void* d_k, const void* d_v, const void* d_q,
                                       float sm_scale, float* d_out, void* d_ws, size_t ws_bytes, hipStream_t stream) {
    bool skip = false;
    kv_status st = check_decode(pool, layer, B, Hq, max_seq_len, d_ws, ws_bytes, &skip);
    if (st != KV_OK) return st;
    if (!(sm_scale > 0.f) || !std::isfinite(sm_scale)) return fail(KV_E_INVALID, "sm_scale must be finite and > 0");
    if (skip) return ok();
    if (!d_k || !d_v || !d_q || !d_out) return fail(KV_E_INVALID, "null device pointer");
    PoolView pv = pool->view(layer);
    if (!decode_append_supported(pv, int(B), int(Hq)))
        return fail(KV_E_UNSUPPORTED, "append in the decode run needs a matrix-core page stream; use kv_append");
    hipError_t e = launch_decode_run(pv, int(B), int(Hq), int(max_seq_len), d_q, sm_scale, d_out, d_ws, stream, d_k,
                                     d_v);
    if (e != hipSuccess) return fail(KV_E_DEVICE, std::string("decode run launch: ") + hipGetErrorString(e));
    return ok();
}

kv_status paged_attn_verify(const kv_pool* pool, uint32_t layer, uint32_t B, uint32_t Hq,
                            const int32_t* d_table_rows, const int32_t* d_q_pos0, const int32_t* d_cu_q,
                            uint32_t total_q, uint32_t max_q_len, uint32_t max_seq_len, const void* d_q,
                            float sm_scale, float* d_out, void* d_ws, size_t ws_bytes, hipStream_t stream) {
    kv_status st = check_compute(pool, layer, B);
    if (st != KV_OK) return st;
    if (Hq == 0 || Hq % pool->geo.num_kv_heads) return fail(KV_E_GEOMETRY, "Hq must be a multiple of H");
    if (!(sm_scale > 0.f) || !std::isfinite(sm_scale)) return fail(KV_E_INVALID, "sm_scale must be finite and > 0");
    if (B == 0 || total_q == 0) return ok();
    if (!d_table_rows || !d_q_pos0 || !d_cu_q || !d_q || !d_out) return fail(KV_E_INVALID, "null device pointer");
    if (max_seq_len > pool->geo.max_context) return fail(KV_E_INVALID, "max_seq_len beyond max_context");
    if (max_q_len == 0 || max_q_len > max_seq_len) return fail(KV_E_INVALID, "bad max_q_len");
    PoolView pv = pool->view(layer);
    if (!verify_supported(pv, int(Hq))) return fail(KV_E_UNSUPPORTED, "no verify kernel for this shape/profile");
    size_t need = verify_workspace_bytes(pv, int(B), int(Hq), int(max_seq_len), int(max_q_len));
    if (need && (!d_ws || ws_bytes < need)) return fail(KV_E_INVALID, "workspace too small");
    hipError_t e = launch_verify(pv, int(B), int(Hq), d_table_rows, d_q_pos0, d_cu_q, int(total_q), int(max_q_len),
                                 int(max_seq_len), d_q, sm_scale, d_out, d_ws, ws_bytes, stream);
    if (e != hipSuccess) return fail(KV_E_DEVICE, std::string("verify launch: ") + hipGetErrorString(e));
    return ok();
}

}  // extern "C"

// ------------------------------------------------------------ step graph --
// One decode step of many layers as a HIP graph (Paged KV Context Store page:
// plane and table bases stay stable across graph replays; page ids, table
// rows, lengths and positions are data the kernels read on the device, not
// part of what is captured; one graph per exact batch size).  The step is the
// plan of the batch state and, per layer, the append of the step's rows with
// the decode run -- the entry points of an eager step, recorded once on a
// private stream.  Mapping publication stays outside: it carries host values
// in its arguments and is host-side allocator work done before a step.
struct kv_step_graph {
    hipGraphExec_t exec = nullptr;
};

extern "C" {

kv_status kv_decode_step_graph_create(const kv_pool* pool, uint32_t B, uint32_t Hq, uint32_t max_seq_len,
                                      const int32_t* d_table_rows, const int32_t* d_seq_lens, uint32_t n_layers,
                                      const void* const* d_k, const void* const* d_v, const int32_t* d_pos0,
                                      const int32_t* d_cu_tokens, uint32_t total_tokens, const void* const* d_q,
                                      float sm_scale, float* const* d_out, void* d_ws, size_t ws_bytes,
                                      kv_step_graph** out) {
    if (!out) return fail(KV_E_INVALID, "null argument");
    *out = nullptr;
    kv_status st = check_compute(pool, 0, B);
    if (st != KV_OK) return st;
    if (!d_q || !d_out || n_layers == 0 || n_layers > pool->geo.num_layers || B == 0)
        return fail(KV_E_INVALID, "layers, batch or pointer arrays");
    const bool append = d_k != nullptr;
    if (append != (d_v != nullptr)) return fail(KV_E_INVALID, "d_k and d_v go together");
    // which append form: without positions, one row per entry at seq_len - 1
    // inside the run (the matrix-core page streams); with them, kv_append + run
    if ((d_pos0 == nullptr) != (d_cu_tokens == nullptr))
        return fail(KV_E_INVALID, "d_pos0 and d_cu_tokens go together");
    const bool fused = append && !d_pos0;
    if (fused && (total_tokens != B || !decode_append_supported(pool->view(0), int(B), int(Hq))))
        return fail(KV_E_UNSUPPORTED,
                    "the append inside the run takes one row per entry on the matrix-core page streams; "
                    "pass d_pos0 and d_cu_tokens for kv_append");

    hipStream_t s = nullptr;
    if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess)
        return fail(KV_E_DEVICE, "capture stream");
    if (hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal) != hipSuccess) {
        (void)hipStreamDestroy(s);
        return fail(KV_E_DEVICE, "begin capture");
    }
    st = paged_attn_decode_plan(pool, B, Hq, d_table_rows, d_seq_lens, max_seq_len, d_ws, ws_bytes, s);
    std::string why = st == KV_OK ? "" : g_last_error;
    for (uint32_t l = 0; l < n_layers && st == KV_OK; ++l) {
        if (!d_q[l] || !d_out[l] || (append && (!d_k[l] || !d_v[l]))) {
            st = KV_E_INVALID;
            why = "null device pointer of a layer";
            break;
        }
        if (fused) {
            st = paged_attn_decode_append_run(pool, l, B, Hq, max_seq_len, d_k[l], d_v[l], d_q[l], sm_scale,
                                              d_out[l], d_ws, ws_bytes, s);
        } else {
            if (append)
                st = kv_append(pool, l, B, d_table_rows, d_pos0, d_cu_tokens, total_tokens, d_k[l], d_v[l], s);
            if (st == KV_OK)
                st = paged_attn_decode_run(pool, l, B, Hq, max_seq_len, d_q[l], sm_scale, d_out[l], d_ws, ws_bytes,
                                           s);
        }
        if (st != KV_OK) why = g_last_error;
    }
    hipGraph_t graph = nullptr;
    const hipError_t ec = hipStreamEndCapture(s, &graph);
    (void)hipStreamDestroy(s);
    if (st != KV_OK || ec != hipSuccess || !graph) {
        if (graph) (void)hipGraphDestroy(graph);
        if (st != KV_OK) return fail(st, "step graph: " + why);
        return fail(KV_E_DEVICE, std::string("end capture: ") + hipGetErrorString(ec));
    }
    hipGraphExec_t exec = nullptr;
    const hipError_t ei = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (ei != hipSuccess) return fail(KV_E_DEVICE, std::string("instantiate: ") + hipGetErrorString(ei));
    kv_step_graph* g = new (std::nothrow) kv_step_graph();
    if (!g) {
        (void)hipGraphExecDestroy(exec);
        return fail(KV_E_INVALID, "out of host memory");
    }
    g->exec = exec;
    *out = g;
    return ok();
}

kv_status kv_step_graph_launch(kv_step_graph* g, hipStream_t stream) {
    if (!g || !g->exec) return fail(KV_E_INVALID, "null graph");
    const hipError_t e = hipGraphLaunch(g->exec, stream);
    if (e != hipSuccess) return fail(KV_E_DEVICE, std::string("graph launch: ") + hipGetErrorString(e));
    return ok();
}

void kv_step_graph_destroy(kv_step_graph* g) {
    if (!g) return;
    if (g->exec) (void)hipGraphExecDestroy(g->exec);
    delete g;
}

}  // extern "C"
