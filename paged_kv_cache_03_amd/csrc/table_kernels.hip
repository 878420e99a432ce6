// table_kernels.hip -- block-table publication and partial-tail copy.
//
// Mapping publication ("Paged KV Context Store" page, mapping publication
// order): new page ids reach the device as one contiguous row slice, ordered
// on the stream before the consumer.  The slice travels inside the kernel's
// argument block, so the host mirror can change right after the call, no
// pinned staging buffer or memset node is involved, and a captured graph would
// replay the same entries.
//
// Host replica (host replica passage): D2H / H2D copies of full page payloads
// between the planes and a logical-order packed replica in pinned host
// memory.  One block per (page, plane) slice, 16 bytes per lane; the page ids
// travel in the argument block (chunks of kReplicaPages), so a restore copies
// into page groups before any table row names them.
//
// Tail COW (Fork passage): the committed columns [0, F mod 64) of every plane
// slice of the shared page group g are copied into the private group g'.  In
// the page-major order [X, P, H, N] the first `cols` columns of slice (g, h)
// are one contiguous run of cols * X * elem_bytes bytes.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>

#include "internal.h"

namespace kvs {
namespace {

constexpr int kPublishMax = 256;

struct PublishArgs {
    int32_t* dst;
    int32_t n;
    int32_t vals[kPublishMax];
};

__global__ void __launch_bounds__(256) table_publish_kernel(PublishArgs a) {
    int i = threadIdx.x;
    if (i < a.n) a.dst[i] = a.vals[i];
}

__global__ void __launch_bounds__(256) table_fill_kernel(int32_t* dst, int32_t n, int32_t v) {
    int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) dst[i] = v;
}

constexpr int kCopyMaxPlanes = 96;

struct CopyArgs {
    CopyPlane planes[kCopyMaxPlanes];
    int32_t n_planes;
    int32_t H;
    int32_t sg, sh;          // slice number of (g, h): g * sg + h * sh
    int32_t src_g;
    int32_t dst_g;
    int32_t cols;
};

// grid (n_planes, H); block 256 threads copies one contiguous run
__global__ void __launch_bounds__(256) cow_copy_kernel(CopyArgs a) {
    const int pi = blockIdx.x, h = blockIdx.y;
    const CopyPlane p = a.planes[pi];
    const size_t slab = size_t(p.row_bytes) * kPage;
    const char* src = static_cast<const char*>(p.base) + (size_t(a.src_g) * a.sg + size_t(h) * a.sh) * slab;
    char* dst = static_cast<char*>(p.base) + (size_t(a.dst_g) * a.sg + size_t(h) * a.sh) * slab;
    const size_t bytes = size_t(a.cols) * p.row_bytes;
    if ((bytes & 15) == 0) {
        const size_t n = bytes >> 4;
        for (size_t i = threadIdx.x; i < n; i += 256)
            reinterpret_cast<uint4*>(dst)[i] = reinterpret_cast<const uint4*>(src)[i];
    } else {
        const size_t n = bytes >> 2;
        for (size_t i = threadIdx.x; i < n; i += 256)
            reinterpret_cast<uint32_t*>(dst)[i] = reinterpret_cast<const uint32_t*>(src)[i];
    }
}

constexpr int kReplicaPlanes = 96;
constexpr int kReplicaPages = 64;

struct ReplicaArgs {
    ReplicaPlane planes[kReplicaPlanes];
    int32_t pages[kReplicaPages];
    int32_t n_planes;
    int32_t first_page;      // replica index of pages[0]
    uint64_t page_bytes;
    char* host;
    int32_t to_host;
    int32_t H, sg, sh;       // heads; slice number of (g, h): g * sg + h * sh
};

// grid (pages of the chunk, planes of the chunk, heads): slice (g, h) of a
// plane starts at base + (g * sg + h * sh) * head_bytes (page-major: the H
// slices of a group are adjacent), its host image at host_off + h * head_bytes
__global__ void __launch_bounds__(256) replica_copy_kernel(ReplicaArgs a) {
    const int pi = int(blockIdx.x), qi = int(blockIdx.y), h = int(blockIdx.z);
    const ReplicaPlane pl = a.planes[qi];
    const size_t n = pl.head_bytes >> 4;
    const size_t slice = size_t(a.pages[pi]) * a.sg + size_t(h) * a.sh;
    uint4* dev = reinterpret_cast<uint4*>(static_cast<char*>(pl.base) + slice * pl.head_bytes);
    uint4* host = reinterpret_cast<uint4*>(a.host + size_t(a.first_page + pi) * a.page_bytes + pl.host_off +
                                           size_t(h) * pl.head_bytes);
    if (a.to_host) {
        for (size_t i = threadIdx.x; i < n; i += 256) host[i] = dev[i];
    } else {
        for (size_t i = threadIdx.x; i < n; i += 256) dev[i] = host[i];
    }
}

}  // namespace

hipError_t launch_replica_copy(const ReplicaPlane* planes, int n_planes, const int32_t* pages, int n_pages,
                               uint64_t page_bytes, int H, int sg, int sh, char* host, bool to_host, hipStream_t s) {
    for (int p0 = 0; p0 < n_pages; p0 += kReplicaPages) {
        for (int q0 = 0; q0 < n_planes; q0 += kReplicaPlanes) {
            ReplicaArgs a;
            a.n_planes = std::min(kReplicaPlanes, n_planes - q0);
            for (int i = 0; i < a.n_planes; ++i) a.planes[i] = planes[q0 + i];
            const int np = std::min(kReplicaPages, n_pages - p0);
            for (int i = 0; i < np; ++i) a.pages[i] = pages[p0 + i];
            a.first_page = p0;
            a.page_bytes = page_bytes;
            a.host = host;
            a.to_host = to_host ? 1 : 0;
            a.H = H;
            a.sg = sg;
            a.sh = sh;
            replica_copy_kernel<<<dim3(np, a.n_planes, H), 256, 0, s>>>(a);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

hipError_t launch_table_fill(int32_t* d_table, int32_t n, int32_t value, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    table_fill_kernel<<<(n + 255) / 256, 256, 0, s>>>(d_table, n, value);
    return hipGetLastError();
}

hipError_t launch_table_publish(int32_t* d_dst, const int32_t* host_vals, int32_t n, hipStream_t s) {
    for (int32_t off = 0; off < n; off += kPublishMax) {
        PublishArgs a;
        a.dst = d_dst + off;
        a.n = std::min(kPublishMax, n - off);
        std::memcpy(a.vals, host_vals + off, size_t(a.n) * sizeof(int32_t));
        table_publish_kernel<<<1, 256, 0, s>>>(a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_cow_copy(const CopyPlane* planes, int n_planes, int H, int sg, int sh, int src_g, int dst_g,
                           int cols, hipStream_t s) {
    for (int off = 0; off < n_planes; off += kCopyMaxPlanes) {
        CopyArgs a;
        a.n_planes = std::min(kCopyMaxPlanes, n_planes - off);
        for (int i = 0; i < a.n_planes; ++i) a.planes[i] = planes[off + i];
        a.H = H;
        a.sg = sg;
        a.sh = sh;
        a.src_g = src_g;
        a.dst_g = dst_g;
        a.cols = cols;
        cow_copy_kernel<<<dim3(a.n_planes, H), 256, 0, s>>>(a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace kvs
