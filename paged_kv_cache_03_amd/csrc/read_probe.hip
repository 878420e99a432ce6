// read_probe.hip -- a read-only kernel over the paged decode's access pattern.
//
// The page stream reads K and V pages in place, one (page group, KV head)
// slice at a time, in whatever order the block table gives (Paged KV Context
// Store page, consumer rules: no gather into contiguous memory).  This kernel
// reads the same kind of slices and does nothing with them but fold them into
// a checksum, so its rate is the HBM read ceiling for that pattern on this
// chip: the secondary denominator the decode kernel is measured against.
//
// Work split as in the page stream: block i of G takes a contiguous share of
// the slice list; each of its four waves takes every fourth slice of the
// share.  A wave keeps the loads of its next slice in flight while it folds
// the current one: a slice of S bytes is S / 1024 16-byte loads per lane.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.h"
#include "stream_common.h"

namespace kvs {
namespace {

constexpr int kProbeWaves = 4;   // waves per block (256 threads)

struct ProbeArgs {
    const uint8_t* base;
    const int32_t* ids;
    uint32_t* sink;
    int64_t slice_bytes;
    int n;
    int per_block;
};

template <int LOADS>
__global__ __launch_bounds__(256) void read_probe_kernel(ProbeArgs a) {
    const int lane = int(threadIdx.x) & 63;
    const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
    const int first = int(blockIdx.x) * a.per_block;
    const int last = min(a.n, first + a.per_block);
    // a slice past the block's share gets an empty range: its loads return
    // zeros without touching memory, so every step issues the same loads and
    // the compiler's wait counts stay exact (one slice in flight while the
    // previous one is folded)
    auto rsrc_of = [&](int i) __attribute__((always_inline)) {
        const bool in = i < last;
        const int64_t id = in ? int64_t(__builtin_amdgcn_readfirstlane(a.ids[i])) : 0;
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.base) + id * a.slice_bytes, 0,
                                                 in ? int(a.slice_bytes) : 0, kBufferWord3);
    };
    auto load = [&](u32x4 (&r)[LOADS], __amdgpu_buffer_rsrc_t rs) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < LOADS; ++j)
            r[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * lane + 1024 * j, 0,
                                                                                   kNonTemporal));
    };
    uint32_t acc = 0;
    auto fold = [&](const u32x4 (&r)[LOADS]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < LOADS; ++j) acc ^= r[j].x ^ r[j].y ^ r[j].z ^ r[j].w;
    };
    u32x4 r0[LOADS], r1[LOADS];
    int i = first + wave;
    load(r0, rsrc_of(i));
    for (; i < last; i += 2 * kProbeWaves) {
        load(r1, rsrc_of(i + kProbeWaves));
        fold(r0);
        load(r0, rsrc_of(i + 2 * kProbeWaves));
        fold(r1);
    }
    // fold the block's checksum so every load has a use
    __shared__ uint32_t red[256];
    red[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t x = 0;
        for (int t = 0; t < 256; ++t) x ^= red[t];
        a.sink[blockIdx.x] = x;
    }
}

}  // namespace

int read_probe_blocks(int blocks_per_cu) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    return cus * blocks_per_cu;
}

hipError_t launch_read_probe(const void* base, const int32_t* ids, int n, int slice_bytes, int blocks,
                             uint32_t* sink, hipStream_t s) {
    ProbeArgs a{};
    a.base = static_cast<const uint8_t*>(base);
    a.ids = ids;
    a.sink = sink;
    a.slice_bytes = slice_bytes;
    a.n = n;
    a.per_block = (n + blocks - 1) / blocks;
    const dim3 grid(static_cast<unsigned>(blocks));
    switch (slice_bytes) {
        case 8192: read_probe_kernel<8><<<grid, 256, 0, s>>>(a); break;
        case 16384: read_probe_kernel<16><<<grid, 256, 0, s>>>(a); break;
        case 32768: read_probe_kernel<32><<<grid, 256, 0, s>>>(a); break;
        default: return hipErrorNotSupported;
    }
    return hipGetLastError();
}

}  // namespace kvs
