// stream_common.h -- device helpers shared by the matrix-core paged
// attention kernels (decode.hip, verify.hip): vector types, waits on the
// vector-memory counter, scalar metadata loads, the direct-to-LDS page fetch,
// cross-row reductions and the bf16 split of probabilities.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace kvs {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Wave-uniform metadata reads (block table, rows, lengths) as scalar loads:
// they are read-only for the kernel, and they must not join the vector-memory
// counter that the page ring waits on.
typedef const int32_t __attribute__((address_space(4)))* const_i32;

__device__ __forceinline__ int ld_uniform(const int32_t* p, size_t idx) {
    const const_i32 cp = (const_i32)(const void*)p;
    return cp[__builtin_amdgcn_readfirstlane(int(idx))];
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef s16x4_t __attribute__((address_space(3)))* lds_s16x4_ptr;
typedef char __attribute__((address_space(3)))* lds_byte_ptr;

constexpr int kStreamPages = 1024;     // most pages one block of the page stream takes
// Buffer resources (raw, stride 0): word 3 of the descriptor for gfx9-family
// parts, and the cache-policy bit of a load that does not expect reuse (NT).
constexpr int kBufferWord3 = 0x00020000;
constexpr int kNonTemporal = 2;
constexpr float kRescaleLog2 = 8.f;    // lazy rescale: probabilities stay below 2^8

// One page into a ring stage: PER_T direct-to-LDS loads of the K slice and
// PER_T of the V slice, 16 bytes per lane each (LDS[M0 + 16*lane] =
// MEM[base + voff]).  The V stages sit 64 KiB above the K stages, and the k-th
// load of a wave lands 4 KiB above its (k-1)-th.  Written as inline assembly
// so that the compiler does not order every later LDS read after these loads
// (it cannot tell the ring's stages apart and would wait for all loads in
// flight); the kernel waits on the vector-memory counter itself before it
// reads a stage.  M0 is restored afterwards: the compiler does not track it
// through inline assembly.
#define KVS_DMA_PAIR(K, V)                          \
    "s_nop 0\n\t"                                   \
    "global_load_lds_dwordx4 %[" #K "], %[kb]\n\t"  \
    "s_add_u32 m0, m0, 0x10000\n\t"                 \
    "s_nop 0\n\t"                                   \
    "global_load_lds_dwordx4 %[" #V "], %[vb]\n\t"
#define KVS_DMA_NEXT "s_sub_u32 m0, m0, 0xf000\n\t"

__device__ __forceinline__ void fetch_page2(uint32_t lds_k, const void* kb, const void* vb, const uint32_t* ko,
                                            const uint32_t* vo) {
    uint32_t sv;
    asm volatile("s_mov_b32 %[sv], m0\n\t"
                 "s_mov_b32 m0, %[d]\n\t" KVS_DMA_PAIR(k0, v0) KVS_DMA_NEXT KVS_DMA_PAIR(k1, v1)
                 "s_mov_b32 m0, %[sv]"
                 : [sv] "=&s"(sv)
                 : [d] "s"(lds_k), [kb] "s"(kb), [vb] "s"(vb), [k0] "v"(ko[0]), [k1] "v"(ko[1]), [v0] "v"(vo[0]),
                   [v1] "v"(vo[1])
                 : "memory", "scc");
}

__device__ __forceinline__ void fetch_page4(uint32_t lds_k, const void* kb, const void* vb, const uint32_t* ko,
                                            const uint32_t* vo) {
    uint32_t sv;
    asm volatile("s_mov_b32 %[sv], m0\n\t"
                 "s_mov_b32 m0, %[d]\n\t" KVS_DMA_PAIR(k0, v0) KVS_DMA_NEXT KVS_DMA_PAIR(k1, v1)
                     KVS_DMA_NEXT KVS_DMA_PAIR(k2, v2) KVS_DMA_NEXT KVS_DMA_PAIR(k3, v3)
                 "s_mov_b32 m0, %[sv]"
                 : [sv] "=&s"(sv)
                 : [d] "s"(lds_k), [kb] "s"(kb), [vb] "s"(vb), [k0] "v"(ko[0]), [k1] "v"(ko[1]), [k2] "v"(ko[2]),
                   [k3] "v"(ko[3]), [v0] "v"(vo[0]), [v1] "v"(vo[1]), [v2] "v"(vo[2]), [v3] "v"(vo[3])
                 : "memory", "scc");
}
#undef KVS_DMA_PAIR
#undef KVS_DMA_NEXT

// One 16-byte chunk per lane from its own address into LDS[M0 + 16*lane]
// (query rows into the block's query cache), ordered with the page loads on
// the same counter.
__device__ __forceinline__ void fetch_chunk(uint32_t lds_wave, const void* src) {
    uint32_t sv;
    asm volatile("s_mov_b32 %[sv], m0\n\t"
                 "s_mov_b32 m0, %[d]\n\t"
                 "s_nop 0\n\t"
                 "global_load_lds_dwordx4 %[a], off\n\t"
                 "s_mov_b32 m0, %[sv]"
                 : [sv] "=&s"(sv)
                 : [d] "s"(lds_wave), [a] "v"(src)
                 : "memory");
}

// One 16-byte load per lane at base + voff into LDS[M0 + 16*lane], ordered
// with the page loads on the same counter (pages whose planes do not fit the
// fixed K/V stage pattern of fetch_page2/4).
__device__ __forceinline__ void fetch_lds16(uint32_t lds_wave, const void* base, uint32_t voff) {
    uint32_t sv;
    asm volatile("s_mov_b32 %[sv], m0\n\t"
                 "s_mov_b32 m0, %[d]\n\t"
                 "s_nop 0\n\t"
                 "global_load_lds_dwordx4 %[o], %[b]\n\t"
                 "s_mov_b32 m0, %[sv]"
                 : [sv] "=&s"(sv)
                 : [d] "s"(lds_wave), [o] "v"(voff), [b] "s"(base)
                 : "memory");
}

// op over the four 16-lane rows (lanes l%16 + 16k); identical in every lane
__device__ __forceinline__ float rows_max(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float rows_sum(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// two fp32 values as the bf16 pair (hi, lo) with hi = rne(x), lo = rne(x - hi)
__device__ __forceinline__ void split_bf16(float x0, float x1, uint32_t& hi, uint32_t& lo) {
    hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{x0, x1}, bf16x2v_t));
    const float r0 = x0 - __uint_as_float(hi << 16);
    const float r1 = x1 - __uint_as_float(hi & 0xFFFF0000u);
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{r0, r1}, bf16x2v_t));
}

}  // namespace kvs
