// attn_common.h -- wave-level helpers shared by the attention kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace kvs {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// DPP row/quad permutations (gfx9 encodings).
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Maximum over the 64 lanes of a wave, returned wave-uniform: DPP inside each
// row of 16 lanes, then the four row results through readlane.
__device__ __forceinline__ float wave_max_uniform(float v) {
    v = fmaxf(v, dpp<kDppQuadXor1>(v));
    v = fmaxf(v, dpp<kDppQuadXor2>(v));
    v = fmaxf(v, dpp<kDppRowRor4>(v));
    v = fmaxf(v, dpp<kDppRowRor8>(v));
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Workgroup barrier that orders LDS traffic only: every LDS access of this
// wave completes (lgkmcnt 0) before the barrier, and the memory clobber keeps
// the compiler from moving memory operations across it.  __syncthreads() also
// fences global memory, i.e. waits for every outstanding vector-memory load --
// including page loads meant to stay in flight across the barrier; callers of
// this barrier wait for the loads they need themselves (vmcnt).
__device__ __forceinline__ void block_lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Order LDS traffic of one wave without a workgroup barrier (the waves of a
// block work on unrelated items and may run different trip counts).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace kvs
