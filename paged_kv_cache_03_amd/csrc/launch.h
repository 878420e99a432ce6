// launch.h -- kernel launch with the measurement hook.
//
// launch_kernel dispatches `kernel` on stream s.  When the caller armed
// kv_trace_next_kernel and `traced` is set, the two events ride on the
// dispatch packet itself (hipExtLaunchKernel), so the time between them is the
// kernel's execution on the stream, with no marker packets of their own.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "internal.h"

namespace kvs {

template <typename... Params, typename... Args>
hipError_t launch_kernel(bool traced, void (*kernel)(Params...), dim3 grid, dim3 block, hipStream_t s,
                         Args&&... args) {
    hipEvent_t before = nullptr, after = nullptr;
    if (traced && take_trace(&before, &after)) {
        hipExtLaunchKernelGGL(kernel, grid, block, 0, s, before, after, 0, Params(args)...);
    } else {
        kernel<<<grid, block, 0, s>>>(Params(args)...);
    }
    return hipGetLastError();
}

}  // namespace kvs
