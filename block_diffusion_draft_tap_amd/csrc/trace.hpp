// Launch tracing (instrumentation only): the workgroups of a traced launch write
// the device wall clock at their start and end into a slice of a caller-owned
// stamp buffer, so a kernel's duration (first start to last end) can be read
// back after timed graph replays. Off unless the caller switched it on.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace dfl {

enum { TRACE_LM_HEAD = 1, TRACE_ATTENTION = 2, TRACE_PROJECTIONS = 4 };

// Host side: the stamp slice for one launch of `workgroups` workgroups of the
// kernel `name` (kind: one TRACE_* bit), or nullptr when that kind is not
// traced or the buffer is full. bytes: the launch's algorithmic HBM bytes known
// on the host; ctx_row_bytes: bytes per held context row it also reads (the
// attention's cache rows, whose counts live on the device).
uint64_t* trace_launch(int kind, const char* name, int64_t workgroups, double bytes, double ctx_row_bytes);

// Device side. The start time of this workgroup (0 when untraced) ...
__device__ __forceinline__ uint64_t trace_start(const uint64_t* stamps) {
    return stamps ? (uint64_t)wall_clock64() : 0;
}
// ... and, after all of its work, its (start, end) pair at entries 2w, 2w + 1
// (w = the linear workgroup id). stamps is a kernel argument, so the barrier is
// reached by every thread or by none.
__device__ __forceinline__ void trace_end(uint64_t* stamps, uint64_t t0) {
    if (stamps) {
        __syncthreads();
        if (threadIdx.x == 0) {
            const int64_t w = blockIdx.x + (int64_t)gridDim.x * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
            stamps[2 * w] = t0;
            stamps[2 * w + 1] = (uint64_t)wall_clock64();
        }
    }
}

}  // namespace dfl
