// Helpers shared by the weight-streaming kernels.
#pragma once

#include "common.h"

namespace moe {

// Buffer resource over one expert's matrix: 32-bit byte offsets, and an
// offset past `bytes` reads zero without touching memory (the pipelines'
// loads beyond the last chunk use kOutOfRange).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const uint8_t *base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0,
                                             (int)(bytes < 0x7FFFFFFF ? bytes : 0x7FFFFFFF),
                                             0x00020000);
}
constexpr int kOutOfRange = 0x7FFFFFF0;

// Work-group barrier that orders LDS only: weight loads already in flight
// are not drained (a plain __syncthreads waits for every outstanding load).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}


}  // namespace moe
