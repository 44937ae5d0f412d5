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

struct GemvMat {                 // one projection bank, byte addressed
    const uint8_t *q, *s;
    const float *gs;             // NVFP4 global scale [E] or null
    int64_t qe, qr, se, sr;      // expert / row strides (bytes)
    const uint8_t *z;            // asymmetric int4 zero points or null
    int64_t ze, zr;
    const uint32_t *xc;          // NVFP4_CSF: exceptions and their row index
    const int32_t *ri;
    float xs;                    // NVFP4 with quantized inputs: the input scale (else 1)
};

inline GemvMat gemv_mat(const moe_weight_desc_t &d) {
    return GemvMat{(const uint8_t *)d.qweight, (const uint8_t *)d.scale, d.global_scale,
                   d.qweight_expert_stride, d.qweight_row_stride, d.scale_expert_stride,
                   d.scale_row_stride, d.zero_point, d.zero_point_expert_stride,
                   d.zero_point_row_stride, d.csf_exceptions, d.csf_row_index,
                   d.input_scale > 0.0f ? d.input_scale : 1.0f};
}

// Work groups that need more than 64 KB of LDS must say so before launch.
template <typename Kern>
inline void allow_lds(Kern k, size_t lds) {
    if (lds > 65536)
        (void)hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)lds);
}

}  // namespace moe
