// Weighted combine of the routed experts' outputs (page "Step 5 Preview:
// 92 narrow layers, ...", "The shape: narrow and deep": each token adds the
// outputs of its 8 routed experts and of the shared expert), plus the
// optional float32 residual stream (same page, fp32_residual_connection).
//
//   out[t][n] = sum_{k ascending} w[t][k] * y[slot_to_row[t*K+k]][n]
//               (+ shared[t][n]) (+ residual[t][n])
//
// float32 throughout, one fixed order, no atomics: the result does not
// depend on scheduling. A slot whose row is -1 (its id lay outside the
// expert range, so the permutation routed it nowhere) adds nothing.
#include "common.h"

namespace moe {

// The largest K the library accepts (the host rejects more).
constexpr int kCombineMaxK = 16;

template <int OUT>
__global__ void __launch_bounds__(256) combine_kernel(
    const float *__restrict__ y, const int32_t *__restrict__ slot_to_row,
    const float *__restrict__ w, int K, int H, const float *__restrict__ shared,
    const float *__restrict__ residual, void *__restrict__ out) {
    const int t = blockIdx.y;
    const int n = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (n >= H) return;
    // all K rows and weights first (uniform: scalar loads), then all K row
    // loads in flight together, then the sum in ascending k
    int rows[kCombineMaxK];
    float wk[kCombineMaxK];
    float4 v[kCombineMaxK];
#pragma unroll
    for (int k = 0; k < kCombineMaxK; ++k) {
        if (k < K) {
            rows[k] = slot_to_row[(size_t)t * K + k];
            wk[k] = w[(size_t)t * K + k];
        }
    }
#pragma unroll
    for (int k = 0; k < kCombineMaxK; ++k)
        if (k < K && rows[k] >= 0) v[k] = *(const float4 *)(y + (size_t)rows[k] * H + n);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < kCombineMaxK; ++k) {
        if (k < K && rows[k] >= 0) {
            acc.x = __builtin_fmaf(wk[k], v[k].x, acc.x);
            acc.y = __builtin_fmaf(wk[k], v[k].y, acc.y);
            acc.z = __builtin_fmaf(wk[k], v[k].z, acc.z);
            acc.w = __builtin_fmaf(wk[k], v[k].w, acc.w);
        }
    }
    if (shared) {
        const float4 v = *(const float4 *)(shared + (size_t)t * H + n);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    if (residual) {
        const float4 v = *(const float4 *)(residual + (size_t)t * H + n);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    const size_t o = (size_t)t * H + n;
    if (OUT == MOE_F32) {
        *(float4 *)((float *)out + o) = acc;
    } else {
        const uint32_t lo = f32_to_act<OUT>(acc.x) | ((uint32_t)f32_to_act<OUT>(acc.y) << 16);
        const uint32_t hi = f32_to_act<OUT>(acc.z) | ((uint32_t)f32_to_act<OUT>(acc.w) << 16);
        *(uint2 *)((uint16_t *)out + o) = make_uint2(lo, hi);
    }
}

moe_status_t launch_combine(const float *y, const int32_t *slot_to_row, const float *w, int T,
                            int K, int H, const float *shared, const float *residual, void *out,
                            int out_dtype, hipStream_t s) {
    const dim3 grid((H / 4 + 255) / 256, T);
    if (out_dtype == MOE_F32)
        hipLaunchKernelGGL(combine_kernel<MOE_F32>, grid, dim3(256), 0, s, y, slot_to_row, w, K,
                           H, shared, residual, out);
    else if (out_dtype == MOE_BF16)
        hipLaunchKernelGGL(combine_kernel<MOE_BF16>, grid, dim3(256), 0, s, y, slot_to_row, w, K,
                           H, shared, residual, out);
    else
        hipLaunchKernelGGL(combine_kernel<MOE_F16>, grid, dim3(256), 0, s, y, slot_to_row, w, K,
                           H, shared, residual, out);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

}  // namespace moe
