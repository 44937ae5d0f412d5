// Weighted combine of the routed experts' outputs (page "Step 5 Preview:
// 92 narrow layers, ...", "The shape: narrow and deep": each token adds the
// outputs of its 8 routed experts and of the shared expert), plus the
// optional float32 residual stream (same page, fp32_residual_connection).
//
//   out[t][n] = sum_{k ascending} w[t][k] * y[slot_to_row[t*K+k]][n]
//               (+ shared[t][n]) (+ residual[t][n])
//
// float32 throughout, one fixed order, no atomics: the result does not
// depend on scheduling. y is float32, or (Y16, the grouped-GEMM path) fp16
// with a power-of-two scale per (row, 32-column group): y = v * 2^-s with s
// one signed byte of yexp [rows][H / 32], widened exactly. A slot whose row is -1 (its id lay outside the
// expert range, so the permutation routed it nowhere) adds nothing.
#include "common.h"

namespace moe {

// The largest K the library accepts (the host rejects more).
constexpr int kCombineMaxK = 16;

// A thread owns NC consecutive columns of one token: 4 (float32 y, one
// 16-byte load per row) or 8 (fp16 y, one 16-byte load per row).
template <int OUT, bool Y16>
__global__ void __launch_bounds__(256) combine_kernel(
    const float *__restrict__ y, const uint16_t *__restrict__ y16,
    const int8_t *__restrict__ yexp, const int32_t *__restrict__ slot_to_row,
    const float *__restrict__ w, int K, int H, const float *__restrict__ shared,
    const float *__restrict__ residual, void *__restrict__ out) {
    constexpr int NC = Y16 ? 8 : 4;
    const int t = blockIdx.y;
    const int n = (blockIdx.x * 256 + threadIdx.x) * NC;
    if (n >= H) return;
    // all K rows and weights first (uniform: scalar loads), then all K row
    // loads in flight together, then the sum in ascending k
    int rows[kCombineMaxK];
    float wk[kCombineMaxK];
    uint4 v[kCombineMaxK];
    int sh[kCombineMaxK];
#pragma unroll
    for (int k = 0; k < kCombineMaxK; ++k) {
        if (k < K) {
            rows[k] = slot_to_row[(size_t)t * K + k];
            wk[k] = w[(size_t)t * K + k];
        }
    }
#pragma unroll
    for (int k = 0; k < kCombineMaxK; ++k) {
        if (k < K && rows[k] >= 0) {
            if constexpr (Y16) {
                v[k] = *(const uint4 *)(y16 + (size_t)rows[k] * H + n);
                sh[k] = -(int)yexp[(size_t)rows[k] * (H / 32) + n / 32];
            } else {
                v[k] = *(const uint4 *)(y + (size_t)rows[k] * H + n);
            }
        }
    }
    float acc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] = 0.0f;
#pragma unroll
    for (int k = 0; k < kCombineMaxK; ++k) {
        if (k < K && rows[k] >= 0) {
            const uint32_t d[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                float yv;
                if constexpr (Y16)
                    yv = __builtin_ldexpf(
                        (float)__builtin_bit_cast(_Float16, (uint16_t)(d[c >> 1] >> (16 * (c & 1)))),
                        sh[k]);
                else
                    yv = __uint_as_float(d[c]);
                acc[c] = __builtin_fmaf(wk[k], yv, acc[c]);
            }
        }
    }
#pragma unroll
    for (int c0 = 0; c0 < NC; c0 += 4) {
        if (shared) {
            const float4 u = *(const float4 *)(shared + (size_t)t * H + n + c0);
            acc[c0] += u.x; acc[c0 + 1] += u.y; acc[c0 + 2] += u.z; acc[c0 + 3] += u.w;
        }
        if (residual) {
            const float4 u = *(const float4 *)(residual + (size_t)t * H + n + c0);
            acc[c0] += u.x; acc[c0 + 1] += u.y; acc[c0 + 2] += u.z; acc[c0 + 3] += u.w;
        }
        const size_t o = (size_t)t * H + n + c0;
        if (OUT == MOE_F32) {
            *(float4 *)((float *)out + o) = make_float4(acc[c0], acc[c0 + 1], acc[c0 + 2], acc[c0 + 3]);
        } else {
            const uint32_t lo = f32_to_act<OUT>(acc[c0]) | ((uint32_t)f32_to_act<OUT>(acc[c0 + 1]) << 16);
            const uint32_t hi = f32_to_act<OUT>(acc[c0 + 2]) | ((uint32_t)f32_to_act<OUT>(acc[c0 + 3]) << 16);
            *(uint2 *)((uint16_t *)out + o) = make_uint2(lo, hi);
        }
    }
}

moe_status_t launch_combine(const float *y, const uint16_t *y16, const int8_t *yexp,
                            const int32_t *slot_to_row, const float *w, int T, int K, int H,
                            const float *shared, const float *residual, void *out, int out_dtype,
                            hipStream_t s) {
    const int nc = y16 ? 8 : 4;
    const dim3 grid((H / nc + 255) / 256, T);
#define MOE_COMBINE(O, Y)                                                                      \
    hipLaunchKernelGGL((combine_kernel<O, Y>), grid, dim3(256), 0, s, y, y16, yexp, slot_to_row, \
                       w, K, H, shared, residual, out)
    const bool h16 = y16 != nullptr;
    if (out_dtype == MOE_F32) {
        if (h16) MOE_COMBINE(MOE_F32, true); else MOE_COMBINE(MOE_F32, false);
    } else if (out_dtype == MOE_BF16) {
        if (h16) MOE_COMBINE(MOE_BF16, true); else MOE_COMBINE(MOE_BF16, false);
    } else {
        if (h16) MOE_COMBINE(MOE_F16, true); else MOE_COMBINE(MOE_F16, false);
    }
#undef MOE_COMBINE
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

}  // namespace moe
