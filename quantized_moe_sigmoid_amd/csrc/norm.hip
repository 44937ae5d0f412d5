// The 16-bit input of a layer from the float32 residual stream (page "Step 5
// Preview: ...", the paragraph on training the deep stack: the residual
// stream stays fp32, and Step5RMSNorm scales x / rms(x) by the zero-centred
// gain (1 + w), in fp32 or wider):
//   rmsnorm:  out[t][h] = 16-bit( x[t][h] / sqrt(mean_h x[t][h]^2 + eps) * (1 + w[h]) )
//   round:    out[i]    = 16-bit( in[i] )
// The norm is evaluated in float64 (squares of float32 values are exact in
// float64, and the sum of H of them loses about H * 2^-53 relative), then
// rounded once to the 16-bit format, so the result is the correctly rounded
// value of the exact expression except within ~1e-16 of a rounding midpoint.
#include "norm.h"

namespace moe {

__device__ __forceinline__ double block_sum_f64(double v, double *red) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    double s = 0.0;
    for (int i = 0; i < nw; ++i) s += red[i];
    return s;
}

// One workgroup of 256 threads per row; 4 consecutive columns per thread.
template <int OUT>
__global__ void __launch_bounds__(256) rmsnorm_kernel(const float *__restrict__ x,
                                                      const float *__restrict__ w, double eps,
                                                      int H, uint16_t *__restrict__ out) {
    __shared__ double red[4];
    const float *row = x + (size_t)blockIdx.x * H;
    double ss = 0.0;
    for (int i = threadIdx.x * 4; i < H; i += 1024) {
        const float4 v = *(const float4 *)(row + i);
        ss += (double)v.x * v.x + (double)v.y * v.y + (double)v.z * v.z + (double)v.w * v.w;
    }
    const double inv = 1.0 / __builtin_sqrt(block_sum_f64(ss, red) / H + eps);
    uint16_t *o = out + (size_t)blockIdx.x * H;
    for (int i = threadIdx.x * 4; i < H; i += 1024) {
        const float4 v = *(const float4 *)(row + i);
        float4 g = make_float4(0.f, 0.f, 0.f, 0.f);
        if (w) g = *(const float4 *)(w + i);
        const uint32_t lo = f64_to_act<OUT>((double)v.x * inv * (1.0 + (double)g.x)) |
                            ((uint32_t)f64_to_act<OUT>((double)v.y * inv * (1.0 + (double)g.y))
                             << 16);
        const uint32_t hi = f64_to_act<OUT>((double)v.z * inv * (1.0 + (double)g.z)) |
                            ((uint32_t)f64_to_act<OUT>((double)v.w * inv * (1.0 + (double)g.w))
                             << 16);
        *(uint2 *)(o + i) = make_uint2(lo, hi);
    }
}

// float32 -> 16-bit, round to nearest even; 4 elements a thread.
template <int OUT>
__global__ void __launch_bounds__(256) round_kernel(const float *__restrict__ in, size_t n,
                                                    uint16_t *__restrict__ out) {
    const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= n) return;
    if (i + 4 <= n) {
        const float4 v = *(const float4 *)(in + i);
        const uint32_t lo = f32_to_act<OUT>(v.x) | ((uint32_t)f32_to_act<OUT>(v.y) << 16);
        const uint32_t hi = f32_to_act<OUT>(v.z) | ((uint32_t)f32_to_act<OUT>(v.w) << 16);
        *(uint2 *)(out + i) = make_uint2(lo, hi);
    } else {
        for (size_t j = i; j < n; ++j) out[j] = f32_to_act<OUT>(in[j]);
    }
}

moe_status_t launch_rmsnorm(const float *x, const float *w, float eps, int T, int H, int dtype,
                            void *out, hipStream_t s) {
    if (dtype == MOE_BF16)
        hipLaunchKernelGGL(rmsnorm_kernel<MOE_BF16>, dim3(T), dim3(256), 0, s, x, w, (double)eps,
                           H, (uint16_t *)out);
    else
        hipLaunchKernelGGL(rmsnorm_kernel<MOE_F16>, dim3(T), dim3(256), 0, s, x, w, (double)eps,
                           H, (uint16_t *)out);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

moe_status_t launch_round(const float *in, size_t n, int dtype, void *out, hipStream_t s) {
    const dim3 grid((unsigned)((n + 1023) / 1024));
    if (dtype == MOE_BF16)
        hipLaunchKernelGGL(round_kernel<MOE_BF16>, grid, dim3(256), 0, s, in, n, (uint16_t *)out);
    else
        hipLaunchKernelGGL(round_kernel<MOE_F16>, grid, dim3(256), 0, s, in, n, (uint16_t *)out);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

}  // namespace moe
