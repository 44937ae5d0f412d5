// The 16-bit input of a layer from the float32 residual stream (page "Step 5
// Preview: ...", the paragraph on training the deep stack: the residual
// stream stays fp32, and Step5RMSNorm scales x / rms(x) by the zero-centred
// gain (1 + w), computed in fp32):
//   rmsnorm:  out[t][h] = 16-bit( (x[t][h] / sqrt(mean_h x[t][h]^2 + eps)) * (1 + w[h]) )
//   round:    out[i]    = 16-bit( in[i] )
// Every operation of the norm is a float32 operation rounded to nearest
// even (no contraction into FMAs; IEEE division and square root), and its
// sum of squares has one fixed order, the one a 256-lane reduction gives:
// thread p adds the squares of columns 4p .. 4p+3, 1024 + 4p .. in ascending
// order, each wave folds its 64 partial sums in halves (xor-shuffles 32, 16,
// .., 1; partial i gets partial i + m), and the four wave sums are added left
// to right. The fused norm + router kernel follows the same order, so both
// produce the same bits.
#include "common.h"

#pragma clang fp contract(off)

namespace moe {

// One workgroup of 256 threads per row; 4 consecutive columns per thread.
template <int OUT>
__global__ void __launch_bounds__(256) rmsnorm_kernel(const float *__restrict__ x,
                                                      const float *__restrict__ w, float eps,
                                                      int H, uint16_t *__restrict__ out) {
    __shared__ float red[4];
    const float *row = x + (size_t)blockIdx.x * H;
    float ss = 0.0f;
    for (int i = threadIdx.x * 4; i < H; i += 1024) {
        const float4 v = *(const float4 *)(row + i);
        ss = ss + v.x * v.x;
        ss = ss + v.y * v.y;
        ss = ss + v.z * v.z;
        ss = ss + v.w * v.w;
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss = ss + __shfl_xor(ss, m, kWave);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = ((red[0] + red[1]) + red[2]) + red[3];
    const float r = __builtin_sqrtf(tot / (float)H + eps);
    uint16_t *o = out + (size_t)blockIdx.x * H;
    for (int i = threadIdx.x * 4; i < H; i += 1024) {
        const float4 v = *(const float4 *)(row + i);
        float4 g = make_float4(0.f, 0.f, 0.f, 0.f);
        if (w) g = *(const float4 *)(w + i);
        const uint32_t lo = f32_to_act<OUT>(as_f32((v.x / r) * (1.0f + g.x))) |
                            ((uint32_t)f32_to_act<OUT>(as_f32((v.y / r) * (1.0f + g.y))) << 16);
        const uint32_t hi = f32_to_act<OUT>(as_f32((v.z / r) * (1.0f + g.z))) |
                            ((uint32_t)f32_to_act<OUT>(as_f32((v.w / r) * (1.0f + g.w))) << 16);
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
        hipLaunchKernelGGL(rmsnorm_kernel<MOE_BF16>, dim3(T), dim3(256), 0, s, x, w, eps, H,
                           (uint16_t *)out);
    else
        hipLaunchKernelGGL(rmsnorm_kernel<MOE_F16>, dim3(T), dim3(256), 0, s, x, w, eps, H,
                           (uint16_t *)out);
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
