// NVFP4 quantization of activations, for the layers whose experts quantize
// their inputs (page "Step-5-Preview-NVFP4-Local", "Modifications" items
// 2-3: those layers keep an input scale; the W4A16 ones have none). The
// pages give no rule for activations; the one used is the weights' two-level
// rule ("Format": E2M1 value x E4M3 block scale per 16 x a float32 scale),
// the float32 scale being the tensor's input scale g, with every decision
// in float32:
//   per 16-block: t = max|x| / (6 g); bs = E4M3(t), nearest, ties to even,
//   saturating at 448; v = x / (bs g); code = E2M1(v), nearest, ties to
//   even, saturating at 6 (bs = 0 gives code 0, a magnitude that rounds to
//   0 gives +0).
// The kernel writes e2m1 x bs in the activation dtype (exact: at most 6
// significant bits); the expert kernels multiply their accumulators by g
// with the weights' global scale.
#include "decode.h"

#pragma clang fp contract(off)

namespace moe {

// E4M3FN byte of t >= 0: nearest, ties to even, saturating at 448 (0x7E).
// t >= 448 saturates (448 < t <= 464 rounds to 448, beyond to 480 or
// more); below 2^-6 the grid is m 2^-9, m = 0..8 (8 is the smallest
// normal, byte 0x08); above, the mantissa is rounded to 3 bits.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float t) {
    if (!(t < 448.0f)) return 0x7Eu;
    if (t < 0x1p-6f) return (uint32_t)__builtin_rintf(t * 512.0f);
    uint32_t u = __float_as_uint(t);
    u += 0x7FFFFu + ((u >> 20) & 1u);
    const uint32_t e = (u >> 23) - 120u, m = (u >> 20) & 7u;    // re-biased: 127 - 7
    return (e << 3) | m;
}

// E2M1 code of v: nearest of {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even
// code (0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4,
// 5 -> 4), saturating at 6; sign in bit 3 unless the magnitude is 0.
__device__ __forceinline__ uint32_t e2m1_rne_sat(float v) {
    const float a = __builtin_fabsf(v);
    const uint32_t m = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                       (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                       (uint32_t)(a > 5.0f);
    return m ? (m | (v < 0.0f ? 8u : 0u)) : 0u;
}

// One thread per 16-element block of a row (rows of k elements, k % 16 ==
// 0, contiguous). With row_slot, rows whose entry is negative (padding of
// the expert-sorted rows) are skipped. in may equal out.
template <int ACT>
__global__ void __launch_bounds__(256) act_quant_kernel(const uint16_t *in, int64_t nblk,
                                                        int kblk, float g, float six_g,
                                                        uint16_t *out,
                                                        const int32_t *__restrict__ row_slot) {
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= nblk) return;
    if (row_slot && row_slot[b / kblk] < 0) return;
    const uint4 *src = (const uint4 *)(in + b * 16);
    const uint4 p0 = src[0], p1 = src[1];
    const uint32_t w[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    float v[16];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[2 * i] = act_to_f32<ACT>(w[i] & 0xFFFFu);
        v[2 * i + 1] = act_to_f32<ACT>(w[i] >> 16);
        amax = __builtin_fmaxf(amax, __builtin_fabsf(v[2 * i]));
        amax = __builtin_fmaxf(amax, __builtin_fabsf(v[2 * i + 1]));
    }
    const float bs = e4m3_to_f32(e4m3_rne_sat(amax / six_g));
    const float den = bs * g;
    uint32_t o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t c0 = bs > 0.0f ? e2m1_rne_sat(v[2 * i] / den) : 0u;
        const uint32_t c1 = bs > 0.0f ? e2m1_rne_sat(v[2 * i + 1] / den) : 0u;
        // e2m1 x bs: at most 6 significant bits, exact in both 16-bit formats
        o[i] = (uint32_t)f32_to_act<ACT>(e2m1_to_f32(c0) * bs) |
               ((uint32_t)f32_to_act<ACT>(e2m1_to_f32(c1) * bs) << 16);
    }
    uint4 *dst = (uint4 *)(out + b * 16);
    dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
    dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
}

moe_status_t launch_act_quant(const void *in, int dtype, int64_t rows, int k, float g,
                              void *out, const int32_t *row_slot, hipStream_t s) {
    const int64_t nblk = rows * (k / 16);
    if (nblk == 0) return MOE_OK;
    const float six_g = 6.0f * g;
    const dim3 grid((unsigned)((nblk + 255) / 256));
    if (dtype == MOE_BF16)
        hipLaunchKernelGGL(act_quant_kernel<MOE_BF16>, grid, dim3(256), 0, s,
                           (const uint16_t *)in, nblk, k / 16, g, six_g, (uint16_t *)out,
                           row_slot);
    else
        hipLaunchKernelGGL(act_quant_kernel<MOE_F16>, grid, dim3(256), 0, s,
                           (const uint16_t *)in, nblk, k / 16, g, six_g, (uint16_t *)out,
                           row_slot);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

}  // namespace moe
