// Export of one expert's dequantized matrix as float32 [n][k].
//
// It runs the forward kernels' own decoders: int4 words go through the
// biased fp16 pairs (1032 + q for the signed forms, 1024 + q for the
// unsigned one, then the bias, with the zero point, is removed exactly) and
// the scale is applied as one exact float32 product (compressed NVFP4 scales
// are decoded from base, code and exceptions first); int8 bytes go through
// the fp16 pairs 1152 + q the same way; NVFP4 bytes go through the
// hardware E2M1 pair conversion, the E4M3 scale multiplies exactly, and the
// global scale is the single float32 rounding.
#include "decode.h"

namespace moe {

// GS inputs per scale; ASYM: unsigned nibbles (1024 + q) and a zero point
// per 128 inputs, subtracted with the bias: (1024 + q) - (1024 + z) = q - z.
template <int GS, bool ASYM>
__global__ void __launch_bounds__(256) dequant_int4_kernel(
    const uint8_t *__restrict__ qw, int64_t qrow, const uint8_t *__restrict__ sc, int64_t srow,
    const uint8_t *__restrict__ zp, int64_t zrow, int n, int k, float *__restrict__ out) {
    const int words = k / 8;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)n * words) return;
    const int r = (int)(idx / words), j = (int)(idx % words);
    const uint32_t w = *(const uint32_t *)(qw + r * qrow + 4 * (int64_t)j);
    const uint16_t sb = *(const uint16_t *)(sc + r * srow + 2 * (int64_t)((8 * j) / GS));
    const float s = bf16_bits_to_f32(sb);
    uint32_t p[4];
    float bias;
    if (ASYM) {
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = ((w >> (4 * i)) & 0x000F000Fu) | Int4Bias<MOE_F16>::kMagic;
        bias = Int4Bias<MOE_F16>::kMagicValue + (float)zp[r * zrow + (8 * j) / 128];
    } else {
        int4_biased_pairs<MOE_F16>(w, p);
        bias = Int4Bias<MOE_F16>::kBias;
    }
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[i] = (f16_bits_to_f32(p[i] & 0xFFFF) - bias) * s;
        v[i + 4] = (f16_bits_to_f32(p[i] >> 16) - bias) * s;
    }
    float4 *o = (float4 *)(out + (int64_t)r * k + 8 * (int64_t)j);
    o[0] = make_float4(v[0], v[1], v[2], v[3]);
    o[1] = make_float4(v[4], v[5], v[6], v[7]);
}

// 8 inputs per thread: (1152 + q) - 1152 = q exactly, times the bf16 scale
// (at most 8 + 8 significant bits: exact in float32).
__global__ void __launch_bounds__(256) dequant_int8_kernel(
    const uint8_t *__restrict__ qw, int64_t qrow, const uint8_t *__restrict__ sc, int64_t srow,
    int n, int k, float *__restrict__ out) {
    const int items = k / 8;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)n * items) return;
    const int r = (int)(idx / items), j = (int)(idx % items);
    const uint2 w = *(const uint2 *)(qw + r * qrow + 8 * (int64_t)j);
    const float s = bf16_bits_to_f32(*(const uint16_t *)(sc + r * srow + 2 * (int64_t)(j / 16)));
    const uint32_t d[2] = {w.x ^ 0x80808080u, w.y ^ 0x80808080u};
    float v[8];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const uint32_t p0 = int8_pair<MOE_F16, 0>(d[q]), p1 = int8_pair<MOE_F16, 1>(d[q]);
        v[4 * q + 0] = (f16_bits_to_f32(p0 & 0xFFFF) - Int8Bias<MOE_F16>::kBias) * s;
        v[4 * q + 1] = (f16_bits_to_f32(p0 >> 16) - Int8Bias<MOE_F16>::kBias) * s;
        v[4 * q + 2] = (f16_bits_to_f32(p1 & 0xFFFF) - Int8Bias<MOE_F16>::kBias) * s;
        v[4 * q + 3] = (f16_bits_to_f32(p1 >> 16) - Int8Bias<MOE_F16>::kBias) * s;
    }
    float4 *o = (float4 *)(out + (int64_t)r * k + 8 * (int64_t)j);
    o[0] = make_float4(v[0], v[1], v[2], v[3]);
    o[1] = make_float4(v[4], v[5], v[6], v[7]);
}

__global__ void __launch_bounds__(256) dequant_nvfp4_kernel(
    const uint8_t *__restrict__ qw, int64_t qrow, const uint8_t *__restrict__ sc, int64_t srow,
    const float *__restrict__ gsp, int n, int k, float *__restrict__ out) {
    const float gs = *gsp;
    const int dwords = k / 8;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)n * dwords) return;
    const int r = (int)(idx / dwords), j = (int)(idx % dwords);
    const uint32_t w = *(const uint32_t *)(qw + r * qrow + 4 * (int64_t)j);
    const float bs = e4m3_to_f32(sc[r * srow + (8 * j) / 16]);
    const uint32_t p[4] = {fp4_pair<MOE_BF16, 0>(w), fp4_pair<MOE_BF16, 1>(w),
                           fp4_pair<MOE_BF16, 2>(w), fp4_pair<MOE_BF16, 3>(w)};
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = (bf16_bits_to_f32(p[i] & 0xFFFF) * bs) * gs;
        v[2 * i + 1] = (bf16_bits_to_f32(p[i] >> 16) * bs) * gs;
    }
    float4 *o = (float4 *)(out + (int64_t)r * k + 8 * (int64_t)j);
    o[0] = make_float4(v[0], v[1], v[2], v[3]);
    o[1] = make_float4(v[4], v[5], v[6], v[7]);
}

// NVFP4 with compressed scales: a block's scale byte comes from the row's
// exception list when it names the block's position, else it is the row
// base plus the block's 4-bit code (even blocks in the low nibble); the
// rest as dequant_nvfp4_kernel.
__global__ void __launch_bounds__(256) dequant_nvfp4_csf_kernel(
    const uint8_t *__restrict__ qw, int64_t qrow, const uint8_t *__restrict__ fixed,
    const uint32_t *__restrict__ xc, const int32_t *__restrict__ ri,
    const float *__restrict__ gsp, int n, int k, float *__restrict__ out) {
    const float gs = *gsp;
    const int dwords = k / 8, C = k / 16;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)n * dwords) return;
    const int r = (int)(idx / dwords), j = (int)(idx % dwords);
    const int b = (8 * j) / 16;                              // block of these 8 inputs
    const uint8_t *slab = fixed + (size_t)(r >> 4) * 16 * (1 + C / 2);
    const uint32_t code = slab[16 + (r & 15) * (C / 2) + b / 2];
    uint32_t sb = slab[r & 15] + ((b & 1) ? code >> 4 : code & 15u);
    const uint32_t pos = (uint32_t)r * (uint32_t)C + (uint32_t)b;
    for (int x = ri[r]; x < ri[r + 1]; ++x)
        if ((xc[x] & 0xFFFFFFu) == pos) sb = xc[x] >> 24;
    const float bs = e4m3_to_f32(sb);
    const uint32_t w = *(const uint32_t *)(qw + r * qrow + 4 * (int64_t)j);
    const uint32_t p[4] = {fp4_pair<MOE_BF16, 0>(w), fp4_pair<MOE_BF16, 1>(w),
                           fp4_pair<MOE_BF16, 2>(w), fp4_pair<MOE_BF16, 3>(w)};
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = (bf16_bits_to_f32(p[i] & 0xFFFF) * bs) * gs;
        v[2 * i + 1] = (bf16_bits_to_f32(p[i] >> 16) * bs) * gs;
    }
    float4 *o = (float4 *)(out + (int64_t)r * k + 8 * (int64_t)j);
    o[0] = make_float4(v[0], v[1], v[2], v[3]);
    o[1] = make_float4(v[4], v[5], v[6], v[7]);
}

moe_status_t launch_dequant(const moe_weight_desc_t &d, int e, float *out,
                            hipStream_t s) {
    const uint8_t *qw = (const uint8_t *)d.qweight + (int64_t)e * d.qweight_expert_stride;
    const uint8_t *sc = (const uint8_t *)d.scale + (int64_t)e * d.scale_expert_stride;
    const int64_t items = (int64_t)d.n * (d.k / 8);
    const dim3 grid((unsigned)((items + 255) / 256));
    const uint8_t *zp = d.zero_point ? d.zero_point + (int64_t)e * d.zero_point_expert_stride
                                     : nullptr;
    if (d.fmt == MOE_W_INT4_G128)
        hipLaunchKernelGGL((dequant_int4_kernel<128, false>), grid, dim3(256), 0, s, qw,
                           d.qweight_row_stride, sc, d.scale_row_stride, nullptr, 0, d.n, d.k, out);
    else if (d.fmt == MOE_W_INT4_G32)
        hipLaunchKernelGGL((dequant_int4_kernel<32, false>), grid, dim3(256), 0, s, qw,
                           d.qweight_row_stride, sc, d.scale_row_stride, nullptr, 0, d.n, d.k, out);
    else if (d.fmt == MOE_W_INT4_G128_ASYM)
        hipLaunchKernelGGL((dequant_int4_kernel<128, true>), grid, dim3(256), 0, s, qw,
                           d.qweight_row_stride, sc, d.scale_row_stride, zp,
                           d.zero_point_row_stride, d.n, d.k, out);
    else if (d.fmt == MOE_W_INT8_G128)
        hipLaunchKernelGGL(dequant_int8_kernel, grid, dim3(256), 0, s, qw, d.qweight_row_stride,
                           sc, d.scale_row_stride, d.n, d.k, out);
    else if (d.fmt == MOE_W_NVFP4_CSF)
        hipLaunchKernelGGL(dequant_nvfp4_csf_kernel, grid, dim3(256), 0, s, qw,
                           d.qweight_row_stride, sc, d.csf_exceptions,
                           d.csf_row_index + (int64_t)e * (d.n + 1), d.global_scale + e, d.n,
                           d.k, out);
    else
        hipLaunchKernelGGL(dequant_nvfp4_kernel, grid, dim3(256), 0, s, qw, d.qweight_row_stride,
                           sc, d.scale_row_stride, d.global_scale + e, d.n, d.k, out);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

}  // namespace moe
