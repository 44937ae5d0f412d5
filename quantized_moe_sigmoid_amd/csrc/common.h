// Shared device/host helpers of the MoE library (HIP, gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_w4a16.h"

namespace moe {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---- 16-bit float <-> float32 (exact widening; rounding narrowing) -------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
    return __uint_as_float(b16 << 16);
}
__device__ __forceinline__ float f16_bits_to_f32(uint32_t b16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)b16);
}
template <int ACT>
__device__ __forceinline__ float act_to_f32(uint16_t v) {
    return ACT == MOE_BF16 ? bf16_bits_to_f32(v) : f16_bits_to_f32(v);
}
// float32 -> bf16 bits, round to nearest even (inputs finite).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}
template <int ACT>
__device__ __forceinline__ uint16_t f32_to_act(float f) {
    return ACT == MOE_BF16 ? f32_to_bf16_bits(f) : f32_to_f16_bits(f);
}
// A float32 value the compiler must materialise as such: without it, a
// product converted to fp16 is folded into one mixed-precision FMA that
// rounds the exact product to fp16 once (v_fma_mixlo_f16), which is not the
// float32 product rounded to fp16.
__device__ __forceinline__ float as_f32(float v) {
    asm volatile("" : "+v"(v));
    return v;
}

// ---- cross-lane helpers ----------------------------------------------------
__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
    return __shfl_xor(v, mask, kWave);
}

__device__ __forceinline__ float silu_mul(float g, float u) {
    return g / (1.0f + __expf(-g)) * u;
}

// ---- shared-expert (dense BF16) planning ---------------------------------
// Input-range splits of the dense gate/up and down launches, and the float32
// partial-sum buffer they need (0 when neither is split).
struct DenseSplit {
    int s_gateup, s_down;
    size_t part_floats;
};

// ---- launch helpers --------------------------------------------------------
#define MOE_LAUNCH_CHECK()                                   \
    do {                                                     \
        if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP; \
    } while (0)

}  // namespace moe
