// float64 -> 16-bit rounding of the RMSNorm output, shared by the norm
// kernel and the fused norm + router kernel (so both round identically).
#pragma once

#include "common.h"

namespace moe {

constexpr double pow2(int e) {
    double v = 1.0;
    for (; e > 0; --e) v *= 2.0;
    for (; e < 0; ++e) v *= 0.5;
    return v;
}

// float64 -> 16-bit float with MB mantissa bits and exponent bias BIAS
// (bf16: 7, 127; fp16: 10, 15), round to nearest even, overflow to infinity,
// subnormals of the target kept. Finite inputs.
template <int MB, int BIAS>
__device__ __forceinline__ uint16_t f64_to_16(double y) {
    const uint64_t u = (uint64_t)__double_as_longlong(y);
    const uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
    const uint64_t a = u & 0x7FFFFFFFFFFFFFFFull;
    const double ay = __longlong_as_double((long long)a);
    constexpr int kEmin = 1 - BIAS;
    constexpr double kMinNormal = pow2(kEmin), kSubScale = pow2(MB - kEmin);
    if (ay < kMinNormal) {
        // subnormal range: the value is m * 2^(emin - MB), m an integer <= 2^MB
        // (m == 2^MB is the encoding of the smallest normal number)
        const double m = __builtin_rint(ay * kSubScale);
        return sign | (uint16_t)m;
    }
    constexpr int kShift = 52 - MB;
    uint64_t r = (a + ((1ull << (kShift - 1)) - 1) + ((a >> kShift) & 1)) >> kShift;
    r -= (uint64_t)(1023 - BIAS) << MB;                  // re-bias the exponent field
    constexpr uint64_t kInf = (uint64_t)(2 * BIAS + 1) << MB;
    if (r > kInf) r = kInf;
    return sign | (uint16_t)r;
}

template <int OUT>
__device__ __forceinline__ uint16_t f64_to_act(double y) {
    return OUT == MOE_BF16 ? f64_to_16<7, 127>(y) : f64_to_16<10, 15>(y);
}

}  // namespace moe
