// Decoding of the 4-bit weight formats, shared by the dequant export and the
// forward kernels.
//
// int4-g128 (page "NeuroSenko/Step-5-Preview-Int4-g128", "Recipe", "Tensor
// layout"): int32 words along K, nibble j of a word = input 8w+j, a
// two's-complement value in [-8, 7]; one bf16 scale per 128 inputs.
//
// int4-g32 and asymmetric int4-g128 (the same page, "Recipe": the error
// table's variants): g32 has one bf16 scale per 32 inputs; the asymmetric
// form holds unsigned nibbles q in [0, 15] with a zero point z per 128
// inputs, weight = (q - z) * scale.
//
// int8-g128 (the same page, "Recipe": its comparison with 8-bit experts):
// two's-complement bytes, input j at byte j, one bf16 scale per 128 inputs.
//
// NVFP4 (page "Step-5-Preview-NVFP4-Local", "Modifications" item 2,
// "Format"): bytes of two E2M1 codes (low nibble = even input), one E4M3
// block scale per 16 inputs, one float32 global scale per expert; value =
// E2M1 x E4M3 x global scale.
#pragma once

#include "common.h"

namespace moe {

// ---- int4 -------------------------------------------------------------------
__device__ __forceinline__ int int4_q(uint32_t w, int j) {
    return ((int32_t)(w << (28 - 4 * j))) >> 28;          // sign-extend nibble j
}

// The four 16-bit pairs of a word, each pair = inputs (8w+i, 8w+i+4), as the
// exact 16-bit value BIAS + q: XOR 0x8 turns the two's-complement nibble
// into q + 8 in [0, 15]; OR-ing that into the mantissa of 1024 (fp16, ulp 1)
// or 128 (bf16, ulp 1) gives 1032 + q or 136 + q without any rounding.
template <int ACT>
struct Int4Bias;
// kMagicValue: the bias of the unsigned form (no XOR), MAGIC + q.
template <>
struct Int4Bias<MOE_F16> {
    static constexpr uint32_t kMagic = 0x64006400u;   // fp16 1024.0 in each half
    static constexpr float kBias = 1032.0f;
    static constexpr float kMagicValue = 1024.0f;
};
template <>
struct Int4Bias<MOE_BF16> {
    static constexpr uint32_t kMagic = 0x43004300u;   // bf16 128.0 in each half
    static constexpr float kBias = 136.0f;
    static constexpr float kMagicValue = 128.0f;
};

// The int4 family: nibble weights with bf16 scales.
__host__ __device__ constexpr bool is_int4(int fmt) {
    return fmt == MOE_W_INT4_G128 || fmt == MOE_W_INT4_G32 || fmt == MOE_W_INT4_G128_ASYM;
}
__host__ __device__ constexpr int int4_group(int fmt) { return fmt == MOE_W_INT4_G32 ? 32 : 128; }
__host__ __device__ constexpr bool int4_asym(int fmt) { return fmt == MOE_W_INT4_G128_ASYM; }
// The XOR key of the one-op pair decode ((w >> 4i) & 0x000F000F) ^ key: the
// signed forms fold the XOR with 8 into the magic, the unsigned form takes
// the nibble as it is (MAGIC + q).
template <int ACT, int FMT>
__host__ __device__ constexpr uint32_t int4_key() {
    return int4_asym(FMT) ? Int4Bias<ACT>::kMagic : (Int4Bias<ACT>::kMagic | 0x00080008u);
}

template <int ACT>
__device__ __forceinline__ void int4_biased_pairs(uint32_t w, uint32_t out[4]) {
    const uint32_t u = w ^ 0x88888888u;
    out[0] = (u & 0x000F000Fu) | Int4Bias<ACT>::kMagic;
    out[1] = ((u >> 4) & 0x000F000Fu) | Int4Bias<ACT>::kMagic;
    out[2] = ((u >> 8) & 0x000F000Fu) | Int4Bias<ACT>::kMagic;
    out[3] = ((u >> 12) & 0x000F000Fu) | Int4Bias<ACT>::kMagic;
}

// The same pairs with a per-group nibble mask: ((w >> 4i) & m) ^ K equals
// the expression above when m = 0x000F000F (K folds the XOR with 8 into the
// magic, whose bits are disjoint from the nibbles), and gives BIAS + 0 for
// every input when m = 0, i.e. q = 0: how a group with a zero scale is
// dropped. One shift and one three-input bit operation per pair.
template <int ACT>
__device__ __forceinline__ void int4_biased_pairs_masked(uint32_t w, uint32_t m, uint32_t out[4]) {
    constexpr uint32_t K = Int4Bias<ACT>::kMagic | 0x00080008u;
    out[0] = (w & m) ^ K;
    out[1] = ((w >> 4) & m) ^ K;
    out[2] = ((w >> 8) & m) ^ K;
    out[3] = ((w >> 12) & m) ^ K;
}

// ---- NVFP4 family ------------------------------------------------------------
// NVFP4_CSF: the same codes with the block scales in the compressed scale
// format (base + 4-bit code per scale, exceptions), read in place.
__host__ __device__ constexpr bool is_csf(int fmt) { return fmt == MOE_W_NVFP4_CSF; }
__host__ __device__ constexpr bool is_nvfp4(int fmt) {
    return fmt == MOE_W_NVFP4_G16 || fmt == MOE_W_NVFP4_CSF;
}

// ---- int8 -------------------------------------------------------------------
__host__ __device__ constexpr bool is_int8(int fmt) { return fmt == MOE_W_INT8_G128; }
// Inputs per 16-byte weight chunk: 32 for the 4-bit formats, 16 for int8.
__host__ __device__ constexpr int chunk_inputs(int fmt) { return is_int8(fmt) ? 16 : 32; }

// The bias of the decoded int8 pairs: u = q + 128 (the byte XOR 0x80) sits
// in the low mantissa byte of fp16 1024.0 (ulp 1 on [1024, 2048)), so the
// fp16 value is 1152 + q; bf16 has no binade with 8 mantissa bits of ulp 1,
// so there the pair holds u itself (128 + q), converted through float32.
template <int ACT>
struct Int8Bias;
template <>
struct Int8Bias<MOE_F16> {
    static constexpr float kBias = 1152.0f;
};
template <>
struct Int8Bias<MOE_BF16> {
    static constexpr float kBias = 128.0f;
};

// Inputs (2 SEL, 2 SEL + 1) of a word whose bytes are already XOR 0x80 as
// an exact 16-bit pair (element 0 = the even input). fp16: one byte
// permute with the constant 0x64 bytes. bf16: u has at most 8 significant
// bits, so the upper half of its float32 is exactly its bf16.
template <int ACT, int SEL>
__device__ __forceinline__ uint32_t int8_pair(uint32_t u) {
    if constexpr (ACT == MOE_F16) {
        return __builtin_amdgcn_perm(0x64646464u, u, SEL ? 0x04030402u : 0x04010400u);
    } else {
        const float lo = (float)((u >> (16 * SEL)) & 0xFFu);
        const float hi = (float)((u >> (16 * SEL + 8)) & 0xFFu);
        return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
    }
}

// A value the compiler cannot see through, held in a VGPR. gfx950 VOP3
// instructions take no literal and at most one scalar operand, so a
// three-operand bit operation with two constant operands only issues as one
// instruction when one constant already sits in a vector register.
__device__ __forceinline__ uint32_t in_vgpr(uint32_t v) {
    uint32_t r;
    asm("v_mov_b32 %0, %1" : "=v"(r) : "s"(v));
    return r;
}

// ---- NVFP4 ------------------------------------------------------------------
// E4M3FN byte -> float32 (exact): exponent bias 7, so a normal value is
// (8 + m) 2^(e - 10) and a subnormal (e = 0) m 2^-9 = m 2^(1 - 10); written
// with selects and one ldexp so that it never branches.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
    const uint32_t e = (b >> 3) & 0xF, m = b & 7;
    const float mant = (float)(m | (e ? 8u : 0u));
    const float mag = __builtin_amdgcn_ldexpf(mant, (int)(e ? e : 1u) - 10);
    return __uint_as_float(__float_as_uint(mag) | ((b & 0x80u) << 24));
}

// E2M1 code -> float32 (exact): {0, .5, 1, 1.5, 2, 3, 4, 6}, sign bit 3.
__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
    const uint32_t e = (c >> 1) & 3, m = c & 1;
    const float mag = e ? __uint_as_float(((e + 126u) << 23) | (m << 22)) : 0.5f * (float)m;
    return (c & 8) ? -mag : mag;
}

// Two E2M1 codes of byte `SEL` of `w` as a 16-bit pair (element 0 = low
// nibble = even input), exact, via the CDNA4 scaled FP4 conversion with a
// unit scale.
template <int ACT, int SEL>
__device__ __forceinline__ uint32_t fp4_pair(uint32_t w) {
    if constexpr (ACT == MOE_BF16)
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL));
    else
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL));
}

// ---- 16-bit pair dot products with float32 accumulation --------------------
template <int ACT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    if constexpr (ACT == MOE_BF16)
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, a),
                                               __builtin_bit_cast(bf162_t, b), c, false);
    else
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a),
                                      __builtin_bit_cast(half2_t, b), c, false);
}

}  // namespace moe
