// Prefill-sized expert FFN: grouped GEMM over expert tiles on CDNA4 MFMA
// (v_mfma_f32_32x32x16_{bf16,f16}).
//
// Work unit = (tile of 64 expert-sorted slots of one expert, block of 128
// output columns); 4 waves, wave w owns 32 columns and all 64 rows (two
// 32x32 accumulator blocks). The activation tile streams through LDS in
// 128-input groups (double buffered, 16-byte chunks XOR-swizzled by row so
// a wave's 16-byte reads hit every bank once). Weights go straight from HBM
// into registers: each lane loads 16 bytes (32 inputs) of its own output
// column per half-group and decodes them into MFMA operands, so every weight
// is read and decoded exactly once per tile.
//
// The MFMA sums over its 16 k-slots in any order, so A and B only have to
// agree on which input each slot holds: lane half h of MFMA (i, j) of a
// group carries inputs 64i + 32h + 8j .. +7, in the pair order the decoder
// produces.
//
// int4: B holds the exact 16-bit values BIAS + q (decode.h); a group's
//   partial sum P = sum (BIAS + q) x is turned into s_g (P - BIAS sum x) and
//   accumulated in float32, with sum x over the group's 128 inputs of each
//   row computed while staging the activations. The bf16 scale is applied
//   exactly once per group in float32. Asymmetric int4 (uint4 codes, zero
//   point z per group and column): B holds MAGIC + q and the group's term is
//   s_g (P - (MAGIC + z) sum x).
// int8-g128: as int4-g128 with BIAS + q = 1152 + q (fp16) / 128 + q (bf16),
//   the bytes re-paired into the same (i, i + 4) order; twice the weight
//   registers, so that instantiation runs one wave per SIMD.
// int4-g32: one 32x32x16 MFMA takes inputs from two 32-input groups (its
//   two lane halves), so the scale cannot be applied between MFMAs; B holds
//   q s_g instead (exact in fp16, rounded once in bf16), as for NVFP4.
// NVFP4: B holds e2m1 * e4m3 exactly in 16 bits (<= 6 significant bits);
//   the float32 global scale multiplies the accumulators in the epilogue.
//
//   gate/up pass: h = silu(gate) * up for the wave's 32 columns (both
//                 projections of a column in the same lane: SwiGLU fused);
//   down pass:    y rows for the combine: fp16 with a power-of-two scale
//                 per (row, 32-column group), float32 for int4-g32.
#include <functional>

#include "decode.h"
#include "stream.h"

namespace moe {

constexpr int kGemmThreads = 256;
constexpr int kGemmTM = 64;          // rows per tile
constexpr int kGemmBN = 128;         // output columns per block
constexpr int kGemmKS = 256;         // inputs per pipeline step (two int4 groups)
constexpr int kGemmRowBytes = kGemmKS * 2;

// The int4 group path: signed int4-g128, or asymmetric (uint4 codes and a
// 4-bit zero point per group) int4-g128.
__host__ __device__ constexpr bool int4_g128(int fmt) {
    return fmt == MOE_W_INT4_G128 || fmt == MOE_W_INT4_G128_ASYM;
}

// Group-rescaled forms: 128-input groups, exact BIAS + q operands, the
// per-group correction -BIAS sum x (int4 as above; int8-g128 as 1152 + q in
// fp16 and 128 + q in bf16, decode.h).
__host__ __device__ constexpr bool g128_rescaled(int fmt) {
    return int4_g128(fmt) || fmt == MOE_W_INT8_G128;
}

// Every int4 form and int8: the operand pairs hold inputs (i, i + 4) of an
// 8-input group, so x and h are staged in that pair order.
__host__ __device__ constexpr bool int4_pairs(int fmt) {
    return g128_rescaled(fmt) || fmt == MOE_W_INT4_G32;
}

// The down pass stores y in fp16 with a power-of-two scale per (row,
// 32-column group) for the formats whose operands are exact; int4-g32 in
// bf16 already rounds q s into its operands, which uses most of the layer's
// error bound, so its y stays float32.
__host__ __device__ constexpr bool gemm_y16(int fmt) { return fmt != MOE_W_INT4_G32; }

// 16-byte weight loads per matrix and step: 32 inputs of a lane are 16 bytes
// of int4 or 32 of int8.
constexpr int gemm_wloads(int fmt) { return fmt == MOE_W_INT8_G128 ? 8 : 4; }

// The bias of the decoded 16-bit values: signed codes BIAS + q (decode.h),
// asymmetric codes MAGIC + q, whose zero point is added per group and
// column (see GemmCtx::step).
template <int ACT, int FMT>
__device__ __forceinline__ constexpr float g128_bias() {
    return FMT == MOE_W_INT8_G128        ? Int8Bias<ACT>::kBias
           : FMT == MOE_W_INT4_G128_ASYM ? Int4Bias<ACT>::kMagicValue
                                         : Int4Bias<ACT>::kBias;
}

// int8: inputs 0..3 in word lo, 4..7 in word hi, bytes masked (a dropped
// group decodes as q = 0) and re-paired as (0, 4) (1, 5) (2, 6) (3, 7).
template <int ACT>
__device__ __forceinline__ uint4 decode_int8_b(uint32_t lo, uint32_t hi, uint32_t bmask) {
    const uint32_t l = (lo & bmask) ^ 0x80808080u, h = (hi & bmask) ^ 0x80808080u;
    const uint32_t t01 = __builtin_amdgcn_perm(h, l, 0x05010400u);   // l0 h0 l1 h1
    const uint32_t t23 = __builtin_amdgcn_perm(h, l, 0x07030602u);   // l2 h2 l3 h3
    return make_uint4(int8_pair<ACT, 0>(t01), int8_pair<ACT, 1>(t01), int8_pair<ACT, 0>(t23),
                      int8_pair<ACT, 1>(t23));
}

struct GemmMat {
    const uint8_t *q, *s;
    const float *gs;
    int64_t qe, qr, se, sr;
    const uint8_t *z;                            // asymmetric int4: zero points [E][n][k/128]
    int64_t ze, zr;
    float xs;                                    // NVFP4 with quantized inputs: the input
                                                 // scale (else 1), with the global scale
};

template <int ACT>
__device__ __forceinline__ f32x16_t mfma32(uint4 a, uint4 b, f32x16_t c) {
    if constexpr (ACT == MOE_BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// 16-bit pair of two float32 values that are exact in the target format.
template <int ACT>
__device__ __forceinline__ uint32_t pack_exact(float lo, float hi) {
    if constexpr (ACT == MOE_BF16)
        return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
    else
        return (uint32_t)f32_to_f16_bits(lo) | ((uint32_t)f32_to_f16_bits(hi) << 16);
}

// B operand (4 dwords = 8 inputs of one output column) from packed word w.
template <int ACT, int FMT>
__device__ __forceinline__ uint4 decode_b(uint32_t w, float bs, uint32_t qmask) {
    if constexpr (FMT == MOE_W_INT4_G128) {
        uint32_t p[4];
        int4_biased_pairs_masked<ACT>(w, qmask, p);
        (void)bs;
        return make_uint4(p[0], p[1], p[2], p[3]);
    } else if constexpr (FMT == MOE_W_INT4_G32) {
        // the 32-input group's scale goes into the operand: q s in 16 bits.
        // fp16: |q| <= 8 has at most 3 significant bits and the bf16 scale
        // 8, so q s is exact (for scales in fp16's normal range), formed by
        // an exact packed subtraction of the bias and an exact product.
        // bf16: q s is exact in float32 and rounded once to bf16.
        (void)qmask;
        uint32_t p[4];
        int4_biased_pairs<ACT>(w, p);
        uint32_t d[4];
        if constexpr (ACT == MOE_F16) {
            const _Float16 sh = (_Float16)bs;
            const half2_t s2 = {sh, sh};
            const half2_t nb = {(_Float16)(-Int4Bias<MOE_F16>::kBias),
                                (_Float16)(-Int4Bias<MOE_F16>::kBias)};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                d[i] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(half2_t, p[i]) + nb) * s2);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float lo = (__uint_as_float(p[i] << 16) - Int4Bias<MOE_BF16>::kBias) * bs;
                const float hi = (__uint_as_float(p[i] & 0xFFFF0000u) - Int4Bias<MOE_BF16>::kBias) * bs;
                d[i] = (uint32_t)f32_to_act<MOE_BF16>(lo) | ((uint32_t)f32_to_act<MOE_BF16>(hi) << 16);
            }
        }
        return make_uint4(d[0], d[1], d[2], d[3]);
    } else if constexpr (FMT == MOE_W_INT4_G128_ASYM) {
        // unsigned codes: MAGIC + q, the same pair order as the signed form
        (void)bs;
        return make_uint4((w & qmask) | Int4Bias<ACT>::kMagic, ((w >> 4) & qmask) | Int4Bias<ACT>::kMagic,
                          ((w >> 8) & qmask) | Int4Bias<ACT>::kMagic,
                          ((w >> 12) & qmask) | Int4Bias<ACT>::kMagic);
    } else {
        (void)qmask;
        uint32_t d[4];
        const uint32_t e[4] = {fp4_pair<MOE_BF16, 0>(w), fp4_pair<MOE_BF16, 1>(w),
                               fp4_pair<MOE_BF16, 2>(w), fp4_pair<MOE_BF16, 3>(w)};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float lo = __uint_as_float(e[i] << 16) * bs;
            const float hi = __uint_as_float(e[i] & 0xFFFF0000u) * bs;
            d[i] = pack_exact<ACT>(lo, hi);
        }
        return make_uint4(d[0], d[1], d[2], d[3]);
    }
}

__device__ __forceinline__ int xcd_remap(int b, int nreal) {
    // Blocks are dispatched round-robin over the 8 XCDs; give each XCD a
    // contiguous range of logical blocks so blocks sharing a tile (and its
    // activation rows) share that XCD's L2. The grid is sized for the most
    // tiles the routing can produce, so the ranges split only the blocks
    // with real work (nreal): each XCD gets its share among the first
    // blocks it is sent, and the rest (-1) exit.
    const int q = nreal / 8, r = nreal % 8, xcd = b % 8, j = b / 8;
    return j < q + (xcd < r ? 1 : 0) ? xcd * q + min(xcd, r) + j : -1;
}

// Weights of one pipeline step for one lane: four 16-byte loads per matrix
// (inputs 64i + 32h .. +31 of the step) and the step's scales.
template <int FMT>
struct StepW {
    uint4 w[gemm_wloads(FMT)];
    uint32_t s32;      // g128 forms: the step's two bf16 group scales
    uint4 s128;        // NVFP4: the step's sixteen E4M3 block scales
    uint32_t z16;      // asymmetric int4: the step's two zero points (bytes)
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t q, __amdgpu_buffer_rsrc_t s,
                                         __amdgpu_buffer_rsrc_t z, int qoff, int soff, int zoff,
                                         int step, int half) {
        if (FMT == MOE_W_INT4_G128_ASYM)
            z16 = __builtin_amdgcn_raw_buffer_load_b16(z, zoff + step * 2, 0, 0);
        if (FMT == MOE_W_INT8_G128) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                w[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                    q, qoff + step * kGemmKS + (i >> 1) * 64 + half * 32 + (i & 1) * 16, 0, 0));
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                w[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                    q, qoff + step * (kGemmKS / 2) + i * 32 + half * 16, 0, 0));
        }
        if (g128_rescaled(FMT))
            s32 = __builtin_amdgcn_raw_buffer_load_b32(s, soff + step * 4, 0, 0);
        else
            s128 = __builtin_bit_cast(uint4,
                                      __builtin_amdgcn_raw_buffer_load_b128(s, soff + step * 16, 0, 0));
    }
};

__device__ __forceinline__ uint32_t half_of(uint4 v, int i) {
    const uint32_t d = i < 4 ? (i < 2 ? v.x : v.y) : (i < 6 ? v.z : v.w);
    return (d >> (16 * (i & 1))) & 0xFFFF;
}

__device__ __forceinline__ uint32_t byte_of(uint4 v, int i) {
    const uint32_t d = i < 8 ? (i < 4 ? v.x : v.y) : (i < 12 ? v.z : v.w);
    return (d >> (8 * (i & 3))) & 0xFF;
}

// LDS layout of one 256-input step of the 64-row activation tile: eight
// 1 KB column groups (4 chunks of 16 bytes = 32 inputs each), and inside a
// group 64 rows of 64 bytes. The chunk slot of a row is XOR-swizzled so
// that one 16-byte read of a chunk by 16 consecutive rows (the lanes one
// cycle of a 64-bank LDS serves) touches 16 different 4-bank groups:
// the group is 4 * (row & 3) + (slot), and the swizzle makes the slot take
// all four values over rows of equal row & 3 (it also spreads 8 rows over
// a 32-bank LDS).
__device__ __forceinline__ int a_swz(int row) { return ((row >> 1) & 3) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int a_offset(int row, int chunk) {
    return ((chunk >> 2) * kGemmTM + row) * 64 + (((chunk & 3) ^ a_swz(row)) << 4);
}

// One step of the 64-row activation tile through registers into LDS.
// Thread t owns row t/4 and chunk slot t%4 of each of the eight column
// groups; the slot holds input chunk (t%4) ^ swz(row), so the four threads
// of a row read 64 contiguous bytes per group and a wave writes 1 KB of LDS
// contiguously. The row's bytes come through a buffer resource at byte
// offset xoff; a padded row's xoff lies past the resource, so its loads
// return zeros without fetching anything (its output row is never
// stored). Thread t < 64 also carries row t's two (-BIAS * group sum)
// values (int4).
template <int FMT>
struct Stager {
    u32x4_t v[8];      // a native vector type: HIP's uint4 struct copies become
                       // memcpy through scratch memory
    float rs0, rs1;
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rx, uint32_t xoff,
                                         const float *sum_row, int step) {
        const int row = threadIdx.x >> 2;
        const int kc = (threadIdx.x & 3) ^ a_swz(row);
#pragma unroll
        for (int g = 0; g < 8; ++g)
            v[g] = __builtin_bit_cast(
                u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                             rx, (int)(xoff + (uint32_t)(step * kGemmKS + (g * 4 + kc) * 8) * 2u),
                             0, 0));
        if (g128_rescaled(FMT) && threadIdx.x < kGemmTM) {
            rs0 = sum_row[2 * step];
            rs1 = sum_row[2 * step + 1];
        }
    }
    __device__ __forceinline__ void store(uint8_t *buf, float *xs) {
        const int row = threadIdx.x >> 2;
#pragma unroll
        for (int g = 0; g < 8; ++g)
            *(u32x4_t *)(buf + (g * kGemmTM + row) * 64 + ((threadIdx.x & 3) << 4)) = v[g];
        if (g128_rescaled(FMT) && threadIdx.x < kGemmTM) {
            xs[threadIdx.x] = rs0;
            xs[kGemmTM + threadIdx.x] = rs1;
        }
    }
};

template <int ACT, int FMT, bool GATEUP>
struct GemmCtx {
    f32x16_t da[2], db[2];
    float sprev_a, sprev_b;
    int half, l32;
    bool two_mb;

    // One 256-input step: MFMAs over the LDS tile `buf` with weights (wa, wb).
    __device__ __forceinline__ void step(const uint8_t *buf, const float *xs,
                                         const StepW<FMT> &wa_s, const StepW<FMT> &wb_s) {
#pragma unroll
        for (int gi = 0; gi < 2; ++gi) {            // two 128-input groups per step
            uint32_t ma = 0, mbk = 0;
            if (g128_rescaled(FMT)) {
                float sa_g = bf16_bits_to_f32(gi ? wa_s.s32 >> 16 : wa_s.s32 & 0xFFFF);
                float sb_g = bf16_bits_to_f32(gi ? wb_s.s32 >> 16 : wb_s.s32 & 0xFFFF);
                // a zero scale drops the group: its codes decode as q = 0
                constexpr uint32_t kKeep = FMT == MOE_W_INT8_G128 ? 0xFFFFFFFFu : 0x000F000Fu;
                ma = sa_g == 0.0f ? 0u : kKeep;
                mbk = sb_g == 0.0f ? 0u : kKeep;
                // and runs with the scale 2^-24 instead: its codes are zeroed,
                // but P - BIAS sum x cancels only up to float32 rounding
                // (~1e-2 of the group's sum), which this scale makes
                // negligible; a power of two keeps every rescale exact
                sa_g = sa_g == 0.0f ? 0x1p-24f : sa_g;
                sb_g = sb_g == 0.0f ? 0x1p-24f : sb_g;
                const float ra = sprev_a * __builtin_amdgcn_rcpf(sa_g);
                const float rb = sprev_b * __builtin_amdgcn_rcpf(sb_g);
                // asymmetric: the group's correction is -(MAGIC + z) sum x, the
                // staged -MAGIC sum x times (MAGIC + z) / MAGIC (exact: MAGIC is
                // a power of two); a dropped group keeps q = 0 and factor 1
                float za = 1.0f, zb = 1.0f;
                if (FMT == MOE_W_INT4_G128_ASYM) {
                    constexpr float kM = Int4Bias<ACT>::kMagicValue;
                    if (ma) za = (kM + (float)((wa_s.z16 >> (8 * gi)) & 0xFFu)) * (1.0f / kM);
                    if (mbk) zb = (kM + (float)((wb_s.z16 >> (8 * gi)) & 0xFFu)) * (1.0f / kM);
                }
                sprev_a = sa_g;
                sprev_b = sb_g;
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) {
                    if (mb == 1 && !two_mb) break;
#pragma unroll
                    for (int b4 = 0; b4 < 4; ++b4) {
                        const float4 x4 = *(const float4 *)&xs[gi * kGemmTM + mb * 32 + 8 * b4 + 4 * half];
                        const float xv[4] = {x4.x, x4.y, x4.z, x4.w};
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float xa = FMT == MOE_W_INT4_G128_ASYM ? xv[r] * za : xv[r];
                            const float xb = FMT == MOE_W_INT4_G128_ASYM ? xv[r] * zb : xv[r];
                            da[mb][4 * b4 + r] = __builtin_fmaf(da[mb][4 * b4 + r], ra, xa);
                            db[mb][4 * b4 + r] = __builtin_fmaf(db[mb][4 * b4 + r], rb, xb);
                        }
                    }
                }
            }
#pragma unroll
            for (int i2 = 0; i2 < 2; ++i2) {
                const int i = 2 * gi + i2;
                // the lane's 32 inputs of 64-input chunk i: one 16-byte word
                // of int4 (8 inputs per dword) or two of int8 (4 per dword)
                constexpr int kW = gemm_wloads(FMT) / 4;
                const uint4 wa = wa_s.w[kW * i], wb = wb_s.w[kW * i];
                const uint4 wa2 = wa_s.w[kW * i + kW - 1], wb2 = wb_s.w[kW * i + kW - 1];
                const uint32_t wav[8] = {wa.x, wa.y, wa.z, wa.w, wa2.x, wa2.y, wa2.z, wa2.w};
                const uint32_t wbv[8] = {wb.x, wb.y, wb.z, wb.w, wb2.x, wb2.y, wb2.z, wb2.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int chunk = i * 8 + half * 4 + j;
                    // int4-g128: both row blocks' activation words first (the
                    // second is read even when unused), so their LDS latency
                    // runs under the decode below (2-3 % at T=2048; the other
                    // formats measured slower this way)
                    constexpr bool kEarlyA = int4_g128(FMT);
                    uint4 avv[2];
                    if constexpr (kEarlyA) {
#pragma unroll
                        for (int mb = 0; mb < 2; ++mb)
                            avv[mb] = *(const uint4 *)(buf + a_offset(mb * 32 + l32, chunk));
                        // issued here, not sunk into the branch that uses the second
                        asm volatile("" ::: "memory");
                    }
                    float bsa = 0.0f, bsb = 0.0f;
                    if (FMT == MOE_W_NVFP4_G16) {
                        const int blk = i * 4 + half * 2 + (j >> 1);
                        bsa = e4m3_to_f32(byte_of(wa_s.s128, blk));
                        bsb = e4m3_to_f32(byte_of(wb_s.s128, blk));
                    }
                    if (FMT == MOE_W_INT4_G32) {
                        // this lane's 32 inputs of the chunk: group 2 i + half
                        bsa = bf16_bits_to_f32(half_of(wa_s.s128, 2 * i + half));
                        bsb = bf16_bits_to_f32(half_of(wb_s.s128, 2 * i + half));
                    }
                    uint4 ob, obb;
                    if constexpr (FMT == MOE_W_INT8_G128) {
                        ob = decode_int8_b<ACT>(wav[2 * j], wav[2 * j + 1], ma);
                        obb = decode_int8_b<ACT>(wbv[2 * j], wbv[2 * j + 1], mbk);
                    } else {
                        ob = decode_b<ACT, FMT>(wav[j], bsa, ma);
                        obb = decode_b<ACT, FMT>(wbv[j], bsb, mbk);
                    }
#pragma unroll
                    for (int mb = 0; mb < 2; ++mb) {
                        if (mb == 1 && !two_mb) break;
                        const uint4 av =
                            kEarlyA ? avv[mb]
                                    : *(const uint4 *)(buf + a_offset(mb * 32 + l32, chunk));
                        da[mb] = mfma32<ACT>(av, ob, da[mb]);
                        db[mb] = mfma32<ACT>(av, obb, db[mb]);
                    }
                }
            }
        }
    }
};

// GATEUP: A = gate, B = up, both for the wave's 32 columns; the epilogue
// writes h = silu(gate) * up. Otherwise A and B are the same down matrix at
// columns c and c + 32, so a wave owns 64 output columns and every
// activation fragment read from LDS feeds two MFMAs in both passes.
// The asymmetric form needs a few registers more than the 256 that keep two
// waves per SIMD; held to two waves it spills 1 - 2 registers, which costs
// less than running one wave per SIMD (T = 2048 gate/up: 824 against 1028
// us). The other formats fit without the bound, and get none.
template <int ACT, int FMT, bool GATEUP>
__global__ void __launch_bounds__(kGemmThreads)
    __attribute__((amdgpu_waves_per_eu(FMT == MOE_W_INT4_G128_ASYM ? 2 : 1))) gemm_kernel(
    GemmMat A, GemmMat Bm, int n_rows, int kin,
    // xin and rowsum_in are not __restrict__: as restrict read-only kernel
    // arguments their loads count as invariant and get sunk below the MFMAs
    // that should hide their latency
    const uint16_t *xin, int64_t x_bytes, int x_from_slots, int topk, const float *rowsum_in,
    const int32_t *__restrict__ sorted_slots, const int32_t *__restrict__ tile_expert,
    const int32_t *__restrict__ num_tiles, int n_blocks, uint16_t *__restrict__ hout,
    float *__restrict__ hsum_out, float *__restrict__ yout, uint16_t *__restrict__ y16,
    int8_t *__restrict__ yexp) {
    constexpr int BN = GATEUP ? kGemmBN : 2 * kGemmBN;      // output columns per block
    // two separate LDS objects per double buffer: the compiler then knows a
    // DMA into one does not alias reads of the other, and does not make the
    // reads wait for the DMA
    __shared__ __attribute__((aligned(16))) uint8_t abuf0[kGemmTM * kGemmRowBytes];
    __shared__ __attribute__((aligned(16))) uint8_t abuf1[kGemmTM * kGemmRowBytes];
    __shared__ __attribute__((aligned(16))) float xsum0[2 * kGemmTM];
    __shared__ __attribute__((aligned(16))) float xsum1[2 * kGemmTM];
    __shared__ int m_sh;

    const int lid = xcd_remap(blockIdx.x, num_tiles[0] * n_blocks);
    if (lid < 0) return;
    const int tile = lid / n_blocks, nb = lid - tile * n_blocks;
    const int e = tile_expert[tile];
    const int groups = kin / 128;

    // this thread's staging row: its byte offset in xin, or past the end
    // for a padded row (loads of zeros that fetch nothing; the host keeps
    // x_bytes below 2^31)
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const __amdgpu_buffer_rsrc_t rx = buffer_rsrc((const uint8_t *)xin, x_bytes);
    uint32_t xoff;
    {
        const int row = threadIdx.x >> 2;
        const int sl = sorted_slots[tile * kGemmTM + row];
        xoff = sl < 0 ? (uint32_t)kOutOfRange
                      : (uint32_t)((x_from_slots ? (size_t)(sl / topk)
                                                 : (size_t)tile * kGemmTM + row) *
                                   kin * 2);
    }
    const float *sum_row = nullptr;
    if (threadIdx.x < kGemmTM) {
        int sl = sorted_slots[tile * kGemmTM + threadIdx.x];
        int prow = threadIdx.x;
        const uint64_t live = __ballot(sl >= 0);
        if (threadIdx.x == 0) m_sh = __popcll(live);
        if (sl < 0) { sl = sorted_slots[tile * kGemmTM]; prow = 0; }
        if (g128_rescaled(FMT))
            sum_row = rowsum_in +
                      (x_from_slots ? (size_t)(sl / topk) : (size_t)tile * kGemmTM + prow) * groups;
    }

    GemmCtx<ACT, FMT, GATEUP> cx;
    cx.half = lane >> 5;
    cx.l32 = lane & 31;
    const int col_a = nb * BN + wave * (GATEUP ? 32 : 64) + cx.l32;
    const int col_b = GATEUP ? col_a : col_a + 32;
    const bool ok_a = col_a < n_rows, ok_b = col_b < n_rows;
    const __amdgpu_buffer_rsrc_t rqa = buffer_rsrc(A.q + e * A.qe, (int64_t)n_rows * A.qr);
    const __amdgpu_buffer_rsrc_t rsa = buffer_rsrc(A.s + e * A.se, (int64_t)n_rows * A.sr);
    const __amdgpu_buffer_rsrc_t rqb = buffer_rsrc(Bm.q + e * Bm.qe, (int64_t)n_rows * Bm.qr);
    const __amdgpu_buffer_rsrc_t rsb = buffer_rsrc(Bm.s + e * Bm.se, (int64_t)n_rows * Bm.sr);
    const int qoff_a = (ok_a ? col_a : 0) * (int)A.qr, soff_a = (ok_a ? col_a : 0) * (int)A.sr;
    const int qoff_b = (ok_b ? col_b : 0) * (int)Bm.qr, soff_b = (ok_b ? col_b : 0) * (int)Bm.sr;
    const bool asym = FMT == MOE_W_INT4_G128_ASYM;
    const __amdgpu_buffer_rsrc_t rza = buffer_rsrc(asym ? A.z + e * A.ze : A.q, asym ? (int64_t)n_rows * A.zr : 0);
    const __amdgpu_buffer_rsrc_t rzb = buffer_rsrc(asym ? Bm.z + e * Bm.ze : Bm.q, asym ? (int64_t)n_rows * Bm.zr : 0);
    const int zoff_a = asym ? (ok_a ? col_a : 0) * (int)A.zr : 0;
    const int zoff_b = asym ? (ok_b ? col_b : 0) * (int)Bm.zr : 0;

#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int v = 0; v < 16; ++v) cx.da[mb][v] = cx.db[mb][v] = 0.0f;
    cx.sprev_a = cx.sprev_b = 1.0f;

    // Pipeline: while step s computes, the activations and the weights of
    // step s+1 load into registers; after the MFMAs the activations go to
    // the other LDS buffer and an LDS-only barrier closes the step, so the
    // weight loads stay in flight until their first use.
    const int nsteps = kin / kGemmKS;
    Stager<FMT> st;
    StepW<FMT> wa0, wb0, wa1, wb1;
    st.load(rx, xoff, sum_row, 0);
    wa0.load(rqa, rsa, rza, qoff_a, soff_a, zoff_a, 0, cx.half);
    wb0.load(rqb, rsb, rzb, qoff_b, soff_b, zoff_b, 0, cx.half);
    st.store(abuf0, xsum0);
    __syncthreads();
    cx.two_mb = m_sh > 32;

#define MOE_GEMM_STEP(S, BUF, XS, NBUF, NXS, WA, WB, NWA, NWB)                          \
    {                                                                                  \
        const int s_ = (S);                                                            \
        if (s_ >= nsteps) break;                                                       \
        const bool more = s_ + 1 < nsteps;                                             \
        /* unconditional (the last step reloads itself): conditional loads */         \
        /* would merge with the old register values and force early waits */         \
        const int sn = more ? s_ + 1 : s_;                                             \
        st.load(rx, xoff, sum_row, sn);                                                \
        NWA.load(rqa, rsa, rza, qoff_a, soff_a, zoff_a, sn, cx.half);                  \
        NWB.load(rqb, rsb, rzb, qoff_b, soff_b, zoff_b, sn, cx.half);                  \
        /* keep the compiler from sinking the prefetch below the MFMAs */             \
        /* (no memory clobber: it would pin the staging registers to memory) */       \
        __builtin_amdgcn_sched_barrier(0);                                             \
        cx.step(BUF, XS, WA, WB);                                                      \
        /* unconditional too, so the loads are not sunk into a branch */              \
        st.store(NBUF, NXS);                                                           \
        lds_barrier();                                                                 \
    }

    for (int step = 0; step < nsteps; step += 2) {
        MOE_GEMM_STEP(step, abuf0, xsum0, abuf1, xsum1, wa0, wb0, wa1, wb1)
        MOE_GEMM_STEP(step + 1, abuf1, xsum1, abuf0, xsum0, wa1, wb1, wa0, wb0)
    }
#undef MOE_GEMM_STEP

    const int m_valid = m_sh;
    const int half = cx.half;
    // NVFP4: the global scale; int4-g128: the last group's scale (the
    // accumulators are kept in its units); int4-g32: 1 (scales in the operands)
    const float ga = FMT == MOE_W_NVFP4_G16 ? A.gs[e] * A.xs : cx.sprev_a;
    const float gb = FMT == MOE_W_NVFP4_G16 ? Bm.gs[e] * Bm.xs : cx.sprev_b;
    float *hs = (float *)abuf0;                    // [64 rows][128 cols] for the row sums
    // position of column c inside the pair-permuted layout of its 8-group
    // (int4 MFMA path only): (c0 c4 c1 c5 c2 c6 c3 c7)
    const int hcol = int4_pairs(FMT) ? (col_a & ~7) | ((col_a & 3) << 1) | ((col_a >> 2) & 1)
                                            : col_a;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int m = mb * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
            const size_t r = (size_t)tile * kGemmTM + m;
            if (GATEUP) {
                const uint16_t hb = f32_to_act<ACT>(silu_mul(cx.da[mb][v] * ga, cx.db[mb][v] * gb));
                if (m < m_valid && ok_a) hout[r * n_rows + hcol] = hb;
                if (g128_rescaled(FMT))
                    hs[m * kGemmBN + wave * 32 + cx.l32] = m < m_valid ? act_to_f32<ACT>(hb) : 0.0f;
            } else if (!gemm_y16(FMT) && m < m_valid) {
                if (ok_a) yout[r * n_rows + col_a] = cx.da[mb][v] * ga;
                if (ok_b) yout[r * n_rows + col_b] = cx.db[mb][v] * gb;
            }
        }
    }
    if (!GATEUP && gemm_y16(FMT)) {
        // y rows in fp16 with a power-of-two scale per (row, 32-column
        // group), y = fp16 * 2^-s: 32 rows of the wave's 64 x 64 tile at a
        // time go through LDS (rows padded to 65 floats, so the column-wise
        // writes and the row-wise reads each touch every bank once); lane L
        // then owns row L % 32, columns 32 (L / 32) .. + 31. Their largest
        // magnitude fixes s (it lands in [2^14, 2^15)), the scaled values
        // round once to fp16 and go out as 64 contiguous bytes, s as one
        // signed byte. The ring buffers are free: the loop ended on a barrier.
        float *tb = (wave < 2 ? (float *)abuf0 : (float *)abuf1) + (wave & 1) * (32 * 65);
        const int colw = nb * BN + wave * 64;
        const int rr = cx.l32, g = half;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            if (mb == 1 && m_valid <= 32) break;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = 8 * (v >> 2) + 4 * half + (v & 3);
                tb[r * 65 + cx.l32] = cx.da[mb][v] * ga;
                tb[r * 65 + 32 + cx.l32] = cx.db[mb][v] * gb;
            }
            float vals[32];
            float mx = 0.0f;
#pragma unroll
            for (int c = 0; c < 32; ++c) {
                vals[c] = tb[rr * 65 + 32 * g + c];
                mx = fmaxf(mx, fabsf(vals[c]));
            }
            int sh = 0;
            if (mx > 0.0f) {
                sh = 15 - __builtin_amdgcn_frexp_expf(mx);
                sh = sh < -127 ? -127 : (sh > 127 ? 127 : sh);
            }
            const int m = mb * 32 + rr;
            if (m < m_valid && colw + 32 * g < n_rows) {
                const size_t r = (size_t)tile * kGemmTM + m;
                uint32_t pk[16];
#pragma unroll
                for (int c = 0; c < 16; ++c) {
                    const _Float16 lo = (_Float16)__builtin_ldexpf(vals[2 * c], sh);
                    const _Float16 hi = (_Float16)__builtin_ldexpf(vals[2 * c + 1], sh);
                    pk[c] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
                }
                uint4 *dst = (uint4 *)(y16 + r * n_rows + colw + 32 * g);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    dst[q] = make_uint4(pk[4 * q], pk[4 * q + 1], pk[4 * q + 2], pk[4 * q + 3]);
                yexp[r * (n_rows / 32) + (colw + 32 * g) / 32] = (int8_t)sh;
            }
        }
    }
    if (GATEUP && g128_rescaled(FMT)) {
        // -BIAS * sum of the rounded h over this block's 128 columns: the
        // down projection's 128-input group nb of row m
        __syncthreads();
        const int row = threadIdx.x >> 2, qtr = threadIdx.x & 3;
        float t = 0.0f;
#pragma unroll 8
        for (int c = 0; c < 32; ++c) t += hs[row * kGemmBN + qtr * 32 + c];
        t += shfl_xor_f(t, 1);
        t += shfl_xor_f(t, 2);
        if (qtr == 0 && row < m_valid)
            hsum_out[((size_t)tile * kGemmTM + row) * n_blocks + nb] = -g128_bias<ACT, FMT>() * t;
    }
}

// int4 MFMA path, once per token: x with the inputs of every 8-group in
// the decoder's pair order (x0 x4 x1 x5 x2 x6 x3 x7), and -BIAS times the
// sum of each 128-input group (float32).
template <int ACT, int FMT>
__global__ void __launch_bounds__(256) prep_x_kernel(const uint16_t *__restrict__ x, int H,
                                                     uint16_t *__restrict__ xp,
                                                     float *__restrict__ sums) {
    const int t = blockIdx.x;
    const int groups = H / 128;
    for (int g0 = 0; g0 < groups; g0 += 16) {
        const int g = g0 + (threadIdx.x >> 4), sub = threadIdx.x & 15;
        float s = 0.0f;
        if (g < groups) {
            const size_t off = (size_t)t * H + g * 128 + sub * 8;
            const uint4 v = *(const uint4 *)(x + off);
            uint4 p;
            p.x = (v.x & 0xFFFFu) | (v.z << 16);
            p.y = (v.x >> 16) | (v.z & 0xFFFF0000u);
            p.z = (v.y & 0xFFFFu) | (v.w << 16);
            p.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
            *(uint4 *)(xp + off) = p;
            const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                s += act_to_f32<ACT>(d[i] & 0xFFFF) + act_to_f32<ACT>(d[i] >> 16);
        }
#pragma unroll
        for (int m = 8; m >= 1; m >>= 1) s += shfl_xor_f(s, m);
        if (g < groups && sub == 0) sums[(size_t)t * groups + g] = -g128_bias<ACT, FMT>() * s;
    }
}

inline GemmMat gemm_mat(const moe_weight_desc_t &d) {
    return GemmMat{(const uint8_t *)d.qweight, (const uint8_t *)d.scale, d.global_scale,
                   d.qweight_expert_stride, d.qweight_row_stride, d.scale_expert_stride,
                   d.scale_row_stride, d.zero_point, d.zero_point_expert_stride,
                   d.zero_point_row_stride, d.input_scale > 0.0f ? d.input_scale : 1.0f};
}

template <int ACT, int FMT>
moe_status_t gemm_forward_t(const moe_ffn_desc_t &ex, const uint16_t *x, int T, int K,
                            const moe_perm_t &p, int max_tiles, uint16_t *h, float *y,
                            uint16_t *y16, int8_t *yexp, uint16_t *xperm, float *xsum, float *hsum,
                            hipStream_t s, const std::function<moe_status_t(int)> &mark) {
    const int F = ex.gate.n, H = ex.gate.k;
    const uint16_t *xa = x;
    if (int4_pairs(FMT)) {
        hipLaunchKernelGGL((prep_x_kernel<ACT, FMT>), dim3(T), dim3(256), 0, s, x, H, xperm, xsum);
        MOE_LAUNCH_CHECK();
        xa = xperm;
    }
    {
        const int nbk = F / kGemmBN;
        hipLaunchKernelGGL((gemm_kernel<ACT, FMT, true>), dim3(max_tiles * nbk),
                           dim3(kGemmThreads), 0, s, gemm_mat(ex.gate), gemm_mat(ex.up), F, H, xa,
                           (int64_t)T * H * 2, 1, K, xsum, p.sorted_slots, p.tile_expert,
                           p.num_tiles, nbk, h, hsum, nullptr, nullptr, nullptr);
        MOE_LAUNCH_CHECK();
    }
    if (mark && mark(1) != MOE_OK) return MOE_ERR_HIP;
    {
        const int nbk = H / (2 * kGemmBN);
        // A and B are the same down matrix; the kernel offsets B by 32 columns
        const GemmMat d = gemm_mat(ex.down);
        hipLaunchKernelGGL((gemm_kernel<ACT, FMT, false>), dim3(max_tiles * nbk),
                           dim3(kGemmThreads), 0, s, d, d, H, F, h,
                           (int64_t)max_tiles * kGemmTM * F * 2, 0, K, hsum, p.sorted_slots,
                           p.tile_expert, p.num_tiles, nbk, nullptr, nullptr, y, y16, yexp);
        MOE_LAUNCH_CHECK();
    }
    if (mark && mark(2) != MOE_OK) return MOE_ERR_HIP;
    return MOE_OK;
}

int gemm_tile_m() { return kGemmTM; }
int gemm_group() { return kGemmKS; }
int gemm_bn() { return kGemmBN; }

bool gemm_stores_y16(int fmt) { return gemm_y16(fmt); }

moe_status_t launch_gemm_forward(const moe_ffn_desc_t &ex, const void *x, int act, int T, int K,
                                 const moe_perm_t &p, int max_tiles, void *h, float *y,
                                 uint16_t *y16, int8_t *yexp, void *xperm, float *xsum,
                                 float *hsum, hipStream_t s,
                                 const std::function<moe_status_t(int)> &mark) {
    const uint16_t *xx = (const uint16_t *)x;
    uint16_t *hh = (uint16_t *)h;
#define MOE_GEMM_FWD(A, F)                                                                    \
    gemm_forward_t<A, F>(ex, xx, T, K, p, max_tiles, hh, y, y16, yexp, (uint16_t *)xperm, xsum, \
                         hsum, s, mark)
    const int f = ex.gate.fmt;
    if (act == MOE_BF16)
        return f == MOE_W_NVFP4_G16        ? MOE_GEMM_FWD(MOE_BF16, MOE_W_NVFP4_G16)
               : f == MOE_W_INT4_G128_ASYM ? MOE_GEMM_FWD(MOE_BF16, MOE_W_INT4_G128_ASYM)
               : f == MOE_W_INT4_G32       ? MOE_GEMM_FWD(MOE_BF16, MOE_W_INT4_G32)
               : f == MOE_W_INT8_G128      ? MOE_GEMM_FWD(MOE_BF16, MOE_W_INT8_G128)
                                           : MOE_GEMM_FWD(MOE_BF16, MOE_W_INT4_G128);
    return f == MOE_W_NVFP4_G16        ? MOE_GEMM_FWD(MOE_F16, MOE_W_NVFP4_G16)
           : f == MOE_W_INT4_G128_ASYM ? MOE_GEMM_FWD(MOE_F16, MOE_W_INT4_G128_ASYM)
           : f == MOE_W_INT4_G32       ? MOE_GEMM_FWD(MOE_F16, MOE_W_INT4_G32)
           : f == MOE_W_INT8_G128      ? MOE_GEMM_FWD(MOE_F16, MOE_W_INT8_G128)
                                       : MOE_GEMM_FWD(MOE_F16, MOE_W_INT4_G128);
#undef MOE_GEMM_FWD
}

}  // namespace moe
