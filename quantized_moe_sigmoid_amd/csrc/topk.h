// Sigmoid top-K selection of one token's expert scores by one wave (page
// "Step-5-Preview-Spark", "At a glance": a sigmoid router choosing the top
// 8 of 352 routed experts): the K largest logits by (logit desc, expert
// asc), per round a wave maximum of the logits' order-preserving 32-bit
// images, ties resolved to the lowest expert index by ballots, -0 folded to
// +0 first; weights sigmoid of the selected logits, renormalised to sum to
// one when asked (summed in ascending k). Shared by the router's top-K
// kernel and the fused top-K + permutation.
#pragma once

#include "common.h"

#pragma clang fp contract(off)

namespace moe {

constexpr int kMaxE = 512;

// Inputs per block of the canonical logit sum, and the most blocks whose
// sums the top-K adds up (the block-sum paths take H <= 4096).
constexpr int kRouterBlock = 512;
constexpr int kMaxRouterBlocks = 8;

// Order-preserving image of a float in uint32 (a larger float maps to a
// larger value; -0 is folded to +0 first); 0 lies below every image.
__device__ __forceinline__ uint32_t ord32(float f) {
    const uint32_t u = __float_as_uint(f + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ord32_value(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// Maximum over the wave: four DPP butterflies inside each 16-lane row
// (quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror;
// every lane then holds its row's maximum), then the four rows through
// scalar registers.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_max(uint32_t v) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
    return v > o ? v : o;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = dpp_max<0xB1>(v);
    v = dpp_max<0x4E>(v);
    v = dpp_max<0x141>(v);
    v = dpp_max<0x140>(v);
    const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
    const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
    const uint32_t a = r0 > r1 ? r0 : r1, b = r2 > r3 ? r2 : r3;
    return a > b ? a : b;
}

// Lane l owns experts l, l+64, ... (slot j: expert 64 j + lane).
constexpr int kTopkSlots = kMaxE / kWave;

// The selection over the order images o (0 for experts past E): each round
// takes the wave maximum, then the lowest expert holding it (the first slot
// whose ballot hits, at its lowest lane). Writes the token's K ids and
// weights, and the ids also to ids_lds when that is not null.
__device__ __forceinline__ void wave_topk_keys(uint32_t (&o)[kTopkSlots], int K, int renorm,
                                               int32_t *ids, float *wts, int32_t *ids_lds) {
    constexpr int NJ = kTopkSlots;
    const int lane = threadIdx.x & (kWave - 1);
    float my_logit = 0.0f;
    int my_id = 0;
    for (int r = 0; r < K; ++r) {
        uint32_t m = o[0];
#pragma unroll
        for (int j = 1; j < NJ; ++j) m = o[j] > m ? o[j] : m;
        const uint32_t best = wave_max_u32(m);
        int win = -1;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const uint64_t b = __ballot(o[j] == best);
            if (win < 0 && b) win = j * kWave + __ffsll((unsigned long long)b) - 1;
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            if (j * kWave + lane == win) o[j] = 0u;
        if (lane == r) { my_id = win; my_logit = ord32_value(best); }
    }
    float p = 1.0f / (1.0f + expf(-my_logit));
    if (renorm) {
        // sum over lanes 0..K-1 in ascending order (deterministic)
        float s = 0.0f;
        for (int r = 0; r < K; ++r) s += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), r));
        p = p / s;
    }
    if (lane < K) {
        ids[lane] = my_id;
        wts[lane] = p;
        if (ids_lds) ids_lds[lane] = my_id;
    }
}

// One token's top-K from its scores: row[e] (the logits, P = 1) or the P
// block sums row[p * pstride + e], added in block order, then the bias.
// Every slot's values (and bias) are loaded before any addition, as
// unconditional loads at clamped addresses (the extra ones unused): with
// the loads behind per-block branches each slot waited out its own round
// trip (17.4 against 7.2 us at T = 32).
__device__ __forceinline__ void token_topk(const float *row, size_t pstride, int P,
                                           const float *bias, int E, int K, int renorm,
                                           int32_t *ids, float *wts, int32_t *ids_lds) {
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t o[kTopkSlots];
    if (P == 1) {
        float q[kTopkSlots], bv[kTopkSlots];
#pragma unroll
        for (int j = 0; j < kTopkSlots; ++j) {
            const int e = min(lane + j * kWave, E - 1);
            q[j] = row[e];
            bv[j] = bias ? bias[e] : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < kTopkSlots; ++j)
            o[j] = lane + j * kWave < E ? ord32(bias ? q[j] + bv[j] : q[j]) : 0u;
    } else {
        float q[kTopkSlots][kMaxRouterBlocks], bv[kTopkSlots];
#pragma unroll
        for (int j = 0; j < kTopkSlots; ++j) {
            const int e = min(lane + j * kWave, E - 1);
#pragma unroll
            for (int p = 0; p < kMaxRouterBlocks; ++p)
                q[j][p] = row[min(p, P - 1) * pstride + e];
            bv[j] = bias ? bias[e] : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < kTopkSlots; ++j) {
            float v = q[j][0];
#pragma unroll
            for (int p = 1; p < kMaxRouterBlocks; ++p)
                if (p < P) v = v + q[j][p];
            if (bias) v = v + bv[j];
            o[j] = lane + j * kWave < E ? ord32(v) : 0u;
        }
    }
    wave_topk_keys(o, K, renorm, ids, wts, ids_lds);
}

}  // namespace moe
