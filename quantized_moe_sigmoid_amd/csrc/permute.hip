// Expert histogram and stable expert-sorted permutation of the T*K slots.
//
// The pages do not describe this step; it follows from the layer: the
// routed experts are nearly all of the weight bytes (page
// "NeuroSenko/Step-5-Preview-Int4-g128", "Recipe": 96.7 % of the model), so
// all slots of one expert are gathered into padded tiles and the expert's
// weights stream from HBM once.
//
// Two launches, one block per expert in each, no atomics:
//   count:   block e counts the slots routed to e (compare + ballot).
//   scatter: block e derives its offsets from all counts, then walks the
//            slots in ascending order and compacts its own (ballot prefix
//            inside a wave, wave prefix through LDS), so the order inside
//            an expert is the slot order. It also pads its segment with -1,
//            writes its tile map entries and its place among active experts;
//            the last block writes the totals.
#include "common.h"

namespace moe {

constexpr int kPermThreads = 256;
constexpr int kPermWaves = kPermThreads / kWave;

__device__ __forceinline__ int block_sum(int v, int *red) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    int s = 0;
#pragma unroll
    for (int w = 0; w < kPermWaves; ++w) s += red[w];
    return s;
}

__global__ void __launch_bounds__(kPermThreads) perm_count_kernel(
    const int32_t *__restrict__ ids, int n, int32_t *__restrict__ counts) {
    __shared__ int red[kPermWaves];
    const int e = blockIdx.x;
    int c = 0;
    for (int i = threadIdx.x; i < n; i += kPermThreads) c += (ids[i] == e);
    c = block_sum(c, red);
    if (threadIdx.x == 0) counts[e] = c;
}

__global__ void __launch_bounds__(kPermThreads) perm_scatter_kernel(
    const int32_t *__restrict__ ids, int n, int E, int tile_m,
    const int32_t *__restrict__ counts, int32_t *__restrict__ expert_offsets,
    int32_t *__restrict__ padded_offsets, int32_t *__restrict__ sorted_slots,
    int32_t *__restrict__ slot_to_row, int32_t *__restrict__ tile_expert,
    int32_t *__restrict__ num_tiles, int32_t *__restrict__ active_experts,
    int32_t *__restrict__ num_active) {
    __shared__ int red[kPermWaves];
    __shared__ int wave_cnt[kPermWaves];
    const int e = blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;

    // Offsets of e from the counts of all experts below it.
    int below = 0, below_pad = 0, below_act = 0;
    for (int j = threadIdx.x; j < e; j += kPermThreads) {
        const int c = counts[j];
        below += c;
        below_pad += (c + tile_m - 1) / tile_m * tile_m;
        below_act += (c > 0);
    }
    below = block_sum(below, red);
    below_pad = block_sum(below_pad, red);
    below_act = block_sum(below_act, red);
    const int cnt = counts[e];
    const int pad_cnt = (cnt + tile_m - 1) / tile_m * tile_m;
    if (threadIdx.x == 0) {
        expert_offsets[e] = below;
        padded_offsets[e] = below_pad;
        if (cnt > 0) active_experts[below_act] = e;
        if (e == E - 1) {
            expert_offsets[E] = below + cnt;
            padded_offsets[E] = below_pad + pad_cnt;
            num_tiles[0] = (below_pad + pad_cnt) / tile_m;
            num_active[0] = below_act + (cnt > 0);
        }
    }
    for (int i = threadIdx.x; i < pad_cnt / tile_m; i += kPermThreads)
        tile_expert[below_pad / tile_m + i] = e;
    for (int i = cnt + threadIdx.x; i < pad_cnt; i += kPermThreads)
        sorted_slots[below_pad + i] = -1;
    if (cnt == 0) return;

    // Stable compaction of the slots routed to e.
    int base = 0;
    for (int s0 = 0; s0 < n; s0 += kPermThreads) {
        const int s = s0 + threadIdx.x;
        const bool hit = s < n && ids[s] == e;
        const uint64_t m = __ballot(hit);
        const int rank = __popcll(m & ((1ull << lane) - 1ull));
        __syncthreads();
        if (lane == 0) wave_cnt[wave] = __popcll(m);
        __syncthreads();
        int pre = 0;
#pragma unroll
        for (int w = 0; w < kPermWaves; ++w) pre += (w < wave) ? wave_cnt[w] : 0;
        if (hit) {
            const int row = below_pad + base + pre + rank;
            sorted_slots[row] = s;
            slot_to_row[s] = row;
        }
        int tot = 0;
#pragma unroll
        for (int w = 0; w < kPermWaves; ++w) tot += wave_cnt[w];
        base += tot;
        if (base >= cnt) break;          // uniform across the block
    }
}

moe_status_t launch_permute(const int32_t *ids, int T, int K, int E, const moe_perm_t &p,
                            hipStream_t s) {
    const int n = T * K;
    hipLaunchKernelGGL(perm_count_kernel, dim3(E), dim3(kPermThreads), 0, s, ids, n, p.counts);
    MOE_LAUNCH_CHECK();
    hipLaunchKernelGGL(perm_scatter_kernel, dim3(E), dim3(kPermThreads), 0, s, ids, n, E,
                       p.tile_m, p.counts, p.expert_offsets, p.padded_offsets, p.sorted_slots,
                       p.slot_to_row, p.tile_expert, p.num_tiles, p.active_experts,
                       p.num_active);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

}  // namespace moe
