// Expert histogram and stable expert-sorted permutation of the T*K slots.
//
// The pages do not describe this step; it follows from the layer: the
// routed experts are nearly all of the weight bytes (page
// "NeuroSenko/Step-5-Preview-Int4-g128", "Recipe": 96.7 % of the model), so
// all slots of one expert are gathered into padded tiles and the expert's
// weights stream from HBM once.
//
// Batches of up to 1024 slots (decode): one work group. Every slot sets
// its bit in its expert's slot mask in LDS (an OR, so the masks do not
// depend on the order the bits arrive in); an expert's count is the
// popcount of its mask, the offsets come from one block scan, and a slot's
// rank inside its expert is the number of its expert's bits below its own,
// so the order inside an expert is the slot order.
//
// Larger batches: two launches, one block per expert in each, no atomics:
//   count:   block e counts the slots routed to e (compare + ballot).
//   scatter: block e derives its offsets from all counts, then walks the
//            slots in ascending order and compacts its own (ballot prefix
//            inside a wave, wave prefix through LDS), so the order inside
//            an expert is the slot order. It also pads its segment with -1,
//            writes its tile map entries and its place among active experts;
//            the last block writes the totals.
// Ids outside [0, E) are not routed anywhere in either form.
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

constexpr int kPermSmallThreads = 1024;
constexpr int kPermSmallSlots = 1024;

__global__ void __launch_bounds__(kPermSmallThreads) perm_small_kernel(
    const int32_t *__restrict__ ids, int n, int E, int tile_m, int32_t *__restrict__ counts,
    int32_t *__restrict__ expert_offsets, int32_t *__restrict__ padded_offsets,
    int32_t *__restrict__ sorted_slots, int32_t *__restrict__ slot_to_row,
    int32_t *__restrict__ tile_expert, int32_t *__restrict__ num_tiles,
    int32_t *__restrict__ active_experts, int32_t *__restrict__ num_active) {
    extern __shared__ uint64_t sm_masks[];
    const int W = (n + 63) / 64 > 0 ? (n + 63) / 64 : 1;     // mask words per expert
    uint64_t *mask = sm_masks;                               // [E][W]
    int *wtot = (int *)(mask + (size_t)E * W);               // [waves][3]
    int *poff = wtot + 3 * (kPermSmallThreads / kWave);      // [E] padded offsets
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;

    for (int i = tid; i < E * W; i += kPermSmallThreads) mask[i] = 0ull;
    __syncthreads();
    for (int s = tid; s < n; s += kPermSmallThreads) {
        const int e = ids[s];
        if (e >= 0 && e < E)
            atomicOr((unsigned long long *)&mask[e * W + (s >> 6)], 1ull << (s & 63));
    }
    __syncthreads();

    // thread e: count, padded count, active flag; exclusive scans over e
    const int e = tid;
    int c = 0;
    if (e < E)
        for (int w = 0; w < W; ++w) c += __popcll(mask[e * W + w]);
    const int pc = (c + tile_m - 1) / tile_m * tile_m, a = c > 0;
    int ic = c, ip = pc, ia = a;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int tc = __shfl_up(ic, d, kWave), tp = __shfl_up(ip, d, kWave);
        const int ta = __shfl_up(ia, d, kWave);
        if (lane >= d) { ic += tc; ip += tp; ia += ta; }
    }
    if (lane == kWave - 1) {
        wtot[3 * wave] = ic;
        wtot[3 * wave + 1] = ip;
        wtot[3 * wave + 2] = ia;
    }
    __syncthreads();
    int bc = 0, bp = 0, ba = 0;
    for (int w = 0; w < wave; ++w) {
        bc += wtot[3 * w];
        bp += wtot[3 * w + 1];
        ba += wtot[3 * w + 2];
    }
    const int xc = bc + ic - c, xp = bp + ip - pc, xa = ba + ia - a;
    if (e < E) {
        poff[e] = xp;
        counts[e] = c;
        expert_offsets[e] = xc;
        padded_offsets[e] = xp;
        if (c > 0) active_experts[xa] = e;
        for (int i = 0; i < pc / tile_m; ++i) tile_expert[xp / tile_m + i] = e;
        for (int i = c; i < pc; ++i) sorted_slots[xp + i] = -1;
        if (e == E - 1) {
            expert_offsets[E] = xc + c;
            padded_offsets[E] = xp + pc;
            num_tiles[0] = (xp + pc) / tile_m;
            num_active[0] = xa + a;
        }
    }
    __syncthreads();

    // a slot's rank among its expert's slots: that expert's bits below it
    for (int s = tid; s < n; s += kPermSmallThreads) {
        const int ee = ids[s];
        if (ee < 0 || ee >= E) continue;
        const uint64_t *m = mask + (size_t)ee * W;
        int r = __popcll(m[s >> 6] & ((1ull << (s & 63)) - 1ull));
        for (int w = 0; w < (s >> 6); ++w) r += __popcll(m[w]);
        const int row = poff[ee] + r;
        sorted_slots[row] = s;
        slot_to_row[s] = row;
    }
}

moe_status_t launch_permute(const int32_t *ids, int T, int K, int E, const moe_perm_t &p,
                            hipStream_t s) {
    const int n = T * K;
    if (n <= kPermSmallSlots && E <= kPermSmallThreads) {
        const int W = n > 0 ? (n + 63) / 64 : 1;
        const size_t lds = (size_t)E * W * 8 + 3 * (kPermSmallThreads / kWave) * 4 + (size_t)E * 4;
        if (lds > 65536 &&
            hipFuncSetAttribute((const void *)perm_small_kernel,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
            return MOE_ERR_HIP;
        hipLaunchKernelGGL(perm_small_kernel, dim3(1), dim3(kPermSmallThreads), lds, s, ids, n, E,
                           p.tile_m, p.counts, p.expert_offsets, p.padded_offsets, p.sorted_slots,
                           p.slot_to_row, p.tile_expert, p.num_tiles, p.active_experts,
                           p.num_active);
        MOE_LAUNCH_CHECK();
        return MOE_OK;
    }
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
