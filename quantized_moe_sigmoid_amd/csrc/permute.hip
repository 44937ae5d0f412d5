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
// Larger batches: one launch, one block per expert. Up to 32768 slots the
// block first copies the ids into LDS. Block e counts every expert's slots
// in LDS (integer adds: the counts do
// not depend on the order they arrive in), derives its offsets from the
// counts below it, then walks the slots in ascending order and compacts
// its own (ballot prefix inside a wave, wave prefix through LDS), so the
// order inside an expert is the slot order. It also pads its segment with
// -1, writes its tile map entries and its place among active experts; the
// last block writes the totals.
// Ids outside [0, E) are not routed anywhere in either form: such a slot
// gets slot_to_row -1 and no row, and the combine adds nothing for it.
#include "topk.h"

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

// Larger batches: one block per expert. Each block builds the histogram of
// all slots in LDS (integer adds, whose sum does not depend on their
// order), takes its offsets from the counts of the experts below it, and
// compacts its own slots in slot order, kPermPass slots per pass: thread t
// holds slots s0 + 256 j + t (j < 8), ranked by one ballot per j and wave.
constexpr int kPermPerThread = 8, kPermPass = kPermThreads * kPermPerThread;
constexpr int kPermStageMax = 32768;          // slots whose ids a block stages in LDS (64 KB)

// STAGE: the block first copies all ids into LDS (16-bit; E <= 512, a
// foreign id becomes 0xFFFF), so its passes read LDS instead of L2.
template <bool STAGE>
__global__ void __launch_bounds__(kPermThreads) perm_large_kernel(
    const int32_t *__restrict__ ids, int n, int E, int tile_m, int32_t *__restrict__ counts,
    int32_t *__restrict__ expert_offsets, int32_t *__restrict__ padded_offsets,
    int32_t *__restrict__ sorted_slots, int32_t *__restrict__ slot_to_row,
    int32_t *__restrict__ tile_expert, int32_t *__restrict__ num_tiles,
    int32_t *__restrict__ active_experts, int32_t *__restrict__ num_active) {
    extern __shared__ int hist[];                              // [E], then STAGE: ids [n]
    uint16_t *sid = (uint16_t *)(hist + ((E + 3) & ~3));
    __shared__ int red[kPermWaves];
    __shared__ int wcnt[2][kPermPerThread][kPermWaves];        // by pass parity
    const int e = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid >> 6;
    auto id_at = [&](int s) -> int {
        if constexpr (STAGE) {
            const int v = sid[s];
            return v == 0xFFFF ? -1 : v;
        } else {
            return ids[s];
        }
    };

    for (int j = tid; j < E; j += kPermThreads) hist[j] = 0;
    if constexpr (STAGE) {
        // 16 loads in flight per thread
        for (int s0 = 0; s0 < n; s0 += 16 * kPermThreads) {
            int v[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int s = s0 + j * kPermThreads + tid;
                v[j] = s < n ? ids[s] : -1;
            }
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int s = s0 + j * kPermThreads + tid;
                if (s < n) sid[s] = (uint16_t)(v[j] >= 0 && v[j] < E ? v[j] : 0xFFFF);
            }
        }
    }
    __syncthreads();
    for (int s0 = 0; s0 < n; s0 += kPermPass) {
        int v[kPermPerThread];
#pragma unroll
        for (int j = 0; j < kPermPerThread; ++j) {
            const int s = s0 + j * kPermThreads + tid;
            v[j] = s < n ? id_at(s) : -1;
        }
#pragma unroll
        for (int j = 0; j < kPermPerThread; ++j)
            if (v[j] >= 0 && v[j] < E) atomicAdd(&hist[v[j]], 1);
    }
    // slots with a foreign id, spread over the blocks: no row
    for (int i = e * kPermThreads + tid; i < n; i += E * kPermThreads) {
        const int id = ids[i];
        if (id < 0 || id >= E) slot_to_row[i] = -1;
    }
    __syncthreads();

    // Offsets of e from the counts of the experts below it.
    int below = 0, below_pad = 0, below_act = 0;
    for (int j = tid; j < e; j += kPermThreads) {
        const int c = hist[j];
        below += c;
        below_pad += (c + tile_m - 1) / tile_m * tile_m;
        below_act += (c > 0);
    }
    below = block_sum(below, red);
    below_pad = block_sum(below_pad, red);
    below_act = block_sum(below_act, red);
    const int cnt = hist[e];
    const int pad_cnt = (cnt + tile_m - 1) / tile_m * tile_m;
    if (tid == 0) {
        counts[e] = cnt;
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
    for (int i = tid; i < pad_cnt / tile_m; i += kPermThreads)
        tile_expert[below_pad / tile_m + i] = e;
    for (int i = cnt + tid; i < pad_cnt; i += kPermThreads) sorted_slots[below_pad + i] = -1;

    // Stable compaction of the slots routed to e. Pass i writes wave counts
    // into wcnt[i % 2] and reads them after one barrier; pass i + 2 writes
    // the same half only after every thread has passed pass i + 1's barrier.
    const uint64_t below_lane = (1ull << lane) - 1ull;
    int base = 0, par = 0;
    for (int s0 = 0; s0 < n && base < cnt; s0 += kPermPass) {   // base: uniform
        bool hit[kPermPerThread];
        int rank[kPermPerThread];
#pragma unroll
        for (int j = 0; j < kPermPerThread; ++j) {
            const int s = s0 + j * kPermThreads + tid;
            hit[j] = s < n && id_at(s) == e;
            const uint64_t m = __ballot(hit[j]);
            rank[j] = __popcll(m & below_lane);
            if (lane == 0) wcnt[par][j][wave] = __popcll(m);
        }
        __syncthreads();
        int before = 0;                          // slots of e earlier in this pass
#pragma unroll
        for (int j = 0; j < kPermPerThread; ++j) {
            int pre = 0, tot = 0;
#pragma unroll
            for (int w = 0; w < kPermWaves; ++w) {
                const int c = wcnt[par][j][w];
                pre += w < wave ? c : 0;
                tot += c;
            }
            if (hit[j]) {
                const int s = s0 + j * kPermThreads + tid;
                const int row = below_pad + base + before + pre + rank[j];
                sorted_slots[row] = s;
                slot_to_row[s] = row;
            }
            before += tot;
        }
        base += before;
        par ^= 1;
    }
}

constexpr int kPermSmallThreads = 1024;
constexpr int kPermSmallSlots = 1024;

// LDS bytes of the one-group permutation of n slots over E experts: the
// slot masks [E][W], the per-wave scan totals, the padded offsets [E].
__host__ __device__ inline size_t perm_small_lds(int n, int E) {
    const int W = n > 0 ? (n + 63) / 64 : 1;
    return (size_t)E * W * 8 + 3 * (kPermSmallThreads / kWave) * 4 + (size_t)E * 4;
}

// The one-group permutation (NT threads, at least E) of n slots whose ids
// id_at(s) returns, LDS at sm (perm_small_lds bytes).
template <int NT, typename IdFn>
__device__ __forceinline__ void perm_small_body(
    IdFn id_at, int n, int E, int tile_m, uint64_t *sm, int32_t *__restrict__ counts,
    int32_t *__restrict__ expert_offsets, int32_t *__restrict__ padded_offsets,
    int32_t *__restrict__ sorted_slots, int32_t *__restrict__ slot_to_row,
    int32_t *__restrict__ tile_expert, int32_t *__restrict__ num_tiles,
    int32_t *__restrict__ active_experts, int32_t *__restrict__ num_active) {
    const int W = (n + 63) / 64 > 0 ? (n + 63) / 64 : 1;     // mask words per expert
    uint64_t *mask = sm;                                     // [E][W]
    int *wtot = (int *)(mask + (size_t)E * W);               // [waves][3]
    int *poff = wtot + 3 * (kPermSmallThreads / kWave);      // [E] padded offsets
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;

    for (int i = tid; i < E * W; i += NT) mask[i] = 0ull;
    __syncthreads();
    for (int s = tid; s < n; s += NT) {
        const int e = id_at(s);
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
    for (int s = tid; s < n; s += NT) {
        const int ee = id_at(s);
        if (ee < 0 || ee >= E) {
            slot_to_row[s] = -1;
            continue;
        }
        const uint64_t *m = mask + (size_t)ee * W;
        int r = __popcll(m[s >> 6] & ((1ull << (s & 63)) - 1ull));
        for (int w = 0; w < (s >> 6); ++w) r += __popcll(m[w]);
        const int row = poff[ee] + r;
        sorted_slots[row] = s;
        slot_to_row[s] = row;
    }
}

__global__ void __launch_bounds__(kPermSmallThreads) perm_small_kernel(
    const int32_t *__restrict__ ids, int n, int E, int tile_m, int32_t *__restrict__ counts,
    int32_t *__restrict__ expert_offsets, int32_t *__restrict__ padded_offsets,
    int32_t *__restrict__ sorted_slots, int32_t *__restrict__ slot_to_row,
    int32_t *__restrict__ tile_expert, int32_t *__restrict__ num_tiles,
    int32_t *__restrict__ active_experts, int32_t *__restrict__ num_active) {
    extern __shared__ uint64_t sm_masks[];
    perm_small_body<kPermSmallThreads>([&](int s) { return ids[s]; }, n, E, tile_m, sm_masks, counts,
                    expert_offsets, padded_offsets, sorted_slots, slot_to_row, tile_expert,
                    num_tiles, active_experts, num_active);
}

// Top-K and permutation of a batch of up to 16 tokens in one launch: wave t
// selects token t's experts from its scores (the logits, or P block sums
// [P][T][E] added in block order, then the bias) and keeps the ids in LDS
// too; after one barrier the group permutes them as perm_small_kernel does.
// Bitwise the results of route_given_kernel followed by perm_small_kernel.
constexpr int kRoutePermMaxT = kPermSmallThreads / kWave;
// Up to 6 tokens over at most 384 experts: 6 waves instead of 16 (fewer
// waves to launch and to meet at each barrier; the same results).
constexpr int kRoutePermFewT = 6, kRoutePermFewThreads = kRoutePermFewT * kWave;

template <int NT>
__global__ void __launch_bounds__(NT) route_perm_small_kernel(
    const float *__restrict__ scores, const float *__restrict__ bias, int T, int E, int K,
    int renorm, int P, int32_t *__restrict__ ids, float *__restrict__ wts, int tile_m,
    int32_t *__restrict__ counts, int32_t *__restrict__ expert_offsets,
    int32_t *__restrict__ padded_offsets, int32_t *__restrict__ sorted_slots,
    int32_t *__restrict__ slot_to_row, int32_t *__restrict__ tile_expert,
    int32_t *__restrict__ num_tiles, int32_t *__restrict__ active_experts,
    int32_t *__restrict__ num_active) {
    extern __shared__ uint64_t sm_masks[];
    const int n = T * K;
    int32_t *sid = (int32_t *)((char *)sm_masks + perm_small_lds(n, E));   // [n]
    const int t = threadIdx.x >> 6;
    if (t < T)
        token_topk(scores + (size_t)t * E, (size_t)T * E, P, bias, E, K, renorm,
                   ids + (size_t)t * K, wts + (size_t)t * K, sid + t * K);
    __syncthreads();
    perm_small_body<NT>([&](int s) { return sid[s]; }, n, E, tile_m, sm_masks, counts,
                    expert_offsets, padded_offsets, sorted_slots, slot_to_row, tile_expert,
                    num_tiles, active_experts, num_active);
}

bool route_perm_fused(int T, int K) { return T <= kRoutePermMaxT && T * K <= kPermSmallSlots; }

moe_status_t launch_route_perm_small(const float *scores, const float *bias, int T, int E, int K,
                                     int renorm, int P, int32_t *ids, float *wts,
                                     const moe_perm_t &p, hipStream_t s) {
    if (T == 0) return MOE_OK;
    const size_t lds = perm_small_lds(T * K, E) + (size_t)T * K * 4;
    const bool few = T <= kRoutePermFewT && E <= kRoutePermFewThreads;
    const void *k = few ? (const void *)route_perm_small_kernel<kRoutePermFewThreads>
                        : (const void *)route_perm_small_kernel<kPermSmallThreads>;
    if (lds > 65536 &&
        hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
        return MOE_ERR_HIP;
#define MOE_ROUTE_PERM(NT)                                                                      \
    hipLaunchKernelGGL(route_perm_small_kernel<NT>, dim3(1), dim3(NT), lds, s, scores, bias, T, E, \
                       K, renorm, P, ids, wts, p.tile_m, p.counts, p.expert_offsets,           \
                       p.padded_offsets, p.sorted_slots, p.slot_to_row, p.tile_expert,          \
                       p.num_tiles, p.active_experts, p.num_active)
    if (few)
        MOE_ROUTE_PERM(kRoutePermFewThreads);
    else
        MOE_ROUTE_PERM(kPermSmallThreads);
#undef MOE_ROUTE_PERM
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

moe_status_t launch_permute(const int32_t *ids, int T, int K, int E, const moe_perm_t &p,
                            hipStream_t s) {
    const int n = T * K;
    if (n <= kPermSmallSlots && E <= kPermSmallThreads) {
        const size_t lds = perm_small_lds(n, E);
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
    const size_t hist_b = (size_t)((E + 3) & ~3) * sizeof(int);
    if (n <= kPermStageMax) {
        const size_t lds = hist_b + (size_t)n * sizeof(uint16_t);
        if (lds > 65536 &&
            hipFuncSetAttribute((const void *)perm_large_kernel<true>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
            return MOE_ERR_HIP;
        hipLaunchKernelGGL(perm_large_kernel<true>, dim3(E), dim3(kPermThreads), lds, s, ids, n, E,
                           p.tile_m, p.counts, p.expert_offsets, p.padded_offsets, p.sorted_slots,
                           p.slot_to_row, p.tile_expert, p.num_tiles, p.active_experts,
                           p.num_active);
    } else {
        hipLaunchKernelGGL(perm_large_kernel<false>, dim3(E), dim3(kPermThreads), hist_b, s, ids,
                           n, E, p.tile_m, p.counts, p.expert_offsets, p.padded_offsets,
                           p.sorted_slots, p.slot_to_row, p.tile_expert, p.num_tiles,
                           p.active_experts, p.num_active);
    }
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

}  // namespace moe
