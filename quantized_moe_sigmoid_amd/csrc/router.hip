// Sigmoid top-K router (page "Step-5-Preview-Spark", "At a glance": a
// sigmoid router choosing the top 8 of 352 routed experts).
//
// Logits are either computed here from the 16-bit activations and the
// float32 router weight stored transposed ([H][E]), or given. The logit of
// (t, e) is the float32 chain acc = fma(x[t][k], wT[k][e], acc) over k
// ascending from +0: one fixed order, so the chosen experts are the same on
// every run and on the CPU reference. The pages show why the order matters:
// a different summation order inside the MoE flips near-tied expert choices
// ("Step-5-Preview-Spark", "Quality", noise-floor paragraph).
//
// Selection: the K largest logits by (logit desc, expert asc), as 64-bit
// keys (order-preserving float bits << 32 | ~expert) reduced across a wave;
// -0 is folded to +0 first. Weights: sigmoid of the selected logits,
// renormalised to sum to one when asked.
#include "common.h"

#pragma clang fp contract(off)

namespace moe {

constexpr int kRouteTok = 8;       // tokens per block in the logit kernel
constexpr int kRouteKC = 256;      // k-chunk of x staged in LDS
constexpr int kMaxE = 512;
constexpr int kMaxK = 16;

__device__ __forceinline__ uint64_t topk_key(float f, int e) {
    uint32_t u = __float_as_uint(f + 0.0f);          // -0 -> +0
    uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)ord << 32) | (uint32_t)(~(uint32_t)e);
}
__device__ __forceinline__ float key_value(uint64_t key) {
    uint32_t ord = (uint32_t)(key >> 32);
    uint32_t u = (ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord;
    return __uint_as_float(u);
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        uint32_t lo = __shfl_xor((uint32_t)v, m, kWave);
        uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, kWave);
        uint64_t o = ((uint64_t)hi << 32) | lo;
        v = o > v ? o : v;
    }
    return v;
}

// One wave selects the top K of E logits held in `lg` (LDS or global).
// Lane l owns experts l, l+64, ... Writes ids / weights for one token.
template <typename LoadFn>
__device__ __forceinline__ void wave_topk(LoadFn load, int E, int K, int renorm,
                                          int32_t *ids, float *wts) {
    const int lane = threadIdx.x & (kWave - 1);
    uint64_t keys[kMaxE / kWave];
#pragma unroll
    for (int j = 0; j < kMaxE / kWave; ++j) {
        int e = lane + j * kWave;
        keys[j] = e < E ? topk_key(load(e), e) : 0ull;    // 0 = below any real key
    }
    float my_logit = 0.0f;
    int my_id = 0;
    for (int r = 0; r < K; ++r) {
        uint64_t best = 0;
#pragma unroll
        for (int j = 0; j < kMaxE / kWave; ++j) best = keys[j] > best ? keys[j] : best;
        best = wave_max_u64(best);
        const int e = (int)(~(uint32_t)best);
#pragma unroll
        for (int j = 0; j < kMaxE / kWave; ++j)
            if (keys[j] == best) keys[j] = 0;
        if (lane == r) { my_id = e; my_logit = key_value(best); }
    }
    float p = 1.0f / (1.0f + expf(-my_logit));
    if (renorm) {
        // sum over lanes 0..K-1 in ascending order (deterministic)
        float s = 0.0f;
        for (int r = 0; r < K; ++r) s += __shfl(p, r, kWave);
        p = p / s;
    }
    if (lane < K) { ids[lane] = my_id; wts[lane] = p; }
}

// Logits given: one wave per token.
__global__ void __launch_bounds__(256) route_given_kernel(
    const float *__restrict__ logits, const float *__restrict__ bias, int T, int E, int K,
    int renorm, int32_t *__restrict__ ids, float *__restrict__ wts) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const float *row = logits + (size_t)t * E;
    auto load = [&](int e) {
        float v = row[e];
        if (bias) v = v + bias[e];
        return v;
    };
    wave_topk(load, E, K, renorm, ids + (size_t)t * K, wts + (size_t)t * K);
}

// Logits computed: a block owns kRouteTok tokens and all experts; thread e
// runs the kRouteTok fma chains of expert e in k order, then waves select.
template <int ACT>
__global__ void __launch_bounds__(512) route_logits_kernel(
    const uint16_t *__restrict__ x, const float *__restrict__ wT,
    const float *__restrict__ bias, int T, int H, int E, int K, int renorm,
    int32_t *__restrict__ ids, float *__restrict__ wts) {
    __shared__ float xs[kRouteKC][kRouteTok];     // token-minor: 2 x b128 reads
    __shared__ float lg[kRouteTok][kMaxE];
    const int t0 = blockIdx.x * kRouteTok;
    const int e = threadIdx.x;
    const int nthr = blockDim.x;
    float acc[kRouteTok];
#pragma unroll
    for (int i = 0; i < kRouteTok; ++i) acc[i] = 0.0f;

    for (int k0 = 0; k0 < H; k0 += kRouteKC) {
        const int kc = min(kRouteKC, H - k0);
        __syncthreads();
        for (int i = threadIdx.x; i < kRouteTok * kc; i += nthr) {
            const int tt = i / kc, kk = i - tt * kc;
            const int t = t0 + tt;
            xs[kk][tt] = t < T ? act_to_f32<ACT>(x[(size_t)t * H + k0 + kk]) : 0.0f;
        }
        __syncthreads();
        if (e < E) {
            const float *w = wT + (size_t)k0 * E + e;
#pragma unroll 8
            for (int kk = 0; kk < kc; ++kk) {
                const float wv = w[(size_t)kk * E];
#pragma unroll
                for (int i = 0; i < kRouteTok; ++i) acc[i] = __builtin_fmaf(xs[kk][i], wv, acc[i]);
            }
        }
    }
    if (e < E) {
        const float b = bias ? bias[e] : 0.0f;
#pragma unroll
        for (int i = 0; i < kRouteTok; ++i) lg[i][e] = bias ? acc[i] + b : acc[i];
    }
    __syncthreads();
    const int wave = threadIdx.x >> 6, nwave = nthr >> 6;
    for (int i = wave; i < kRouteTok; i += nwave) {
        const int t = t0 + i;
        if (t >= T) break;
        auto load = [&](int ee) { return lg[i][ee]; };
        wave_topk(load, E, K, renorm, ids + (size_t)t * K, wts + (size_t)t * K);
    }
}

moe_status_t launch_route(const void *x, int x_dtype, const float *wT, const float *logits,
                          const float *bias, int T, int H, int E, int K, int renorm,
                          int32_t *ids, float *wts, hipStream_t s) {
    if (T == 0) return MOE_OK;
    if (logits) {
        hipLaunchKernelGGL(route_given_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, bias,
                           T, E, K, renorm, ids, wts);
    } else {
        const int threads = ((E + kWave - 1) / kWave) * kWave;
        const dim3 grid((T + kRouteTok - 1) / kRouteTok);
        if (x_dtype == MOE_BF16)
            hipLaunchKernelGGL(route_logits_kernel<MOE_BF16>, grid, dim3(threads), 0, s,
                               (const uint16_t *)x, wT, bias, T, H, E, K, renorm, ids, wts);
        else
            hipLaunchKernelGGL(route_logits_kernel<MOE_F16>, grid, dim3(threads), 0, s,
                               (const uint16_t *)x, wT, bias, T, H, E, K, renorm, ids, wts);
    }
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

}  // namespace moe
