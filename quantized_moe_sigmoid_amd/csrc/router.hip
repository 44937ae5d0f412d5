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
// Selection: the K largest logits by (logit desc, expert asc): per round a
// wave maximum of the logits' order-preserving 32-bit images, ties resolved
// to the lowest expert index by ballots; -0 is folded to +0 first.
// Weights: sigmoid of the selected logits, renormalised to sum to one when
// asked.
#include "common.h"

#pragma clang fp contract(off)

namespace moe {

constexpr int kMaxE = 512;

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

// One wave selects the top K of E logits held in `lg` (LDS or global).
// Lane l owns experts l, l+64, ... Each round takes the wave maximum of the
// logits' order images, then the lowest expert holding it: experts of slot
// j are 64 j + lane, so the first slot whose ballot hits, at its lowest
// lane (ties go to the lower index). Writes ids / weights for one token.
template <typename LoadFn>
__device__ __forceinline__ void wave_topk(LoadFn load, int E, int K, int renorm,
                                          int32_t *ids, float *wts) {
    constexpr int NJ = kMaxE / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t o[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int e = lane + j * kWave;
        o[j] = e < E ? ord32(load(e)) : 0u;
    }
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

// Logits computed: a plain fp32 SIMT GEMM, logits[t][e] = x[t] . wT[:, e],
// in which every output is one fma chain over k in ascending order (so the
// input range cannot be split across threads). Block tile: 64 experts (one
// per lane) x 16 tokens (4 per wave): at T = 2048 and E = 352 that is 768
// work groups, three per CU in one round, and each wave's serial chain
// work stays short. k advances in chunks of 64 staged in LDS (double
// buffered): the 64 x 64 slice of wT read by all four waves, and x widened
// to float32, token-minor, so a wave reads its 4 tokens' inputs with one
// broadcast 16-byte LDS read per k.
constexpr int kRtExp = 64, kRtTok = 16, kRtKC = 64;

template <int ACT>
__global__ void __launch_bounds__(256) router_logits_kernel(
    const uint16_t *__restrict__ x, const float *__restrict__ wT,
    const float *__restrict__ bias, int T, int H, int E, float *__restrict__ logits) {
    // xs rows padded to 20 floats: the transposing stores of the four k rows
    // a wave writes (4 apart) then fall on four different 16-bank groups;
    // 20 * 4 bytes keeps every 4-token group 16-byte aligned for the
    // broadcast reads
    __shared__ __attribute__((aligned(16))) float ws[2][kRtKC][kRtExp];
    __shared__ __attribute__((aligned(16))) float xs[2][kRtKC][kRtTok + 4];
    const int t0 = blockIdx.x * kRtTok, e0 = blockIdx.y * kRtExp;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

    // staging roles: wT float4 column tid%16 of rows tid/16 + 16 i (each
    // store instruction writes 4 whole 256-byte rows: no bank conflicts);
    // x: token tid%16, 4 consecutive k starting at 4 * (tid/16)
    const int wk = threadIdx.x >> 4, we = (threadIdx.x & 15) * 4;
    const int xt = threadIdx.x & 15, xk = (threadIdx.x >> 4) * 4;
    float4 wreg[4];
    uint2 xreg;
    auto load = [&](int k0) {
        const int e = e0 + we;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float *wp = wT + (size_t)(k0 + wk + 16 * i) * E + e;
            wreg[i] = e + 3 < E ? *(const float4 *)wp
                                : make_float4(e < E ? wp[0] : 0.f, e + 1 < E ? wp[1] : 0.f,
                                              e + 2 < E ? wp[2] : 0.f, 0.f);
        }
        const int t = t0 + xt;
        xreg = t < T ? *(const uint2 *)(x + (size_t)t * H + k0 + xk) : make_uint2(0, 0);
    };
    auto store = [&](int b) {
#pragma unroll
        for (int i = 0; i < 4; ++i) *(float4 *)&ws[b][wk + 16 * i][we] = wreg[i];
        const uint32_t d[2] = {xreg.x, xreg.y};
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            xs[b][xk + 2 * i][xt] = act_to_f32<ACT>(d[i] & 0xFFFF);
            xs[b][xk + 2 * i + 1][xt] = act_to_f32<ACT>(d[i] >> 16);
        }
    };

    float acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = 0.0f;
    const int nch = H / kRtKC;
    load(0);
    store(0);
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        const int b = c & 1;
        if (c + 1 < nch) load((c + 1) * kRtKC);
#pragma unroll 16
        for (int k = 0; k < kRtKC; ++k) {
            const float w = ws[b][k][lane];
            const float4 xa = *(const float4 *)&xs[b][k][4 * wave];
            acc[0] = __builtin_fmaf(xa.x, w, acc[0]);
            acc[1] = __builtin_fmaf(xa.y, w, acc[1]);
            acc[2] = __builtin_fmaf(xa.z, w, acc[2]);
            acc[3] = __builtin_fmaf(xa.w, w, acc[3]);
        }
        if (c + 1 < nch) store(b ^ 1);
        __syncthreads();
    }
    const int e = e0 + lane;
    if (e >= E) return;
    const float bv = bias ? bias[e] : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = t0 + 4 * wave + i;
        if (t < T) logits[(size_t)t * E + e] = bias ? acc[i] + bv : acc[i];
    }
}

// bf16 activations: the wave's 4 token rows are wave-uniform, so they are
// read with scalar loads straight into SGPRs and widened there (bf16 -> f32
// is a shift), and every FMA takes its x operand from an SGPR. Only wT goes
// through LDS (one lane-varying 4-byte read per k), which removes the
// broadcast x reads that bound the LDS return path above. Same tiles, same
// per-(t, e) chain order.
//
// TPW tokens per wave: 4 for large batches; 1 for small ones, where the
// tiled grid would otherwise be a handful of work groups whose waves each
// run four 4096-step chains back to back (T = 32: 12 groups, 116 us); with
// one token per wave the grid has four times the waves and each wave a
// quarter of the serial work.
template <int TPW>
__global__ void __launch_bounds__(256) router_logits_bf16_kernel(
    const uint16_t *__restrict__ x, const float *__restrict__ wT,
    const float *__restrict__ bias, int T, int H, int E, float *__restrict__ logits) {
    __shared__ __attribute__((aligned(16))) float ws[2][kRtKC][kRtExp];
    const int t0 = blockIdx.x * (4 * TPW), e0 = blockIdx.y * kRtExp;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // the wave's token rows as 32-bit pairs (rows past T read row t0; their
    // logits are not stored)
    const uint32_t *xr[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int t = t0 + TPW * wave + i;
        xr[i] = (const uint32_t *)(x + (size_t)(t < T ? t : t0) * H);
    }
    // E % 4 == 0: a float4 column group is either inside the matrix or past
    // it; groups past it read the last group and store zeros (no branch)
    const int wk = threadIdx.x >> 4, we = (threadIdx.x & 15) * 4;
    const bool w_in = e0 + we < E;
    const int w_col = w_in ? e0 + we : E - 4;
    float4 wreg[4];
    // the next chunk's x bytes of the wave's rows (TPW rows x 128 B) are also
    // touched with vector loads one chunk ahead, so the scalar loads that
    // consume them hit L2 instead of waiting for HBM; the loaded words only
    // feed `sink`
    uint32_t sink = 0, xtouch = 0;
    const int tpf = t0 + TPW * wave + ((lane >> 3) % TPW);
    const uint16_t *xpf = x + (size_t)(tpf < T ? tpf : t0) * H + (lane & 7) * 8;
    auto load = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            wreg[i] = *(const float4 *)(wT + (size_t)(k0 + wk + 16 * i) * E + w_col);
        xtouch = *(const uint32_t *)(xpf + k0);
    };
    auto store = [&](int b) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *(float4 *)&ws[b][wk + 16 * i][we] = w_in ? wreg[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        sink ^= xtouch;
    };

    float acc[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) acc[i] = 0.0f;
    const int nch = H / kRtKC;
    load(0);
    store(0);
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        const int b = c & 1;
        if (c + 1 < nch) load((c + 1) * kRtKC);
        const int p0 = c * (kRtKC / 2);
        // one token per wave: the whole chunk unrolled, so its LDS and
        // scalar reads are issued ahead of the FMA chain instead of
        // between its pieces
        constexpr int kUnroll = TPW == 1 ? kRtKC / 2 : 8;
#pragma unroll kUnroll
        for (int k2 = 0; k2 < kRtKC / 2; ++k2) {
            uint32_t xp[TPW];
#pragma unroll
            for (int i = 0; i < TPW; ++i) xp[i] = xr[i][p0 + k2];
            const float w0 = ws[b][2 * k2][lane], w1 = ws[b][2 * k2 + 1][lane];
#pragma unroll
            for (int i = 0; i < TPW; ++i)
                acc[i] = __builtin_fmaf(__uint_as_float(xp[i] << 16), w0, acc[i]);
#pragma unroll
            for (int i = 0; i < TPW; ++i)
                acc[i] = __builtin_fmaf(__uint_as_float(xp[i] & 0xFFFF0000u), w1, acc[i]);
        }
        if (c + 1 < nch) store(b ^ 1);
        __syncthreads();
    }
    const int e = e0 + lane;
    if (sink == 0x9E3779B9u && H == 0) logits[0] = 0.0f;    // never true: keeps the prefetch
    if (e >= E) return;
    const float bv = bias ? bias[e] : 0.0f;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int t = t0 + TPW * wave + i;
        if (t < T) logits[(size_t)t * E + e] = bias ? acc[i] + bv : acc[i];
    }
}

// bf16 batches up to this many tokens run one token per wave.
constexpr int kRtSmallT = 512;

moe_status_t launch_router_logits(const void *x, int x_dtype, const float *wT, const float *bias,
                                  int T, int H, int E, float *logits, hipStream_t s) {
    if (T == 0) return MOE_OK;
    const dim3 grid((T + kRtTok - 1) / kRtTok, (E + kRtExp - 1) / kRtExp);
    if (x_dtype == MOE_BF16 && T <= kRtSmallT)
        hipLaunchKernelGGL(router_logits_bf16_kernel<1>, dim3((T + 3) / 4, grid.y), dim3(256), 0,
                           s, (const uint16_t *)x, wT, bias, T, H, E, logits);
    else if (x_dtype == MOE_BF16)
        hipLaunchKernelGGL(router_logits_bf16_kernel<4>, grid, dim3(256), 0, s,
                           (const uint16_t *)x, wT, bias, T, H, E, logits);
    else
        hipLaunchKernelGGL(router_logits_kernel<MOE_F16>, grid, dim3(256), 0, s,
                           (const uint16_t *)x, wT, bias, T, H, E, logits);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

// Top-K of logits that are already final (bias, if any, folded in by the
// caller) or given plus an optional bias.
moe_status_t launch_topk(const float *logits, const float *bias, int T, int E, int K, int renorm,
                         int32_t *ids, float *wts, hipStream_t s) {
    if (T == 0) return MOE_OK;
    hipLaunchKernelGGL(route_given_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, bias, T, E,
                       K, renorm, ids, wts);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

}  // namespace moe
