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

// The 64-expert column block of wT streamed through a two-stage LDS buffer
// in chunks of KC rows, NP chunks ahead in registers. Chunk m sits in
// register slot m % NP; step c stores chunk c + 1 into the stage that step
// c - 1 finished reading, reloads the freed slot with chunk c + 1 + NP, then
// runs the chain over chunk c. A load thus has NP steps of chain work to
// arrive. Every step issues the same loads (chunk indices past the end are
// clamped to the last chunk, steps past the end only store and
// synchronize), so the compiler's wait before a store counts exactly the
// NP - 1 younger chunks instead of draining every load in flight.
// Staging roles (NT threads): float4 column tid % 16 of rows tid / 16 +
// (NT / 16) i, so each store instruction writes NT / 16 whole 256-byte rows.
// E % 4 == 0: a column
// group past E stages a copy of the last group; the lanes that read it
// compute logits that are never stored.
// XT = kXStage (NT = 256, KC = 64): the chunk's inputs of 16 tokens ride
// along with the weights, 4 bf16 per thread (token tid / 16, inputs 4 (tid %
// 16) .. + 3 of the chunk), and are stored widened to float32 into `xs`
// [stage][16][KC] with the weights.
constexpr int kXNone = 0, kXStage = 1;

template <int KC, int NP, int XT, int NT = 256>
struct RouterWeightPipe {
    static constexpr int kStride = NT / 16;      // rows apart of a thread's loads
    static constexpr int kRows = KC / kStride;   // float4 loads per thread and chunk
    f32x4_t r[NP][kRows];
    uint2 xw[NP];
    const float *src;                            // wT + (tid / 16) * E + column
    const uint16_t *xt;                          // kXStage: this thread's 4 inputs
    float *xs;                                   // kXStage: [2][16][KC] in LDS
    size_t row;                                  // one row of wT, in floats (E)
    int wk, we, nch;

    __device__ __forceinline__ RouterWeightPipe(const float *wT, int E, int e0, int H, int tid,
                                                const uint16_t *xsrc = nullptr,
                                                float *xstage = nullptr) {
        wk = tid >> 4;
        we = (tid & 15) * 4;
        src = wT + (size_t)wk * E + (e0 + we < E ? e0 + we : E - 4);
        row = (size_t)E;
        nch = H / KC;
        xt = xsrc;
        xs = xstage;
    }
    __device__ __forceinline__ void load(int slot, int chunk) {
        chunk = chunk < nch ? chunk : nch - 1;
        const float *p = src + (size_t)chunk * KC * row;
#pragma unroll
        for (int i = 0; i < kRows; ++i) r[slot][i] = *(const f32x4_t *)(p + i * kStride * row);
        if (XT == kXStage) xw[slot] = *(const uint2 *)(xt + (size_t)chunk * KC);
    }
    __device__ __forceinline__ void store(float (*ws)[KC][kRtExp], int stage, int slot) {
#pragma unroll
        for (int i = 0; i < kRows; ++i)
            *(f32x4_t *)&ws[stage][wk + kStride * i][we] = r[slot][i];
        if (XT == kXStage)
            *(f32x4_t *)&xs[(stage * 16 + wk) * KC + we] =
                f32x4_t{__uint_as_float(xw[slot].x << 16), __uint_as_float(xw[slot].x & 0xFFFF0000u),
                        __uint_as_float(xw[slot].y << 16), __uint_as_float(xw[slot].y & 0xFFFF0000u)};
    }
    // chunks 0 .. NP-1 in flight
    __device__ __forceinline__ void prime() {
#pragma unroll
        for (int j = 0; j < NP; ++j) load(j, j);
    }
    // after prime(): chunk 0 into stage 0, then every step; chunk(c, stage)
    // runs the chain over chunk c. Ends with a barrier.
    template <typename Chunk>
    __device__ __forceinline__ void run(float (*ws)[KC][kRtExp], Chunk &&chunk) {
        store(ws, 0, 0);
        load(0, NP);
        __syncthreads();
        for (int c0 = 0; c0 < nch; c0 += NP) {
#pragma unroll
            for (int j = 0; j < NP; ++j) {
                const int c = c0 + j;
                store(ws, (c + 1) & 1, (j + 1) % NP);
                load((j + 1) % NP, c + 1 + NP);
                if (c < nch) chunk(c, ws[c & 1]);  // uniform over the block
                __syncthreads();
            }
        }
    }
};

// Larger bf16 batches: 64 experts x 16 tokens a work group, 4 tokens per
// wave. Each 64-input chunk stages the weight tile and the 16 tokens'
// inputs (widened to float32) in LDS; a wave reads, per 16 inputs, 16
// weights (8 pair reads, shared by its 4 tokens) and one 4-byte input word
// per token (lane j of every 16-lane row: input j), and runs the 4 tokens'
// chains interleaved, each FMA taking its input by DPP row_newbcast: about
// 4.75 instructions per input position for 4 FMAs, where scalar loads of x
// cost 8.5 (an unpacking SALU op per FMA). Same per-(t, e) chain order.
//
// acc[i] = fma(x_i,j, w[j - J], acc[i]) for j = J .. J+3 in this order, i =
// 0 .. 3 interleaved (independent chains), x_i,j = lane j of xq[i]'s 16-lane
// row; as fma16_row_bcast.
template <int J>
__device__ __forceinline__ void fma4x4_row_bcast(float (&acc)[4], const float (&xq)[4],
                                                 const float *w);
template <>
__device__ __forceinline__ void fma4x4_row_bcast<0>(float (&acc)[4], const float (&xq)[4],
                                                    const float *w) {
    asm("s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %4, %8 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %8 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %8 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %8 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %9 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %9 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %9 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %9 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %10 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %10 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %10 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %10 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %11 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %11 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %11 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %11 row_newbcast:3 row_mask:0xf bank_mask:0xf"
        : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3])
        : "v"(xq[0]), "v"(xq[1]), "v"(xq[2]), "v"(xq[3]), "v"(w[0]), "v"(w[1]), "v"(w[2]),
          "v"(w[3])
        : "memory");
}

template <>
__device__ __forceinline__ void fma4x4_row_bcast<4>(float (&acc)[4], const float (&xq)[4],
                                                    const float *w) {
    asm("s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %4, %8 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %8 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %8 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %8 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %9 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %9 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %9 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %9 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %10 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %10 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %10 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %10 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %11 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %11 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %11 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %11 row_newbcast:7 row_mask:0xf bank_mask:0xf"
        : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3])
        : "v"(xq[0]), "v"(xq[1]), "v"(xq[2]), "v"(xq[3]), "v"(w[0]), "v"(w[1]), "v"(w[2]),
          "v"(w[3])
        : "memory");
}

template <>
__device__ __forceinline__ void fma4x4_row_bcast<8>(float (&acc)[4], const float (&xq)[4],
                                                    const float *w) {
    asm("s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %4, %8 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %8 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %8 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %8 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %9 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %9 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %9 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %9 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %10 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %10 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %10 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %10 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %11 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %11 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %11 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %11 row_newbcast:11 row_mask:0xf bank_mask:0xf"
        : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3])
        : "v"(xq[0]), "v"(xq[1]), "v"(xq[2]), "v"(xq[3]), "v"(w[0]), "v"(w[1]), "v"(w[2]),
          "v"(w[3])
        : "memory");
}

template <>
__device__ __forceinline__ void fma4x4_row_bcast<12>(float (&acc)[4], const float (&xq)[4],
                                                    const float *w) {
    asm("s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %4, %8 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %8 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %8 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %8 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %9 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %9 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %9 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %9 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %10 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %10 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %10 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %10 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %11 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %11 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %11 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %11 row_newbcast:15 row_mask:0xf bank_mask:0xf"
        : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3])
        : "v"(xq[0]), "v"(xq[1]), "v"(xq[2]), "v"(xq[3]), "v"(w[0]), "v"(w[1]), "v"(w[2]),
          "v"(w[3])
        : "memory");
}

template <int NP>
__global__ void __launch_bounds__(256) router_tiled_kernel(
    const uint16_t *__restrict__ x, const float *__restrict__ wT,
    const float *__restrict__ bias, int T, int H, int E, float *__restrict__ logits) {
    __shared__ __attribute__((aligned(16))) float ws[2][kRtKC][kRtExp];
    __shared__ __attribute__((aligned(16))) float xs[2][16][kRtKC];
    // Work groups go round-robin over the 8 XCDs; each XCD takes a
    // contiguous range of (expert block, token block) pairs, expert block
    // major, so it reads the weight slices of one or two expert blocks
    // from its own L2 instead of all of them.
    const int nb = gridDim.x, b = blockIdx.x, xq = nb / 8, xr = nb % 8, xcd = b % 8;
    const int lid = xcd * xq + (xcd < xr ? xcd : xr) + b / 8;
    const int ntb = (T + 15) / 16, eb = lid / ntb;
    const int t0 = (lid - eb * ntb) * 16, e0 = eb * kRtExp;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // this thread's staging share of x (rows past T read row t0; their
    // logits are not stored)
    const int ts = t0 + (tid >> 4);
    const uint16_t *xsrc = x + (size_t)(ts < T ? ts : t0) * H + 4 * (tid & 15);
    RouterWeightPipe<kRtKC, NP, kXStage> pipe(wT, E, e0, H, tid, xsrc, &xs[0][0][0]);
    pipe.prime();

    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    pipe.run(ws, [&](int c, float (*st)[kRtExp]) {
        const float *xw = &xs[c & 1][4 * wave][lane & 15];
        float xq[2][4], w[2][16];
        auto read = [&](int m, int b) {
#pragma unroll
            for (int i = 0; i < 4; ++i) xq[b][i] = xw[i * kRtKC + 16 * m];
#pragma unroll
            for (int j = 0; j < 16; ++j) w[b][j] = st[16 * m + j][lane];
        };
        read(0, 0);
#pragma unroll
        for (int m = 0; m < kRtKC / 16; ++m) {
            if (m + 1 < kRtKC / 16) read(m + 1, (m + 1) & 1);
            fma4x4_row_bcast<0>(acc, xq[m & 1], &w[m & 1][0]);
            fma4x4_row_bcast<4>(acc, xq[m & 1], &w[m & 1][4]);
            fma4x4_row_bcast<8>(acc, xq[m & 1], &w[m & 1][8]);
            fma4x4_row_bcast<12>(acc, xq[m & 1], &w[m & 1][12]);
        }
    });
    const int e = e0 + lane;
    if (e >= E) return;
    const float bv = bias ? bias[e] : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = t0 + 4 * wave + i;
        if (t < T) logits[(size_t)t * E + e] = bias ? acc[i] + bv : acc[i];
    }
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

// acc = fma(x_j, w[j], acc) for j = 0 .. 15 in this order, where x_j is the
// value of lane j of the lane's 16-lane row in xq, delivered to the FMA by
// DPP row_newbcast:j. With the same 16 inputs in every row this broadcasts
// input j to the whole wave inside the FMA: one instruction per input and
// no LDS or scalar traffic for x. The FMA is the same single-rounding fp32
// fma the compiler emits for __builtin_fmaf. The leading s_nop covers the
// two wait states a DPP read needs after a VALU write of its source. The
// memory clobber keeps the caller's loads on their side of the block, so
// the reads of the next 16 inputs overlap these FMAs.
__device__ __forceinline__ void fma16_row_bcast(float &acc, float xq, const float (&w)[16]) {
    asm("s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %1, %2 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %3 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %4 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %5 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %6 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %7 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %8 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %9 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %10 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %11 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %12 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %13 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %14 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %15 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %16 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %17 row_newbcast:15 row_mask:0xf bank_mask:0xf"
        : "+v"(acc)
        : "v"(xq), "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]), "v"(w[4]), "v"(w[5]), "v"(w[6]), "v"(w[7]), "v"(w[8]), "v"(w[9]), "v"(w[10]), "v"(w[11]), "v"(w[12]), "v"(w[13]), "v"(w[14]), "v"(w[15])
        : "memory");
}

// ---- small batches: rows staged in LDS, one token per wave ------------------
// W tokens x 64 experts a work group of W waves (W = 2 or 4), one token per
// wave: a batch of a few tokens has too few waves for the tiled kernels
// above, and each wave runs one 4096-step chain. The group first stages its W rows in LDS
// as float32: the bf16 activations widened (NORM = false) or, fused, the
// RMSNorm of W fp32 residual rows (NORM = true), whose float32 sums of
// squares follow rmsnorm_kernel's 256-thread order exactly (each thread
// stands in for 4 / W of those threads: same columns, same wave shuffles,
// same block sum), so the 16-bit rows are bitwise the ones moe_rmsnorm
// writes; the groups of the first expert block also write them to a_out for
// the experts. In the chain each input costs one FMA (x broadcast by DPP
// from one 4-byte LDS read per 16 inputs) and half a 4-byte-pair LDS read
// of weights; what bounds it is that instruction stream of one wave (about
// 19 cycles per input measured, against the 6.5-cycle latency of the FMA
// chain), not LDS bandwidth or the weight loads: prefetch depth and chunk
// size change nothing, and neither does W, apart from the number of groups.
// Same chain, same order as the other router kernels.
constexpr int kRowsMaxT = 192;                   // batches up to this size (beyond it
                                                 // router_tiled_kernel is faster: T = 256,
                                                 // 64 us against 69)
constexpr int kRowsMaxH = 4096;                  // W float32 rows in LDS

template <bool NORM, int W>
__global__ void __launch_bounds__(64 * W) router_rows_kernel(
    const void *__restrict__ xin, const float *__restrict__ gain, float eps,
    const float *__restrict__ wT, const float *__restrict__ bias, int T, int H, int E,
    uint16_t *__restrict__ a_out, float *__restrict__ logits) {
    constexpr int NT = 64 * W, KC = 64, NP = 2;
    static_assert(W == 1 || W == 2 || W == 4, "norm threads must split evenly");
    constexpr int kVT = 4 / W;                   // 256-thread norm threads per thread
    constexpr int kCols = kRowsMaxH / 1024;      // float4 groups of a row per norm thread
    __shared__ __attribute__((aligned(16))) float ws[2][KC][kRtExp];
    __shared__ __attribute__((aligned(16))) float as[W][kRowsMaxH];
    __shared__ float red[W][4];
    const int t0 = blockIdx.x * W, e0 = blockIdx.y * kRtExp;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // the router weight's first chunks are in flight while the rows stage
    RouterWeightPipe<KC, NP, kXNone, NT> pipe(wT, E, e0, H, tid);
    pipe.prime();

    if (!NORM) {
        // bf16 rows widened (rows past T repeat row t0; never stored)
        const uint16_t *x = (const uint16_t *)xin;
#pragma unroll
        for (int i = 0; i < W; ++i) {
            const int t = t0 + i < T ? t0 + i : t0;
            for (int c = tid * 4; c < H; c += 4 * NT) {
                const uint2 v = *(const uint2 *)(x + (size_t)t * H + c);
                *(f32x4_t *)&as[i][c] = f32x4_t{__uint_as_float(v.x << 16),
                                                __uint_as_float(v.x & 0xFFFF0000u),
                                                __uint_as_float(v.y << 16),
                                                __uint_as_float(v.y & 0xFFFF0000u)};
            }
        }
    } else {
        // RMSNorm of the W rows (rows past T repeat row t0; not stored).
        // Norm thread tid + NT u of rmsnorm_kernel's 256 (its wave: wave +
        // W u, its lane: lane) owns columns 4 (tid + NT u) + 1024 j. All of a
        // thread's values are loaded at once.
        const float *res = (const float *)xin;
        f32x4_t v[W][kVT][kCols], g[kVT][kCols];
#pragma unroll
        for (int u = 0; u < kVT; ++u)
#pragma unroll
            for (int j = 0; j < kCols; ++j) {
                const int c = (tid + NT * u) * 4 + 1024 * j;
                g[u][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                if (c < H) {
                    if (gain) g[u][j] = *(const f32x4_t *)(gain + c);
#pragma unroll
                    for (int i = 0; i < W; ++i) {
                        const int t = t0 + i < T ? t0 + i : t0;
                        v[i][u][j] = *(const f32x4_t *)(res + (size_t)t * H + c);
                    }
                }
            }
#pragma unroll
        for (int i = 0; i < W; ++i)
#pragma unroll
            for (int u = 0; u < kVT; ++u) {
                float ss = 0.0f;
#pragma unroll
                for (int j = 0; j < kCols; ++j) {
                    if ((tid + NT * u) * 4 + 1024 * j < H) {
                        const f32x4_t q = v[i][u][j];
                        ss = ss + q.x * q.x;
                        ss = ss + q.y * q.y;
                        ss = ss + q.z * q.z;
                        ss = ss + q.w * q.w;
                    }
                }
#pragma unroll
                for (int m = 32; m >= 1; m >>= 1) ss = ss + __shfl_xor(ss, m, kWave);
                if (lane == 0) red[i][wave + W * u] = ss;
            }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < W; ++i) {
            const float tot = ((red[i][0] + red[i][1]) + red[i][2]) + red[i][3];
            const float r = __builtin_sqrtf(tot / (float)H + eps);
#pragma unroll
            for (int u = 0; u < kVT; ++u)
#pragma unroll
                for (int j = 0; j < kCols; ++j) {
                    const int c = (tid + NT * u) * 4 + 1024 * j;
                    if (c < H) {
                        const f32x4_t q = v[i][u][j], gg = g[u][j];
                        const uint32_t lo =
                            f32_to_bf16_bits((q.x / r) * (1.0f + gg.x)) |
                            ((uint32_t)f32_to_bf16_bits((q.y / r) * (1.0f + gg.y)) << 16);
                        const uint32_t hi =
                            f32_to_bf16_bits((q.z / r) * (1.0f + gg.z)) |
                            ((uint32_t)f32_to_bf16_bits((q.w / r) * (1.0f + gg.w)) << 16);
                        *(f32x4_t *)&as[i][c] = f32x4_t{__uint_as_float(lo << 16),
                                                        __uint_as_float(lo & 0xFFFF0000u),
                                                        __uint_as_float(hi << 16),
                                                        __uint_as_float(hi & 0xFFFF0000u)};
                        if (blockIdx.y == 0 && t0 + i < T)
                            *(uint2 *)(a_out + (size_t)(t0 + i) * H + c) = make_uint2(lo, hi);
                    }
                }
        }
    }
    // the rows reach LDS before the chains read them: run() stores the first
    // chunk and synchronizes before its first step

    // lane j of every 16-lane row reads inputs 16 m + j of the chunk
    const float *xr = &as[wave][lane & 15];
    float acc = 0.0f;
    pipe.run(ws, [&](int c, float (*st)[kRtExp]) {
        // 16 inputs at a time, the reads of the next 16 issued before the
        // FMAs of these (double-buffered in registers)
        float xq[2], w[2][16];
        auto read = [&](int m, int b) {
            xq[b] = xr[c * KC + 16 * m];
#pragma unroll
            for (int j = 0; j < 16; ++j) w[b][j] = st[16 * m + j][lane];
        };
        read(0, 0);
#pragma unroll
        for (int m = 0; m < KC / 16; ++m) {
            if (m + 1 < KC / 16) read(m + 1, (m + 1) & 1);
            fma16_row_bcast(acc, xq[m & 1], w[m & 1]);
        }
    });
    const int e = e0 + lane, t = t0 + wave;
    if (e < E && t < T) logits[(size_t)t * E + e] = bias ? acc + bias[e] : acc;
}

// tokens per work group, measured at H = 4096, E = 352: W = 2 up to 64
// tokens (T = 32: 36 us against 39 us at W = 4 and 41 us at W = 1, whose
// single wave per group gains no LDS bandwidth worth its lost sharing),
// W = 4 beyond (T = 256: 68 us against 79 us at W = 2)
constexpr int kRowsW2MaxT = 64;

template <bool NORM>
static void launch_rows(const void *xin, const float *gain, float eps, int T, int H,
                        const float *wT, const float *bias, int E, void *a_out, float *logits,
                        hipStream_t s) {
    const int eb = (E + kRtExp - 1) / kRtExp;
    if (T <= kRowsW2MaxT)
        hipLaunchKernelGGL((router_rows_kernel<NORM, 2>), dim3((T + 1) / 2, eb), dim3(128), 0, s,
                           xin, gain, eps, wT, bias, T, H, E, (uint16_t *)a_out, logits);
    else
        hipLaunchKernelGGL((router_rows_kernel<NORM, 4>), dim3((T + 3) / 4, eb), dim3(256), 0, s,
                           xin, gain, eps, wT, bias, T, H, E, (uint16_t *)a_out, logits);
}

moe_status_t launch_router_logits(const void *x, int x_dtype, const float *wT, const float *bias,
                                  int T, int H, int E, float *logits, hipStream_t s) {
    if (T == 0) return MOE_OK;
    const dim3 grid((T + kRtTok - 1) / kRtTok, (E + kRtExp - 1) / kRtExp);
    if (x_dtype == MOE_BF16 && T <= kRowsMaxT && H <= kRowsMaxH)
        launch_rows<false>(x, nullptr, 0.f, T, H, wT, bias, E, nullptr, logits, s);
    else if (x_dtype == MOE_BF16)
        hipLaunchKernelGGL((router_tiled_kernel<2>), dim3(grid.x * grid.y), dim3(256), 0, s,
                           (const uint16_t *)x, wT, bias, T, H, E, logits);
    else
        hipLaunchKernelGGL(router_logits_kernel<MOE_F16>, grid, dim3(256), 0, s,
                           (const uint16_t *)x, wT, bias, T, H, E, logits);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

bool norm_route_fused(int T, int H, int E) { return T <= kRowsMaxT && H <= kRowsMaxH; }

moe_status_t launch_norm_router_logits(const float *res, const float *gain, float eps, int T,
                                       int H, const float *wT, const float *bias, int E,
                                       void *a_out, float *logits, hipStream_t s) {
    if (T == 0) return MOE_OK;
    launch_rows<true>(res, gain, eps, T, H, wT, bias, E, a_out, logits, s);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

}  // namespace moe
