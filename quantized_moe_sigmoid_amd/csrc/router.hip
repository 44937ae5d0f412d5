// Sigmoid top-K router (page "Step-5-Preview-Spark", "At a glance": a
// sigmoid router choosing the top 8 of 352 routed experts).
//
// Logits are either computed here from the 16-bit activations and the
// float32 router weight stored transposed ([H][E]), or given. The logit of
// (t, e) is a sum in one fixed order: the inputs in blocks of 512, each
// block one float32 chain s = fma(x[t][k], wT[k][e], s) over its k
// ascending from +0, the block sums added in ascending block order (then
// the bias, if any). The chosen experts are thus the same on every run and
// on the CPU reference, and a small batch can run a token's 8 block chains
// side by side instead of one 4096-step chain. The pages show why the order
// matters: a different summation order inside the MoE flips near-tied
// expert choices ("Step-5-Preview-Spark", "Quality", noise-floor
// paragraph). The selection and the weights are in topk.h.
#include "topk.h"

#pragma clang fp contract(off)

namespace moe {

// After the chain over 64-input chunk c (of nch) has run into acc: at the
// end of a 512-input block, fold the block's sum into tot (the first block
// sets it) and start a fresh chain.
template <int N>
__device__ __forceinline__ void block_end(int c, int nch, float (&acc)[N], float (&tot)[N]) {
    if (((c + 1) & (kRouterBlock / 64 - 1)) == 0 || c + 1 == nch) {
        const bool first = c < kRouterBlock / 64;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            tot[i] = first ? acc[i] : tot[i] + acc[i];
            acc[i] = 0.0f;
        }
    }
}

// Logits given, or P block sums of them ([P][T][E], added in block
// order): one wave per token.
__global__ void __launch_bounds__(256) route_given_kernel(
    const float *__restrict__ logits, const float *__restrict__ bias, int T, int E, int K,
    int renorm, int P, int32_t *__restrict__ ids, float *__restrict__ wts) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    token_topk(logits + (size_t)t * E, (size_t)T * E, P, bias, E, K, renorm, ids + (size_t)t * K,
               wts + (size_t)t * K, nullptr);
}

// Logits computed: a plain fp32 SIMT GEMM, logits[t][e] = x[t] . wT[:, e],
// every output the canonical sum (fma chains over k ascending, restarted
// every 512 inputs, the block sums added in order). Block tile: 64 experts (one
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

    float acc[4], tot[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = tot[i] = 0.0f;
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
        block_end(c, nch, acc, tot);
        if (c + 1 < nch) store(b ^ 1);
        __syncthreads();
    }
    const int e = e0 + lane;
    if (e >= E) return;
    const float bv = bias ? bias[e] : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = t0 + 4 * wave + i;
        if (t < T) logits[(size_t)t * E + e] = bias ? tot[i] + bv : tot[i];
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
// [stage][16][KC] with the weights. XT = kXStage2: two tokens per thread,
// tid / 16 from xsrc and tid / 16 + 16 from xsrc2, into [stage][32][KC].
constexpr int kXNone = 0, kXStage = 1, kXStage2 = 2;

template <int KC, int NP, int XT, int NT = 256>
struct RouterWeightPipe {
    static constexpr int kStride = NT / 16;      // rows apart of a thread's loads
    static constexpr int kRows = KC / kStride;   // float4 loads per thread and chunk
    static constexpr int kXR = XT == kXStage2 ? 2 : 1;  // staged token rows per thread
    f32x4_t r[NP][kRows];
    uint2 xw[NP][kXR];
    const float *src;                            // wT + (tid / 16) * E + column
    const uint16_t *xt[kXR];                     // this thread's 4 inputs of each row
    float *xs;                                   // kXStage: [2][16][KC] in LDS
    size_t row;                                  // one row of wT, in floats (E)
    int wk, we, nch;

    __device__ __forceinline__ RouterWeightPipe(const float *wT, int E, int e0, int H, int tid,
                                                const uint16_t *xsrc = nullptr,
                                                float *xstage = nullptr,
                                                const uint16_t *xsrc2 = nullptr) {
        wk = tid >> 4;
        we = (tid & 15) * 4;
        src = wT + (size_t)wk * E + (e0 + we < E ? e0 + we : E - 4);
        row = (size_t)E;
        nch = H / KC;
        xt[0] = xsrc;
        xt[kXR - 1] = XT == kXStage2 ? xsrc2 : xsrc;
        xs = xstage;
    }
    __device__ __forceinline__ void load(int slot, int chunk) {
        chunk = chunk < nch ? chunk : nch - 1;
        const float *p = src + (size_t)chunk * KC * row;
#pragma unroll
        for (int i = 0; i < kRows; ++i) r[slot][i] = *(const f32x4_t *)(p + i * kStride * row);
        if (XT != kXNone)
#pragma unroll
            for (int q = 0; q < kXR; ++q) xw[slot][q] = *(const uint2 *)(xt[q] + (size_t)chunk * KC);
    }
    __device__ __forceinline__ void store(float (*ws)[KC][kRtExp], int stage, int slot) {
#pragma unroll
        for (int i = 0; i < kRows; ++i)
            *(f32x4_t *)&ws[stage][wk + kStride * i][we] = r[slot][i];
        if (XT != kXNone)
#pragma unroll
            for (int q = 0; q < kXR; ++q) {
                const uint2 v = xw[slot][q];
                *(f32x4_t *)&xs[(stage * 16 * kXR + wk + 16 * q) * KC + we] =
                    f32x4_t{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u),
                            __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xFFFF0000u)};
            }
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
// wave (or 32 tokens, 8 per wave, two 4-token groups per weight read). Each 64-input chunk stages the weight tile and the 16 tokens'
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

// PART: one 512-input block per work group (the grid spans the blocks
// too) and the chains' values to logits as block sums [block][T][E] for
// the top-K; else all blocks in turn and the logits. TPW tokens per wave
// (4 or 8), 4 TPW per work group.
template <int NP, bool PART, int TPW>
__global__ void __launch_bounds__(256) router_tiled_kernel(
    const uint16_t *__restrict__ x, const float *__restrict__ wT,
    const float *__restrict__ bias, int T, int H, int E, float *__restrict__ logits) {
    constexpr int BT = 4 * TPW;
    __shared__ __attribute__((aligned(16))) float ws[2][kRtKC][kRtExp];
    __shared__ __attribute__((aligned(16))) float xs[2][BT][kRtKC];
    // Work groups go round-robin over the 8 XCDs; each XCD takes a
    // contiguous range of (expert block[, input block], token block)
    // tuples, expert block major, so it reads the weight slices of one or
    // two expert blocks from its own L2 instead of all of them.
    const int nb = gridDim.x, b = blockIdx.x, xq = nb / 8, xr = nb % 8, xcd = b % 8;
    const int lid = xcd * xq + (xcd < xr ? xcd : xr) + b / 8;
    const int ntb = (T + BT - 1) / BT, P = PART ? (H + kRouterBlock - 1) / kRouterBlock : 1;
    const int rest = lid / ntb, pb = rest % P, eb = rest / P;
    const int t0 = (lid - rest * ntb) * BT, e0 = eb * kRtExp;
    const int k0 = pb * kRouterBlock, kn = PART ? min(kRouterBlock, H - k0) : H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // this thread's staging share of x (rows past T read row t0; their
    // logits are not stored)
    const int ts = t0 + (tid >> 4), ts2 = ts + 16;
    const uint16_t *xsrc = x + (size_t)(ts < T ? ts : t0) * H + k0 + 4 * (tid & 15);
    const uint16_t *xsrc2 = x + (size_t)(ts2 < T ? ts2 : t0) * H + k0 + 4 * (tid & 15);
    RouterWeightPipe<kRtKC, NP, TPW == 8 ? kXStage2 : kXStage> pipe(
        wT + (size_t)k0 * E, E, e0, kn, tid, xsrc, &xs[0][0][0], xsrc2);
    pipe.prime();

    float acc[TPW], tot[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) acc[i] = tot[i] = 0.0f;
    pipe.run(ws, [&](int c, float (*st)[kRtExp]) {
        const float *xw = &xs[c & 1][TPW * wave][lane & 15];
        float xq[2][TPW], w[2][16];
        auto read = [&](int m, int b) {
#pragma unroll
            for (int i = 0; i < TPW; ++i) xq[b][i] = xw[i * kRtKC + 16 * m];
#pragma unroll
            for (int j = 0; j < 16; ++j) w[b][j] = st[16 * m + j][lane];
        };
        read(0, 0);
#pragma unroll
        for (int m = 0; m < kRtKC / 16; ++m) {
            if (m + 1 < kRtKC / 16) read(m + 1, (m + 1) & 1);
#pragma unroll
            for (int g = 0; g < TPW / 4; ++g) {
                float(&a4)[4] = *reinterpret_cast<float(*)[4]>(&acc[4 * g]);
                const float(&x4)[4] = *reinterpret_cast<const float(*)[4]>(&xq[m & 1][4 * g]);
                fma4x4_row_bcast<0>(a4, x4, &w[m & 1][0]);
                fma4x4_row_bcast<4>(a4, x4, &w[m & 1][4]);
                fma4x4_row_bcast<8>(a4, x4, &w[m & 1][8]);
                fma4x4_row_bcast<12>(a4, x4, &w[m & 1][12]);
            }
        }
        if (!PART) block_end(c, pipe.nch, acc, tot);
    });
    const int e = e0 + lane;
    if (e >= E) return;
    const float bv = bias && !PART ? bias[e] : 0.0f;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int t = t0 + TPW * wave + i;
        if (t >= T) continue;
        if (PART)
            logits[((size_t)pb * T + t) * E + e] = acc[i];
        else
            logits[(size_t)t * E + e] = bias ? tot[i] + bv : tot[i];
    }
}

// Top-K of logits that are already final (bias, if any, folded in by the
// caller) or given plus an optional bias.
moe_status_t launch_topk(const float *logits, const float *bias, int T, int E, int K, int renorm,
                         int32_t *ids, float *wts, hipStream_t s, int P) {
    if (T == 0) return MOE_OK;
    hipLaunchKernelGGL(route_given_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, bias, T, E,
                       K, renorm, P, ids, wts);
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
// wave, the logits of moe_router_logits: a batch of a few tokens has too few
// waves for the tiled kernel above. The group stages its W bf16 rows in LDS
// widened to float32; each wave runs its token's blocks in turn. In the
// chain each input costs one FMA (x broadcast by DPP from one 4-byte LDS
// read per 16 inputs) and half a 4-byte-pair LDS read of weights; what
// bounds it is that instruction stream of one wave (about 19 cycles per
// input measured, against 7 for the bare DPP FMA chain). The routing calls
// run the block sums side by side instead (router_block_kernel below).
constexpr int kRowsMaxT = 192;                   // batches up to this size (beyond it
                                                 // router_tiled_kernel is faster: T = 256,
                                                 // 64 us against 69)
constexpr int kRowsMaxH = 4096;                  // W float32 rows in LDS

template <int W>
__global__ void __launch_bounds__(64 * W) router_rows_kernel(
    const uint16_t *__restrict__ x, const float *__restrict__ wT,
    const float *__restrict__ bias, int T, int H, int E, float *__restrict__ logits) {
    constexpr int NT = 64 * W, KC = 64, NP = 2;
    __shared__ __attribute__((aligned(16))) float ws[2][KC][kRtExp];
    __shared__ __attribute__((aligned(16))) float as[W][kRowsMaxH];
    const int t0 = blockIdx.x * W, e0 = blockIdx.y * kRtExp;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // the router weight's first chunks are in flight while the rows stage
    RouterWeightPipe<KC, NP, kXNone, NT> pipe(wT, E, e0, H, tid);
    pipe.prime();
    // bf16 rows widened (rows past T repeat row t0; never stored)
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
    // the rows reach LDS before the chains read them: run() stores the first
    // chunk and synchronizes before its first step

    // lane j of every 16-lane row reads inputs 16 m + j of the chunk
    const float *xr = &as[wave][lane & 15];
    float acc[1] = {0.0f}, tot[1] = {0.0f};
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
            fma16_row_bcast(acc[0], xq[m & 1], w[m & 1]);
        }
        block_end(c, pipe.nch, acc, tot);
    });
    const int e = e0 + lane, t = t0 + wave;
    if (e < E && t < T) logits[(size_t)t * E + e] = bias ? tot[0] + bias[e] : tot[0];
}

// tokens per work group, measured at H = 4096, E = 352: W = 2 up to 64
// tokens (T = 32: 36 us against 39 us at W = 4 and 41 us at W = 1, whose
// single wave per group gains no LDS bandwidth worth its lost sharing),
// W = 4 beyond (T = 256: 68 us against 79 us at W = 2)
constexpr int kRowsW2MaxT = 64;

static void launch_rows(const void *x, int T, int H, const float *wT, const float *bias, int E,
                        float *logits, hipStream_t s) {
    const int eb = (E + kRtExp - 1) / kRtExp;
    if (T <= kRowsW2MaxT)
        hipLaunchKernelGGL((router_rows_kernel<2>), dim3((T + 1) / 2, eb), dim3(128), 0, s,
                           (const uint16_t *)x, wT, bias, T, H, E, logits);
    else
        hipLaunchKernelGGL((router_rows_kernel<4>), dim3((T + 3) / 4, eb), dim3(256), 0, s,
                           (const uint16_t *)x, wT, bias, T, H, E, logits);
}

// ---- small batches, block sums side by side --------------------------------
// One work group per (4 TW tokens, 64 experts, 512-input block), TW tokens
// per wave: the tiled kernel's layout (x by DPP row broadcast, the weight
// chunk shared through LDS by the group's waves) over one block of the
// canonical sum, whose chains' values go to part [block][T][E] for the
// top-K to add up in block order. A token's 8 chains of 512 steps run side
// by side instead of one chain of 4096. Fewer tokens per wave shorten a
// wave's instruction stream (TW DPP FMAs per input); more tokens per group
// read each 128 KB weight slice for more tokens (the batch streams the
// 5.8 MB router weight once per 4 TW tokens). Groups are ordered (expert
// block, input block) major in contiguous ranges per XCD, so the groups
// sharing a weight slice share an L2.
// The group first stages its rows' block inputs in LDS as float32: the
// bf16 activations widened (NORM = false), or (NORM = true) the RMSNorm of
// the float32 residual rows, bf16-rounded and widened. The norm's sums of
// squares follow rmsnorm_kernel exactly (the group's 256 threads are that
// kernel's 256 threads, one row after the other), so the rows are bitwise
// the ones moe_rmsnorm writes; the groups of the first expert block write
// their block's columns of them to a_out for the experts.
constexpr int kBlkPitch = kRouterBlock + 4;      // floats per staged row: the 4 pad
                                                 // floats keep 16-byte alignment

// TW tokens per wave, 4 TW per group; a wave runs its tokens' chains one
// 16-input DPP broadcast FMA block after the other.
template <bool NORM, int TW>
__global__ void __launch_bounds__(256) router_block_kernel(
    const void *__restrict__ xin, const float *__restrict__ gain, float eps,
    const float *__restrict__ wT, int T, int H, int E, uint16_t *__restrict__ a_out,
    float *__restrict__ part) {
    constexpr int BT = 4 * TW;                   // tokens per group
    constexpr int TPR = 256 / BT;                // staging threads per row
    static_assert(TW == 1 || TW == 2, "tokens per wave");
    __shared__ __attribute__((aligned(16))) float ws[2][kRtKC][kRtExp];
    __shared__ __attribute__((aligned(16))) float xs[BT][kBlkPitch];
    __shared__ float red[BT][4];
    const int nb = gridDim.x, b = blockIdx.x, xq8 = nb / 8, xr8 = nb % 8, xcd = b % 8;
    const int lid = xcd * xq8 + (xcd < xr8 ? xcd : xr8) + b / 8;
    const int ntb = (T + BT - 1) / BT, P = (H + kRouterBlock - 1) / kRouterBlock;
    const int tb = lid % ntb, rest = lid / ntb, pb = rest % P, eb = rest / P;
    const int t0 = tb * BT, e0 = eb * kRtExp;
    const int k0 = pb * kRouterBlock, kn = min(kRouterBlock, H - k0);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // the block's first weight chunks are in flight while the rows stage
    RouterWeightPipe<kRtKC, 2, kXNone> pipe(wT + (size_t)k0 * E, E, e0, kn, tid);
    pipe.prime();

    // staging roles: row tid / TPR, columns 4 (tid % TPR) + 4 TPR i of the
    // block (rows past T repeat row t0; their logits are not stored)
    const int sr = tid / TPR, sc = (tid % TPR) * 4;
    const int st_row = t0 + sr < T ? t0 + sr : t0;
    if (!NORM) {
        const uint16_t *x = (const uint16_t *)xin + (size_t)st_row * H + k0;
        for (int c = sc; c < kn; c += 4 * TPR) {
            const uint2 v = *(const uint2 *)(x + c);
            *(f32x4_t *)&xs[sr][c] = f32x4_t{__uint_as_float(v.x << 16),
                                             __uint_as_float(v.x & 0xFFFF0000u),
                                             __uint_as_float(v.y << 16),
                                             __uint_as_float(v.y & 0xFFFF0000u)};
        }
    } else {
        const float *res = (const float *)xin;
        // sums of squares, row after row: thread p adds columns 4p .. 4p+3,
        // 1024 + 4p .. in order, the wave folds by xor-shuffles 32 .. 1, the
        // four wave sums add left to right (after the barrier); four rows'
        // loads in flight at a time
        constexpr int kCols = kRowsMaxH / 1024;
        for (int r0 = 0; r0 < BT; r0 += 4) {
            f32x4_t v[4][kCols];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = t0 + r0 + i < T ? t0 + r0 + i : t0;
#pragma unroll
                for (int j = 0; j < kCols; ++j) {
                    const int c = tid * 4 + 1024 * j;
                    if (c < H) v[i][j] = *(const f32x4_t *)(res + (size_t)t * H + c);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float ss = 0.0f;
#pragma unroll
                for (int j = 0; j < kCols; ++j) {
                    if (tid * 4 + 1024 * j < H) {
                        const f32x4_t q = v[i][j];
                        ss = ss + q.x * q.x;
                        ss = ss + q.y * q.y;
                        ss = ss + q.z * q.z;
                        ss = ss + q.w * q.w;
                    }
                }
#pragma unroll
                for (int m = 32; m >= 1; m >>= 1) ss = ss + __shfl_xor(ss, m, kWave);
                if (lane == 0) red[r0 + i][wave] = ss;
            }
        }
        __syncthreads();
        const float tot = ((red[sr][0] + red[sr][1]) + red[sr][2]) + red[sr][3];
        const float rr = __builtin_sqrtf(tot / (float)H + eps);
        const float *rrow = res + (size_t)st_row * H + k0;
        for (int c = sc; c < kn; c += 4 * TPR) {
            const f32x4_t q = *(const f32x4_t *)(rrow + c);
            f32x4_t gg = f32x4_t{0.f, 0.f, 0.f, 0.f};
            if (gain) gg = *(const f32x4_t *)(gain + k0 + c);
            const uint32_t lo = f32_to_bf16_bits((q.x / rr) * (1.0f + gg.x)) |
                                ((uint32_t)f32_to_bf16_bits((q.y / rr) * (1.0f + gg.y)) << 16);
            const uint32_t hi = f32_to_bf16_bits((q.z / rr) * (1.0f + gg.z)) |
                                ((uint32_t)f32_to_bf16_bits((q.w / rr) * (1.0f + gg.w)) << 16);
            *(f32x4_t *)&xs[sr][c] = f32x4_t{__uint_as_float(lo << 16),
                                             __uint_as_float(lo & 0xFFFF0000u),
                                             __uint_as_float(hi << 16),
                                             __uint_as_float(hi & 0xFFFF0000u)};
            if (eb == 0 && t0 + sr < T)
                *(uint2 *)(a_out + (size_t)(t0 + sr) * H + k0 + c) = make_uint2(lo, hi);
        }
    }
    // the rows reach LDS before the chains read them: run() stores the first
    // chunk and synchronizes before its first step

    float acc[TW];
#pragma unroll
    for (int i = 0; i < TW; ++i) acc[i] = 0.0f;
    pipe.run(ws, [&](int c, float (*st)[kRtExp]) {
        // lane j of every 16-lane row reads inputs 16 m + j of the chunk
        const float *xw = &xs[TW * wave][c * kRtKC + (lane & 15)];
        float xq[2][TW], w[2][16];
        auto read = [&](int m, int bb) {
#pragma unroll
            for (int i = 0; i < TW; ++i) xq[bb][i] = xw[i * kBlkPitch + 16 * m];
#pragma unroll
            for (int j = 0; j < 16; ++j) w[bb][j] = st[16 * m + j][lane];
        };
        read(0, 0);
#pragma unroll
        for (int m = 0; m < kRtKC / 16; ++m) {
            if (m + 1 < kRtKC / 16) read(m + 1, (m + 1) & 1);
#pragma unroll
            for (int i = 0; i < TW; ++i) fma16_row_bcast(acc[i], xq[m & 1][i], w[m & 1]);
        }
    });
    const int e = e0 + lane;
    if (e >= E) return;
#pragma unroll
    for (int i = 0; i < TW; ++i) {
        const int t = t0 + TW * wave + i;
        if (t < T) part[((size_t)pb * T + t) * E + e] = acc[i];
    }
}

template <bool NORM, int TW>
static void launch_block_tw(const void *xin, const float *gain, float eps, int T, int H,
                            const float *wT, int E, void *a_out, float *part, hipStream_t s) {
    const int n = ((T + 4 * TW - 1) / (4 * TW)) * ((E + kRtExp - 1) / kRtExp) *
                  ((H + kRouterBlock - 1) / kRouterBlock);
    hipLaunchKernelGGL((router_block_kernel<NORM, TW>), dim3(n), dim3(256), 0, s, xin, gain, eps,
                       wT, T, H, E, (uint16_t *)a_out, part);
}

// Tokens per wave, measured on moe_norm_route (H = 4096, E = 352, graph
// replay, with the top-K): one up to 64 tokens (T = 1: 14.1 us, T = 32:
// 18.7 us, against 17.6 and 19.2 with two and 24.9 and 26.5 with four; the
// kernels with one 4096-step chain per token took 42 and 44 us), two
// beyond (T = 128: 29.0 us against 36.0 with one and 33.5 with four; T =
// 192: 41.6 against 49.1 and 50.1).
constexpr int kBlkTw1MaxT = 64;

template <bool NORM>
static void launch_block(const void *xin, const float *gain, float eps, int T, int H,
                         const float *wT, int E, void *a_out, float *part, hipStream_t s) {
    if (T <= kBlkTw1MaxT)
        launch_block_tw<NORM, 1>(xin, gain, eps, T, H, wT, E, a_out, part, s);
    else
        launch_block_tw<NORM, 2>(xin, gain, eps, T, H, wT, E, a_out, part, s);
}

moe_status_t launch_router_logits(const void *x, int x_dtype, const float *wT, const float *bias,
                                  int T, int H, int E, float *logits, hipStream_t s) {
    if (T == 0) return MOE_OK;
    const dim3 grid((T + kRtTok - 1) / kRtTok, (E + kRtExp - 1) / kRtExp);
    if (x_dtype == MOE_BF16 && T <= kRowsMaxT && H <= kRowsMaxH)
        launch_rows(x, T, H, wT, bias, E, logits, s);
    else if (x_dtype == MOE_BF16)
        hipLaunchKernelGGL((router_tiled_kernel<2, false, 4>), dim3(grid.x * grid.y), dim3(256), 0, s,
                           (const uint16_t *)x, wT, bias, T, H, E, logits);
    else
        hipLaunchKernelGGL(router_logits_kernel<MOE_F16>, grid, dim3(256), 0, s,
                           (const uint16_t *)x, wT, bias, T, H, E, logits);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

bool norm_route_fused(int T, int H, int E) { return T <= kRowsMaxT && H <= kRowsMaxH; }

int router_blocks(int H) { return (H + kRouterBlock - 1) / kRouterBlock; }

static_assert(kRowsMaxH / kRouterBlock <= kMaxRouterBlocks, "block sums the top-K adds");

// The block-sum path: small bf16 batches.
static bool block_path(int T, int H, int x_dtype) {
    return x_dtype == MOE_BF16 && T <= kRowsMaxT && H <= kRowsMaxH;
}
// Block sums (small batches by router_block_kernel, larger ones by the
// tiled kernel): bf16 and H <= 4096.
static bool sums_path(int H, int x_dtype) { return x_dtype == MOE_BF16 && H <= kRowsMaxH; }

// Workspace floats of the routing calls: the block sums on that path,
// else the logits; and the most any H <= kMaxDim can need.
size_t router_ws_floats(int T, int H, int E, int x_dtype) {
    return (size_t)(sums_path(H, x_dtype) ? router_blocks(H) : 1) * T * E;
}
size_t router_ws_floats_max(int T, int E) {
    return (size_t)(kRowsMaxH / kRouterBlock) * T * E;
}

// Tokens per wave of the tiled kernel's block sums: 8 from this batch size
// up (twice the independent chains per lane and half the LDS weight reads
// per FMA, at 3 work groups per CU instead of 4: routing at H = 4096, E =
// 352 took 41.4 / 70.7 / 130.6 / 240.1 us at 512 / 1024 / 2048 / 4096
// tokens against 44.2 / 79.0 / 141.4 / 263.3 with 4), else 4 (256 tokens:
// 28.3 us against 31.5).
constexpr int kTiled8MinT = 512;

// Block sums of bf16 inputs with H <= 4096, [router_blocks(H)][T][E] into
// `part`, *P = router_blocks(H): router_block_kernel up to 192 tokens, the
// tiled kernel with one 512-input block per work group beyond (8x the work
// groups of one chain over all inputs: at 256 tokens 28 us against 72, at
// 4096 tokens 263 against 276 with 4 tokens per wave). Otherwise the logits
// (no bias) with *P = 1. Either way route_given_kernel adds them up in
// block order.
moe_status_t launch_router_scores(const void *x, int x_dtype, const float *wT, int T, int H,
                                  int E, float *part, int *P, hipStream_t s) {
    if (block_path(T, H, x_dtype)) {
        *P = router_blocks(H);
        if (T == 0) return MOE_OK;
        launch_block<false>(x, nullptr, 0.f, T, H, wT, E, nullptr, part, s);
        MOE_LAUNCH_CHECK();
        return MOE_OK;
    }
    if (x_dtype == MOE_BF16 && H <= kRowsMaxH) {
        *P = router_blocks(H);
        if (T == 0) return MOE_OK;
        const int bt = T >= kTiled8MinT ? 32 : 16;
        const int n = ((T + bt - 1) / bt) * ((E + kRtExp - 1) / kRtExp) * *P;
        if (bt == 32)
            hipLaunchKernelGGL((router_tiled_kernel<2, true, 8>), dim3(n), dim3(256), 0, s,
                               (const uint16_t *)x, wT, nullptr, T, H, E, part);
        else
            hipLaunchKernelGGL((router_tiled_kernel<2, true, 4>), dim3(n), dim3(256), 0, s,
                               (const uint16_t *)x, wT, nullptr, T, H, E, part);
        MOE_LAUNCH_CHECK();
        return MOE_OK;
    }
    *P = 1;
    return launch_router_logits(x, x_dtype, wT, nullptr, T, H, E, part, s);
}

// The fused norm and router, block sums [router_blocks(H)][T][E] into part.
moe_status_t launch_norm_router_scores(const float *res, const float *gain, float eps, int T,
                                       int H, const float *wT, int E, void *a_out, float *part,
                                       hipStream_t s) {
    if (T == 0) return MOE_OK;
    launch_block<true>(res, gain, eps, T, H, wT, E, a_out, part, s);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

}  // namespace moe
