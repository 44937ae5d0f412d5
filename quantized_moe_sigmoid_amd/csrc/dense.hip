// The shared expert: a dense BF16 SwiGLU over every token (page "Step 5
// Preview: 92 narrow layers, ...", "The shape: narrow and deep": one shared
// expert per MoE layer, a SwiGLU of width 1536; it stays BF16, page
// "NeuroSenko/Step-5-Preview-Int4-g128", "What stays in BF16"), on MFMA
// v_mfma_f32_32x32x16_bf16.
//
// Work unit = (64 tokens, 128 gate/up columns | 256 down columns, one slice
// of the inputs); 4 waves, each owning 32 columns of gate and of up (64
// columns of down) and all 64 rows. Token rows stream through LDS in
// 64-input steps (double buffered, 16-byte chunks XOR-swizzled by row);
// each lane loads its own weight rows straight from HBM, 64 contiguous bytes
// per step, one step ahead.
//
// Few tokens give few work units, so the input range is split S ways
// (blockIdx.z) until the grid covers the chip; each slice then writes float32
// partial sums, and a second pass adds the S slices in ascending order (no
// atomics: the result does not depend on scheduling) and applies the SwiGLU.
#include "common.h"

namespace moe {

constexpr int kDnThreads = 256;
constexpr int kDnTM = 64;
constexpr int kDnBN = 128;
constexpr int kDnKS = 64;                      // inputs per step
constexpr int kDnRowBytes = kDnKS * 2;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int dn_swz(int row) { return ((row >> 1) & 7) ^ ((row & 1) << 2); }
__device__ __forceinline__ int dn_offset(int row, int chunk) {
    return row * kDnRowBytes + ((chunk ^ dn_swz(row)) << 4);
}

__device__ __forceinline__ f32x16_t dn_mfma(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ void dn_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// GATEUP: A = gate, B = up (same columns). Otherwise A and B are the down
// matrix at columns c and c + 32. Steps [step0, step0 + nsteps) of the
// inputs. PARTIAL: float32 sums to part[z][T][ncols] (gate at column c, up
// at F + c; down at c); else the final result: h = silu(gate) * up as bf16,
// or y float32.
template <bool GATEUP, bool PARTIAL>
__global__ void __launch_bounds__(kDnThreads) dense_kernel(
    const uint8_t *__restrict__ wa, int64_t ra, const uint8_t *__restrict__ wb, int64_t rb,
    int n_rows, int kin, int nsteps, const uint16_t *xin, int T, uint16_t *__restrict__ hout,
    float *__restrict__ yout, float *__restrict__ part) {
    constexpr int BN = GATEUP ? kDnBN : 2 * kDnBN;
    __shared__ __attribute__((aligned(16))) uint8_t abuf[2 * kDnTM * kDnRowBytes];
    const int t0 = blockIdx.x * kDnTM, nb = blockIdx.y, z = blockIdx.z;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int half = lane >> 5, l32 = lane & 31;
    const int m_valid = min(kDnTM, T - t0);
    const bool two_mb = m_valid > 32;
    const int step0 = z * nsteps;

    // staging: thread t owns row t/4 and chunk slots 2(t%4), 2(t%4)+1;
    // rows past T repeat token t0 (their outputs are never stored)
    const int srow = threadIdx.x >> 2;
    const uint16_t *src = xin + (size_t)(t0 + (srow < m_valid ? srow : 0)) * kin +
                          (size_t)step0 * kDnKS;
    const int slot0 = (threadIdx.x & 3) * 2;

    const int col_a = nb * BN + wave * (GATEUP ? 32 : 64) + l32;
    const int col_b = GATEUP ? col_a : col_a + 32;
    const uint8_t *pa = wa + (int64_t)col_a * ra + (int64_t)step0 * kDnRowBytes + half * 64;
    const uint8_t *pb = wb + (int64_t)col_b * rb + (int64_t)step0 * kDnRowBytes + half * 64;

    f32x16_t da[2], db[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int v = 0; v < 16; ++v) da[mb][v] = db[mb][v] = 0.0f;

    u32x4_t sv[2], wa0[4], wb0[4], wa1[4], wb1[4];
    auto load_a = [&](int step) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
            sv[i] = *(const u32x4_t *)(src + step * kDnKS + (((slot0 + i) ^ dn_swz(srow)) * 8));
    };
    auto store_a = [&](uint8_t *buf) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
            *(u32x4_t *)(buf + srow * kDnRowBytes + ((slot0 + i) << 4)) = sv[i];
    };
    auto load_w = [&](u32x4_t (&a)[4], u32x4_t (&b)[4], int step) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            a[j] = *(const u32x4_t *)(pa + (int64_t)step * kDnRowBytes + 16 * j);
            b[j] = *(const u32x4_t *)(pb + (int64_t)step * kDnRowBytes + 16 * j);
        }
    };
    // MFMA j of a step takes inputs 8j..8j+7 (lanes 0-31) and 32+8j..32+8j+7
    // (lanes 32-63): A from LDS chunk 4*half + j, B from the lane's own row
    auto compute = [&](const uint8_t *buf, const u32x4_t (&a)[4], const u32x4_t (&b)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int chunk = half * 4 + j;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                if (mb == 1 && !two_mb) break;
                const int row = mb * 32 + l32;
                const u32x4_t av = *(const u32x4_t *)(buf + dn_offset(row, chunk));
                da[mb] = dn_mfma(av, a[j], da[mb]);
                db[mb] = dn_mfma(av, b[j], db[mb]);
            }
        }
    };

    uint8_t *const buf0 = abuf, *const buf1 = abuf + kDnTM * kDnRowBytes;
    load_a(0);
    load_w(wa0, wb0, 0);
    store_a(buf0);
    __syncthreads();
    for (int step = 0; step < nsteps; step += 2) {
        {
            const int sn = step + 1 < nsteps ? step + 1 : step;
            load_a(sn);
            load_w(wa1, wb1, sn);
            __builtin_amdgcn_sched_barrier(0);
            compute(buf0, wa0, wb0);
            store_a(buf1);
            dn_barrier();
            if (step + 1 >= nsteps) break;
        }
        {
            const int sn = step + 2 < nsteps ? step + 2 : step + 1;
            load_a(sn);
            load_w(wa0, wb0, sn);
            __builtin_amdgcn_sched_barrier(0);
            compute(buf1, wa1, wb1);
            store_a(buf0);
            dn_barrier();
        }
    }

    const int ncols = GATEUP ? 2 * n_rows : n_rows;
    float *const pz = PARTIAL ? part + (size_t)z * T * ncols : nullptr;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int m = mb * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
            if (m >= m_valid) continue;
            const size_t r = (size_t)(t0 + m);
            if (PARTIAL) {
                pz[r * ncols + col_a] = da[mb][v];
                pz[r * ncols + (GATEUP ? n_rows + col_a : col_b)] = db[mb][v];
            } else if (GATEUP) {
                hout[r * n_rows + col_a] = f32_to_bf16_bits(silu_mul(da[mb][v], db[mb][v]));
            } else {
                yout[r * n_rows + col_a] = da[mb][v];
                yout[r * n_rows + col_b] = db[mb][v];
            }
        }
    }
}

// Small batches (T <= 32) at the layer's shape: v_mfma_f32_16x16x32_bf16
// with the tokens as the A operand (two 16-token blocks) and 16 weight rows
// as B. A work group owns BPW = 4 / KS blocks of 16 rows and one slice of
// KS * NSW * 32 inputs (blockIdx.y); the KS waves of a row block take NSW
// consecutive 32-input steps each and meet in LDS at the end (added in
// input order). A step's 16 rows x 64 bytes are loaded four lanes per row
// (lane 4 r + c: row r, bytes 16 c) and pass through a per-wave LDS tile
// into the MFMA layout (lane 16 c + r: row r, bytes 16 c; loaded that way
// directly, every 16 lanes of a load would touch 16 cache lines); R steps
// are in flight per lane and matrix. The slice's inputs of the T tokens are
// staged in LDS once. Output: float32 sums [slice][T][ncols] (gate at column
// c, up at n_rows + c), added and SwiGLU'd by swiglu_reduce_kernel, or the
// down projection's y when there is one slice.
constexpr int kDxWaves = 4, kDxThreads = kDxWaves * 64;

__host__ __device__ constexpr int dx_upad(int kz) { return kz / 8 + 1; }

inline size_t dense_small_lds(int kz, int nm, int ks) {
    return (size_t)32 * dx_upad(kz) * 16 + (size_t)kDxWaves * 1024 +
           (ks > 1 ? (size_t)kDxWaves * nm * 2 * 64 * 16 : 0);
}

template <bool GATEUP, int KS, int NSW, int R>
__global__ void __launch_bounds__(kDxThreads) dense_small_kernel(
    const uint8_t *__restrict__ wa, int64_t ra, const uint8_t *__restrict__ wb, int64_t rb,
    int n_rows, int kin, const uint16_t *__restrict__ xin, int T, float *__restrict__ out) {
    constexpr int NM = GATEUP ? 2 : 1, BPW = kDxWaves / KS, KZ = KS * NSW * 32;
    constexpr int UPAD = dx_upad(KZ), UNITS = KZ / 8;
    static_assert(kDxWaves % KS == 0 && NSW % R == 0 && (32 * UNITS) % kDxThreads == 0,
                  "whole wave parts, ring trips and staging rounds");
    extern __shared__ u32x4_t dxs[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kp = wave % KS, rbk = blockIdx.x * BPW + wave / KS;   // input part, row block
    const int z = blockIdx.y, k0 = z * KZ;
    const int r16 = lane & 15, g = lane >> 4, lr = lane >> 2, lc = lane & 3;
    u32x4_t *xs = dxs;                                    // [32 tokens][UPAD] units
    u32x4_t *wt = dxs + 32 * UPAD + wave * 64;            // this wave's 16 x 64-byte tile
    f32x4_t *red = (f32x4_t *)(dxs + 32 * UPAD + kDxWaves * 64);

    // weight ring (first: every thread's staging loads, then the ring's)
    constexpr int SR = 32 * UNITS / kDxThreads;           // staged units per thread
    u32x4_t xv[SR];
#pragma unroll
    for (int i = 0; i < SR; ++i) {
        const int idx = threadIdx.x + kDxThreads * i, t = idx / UNITS, u = idx % UNITS;
        xv[i] = *(const u32x4_t *)(xin + (size_t)(t < T ? t : 0) * kin + k0 + 8 * u);
    }
    const uint8_t *mats[2] = {wa, wb};
    const int64_t strides[2] = {ra, rb};
    int qo[NM];
#pragma unroll
    for (int k = 0; k < NM; ++k)
        qo[k] = (rbk * 16 + lr) * (int)strides[k] + 2 * k0 + 16 * lc;
    __amdgpu_buffer_rsrc_t rq[NM];
#pragma unroll
    for (int k = 0; k < NM; ++k)
        rq[k] = __builtin_amdgcn_make_buffer_rsrc((void *)mats[k], (short)0,
                                                  (int)min((int64_t)n_rows * strides[k],
                                                           (int64_t)0x7FFFFFFF),
                                                  0x00020000);
    u32x4_t w[R][NM];
    const int j_lo = kp * NSW;
    auto load = [&](int slot, int j) {
#pragma unroll
        for (int k = 0; k < NM; ++k)
            w[slot][k] = __builtin_bit_cast(
                u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq[k], qo[k] + 64 * j, 0, 0));
    };
#pragma unroll
    for (int j = 0; j < R; ++j) load(j, j_lo + j);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < SR; ++i) {
        const int idx = threadIdx.x + kDxThreads * i, t = idx / UNITS, u = idx % UNITS;
        if (t < T) xs[t * UPAD + u] = xv[i];
    }
    dn_barrier();

    // tile: chunk c of row r at unit 4 r + (c ^ (r / 4 % 4))
    u32x4_t *const wt_st = wt + 4 * lr + (lc ^ ((lr >> 2) & 3));
    const u32x4_t *const wt_ld = wt + 4 * r16 + (g ^ ((r16 >> 2) & 3));
    f32x4_t acc[NM][2];
#pragma unroll
    for (int k = 0; k < NM; ++k) acc[k][0] = acc[k][1] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    auto step = [&](int slot, int j, bool refill, int jr) {
        u32x4_t b[NM];
#pragma unroll
        for (int k = 0; k < NM; ++k) {
            *wt_st = w[slot][k];
            b[k] = *wt_ld;
        }
        __builtin_amdgcn_sched_barrier(0);
        if (refill) load(slot, jr);
        const u32x4_t a0 = xs[r16 * UPAD + 4 * j + g], a1 = xs[(16 + r16) * UPAD + 4 * j + g];
#pragma unroll
        for (int k = 0; k < NM; ++k) {
            acc[k][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, a0), __builtin_bit_cast(bf16x8_t, b[k]), acc[k][0], 0, 0, 0);
            acc[k][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, a1), __builtin_bit_cast(bf16x8_t, b[k]), acc[k][1], 0, 0, 0);
        }
    };
#pragma unroll
    for (int i0 = 0; i0 < NSW - R; i0 += R) {
#pragma unroll
        for (int slot = 0; slot < R; ++slot) step(slot, j_lo + i0 + slot, true, j_lo + i0 + slot + R);
    }
#pragma unroll
    for (int slot = 0; slot < R; ++slot) step(slot, j_lo + NSW - R + slot, false, 0);

    if constexpr (KS > 1) {
        if (kp != 0) {
#pragma unroll
            for (int k = 0; k < NM; ++k)
#pragma unroll
                for (int b2 = 0; b2 < 2; ++b2) red[((wave * NM + k) * 2 + b2) * 64 + lane] = acc[k][b2];
        }
        dn_barrier();
        if (kp != 0) return;
#pragma unroll
        for (int q = 1; q < KS; ++q)
#pragma unroll
            for (int k = 0; k < NM; ++k)
#pragma unroll
                for (int b2 = 0; b2 < 2; ++b2) {
                    const f32x4_t o = red[(((wave + q) * NM + k) * 2 + b2) * 64 + lane];
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[k][b2][i] += o[i];
                }
    }
    // lane (r16, g): tokens 16 b2 + 4 g + i of row r16
    const int ncols = NM * n_rows, col = rbk * 16 + r16;
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 16 * b2 + 4 * g + i;
            if (t < T) {
                float *o = out + ((size_t)z * T + t) * ncols + col;
                o[0] = acc[0][b2][i];
                if constexpr (GATEUP) o[n_rows] = acc[1][b2][i];
            }
        }
}

// h[t][c] = bf16(silu(sum_z gate) * sum_z up), z ascending; 4 columns a thread.
__global__ void __launch_bounds__(256) swiglu_reduce_kernel(const float *__restrict__ part,
                                                            int S, int T, int F,
                                                            uint16_t *__restrict__ h) {
    const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= (size_t)T * F) return;
    const size_t t = i / F, c = i % F;
    float4 g = make_float4(0.f, 0.f, 0.f, 0.f), u = g;
    // unrolled so the loads of several slices are in flight together (the
    // sums keep ascending z): one slice at a time, the few work groups of a
    // small batch waited out a cache round trip per slice
#pragma unroll 8
    for (int z = 0; z < S; ++z) {
        const float *p = part + ((size_t)z * T + t) * 2 * F + c;
        const float4 a = *(const float4 *)p, b = *(const float4 *)(p + F);
        g.x += a.x; g.y += a.y; g.z += a.z; g.w += a.w;
        u.x += b.x; u.y += b.y; u.z += b.z; u.w += b.w;
    }
    const uint32_t lo = f32_to_bf16_bits(silu_mul(g.x, u.x)) |
                        ((uint32_t)f32_to_bf16_bits(silu_mul(g.y, u.y)) << 16);
    const uint32_t hi = f32_to_bf16_bits(silu_mul(g.z, u.z)) |
                        ((uint32_t)f32_to_bf16_bits(silu_mul(g.w, u.w)) << 16);
    *(uint2 *)(h + i) = make_uint2(lo, hi);
}

// y[i] = sum_z part[z][i], z ascending; 4 elements a thread.
__global__ void __launch_bounds__(256) sum_reduce_kernel(const float *__restrict__ part, int S,
                                                         size_t n, float *__restrict__ y) {
    const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= n) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
    for (int z = 0; z < S; ++z) {
        const float4 a = *(const float4 *)(part + (size_t)z * n + i);
        acc.x += a.x; acc.y += a.y; acc.z += a.z; acc.w += a.w;
    }
    *(float4 *)(y + i) = acc;
}

// Input-range split for a grid of `units` work units over `steps` steps:
// the largest S that divides the steps, leaves every slice at least 2
// steps, keeps the grid within one work unit per CU and stays at most
// `max_split` (which bounds the partial-sum traffic). Any divisor, not only
// powers of two: the down projection's 24 steps at H = 4096, F = 1536 split
// 12 ways (192 work groups) where doubling stopped at 4 (64).
int dense_split(int64_t units, int steps, int max_split) {
    int S = 1;
    for (int c = 2; c <= max_split; ++c)
        if (steps % c == 0 && steps / c >= 2 && units * c <= 256) S = c;
    return S;
}

// The small-batch kernels' shapes: gate/up slices of 512 inputs (two waves
// of 8 steps per 16 rows), the down pass in one slice (four waves of 12).
constexpr int kDxGuKS = 2, kDxGuNSW = 8, kDxGuR = 4, kDxDnKS = 4, kDxDnNSW = 12, kDxDnR = 6;
static bool dense_small_ok(int T, int H, int F) {
    return T >= 1 && T <= 32 && H % (kDxGuKS * kDxGuNSW * 32) == 0 &&
           F == kDxDnKS * kDxDnNSW * 32 && F % (16 * (kDxWaves / kDxGuKS)) == 0 &&
           H % (16 * (kDxWaves / kDxDnKS)) == 0;
}

DenseSplit dense_plan(int T, int H, int F) {
    DenseSplit d;
    d.part_floats = 0;
    if (dense_small_ok(T, H, F)) {
        d.s_gateup = H / (kDxGuKS * kDxGuNSW * 32);
        d.s_down = 1;
        d.part_floats = (size_t)d.s_gateup * T * 2 * F;
        return d;
    }
    const int64_t tiles = (T + kDnTM - 1) / kDnTM;
    d.s_gateup = dense_split(tiles * (F / kDnBN), H / kDnKS, 16);
    d.s_down = dense_split(tiles * (H / (2 * kDnBN)), F / kDnKS, 12);
    if (d.s_gateup > 1) d.part_floats = (size_t)d.s_gateup * T * 2 * F;
    if (d.s_down > 1 && (size_t)d.s_down * T * H > d.part_floats)
        d.part_floats = (size_t)d.s_down * T * H;
    return d;
}

bool dense_shape_ok(int H, int F) {
    return H % (2 * kDnBN) == 0 && F % kDnBN == 0 && H % kDnKS == 0 && F % kDnKS == 0;
}

moe_status_t launch_dense_swiglu(const moe_ffn_desc_t &sh, const void *x, int T, void *h,
                                 float *y, float *part, hipStream_t s) {
    const int F = sh.gate.n, H = sh.gate.k;
    const DenseSplit d = dense_plan(T, H, F);
    if (dense_small_ok(T, H, F)) {
        const uint8_t *g = (const uint8_t *)sh.gate.qweight, *u = (const uint8_t *)sh.up.qweight;
        const uint8_t *dn = (const uint8_t *)sh.down.qweight;
        {
            auto k = dense_small_kernel<true, kDxGuKS, kDxGuNSW, kDxGuR>;
            const size_t lds = dense_small_lds(kDxGuKS * kDxGuNSW * 32, 2, kDxGuKS);
            if (lds > 65536)
                (void)hipFuncSetAttribute((const void *)k,
                                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            hipLaunchKernelGGL(k, dim3(F / (16 * (kDxWaves / kDxGuKS)), d.s_gateup),
                               dim3(kDxThreads), lds, s, g, sh.gate.qweight_row_stride, u,
                               sh.up.qweight_row_stride, F, H, (const uint16_t *)x, T, part);
            MOE_LAUNCH_CHECK();
            const size_t n4 = ((size_t)T * F) / 4;
            hipLaunchKernelGGL(swiglu_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)),
                               dim3(256), 0, s, (const float *)part, d.s_gateup, T, F,
                               (uint16_t *)h);
            MOE_LAUNCH_CHECK();
        }
        {
            auto k = dense_small_kernel<false, kDxDnKS, kDxDnNSW, kDxDnR>;
            const size_t lds = dense_small_lds(F, 1, kDxDnKS);
            if (lds > 65536)
                (void)hipFuncSetAttribute((const void *)k,
                                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            hipLaunchKernelGGL(k, dim3(H / (16 * (kDxWaves / kDxDnKS)), 1), dim3(kDxThreads), lds,
                               s, dn, sh.down.qweight_row_stride, dn, sh.down.qweight_row_stride, H,
                               F, (const uint16_t *)h, T, y);
            MOE_LAUNCH_CHECK();
        }
        return MOE_OK;
    }
    const unsigned tiles = (unsigned)((T + kDnTM - 1) / kDnTM);
    const uint8_t *g = (const uint8_t *)sh.gate.qweight, *u = (const uint8_t *)sh.up.qweight;
    const uint8_t *dn = (const uint8_t *)sh.down.qweight;
    const int64_t rg = sh.gate.qweight_row_stride, ru = sh.up.qweight_row_stride;
    const int64_t rd = sh.down.qweight_row_stride;
    const dim3 blk(kDnThreads);
    const dim3 ggu(tiles, F / kDnBN, d.s_gateup), gdn(tiles, H / (2 * kDnBN), d.s_down);
    const int gu_steps = H / kDnKS / d.s_gateup, dn_steps = F / kDnKS / d.s_down;
    if (d.s_gateup > 1) {
        hipLaunchKernelGGL((dense_kernel<true, true>), ggu, blk, 0, s, g, rg, u, ru, F, H,
                           gu_steps, (const uint16_t *)x, T, nullptr, nullptr, part);
        MOE_LAUNCH_CHECK();
        const size_t n4 = ((size_t)T * F) / 4;
        hipLaunchKernelGGL(swiglu_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), blk, 0, s,
                           (const float *)part, d.s_gateup, T, F, (uint16_t *)h);
    } else {
        hipLaunchKernelGGL((dense_kernel<true, false>), ggu, blk, 0, s, g, rg, u, ru, F, H,
                           gu_steps, (const uint16_t *)x, T, (uint16_t *)h, nullptr, nullptr);
    }
    MOE_LAUNCH_CHECK();
    if (d.s_down > 1) {
        hipLaunchKernelGGL((dense_kernel<false, true>), gdn, blk, 0, s, dn, rd, dn, rd, H, F,
                           dn_steps, (const uint16_t *)h, T, nullptr, nullptr, part);
        MOE_LAUNCH_CHECK();
        const size_t n = (size_t)T * H;
        hipLaunchKernelGGL(sum_reduce_kernel, dim3((unsigned)((n / 4 + 255) / 256)), blk, 0, s,
                           (const float *)part, d.s_down, n, y);
    } else {
        hipLaunchKernelGGL((dense_kernel<false, false>), gdn, blk, 0, s, dn, rd, dn, rd, H, F,
                           dn_steps, (const uint16_t *)h, T, nullptr, y, nullptr);
    }
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

}  // namespace moe
