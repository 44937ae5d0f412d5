// Decode-sized expert FFN: dequantizing GEMV over expert tiles.
//
// Work unit = (tile of up to TM slots of one expert, block of output rows).
// Each weight row is streamed with 16-byte loads, LPR lanes per row side by
// side along K (LPR * 16 contiguous bytes per row per load), and read once
// per tile; the tile's activation rows sit in LDS in a layout matched to the
// 4-bit decode, so the inner loop is decode + 16-bit dot products with
// float32 accumulation and the LPR partial sums meet in a lane reduction.
//
//   gate/up pass: h[row(s)][n] = silu(g_n) * u_n  for both projections of
//                 the same n in one lane group (SwiGLU fused);
//   down pass:    y[row(s)][n] = sum_j Wd[n][j] h[row(s)][j]  (float32).
//
// int4: a word's nibbles become exact 16-bit values BIAS + q (decode.h),
//   dot2 accumulates sum (BIAS + q) x over a 32-input chunk, and the chunk's
//   sum(x) (kept next to x in LDS) removes BIAS exactly in algebra:
//   acc += s_g * (dot - BIAS * sum x). The bf16 scale s_g applies per chunk
//   in float32 (every chunk lies inside one 128-input group).
// NVFP4: the hardware pair conversion gives exact E2M1 values; the E4M3
//   block scale applies per 16 inputs in float32, the global scale once at
//   the end.
#include <functional>

#include "decode.h"

namespace moe {

constexpr int kGemvThreads = 256;
constexpr int kGemvWaves = kGemvThreads / kWave;

struct GemvMat {                 // one projection bank, byte addressed
    const uint8_t *q, *s;
    const float *gs;             // NVFP4 global scale [E] or null
    int64_t qe, qr, se, sr;      // expert / row strides (bytes)
};

// LDS unit (16 bytes = 4 pair dwords) of input chunk c (32 inputs), word j.
// For a fixed j the LPR chunks read together by one row's lanes are 16-byte
// neighbours, so one wave-wide 16-byte read touches all banks once.
template <int LPR>
__device__ __forceinline__ int xs_unit(int c, int j) {
    return ((c / LPR) * 4 + j) * LPR + (c % LPR);
}
// LDS units per token row: chunks rounded up to a multiple of LPR.
template <int LPR>
__host__ __device__ __forceinline__ int xs_units_pad(int kin) {
    return (kin / 32 + LPR - 1) / LPR * LPR * 4;
}

// Stage the m activation rows of the tile into LDS as 16-bit pairs in the
// order the decoders produce weights, plus (int4) per-chunk sums of x.
template <int FMT, int LPR, int TM>
__device__ __forceinline__ void stage_x(const uint16_t *const *rows, int m, int kin,
                                        uint4 *xs, float *xsum, bool f16) {
    const int units = kin / 8;                   // 8 inputs per unit
    const int upad = xs_units_pad<LPR>(kin);
    for (int idx = threadIdx.x; idx < TM * units; idx += kGemvThreads) {
        const int t = idx / units, g8 = idx - t * units;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (t < m) v = *(const uint4 *)(rows[t] + 8 * g8);
        uint4 p;
        if (FMT == MOE_W_INT4_G128) {            // pairs (i, i+4) of the 8 inputs
            p.x = (v.x & 0xFFFFu) | (v.z << 16);
            p.y = (v.x >> 16) | (v.z & 0xFFFF0000u);
            p.z = (v.y & 0xFFFFu) | (v.w << 16);
            p.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
        } else {                                 // pairs (2i, 2i+1): natural order
            p = v;
        }
        xs[t * upad + xs_unit<LPR>(g8 >> 2, g8 & 3)] = p;
    }
    if (FMT == MOE_W_INT4_G128) {
        __syncthreads();
        const int nch = kin / 32;
        for (int idx = threadIdx.x; idx < TM * nch; idx += kGemvThreads) {
            const int t = idx / nch, c = idx - t * nch;
            float s = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint4 p = xs[t * upad + xs_unit<LPR>(c, j)];
                const uint32_t d[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    s += f16 ? f16_bits_to_f32(d[i] & 0xFFFF) : bf16_bits_to_f32(d[i] & 0xFFFF);
                    s += f16 ? f16_bits_to_f32(d[i] >> 16) : bf16_bits_to_f32(d[i] >> 16);
                }
            }
            xsum[t * nch + c] = s;
        }
    }
    __syncthreads();
}

// Partial dot products of one 16-byte weight chunk against token t's x.
template <int ACT, int FMT>
struct ChunkDot;

template <int ACT>
struct ChunkDot<ACT, MOE_W_INT4_G128> {
    uint32_t p[16];
    __device__ __forceinline__ void decode(uint4 w) {
        int4_biased_pairs<ACT>(w.x, p + 0);
        int4_biased_pairs<ACT>(w.y, p + 4);
        int4_biased_pairs<ACT>(w.z, p + 8);
        int4_biased_pairs<ACT>(w.w, p + 12);
    }
    // s2 = the chunk's scale(s): int4 uses one bf16 scale (as float).
    __device__ __forceinline__ float apply(const uint4 *xu, int stride_j, float xs_sum,
                                           float scale, float, float acc) const {
        float d = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint4 x = xu[j * stride_j];
            d = dot2<ACT>(p[4 * j + 0], x.x, d);
            d = dot2<ACT>(p[4 * j + 1], x.y, d);
            d = dot2<ACT>(p[4 * j + 2], x.z, d);
            d = dot2<ACT>(p[4 * j + 3], x.w, d);
        }
        return __builtin_fmaf(scale, d - Int4Bias<ACT>::kBias * xs_sum, acc);
    }
};

template <int ACT>
struct ChunkDot<ACT, MOE_W_NVFP4_G16> {
    uint32_t p[16];
    __device__ __forceinline__ void decode(uint4 w) {
        const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            p[4 * j + 0] = fp4_pair<ACT, 0>(d[j]);
            p[4 * j + 1] = fp4_pair<ACT, 1>(d[j]);
            p[4 * j + 2] = fp4_pair<ACT, 2>(d[j]);
            p[4 * j + 3] = fp4_pair<ACT, 3>(d[j]);
        }
    }
    __device__ __forceinline__ float apply(const uint4 *xu, int stride_j, float,
                                           float bs0, float bs1, float acc) const {
        float d[2] = {0.0f, 0.0f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint4 x = xu[j * stride_j];
            float &dd = d[j >> 1];
            dd = dot2<ACT>(p[4 * j + 0], x.x, dd);
            dd = dot2<ACT>(p[4 * j + 1], x.y, dd);
            dd = dot2<ACT>(p[4 * j + 2], x.z, dd);
            dd = dot2<ACT>(p[4 * j + 3], x.w, dd);
        }
        return __builtin_fmaf(bs1, d[1], __builtin_fmaf(bs0, d[0], acc));
    }
};

template <int FMT>
__device__ __forceinline__ void chunk_scales(const uint8_t *srow, int c, float &a, float &b) {
    if (FMT == MOE_W_INT4_G128) {
        a = bf16_bits_to_f32(*(const uint16_t *)(srow + 2 * (c >> 2)));
        b = 0.0f;
    } else {
        const uint16_t two = *(const uint16_t *)(srow + 2 * c);
        a = e4m3_to_f32(two & 0xFF);
        b = e4m3_to_f32(two >> 8);
    }
}

// GATEUP: mats a = gate, b = up, output h (16-bit). Otherwise a = down,
// output y (float32).
template <int ACT, int FMT, int LPR, int TM, bool GATEUP>
__global__ void __launch_bounds__(kGemvThreads) gemv_kernel(
    GemvMat A, GemvMat B, int n_rows, int kin, const uint16_t *__restrict__ xin,
    int x_from_slots, int topk, const int32_t *__restrict__ sorted_slots,
    const int32_t *__restrict__ tile_expert, const int32_t *__restrict__ num_tiles,
    uint16_t *__restrict__ hout, float *__restrict__ yout) {
    extern __shared__ uint4 smem[];
    const int tile = blockIdx.y;
    if (tile >= num_tiles[0]) return;
    const int e = tile_expert[tile];

    __shared__ const uint16_t *rows[TM];
    __shared__ int m_sh;
    if (threadIdx.x == 0) {
        int m = 0;
        for (int t = 0; t < TM; ++t) {
            const int s = sorted_slots[tile * TM + t];
            if (s >= 0) m = t + 1;
            rows[t] = x_from_slots ? xin + (size_t)(s >= 0 ? s / topk : 0) * kin
                                   : xin + (size_t)(tile * TM + t) * kin;
        }
        m_sh = m;
    }
    __syncthreads();
    const int m = m_sh;
    uint4 *xs = smem;
    float *xsum = (float *)(smem + TM * xs_units_pad<LPR>(kin));
    stage_x<FMT, LPR, TM>(rows, m, kin, xs, xsum, ACT == MOE_F16);

    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
    const int sub = lane % LPR;
    const int row = (blockIdx.x * kGemvWaves + wave) * (kWave / LPR) + lane / LPR;
    const bool live = row < n_rows;
    const uint8_t *qa = A.q + e * A.qe + (int64_t)row * A.qr;
    const uint8_t *sa = A.s + e * A.se + (int64_t)row * A.sr;
    const uint8_t *qb = GATEUP ? B.q + e * B.qe + (int64_t)row * B.qr : nullptr;
    const uint8_t *sb = GATEUP ? B.s + e * B.se + (int64_t)row * B.sr : nullptr;

    float acc_a[TM], acc_b[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) acc_a[t] = acc_b[t] = 0.0f;

    const int nch = kin / 32;
    const int units = xs_units_pad<LPR>(kin);
    for (int c0 = 0; c0 < nch; c0 += LPR) {
        const int c = c0 + sub;
        if (!live || c >= nch) continue;
        ChunkDot<ACT, FMT> da, db;
        da.decode(*(const uint4 *)(qa + 16 * (int64_t)c));
        float a0, a1, b0 = 0.0f, b1 = 0.0f;
        chunk_scales<FMT>(sa, c, a0, a1);
        if (GATEUP) {
            db.decode(*(const uint4 *)(qb + 16 * (int64_t)c));
            chunk_scales<FMT>(sb, c, b0, b1);
        }
        const int u0 = xs_unit<LPR>(c, 0);
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            if (t < m) {
                const uint4 *xu = xs + t * units + u0;
                const float xsm = FMT == MOE_W_INT4_G128 ? xsum[t * nch + c] : 0.0f;
                acc_a[t] = da.apply(xu, LPR, xsm, a0, a1, acc_a[t]);
                if (GATEUP) acc_b[t] = db.apply(xu, LPR, xsm, b0, b1, acc_b[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < TM; ++t) {
#pragma unroll
        for (int msk = LPR / 2; msk >= 1; msk >>= 1) {
            acc_a[t] += shfl_xor_f(acc_a[t], msk);
            if (GATEUP) acc_b[t] += shfl_xor_f(acc_b[t], msk);
        }
    }
    if (!live || sub != 0) return;
    float ga = 1.0f, gb = 1.0f;
    if (FMT == MOE_W_NVFP4_G16) {
        ga = A.gs[e];
        if (GATEUP) gb = B.gs[e];
    }
#pragma unroll
    for (int t = 0; t < TM; ++t) {
        if (t < m) {
            const size_t r = (size_t)tile * TM + t;
            if (GATEUP)
                hout[r * n_rows + row] = f32_to_act<ACT>(silu_mul(acc_a[t] * ga, acc_b[t] * gb));
            else
                yout[r * n_rows + row] = acc_a[t] * ga;
        }
    }
}

constexpr int kGemvLPR = 8;
constexpr int kGemvTM = 4;

inline GemvMat gemv_mat(const moe_weight_desc_t &d) {
    return GemvMat{(const uint8_t *)d.qweight, (const uint8_t *)d.scale, d.global_scale,
                   d.qweight_expert_stride, d.qweight_row_stride, d.scale_expert_stride,
                   d.scale_row_stride};
}

template <int LPR, int TM>
inline size_t gemv_lds_bytes(int kin) {
    return (size_t)TM * xs_units_pad<LPR>(kin) * 16 + (size_t)TM * (kin / 32) * 4;
}

template <typename Kern>
inline void allow_lds(Kern k, size_t lds) {
    if (lds > 65536)
        (void)hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)lds);
}

template <int ACT, int FMT>
moe_status_t gemv_forward_t(const moe_ffn_desc_t &ex, const uint16_t *x, int K,
                            const moe_perm_t &p, int max_tiles, uint16_t *h, float *y,
                            hipStream_t s, const std::function<moe_status_t(int)> &mark) {
    constexpr int LPR = kGemvLPR, TM = kGemvTM;
    const int F = ex.gate.n, H = ex.gate.k;
    const int rows_per_block = kGemvWaves * (kWave / LPR);
    {
        const size_t lds = gemv_lds_bytes<LPR, TM>(H);
        dim3 grid((F + rows_per_block - 1) / rows_per_block, max_tiles);
        allow_lds(gemv_kernel<ACT, FMT, LPR, TM, true>, lds);
        hipLaunchKernelGGL((gemv_kernel<ACT, FMT, LPR, TM, true>), grid, dim3(kGemvThreads), lds, s,
                           gemv_mat(ex.gate), gemv_mat(ex.up), F, H, x, 1, K, p.sorted_slots,
                           p.tile_expert, p.num_tiles, h, nullptr);
        MOE_LAUNCH_CHECK();
    }
    if (mark && mark(1) != MOE_OK) return MOE_ERR_HIP;
    {
        const size_t lds = gemv_lds_bytes<LPR, TM>(F);
        dim3 grid((H + rows_per_block - 1) / rows_per_block, max_tiles);
        allow_lds(gemv_kernel<ACT, FMT, LPR, TM, false>, lds);
        hipLaunchKernelGGL((gemv_kernel<ACT, FMT, LPR, TM, false>), grid, dim3(kGemvThreads), lds,
                           s, gemv_mat(ex.down), gemv_mat(ex.down), H, F, h, 0, K,
                           p.sorted_slots, p.tile_expert, p.num_tiles, nullptr, y);
        MOE_LAUNCH_CHECK();
    }
    if (mark && mark(2) != MOE_OK) return MOE_ERR_HIP;
    return MOE_OK;
}

int gemv_tile_m() { return kGemvTM; }

moe_status_t launch_gemv_forward(const moe_ffn_desc_t &ex, const void *x, int act, int K,
                                 const moe_perm_t &p, int max_tiles, void *h, float *y,
                                 hipStream_t s, const std::function<moe_status_t(int)> &mark) {
    const uint16_t *xx = (const uint16_t *)x;
    uint16_t *hh = (uint16_t *)h;
    const bool nv = ex.gate.fmt == MOE_W_NVFP4_G16;
    if (act == MOE_BF16)
        return nv ? gemv_forward_t<MOE_BF16, MOE_W_NVFP4_G16>(ex, xx, K, p, max_tiles, hh, y, s, mark)
                  : gemv_forward_t<MOE_BF16, MOE_W_INT4_G128>(ex, xx, K, p, max_tiles, hh, y, s, mark);
    return nv ? gemv_forward_t<MOE_F16, MOE_W_NVFP4_G16>(ex, xx, K, p, max_tiles, hh, y, s, mark)
              : gemv_forward_t<MOE_F16, MOE_W_INT4_G128>(ex, xx, K, p, max_tiles, hh, y, s, mark);
}

}  // namespace moe
