// Prefill-sized expert FFN: grouped GEMM over expert tiles on CDNA4 MFMA
// (v_mfma_f32_32x32x16_{bf16,f16}).
//
// Work unit = (tile of 64 expert-sorted slots of one expert, block of 128
// output columns); 4 waves, wave w owns 32 columns and all 64 rows (two
// 32x32 accumulator blocks). The activation tile streams through LDS in
// 128-input groups (double buffered, 16-byte chunks XOR-swizzled by row so
// a wave's 16-byte reads hit every bank once). Weights go straight from HBM
// into registers: each lane loads 16 bytes (32 inputs) of its own output
// column per half-group and decodes them into MFMA operands, so every weight
// is read and decoded exactly once per tile.
//
// The MFMA sums over its 16 k-slots in any order, so A and B only have to
// agree on which input each slot holds: lane half h of MFMA (i, j) of a
// group carries inputs 64i + 32h + 8j .. +7, in the pair order the decoder
// produces.
//
// int4: B holds the exact 16-bit values BIAS + q (decode.h); a group's
//   partial sum P = sum (BIAS + q) x is turned into s_g (P - BIAS sum x) and
//   accumulated in float32, with sum x over the group's 128 inputs of each
//   row computed while staging the activations. The bf16 scale is applied
//   exactly once per group in float32.
// NVFP4: B holds e2m1 * e4m3 exactly in 16 bits (<= 6 significant bits);
//   the float32 global scale multiplies the accumulators in the epilogue.
//
//   gate/up pass: h = silu(gate) * up for the wave's 32 columns (both
//                 projections of a column in the same lane: SwiGLU fused);
//   down pass:    y rows in float32 for the combine.
#include <functional>

#include "decode.h"

namespace moe {

constexpr int kGemmThreads = 256;
constexpr int kGemmTM = 64;          // rows per tile
constexpr int kGemmBN = 128;         // output columns per block
constexpr int kGemmKG = 128;         // inputs per staged group
constexpr int kGemmRowBytes = kGemmKG * 2;

struct GemmMat {
    const uint8_t *q, *s;
    const float *gs;
    int64_t qe, qr, se, sr;
};

template <int ACT>
using mfma_op_t = typename std::conditional<ACT == MOE_BF16, bf16x8_t, f16x8_t>::type;

template <int ACT>
__device__ __forceinline__ f32x16_t mfma32(uint4 a, uint4 b, f32x16_t c) {
    if constexpr (ACT == MOE_BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// 16-bit pair of two exact float32 values (their low 16 bits are zero for
// bf16 targets; fp16 targets convert exactly).
template <int ACT>
__device__ __forceinline__ uint32_t pack_exact(float lo, float hi) {
    if constexpr (ACT == MOE_BF16)
        return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
    else
        return (uint32_t)f32_to_f16_bits(lo) | ((uint32_t)f32_to_f16_bits(hi) << 16);
}

// B operand (4 dwords = 8 inputs of one output column) from packed word w.
template <int ACT, int FMT>
__device__ __forceinline__ uint4 decode_b(uint32_t w, float bs) {
    if constexpr (FMT == MOE_W_INT4_G128) {
        uint32_t p[4];
        int4_biased_pairs<ACT>(w, p);
        (void)bs;
        return make_uint4(p[0], p[1], p[2], p[3]);
    } else {
        uint32_t d[4];
        const uint32_t e[4] = {fp4_pair<MOE_BF16, 0>(w), fp4_pair<MOE_BF16, 1>(w),
                               fp4_pair<MOE_BF16, 2>(w), fp4_pair<MOE_BF16, 3>(w)};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float lo = __uint_as_float(e[i] << 16) * bs;
            const float hi = __uint_as_float(e[i] & 0xFFFF0000u) * bs;
            d[i] = pack_exact<ACT>(lo, hi);
        }
        return make_uint4(d[0], d[1], d[2], d[3]);
    }
}

// Staging of one 128-input group of the 64-row activation tile into LDS.
// Thread t moves 16-byte chunks q = t + 256 s (s = 0..3): row q/16, chunk
// q%16; the 16 threads of a row also reduce the row's group sum (int4).
template <int ACT, int FMT>
struct Stager {
    uint4 v[4];
    __device__ __forceinline__ void load(const uint16_t *const *rows, int g) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int q = threadIdx.x + kGemmThreads * s;
            const uint16_t *r = rows[q >> 4];
            v[s] = r ? *(const uint4 *)(r + g * kGemmKG + (q & 15) * 8) : make_uint4(0, 0, 0, 0);
        }
    }
    __device__ __forceinline__ void store(uint8_t *buf, float *xs) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int q = threadIdx.x + kGemmThreads * s;
            const int row = q >> 4, c = q & 15;
            uint4 p = v[s];
            if (FMT == MOE_W_INT4_G128) {          // pairs (i, i+4) of the 8 inputs
                p.x = (v[s].x & 0xFFFFu) | (v[s].z << 16);
                p.y = (v[s].x >> 16) | (v[s].z & 0xFFFF0000u);
                p.z = (v[s].y & 0xFFFFu) | (v[s].w << 16);
                p.w = (v[s].y >> 16) | (v[s].w & 0xFFFF0000u);
            }
            *(uint4 *)(buf + row * kGemmRowBytes + ((c ^ (row & 7)) << 4)) = p;
            if (FMT == MOE_W_INT4_G128) {
                const uint32_t one = ACT == MOE_BF16 ? 0x3F803F80u : 0x3C003C00u;
                float t = 0.0f;
                t = dot2<ACT>(v[s].x, one, t);
                t = dot2<ACT>(v[s].y, one, t);
                t = dot2<ACT>(v[s].z, one, t);
                t = dot2<ACT>(v[s].w, one, t);
#pragma unroll
                for (int m = 8; m >= 1; m >>= 1) t += shfl_xor_f(t, m);
                if (c == 0) xs[row] = t;
            }
        }
    }
};

__device__ __forceinline__ int xcd_remap(int b, int nwg) {
    // Blocks are dispatched round-robin over the 8 XCDs; give each XCD a
    // contiguous range of logical blocks so blocks sharing a tile (and its
    // activation rows) share that XCD's L2.
    const int q = nwg / 8, r = nwg % 8, xcd = b % 8;
    return xcd * q + min(xcd, r) + b / 8;
}

template <int ACT, int FMT, bool GATEUP>
__global__ void __launch_bounds__(kGemmThreads) gemm_kernel(
    GemmMat A, GemmMat Bm, int n_rows, int kin, const uint16_t *__restrict__ xin,
    int x_from_slots, int topk, const int32_t *__restrict__ sorted_slots,
    const int32_t *__restrict__ tile_expert, const int32_t *__restrict__ num_tiles,
    int n_blocks, uint16_t *__restrict__ hout, float *__restrict__ yout) {
    __shared__ __attribute__((aligned(16))) uint8_t abuf[2][kGemmTM * kGemmRowBytes];
    __shared__ float xsum[2][kGemmTM];
    __shared__ const uint16_t *rows[kGemmTM];
    __shared__ int m_sh;

    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int tile = lid / n_blocks, nb = lid - tile * n_blocks;
    if (tile >= num_tiles[0]) return;
    const int e = tile_expert[tile];

    if (threadIdx.x < kGemmTM) {
        const int s = sorted_slots[tile * kGemmTM + threadIdx.x];
        rows[threadIdx.x] = s < 0 ? nullptr
                            : x_from_slots ? xin + (size_t)(s / topk) * kin
                                           : xin + (size_t)(tile * kGemmTM + threadIdx.x) * kin;
        const uint64_t live = __ballot(s >= 0);
        if (threadIdx.x == 0) m_sh = __popcll(live);
    }
    __syncthreads();
    const int m_valid = m_sh;                    // valid rows come first in a tile
    const bool two_mb = m_valid > 32;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int half = lane >> 5, l32 = lane & 31;
    const int col = nb * kGemmBN + wave * 32 + l32;
    const bool col_ok = col < n_rows;
    const int colc = col_ok ? col : 0;
    const uint8_t *qa = A.q + e * A.qe + (int64_t)colc * A.qr;
    const uint8_t *sa = A.s + e * A.se + (int64_t)colc * A.sr;
    const uint8_t *qb = GATEUP ? Bm.q + e * Bm.qe + (int64_t)colc * Bm.qr : nullptr;
    const uint8_t *sb = GATEUP ? Bm.s + e * Bm.se + (int64_t)colc * Bm.sr : nullptr;

    f32x16_t acc_a[2], acc_b[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc_a[mb][v] = acc_b[mb][v] = 0.0f;

    const int ngroups = kin / kGemmKG;
    Stager<ACT, FMT> st;
    st.load(rows, 0);
    st.store(abuf[0], xsum[0]);
    __syncthreads();

    for (int g = 0; g < ngroups; ++g) {
        const int cur = g & 1;
        if (g + 1 < ngroups) st.load(rows, g + 1);
        // weights of this group: two 16-byte loads per matrix
        uint4 wa[2], wb[2];
        float sca = 0.0f, scb = 0.0f;
        float bsa[2][2], bsb[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int64_t off = (int64_t)g * (kGemmKG / 2) + i * 32 + half * 16;
            wa[i] = *(const uint4 *)(qa + off);
            if (GATEUP) wb[i] = *(const uint4 *)(qb + off);
            if (FMT == MOE_W_NVFP4_G16) {
                const int blk = g * 8 + i * 4 + half * 2;
                const uint16_t two = *(const uint16_t *)(sa + blk);
                bsa[i][0] = e4m3_to_f32(two & 0xFF);
                bsa[i][1] = e4m3_to_f32(two >> 8);
                if (GATEUP) {
                    const uint16_t tb = *(const uint16_t *)(sb + blk);
                    bsb[i][0] = e4m3_to_f32(tb & 0xFF);
                    bsb[i][1] = e4m3_to_f32(tb >> 8);
                }
            }
        }
        if (FMT == MOE_W_INT4_G128) {
            sca = bf16_bits_to_f32(*(const uint16_t *)(sa + 2 * g));
            if (GATEUP) scb = bf16_bits_to_f32(*(const uint16_t *)(sb + 2 * g));
        }

        f32x16_t pa[2], pb[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int v = 0; v < 16; ++v) pa[mb][v] = pb[mb][v] = 0.0f;
        const uint8_t *buf = abuf[cur];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t wav[4] = {wa[i].x, wa[i].y, wa[i].z, wa[i].w};
            const uint32_t wbv[4] = {wb[i].x, wb[i].y, wb[i].z, wb[i].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float ba = FMT == MOE_W_NVFP4_G16 ? bsa[i][j >> 1] : 0.0f;
                const uint4 ob = decode_b<ACT, FMT>(wav[j], ba);
                uint4 obb = make_uint4(0, 0, 0, 0);
                if (GATEUP) obb = decode_b<ACT, FMT>(wbv[j], FMT == MOE_W_NVFP4_G16 ? bsb[i][j >> 1] : 0.0f);
                const int chunk = i * 8 + half * 4 + j;
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) {
                    if (mb == 1 && !two_mb) break;
                    const int row = mb * 32 + l32;
                    const uint4 av = *(const uint4 *)(buf + row * kGemmRowBytes +
                                                      ((chunk ^ (row & 7)) << 4));
                    if (FMT == MOE_W_INT4_G128) {
                        pa[mb] = mfma32<ACT>(av, ob, pa[mb]);
                        if (GATEUP) pb[mb] = mfma32<ACT>(av, obb, pb[mb]);
                    } else {
                        acc_a[mb] = mfma32<ACT>(av, ob, acc_a[mb]);
                        if (GATEUP) acc_b[mb] = mfma32<ACT>(av, obb, acc_b[mb]);
                    }
                }
            }
        }
        if (FMT == MOE_W_INT4_G128) {
            constexpr float bias = Int4Bias<ACT>::kBias;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                if (mb == 1 && !two_mb) break;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int m = mb * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
                    const float c = bias * xsum[cur][m];
                    acc_a[mb][v] = __builtin_fmaf(sca, pa[mb][v] - c, acc_a[mb][v]);
                    if (GATEUP) acc_b[mb][v] = __builtin_fmaf(scb, pb[mb][v] - c, acc_b[mb][v]);
                }
            }
        }
        if (g + 1 < ngroups) st.store(abuf[cur ^ 1], xsum[cur ^ 1]);
        __syncthreads();
    }

    if (!col_ok) return;
    float ga = 1.0f, gb = 1.0f;
    if (FMT == MOE_W_NVFP4_G16) {
        ga = A.gs[e];
        if (GATEUP) gb = Bm.gs[e];
    }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int m = mb * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
            if (m >= m_valid) continue;
            const size_t r = (size_t)tile * kGemmTM + m;
            if (GATEUP)
                hout[r * n_rows + col] = f32_to_act<ACT>(silu_mul(acc_a[mb][v] * ga,
                                                                  acc_b[mb][v] * gb));
            else
                yout[r * n_rows + col] = acc_a[mb][v] * ga;
        }
    }
}

inline GemmMat gemm_mat(const moe_weight_desc_t &d) {
    return GemmMat{(const uint8_t *)d.qweight, (const uint8_t *)d.scale, d.global_scale,
                   d.qweight_expert_stride, d.qweight_row_stride, d.scale_expert_stride,
                   d.scale_row_stride};
}

template <int ACT, int FMT>
moe_status_t gemm_forward_t(const moe_ffn_desc_t &ex, const uint16_t *x, int K,
                            const moe_perm_t &p, int max_tiles, uint16_t *h, float *y,
                            hipStream_t s, const std::function<moe_status_t(int)> &mark) {
    const int F = ex.gate.n, H = ex.gate.k;
    {
        const int nbk = (F + kGemmBN - 1) / kGemmBN;
        hipLaunchKernelGGL((gemm_kernel<ACT, FMT, true>), dim3(max_tiles * nbk),
                           dim3(kGemmThreads), 0, s, gemm_mat(ex.gate), gemm_mat(ex.up), F, H, x,
                           1, K, p.sorted_slots, p.tile_expert, p.num_tiles, nbk, h, nullptr);
        MOE_LAUNCH_CHECK();
    }
    if (mark && mark(1) != MOE_OK) return MOE_ERR_HIP;
    {
        const int nbk = (H + kGemmBN - 1) / kGemmBN;
        hipLaunchKernelGGL((gemm_kernel<ACT, FMT, false>), dim3(max_tiles * nbk),
                           dim3(kGemmThreads), 0, s, gemm_mat(ex.down), gemm_mat(ex.down), H, F,
                           h, 0, K, p.sorted_slots, p.tile_expert, p.num_tiles, nbk, nullptr, y);
        MOE_LAUNCH_CHECK();
    }
    if (mark && mark(2) != MOE_OK) return MOE_ERR_HIP;
    return MOE_OK;
}

int gemm_tile_m() { return kGemmTM; }
int gemm_group() { return kGemmKG; }

moe_status_t launch_gemm_forward(const moe_ffn_desc_t &ex, const void *x, int act, int K,
                                 const moe_perm_t &p, int max_tiles, void *h, float *y,
                                 hipStream_t s, const std::function<moe_status_t(int)> &mark) {
    const uint16_t *xx = (const uint16_t *)x;
    uint16_t *hh = (uint16_t *)h;
    const bool nv = ex.gate.fmt == MOE_W_NVFP4_G16;
    if (act == MOE_BF16)
        return nv ? gemm_forward_t<MOE_BF16, MOE_W_NVFP4_G16>(ex, xx, K, p, max_tiles, hh, y, s, mark)
                  : gemm_forward_t<MOE_BF16, MOE_W_INT4_G128>(ex, xx, K, p, max_tiles, hh, y, s, mark);
    return nv ? gemm_forward_t<MOE_F16, MOE_W_NVFP4_G16>(ex, xx, K, p, max_tiles, hh, y, s, mark)
              : gemm_forward_t<MOE_F16, MOE_W_INT4_G128>(ex, xx, K, p, max_tiles, hh, y, s, mark);
}

}  // namespace moe
