// Decode-sized expert FFN on the matrix cores: a dequantizing GEMV whose
// contraction over the tile's slots runs on v_mfma_f32_16x16x32_{f16,bf16}
// (int4 with one bf16 scale per 128 inputs, symmetric and asymmetric).
//
// Work unit = (tile of up to TM slots of one expert, a block of rows). A
// wave owns 16 rows at a time, and with KS > 1 only the KS-th part of their
// inputs (the KS waves of a row block meet in LDS at the end: small batches
// have few tiles, and this gives them more waves). Step j covers inputs
// 128 j .. 128 j + 127 of the 16 rows, one scale group. The 16 rows x 64
// bytes of a step are loaded four lanes per row (lane 4 r + c: row r, bytes
// 16 c ..), passed through a per-wave LDS tile into the MFMA layout (lane
// 16 c + r: row r, bytes 16 c ..; loaded that way directly, every 16 lanes
// would touch 16 cache lines and the vector L1 stalls the address unit),
// and each of the lane's four words becomes the eight exact 16-bit values
// BIAS + q (decode.h), the B operand (inputs x rows) of one MFMA whose A
// operand (slots x inputs) holds the same eight inputs of the tile's slots,
// staged in LDS. The four MFMAs of a step sum the group; its scale and the
// bias then apply per output in float32,
//
//   acc[s][r] += scale[r][j] * (t[s][r] - bias * sum_{k in group j} x[s][k]),
//
// where the MFMA output layout gives lane 16 c + r the slots 4 c + i (i < 4)
// of row r. The block's scales (and zero points) are loaded once per block,
// coalesced, and each step's value moves to its MFMA lanes by ds_bpermute.
// The MFMA adds exact products (two 16-bit values) in float32; next to the
// lane-serial dot2 GEMV only the order of the additions inside a group
// differs.
//
// fp16, signed int4: as in the dot2 GEMV, the odd pairs decode in place to
// 1152 + 16 q (mantissa bits 4..7 of 1024.0) against inputs staged times
// 1/16, and the staged group sum carries both biases, 1032 sum(x even) +
// 72 sum(x odd).
//
// NVFP4 (E2M1 codes, one E4M3 scale per 16 inputs, a float32 scale per
// expert): every MFMA spans four 16-input blocks, so the block scale goes
// into the operand. The scaled pair conversion gives 256 e2m1 exactly in
// fp16 (its scale is a power of two), and one packed fp16 multiply by the
// scale's bits moved into an fp16 (b / 256, subnormal for the smaller
// scales) leaves e2m1 x E4M3, at most 6 significant bits inside fp16's
// normal range: exact. The MFMA runs in fp16 for both activation types: bf16
// inputs are staged as fp16 x 2^-p with p per staged row from its largest
// magnitude (largest < 2^15 after the shift), exact for every element within
// 2^29 of that largest, and the epilogue multiplies by the global and input
// scales, then by 2^p. The rows are staged in input order, the MFMAs add
// into the accumulators directly (no group rescale), and a step's block
// scales travel with its weights (two bytes per loading lane, moved to the
// MFMA lanes by ds_bpermute).
//
// A tile's padding slots (t >= m) are neither staged nor stored: the rows
// of an MFMA result are independent, so whatever their LDS rows hold only
// reaches outputs that are dropped.
#include <functional>

#include "decode.h"
#include "stream.h"

namespace moe {

constexpr int kMxWaves = 4, kMxThreads = kMxWaves * kWave;

template <int ACT>
__device__ __forceinline__ f32x4_t mfma16(uint4 a, uint4 b, f32x4_t c) {
    if constexpr (ACT == MOE_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// LDS units (16 bytes = 8 inputs) per staged row, one more than the row
// needs: the copies of one unit in consecutive slots then sit 16 bytes
// apart in the bank cycle, and a wave-wide read of a unit across 16 slots
// touches every bank once.
__host__ __device__ constexpr int mx_upad(int kin) { return kin / 8 + 1; }

// Staged rows, the group sums [group][16 slots] (float32), one 16-row x
// 64-byte weight tile per wave, with KS > 1 the partial sums [wave]
// [matrix][lane] (float32 x 4), and for NVFP4 the staging exponents (per
// slot: the waves' largest magnitudes, then p).
constexpr int kMxF4Bytes = 16 * (kMxWaves + 1) * 4;
inline size_t gemv_mx_lds_bytes(int tm, int kin, int ks, int nm, bool f4) {
    return (size_t)tm * mx_upad(kin) * 16 + (size_t)(kin / 128) * 16 * sizeof(float) +
           (size_t)kMxWaves * 1024 + (ks > 1 ? (size_t)kMxWaves * nm * kWave * 16 : 0) +
           (f4 ? kMxF4Bytes : 0);
}

template <int ACT, int FMT>
__host__ __device__ constexpr bool mx_x16() {
    return ACT == MOE_F16 && FMT == MOE_W_INT4_G128;
}

// Word d of NVFP4 codes (inputs 0..7 in order) as the fp16 pairs e2m1 x
// E4M3: sp holds the block scale as fp16 bits of b / 256 in both halves.
__device__ __forceinline__ uint4 mx_decode_f4(uint32_t d, uint32_t sp) {
    const half2_t s2 = __builtin_bit_cast(half2_t, sp);
    auto mul = [&](half2_t v) { return __builtin_bit_cast(uint32_t, v * s2); };
    return make_uint4(mul(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 256.0f, 0)),
                      mul(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 256.0f, 1)),
                      mul(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 256.0f, 2)),
                      mul(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 256.0f, 3)));
}

// E4M3 byte b as the fp16 bits of b / 256 (exponent and mantissa fields
// moved up by 7 bits, which also maps its subnormals onto fp16's), in both
// halves of a word.
__device__ __forceinline__ uint32_t e4m3_f16_pair(uint32_t b) {
    const uint32_t h = ((b & 0x7Fu) << 7) | ((b & 0x80u) << 8);
    return h | (h << 16);
}

// The four pairs (inputs i, i + 4 of the word, i < 4) of word d as BIAS + q
// (signed) or MAGIC + q (asymmetric); X16: pairs 1 and 3 in place.
template <bool X16>
__device__ __forceinline__ uint4 mx_decode(uint32_t d, uint32_t kv, uint32_t kv1) {
    if constexpr (X16) {
        const uint32_t d8 = d >> 8;
        return make_uint4((d & 0x000F000Fu) ^ kv, (d & 0x00F000F0u) ^ kv1,
                          (d8 & 0x000F000Fu) ^ kv, (d8 & 0x00F000F0u) ^ kv1);
    } else {
        return make_uint4((d & 0x000F000Fu) ^ kv, ((d >> 4) & 0x000F000Fu) ^ kv,
                          ((d >> 8) & 0x000F000Fu) ^ kv, ((d >> 12) & 0x000F000Fu) ^ kv);
    }
}

// NS steps of 128 inputs per row (kin = 128 NS); RP row blocks per wave in
// turn; KS waves per row block, each over NS / KS consecutive steps; R
// steps in flight per lane and matrix.
template <int ACT, int FMT, int TM, bool GATEUP, int NS, int RP, int KS, int R>
__global__ void __launch_bounds__(kMxThreads) gemv_mx_kernel(
    GemvMat A, GemvMat B, int n_rows, const uint16_t *__restrict__ xin, int x_from_slots,
    int topk, const int32_t *__restrict__ sorted_slots, const int32_t *__restrict__ tile_expert,
    const int32_t *__restrict__ num_tiles, uint16_t *__restrict__ hout,
    float *__restrict__ yout) {
    static_assert(TM == 4 || TM == 8 || TM == 16, "tile rows: a power of two up to 16");
    constexpr int kin = NS * 128, UPAD = mx_upad(kin), UNITS = kin / 8;
    constexpr int SPT = (UNITS + kMxThreads - 1) / kMxThreads;   // staged units per thread and slot
    constexpr int NSW = NS / KS, BPW = kMxWaves / KS;            // steps per wave, blocks per pass
    static_assert(UNITS % 16 == 0 && kMxWaves % KS == 0 && NS % KS == 0 && NSW % R == 0,
                  "whole groups, wave parts and ring trips");
    constexpr bool kZ = int4_asym(FMT), X16 = mx_x16<ACT, FMT>();
    constexpr bool kF4 = FMT == MOE_W_NVFP4_G16;
    constexpr int NM = GATEUP ? 2 : 1;           // matrices streamed side by side
    // one matrix: odd ring slots refill themselves and the slot before, so
    // both halves of a 128-byte row line are asked for together (two
    // matrices already ask for two lines per step)
    constexpr bool kPair = NM == 1 && R % 2 == 0;
    // per block and lane, dwords of the block's scales (16 bytes of each row
    // per dword index) and zero points
    constexpr int SL = (2 * NS + 15) / 16, ZL = (NS + 15) / 16;
    extern __shared__ uint4 smem[];
    const int tile = blockIdx.y;
    if (tile >= num_tiles[0]) return;
    const int e = tile_expert[tile];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
    const int kp = wave % KS, wb = wave / KS;    // input part, row block of the wave
    const int j_lo = kp * NSW;                   // the wave's first step
    const int r16 = lane & 15, g = lane >> 4;    // MFMA roles: row / slot, input slice
    const int lr = lane >> 2, lc = lane & 3;     // load roles: row, 16-byte chunk of a step
    int m = 0;                                   // the tile's real rows (slots are -1 past them)
    int tok[TM];                                 // and their input rows
#pragma unroll
    for (int t = 0; t < TM; ++t) {
        const int sl = sorted_slots[tile * TM + t];
        if (sl >= 0) m = t + 1;
        tok[t] = x_from_slots ? (sl >= 0 ? sl / topk : 0) : tile * TM + t;
    }

    uint4 *xs = smem;
    float *xb = (float *)(smem + TM * UPAD);
    uint4 *wt = smem + TM * UPAD + NS * 4 + wave * 64;   // this wave's 16 x 64-byte tile
    f32x4_t *red = (f32x4_t *)(smem + TM * UPAD + NS * 4 + kMxWaves * 64);
    // NVFP4: [slot][wave] largest magnitudes, then [slot] staging exponents
    float *f4m = (float *)(red + (KS > 1 ? kMxWaves * NM * kWave : 0));
    int *f4e = (int *)(f4m + 16 * kMxWaves);
    // NVFP4: the expert's global scale with the input scale, per matrix
    const float ca = kF4 ? A.gs[e] * A.xs : 1.0f, cb = kF4 ? B.gs[e] * B.xs : 1.0f;

    // ---- activation staging: every thread, units t + 256 i of each slot ----
    // (the first four slots' loads go out before the weights')
    u32x4_t xv[4][SPT];
    auto xload = [&](int t, int q) {
        const uint16_t *xr = xin + (size_t)tok[t] * kin;
#pragma unroll
        for (int i = 0; i < SPT; ++i) {
            const int u = threadIdx.x + kMxThreads * i;
            xv[q][i] = *(const u32x4_t *)(xr + 8 * (u < UNITS ? u : 0));   // past the row: unused
        }
    };
#pragma unroll
    for (int q = 0; q < 4 && q < TM; ++q)
        if (q < m) xload(q, q);

    // ---- weight ring ------------------------------------------------------
    // row block of pass p; a lane loads row lr of it, chunk lc of each step
    auto block_of = [&](int p) { return ((blockIdx.x * RP + p) * BPW + wb) * 16; };
    const GemvMat *mats[2] = {&A, &B};
    __amdgpu_buffer_rsrc_t rq[NM], rs[NM], rz[NM];
    int q0[NM], s0[NM], z0[NM], qp[NM], sp[NM], zp[NM], f0[NM];
#pragma unroll
    for (int k = 0; k < NM; ++k) {
        const GemvMat &M = *mats[k];
        rq[k] = buffer_rsrc(M.q + e * M.qe, (int64_t)n_rows * M.qr);
        rs[k] = buffer_rsrc(M.s + e * M.se, (int64_t)n_rows * M.sr);
        rz[k] = buffer_rsrc(kZ ? M.z + e * M.ze : M.q, (int64_t)n_rows * M.zr);
        const int row = block_of(0) + lr;
        q0[k] = row * (int)M.qr + 16 * lc;
        s0[k] = row * (int)M.sr + 4 * lc;
        z0[k] = row * (int)M.zr + 4 * lc;
        qp[k] = 16 * BPW * (int)M.qr;            // the next pass's block
        sp[k] = 16 * BPW * (int)M.sr;
        zp[k] = 16 * BPW * (int)M.zr;
        // NVFP4: a step's eight block scales of row lr, two bytes per lane
        // of the row (blocks 2 lc, 2 lc + 1; 4 rows per 16 lanes, as the
        // weights), passed to the MFMA lanes by ds_bpermute
        f0[k] = row * (int)M.sr + 2 * lc;
    }
    u32x4_t w[R][NM];
    uint32_t wsc[R][NM];
    // step j of pass p into ring slot `slot`; every call issues the same
    // loads, so the compiler's waits count exactly the younger steps
    auto load = [&](int slot, int p, int j) {
#pragma unroll
        for (int k = 0; k < NM; ++k) {
            w[slot][k] = __builtin_bit_cast(
                u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq[k], q0[k] + p * qp[k] + 64 * j, 0, 0));
            if constexpr (kF4)
                wsc[slot][k] = __builtin_amdgcn_raw_buffer_load_b16(rs[k], f0[k] + p * sp[k] + 8 * j, 0, 0);
        }
    };
    // the block's scales (and zero points) of pass p, as loaded: lane 4 r + c
    // holds bytes 16 i + 4 c .. + 3 of row r, i < SL (ZL); bytes past a
    // row's end are never used (past the matrix they read zero)
    uint32_t sreg[NM][SL], zreg[NM][kZ ? ZL : 1];
    auto load_scales = [&](int p) {
        if constexpr (kF4) return;               // NVFP4: with the weights
#pragma unroll
        for (int k = 0; k < NM; ++k) {
#pragma unroll
            for (int i = 0; i < SL; ++i)
                sreg[k][i] = __builtin_amdgcn_raw_buffer_load_b32(rs[k], s0[k] + p * sp[k] + 16 * i, 0, 0);
            if constexpr (kZ) {
#pragma unroll
                for (int i = 0; i < ZL; ++i)
                    zreg[k][i] =
                        __builtin_amdgcn_raw_buffer_load_b32(rz[k], z0[k] + p * zp[k] + 16 * i, 0, 0);
            }
        }
    };
    load_scales(0);
#pragma unroll
    for (int j = 0; j < R; ++j) load(j, 0, j_lo + j);
    // keep every load above in flight before the staging arithmetic starts
    __builtin_amdgcn_sched_barrier(0);

    // ---- activations into LDS: pair order of the decoder, group sums -------
    int pe[4] = {0, 0, 0, 0};                    // NVFP4, bf16: the batch's exponents p
    auto xstage = [&](int t, int q) {
        if constexpr (kF4) {                     // input order; bf16 as fp16 x 2^-p
#pragma unroll
            for (int i = 0; i < SPT; ++i) {
                const u32x4_t v = xv[q][i];
                const int u = threadIdx.x + kMxThreads * i;
                uint32_t o[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    if constexpr (ACT == MOE_BF16) {
                        const uint32_t lo = f32_to_f16_bits(
                            __builtin_amdgcn_ldexpf(bf16_bits_to_f32(v[c] & 0xFFFFu), -pe[q]));
                        const uint32_t hi = f32_to_f16_bits(
                            __builtin_amdgcn_ldexpf(bf16_bits_to_f32(v[c] >> 16), -pe[q]));
                        o[c] = lo | (hi << 16);
                    } else {
                        o[c] = v[c];
                    }
                }
                if (u < UNITS) xs[t * UPAD + u] = make_uint4(o[0], o[1], o[2], o[3]);
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < SPT; ++i) {
            const u32x4_t v = xv[q][i];
            const int u = threadIdx.x + kMxThreads * i;   // unit: inputs 8u .. 8u + 7
            const bool valid = u < UNITS;                 // uniform over 16 lanes
            uint4 pr;                                     // pairs (i, i + 4) of the 8 inputs
            pr.x = (v.x & 0xFFFFu) | (v.z << 16);
            pr.y = (v.x >> 16) | (v.z & 0xFFFF0000u);
            pr.z = (v.y & 0xFFFFu) | (v.w << 16);
            pr.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
            if constexpr (X16) {                 // the odd inputs' pairs, times 1/16
                const half2_t r16v = {(_Float16)0.0625f, (_Float16)0.0625f};
                pr.y = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, pr.y) * r16v);
                pr.w = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, pr.w) * r16v);
            }
            if (valid) xs[t * UPAD + u] = pr;
            const uint32_t d[4] = {v.x, v.y, v.z, v.w};
            float sum;
            if constexpr (X16) {                 // 1032 sum(x even) + 72 sum(x odd)
                float se = 0.0f, so = 0.0f;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    se += act_to_f32<ACT>(d[c] & 0xFFFF);
                    so += act_to_f32<ACT>(d[c] >> 16);
                }
                sum = __builtin_fmaf(1032.0f, se, 72.0f * so);
            } else {
                sum = 0.0f;
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    sum += act_to_f32<ACT>(d[c] & 0xFFFF) + act_to_f32<ACT>(d[c] >> 16);
            }
            // the 16 units of a group sit in 16 consecutive lanes
            sum += shfl_xor_f(sum, 1);
            sum += shfl_xor_f(sum, 2);
            sum += shfl_xor_f(sum, 4);
            sum += shfl_xor_f(sum, 8);
            if (valid && r16 == 0) xb[(u >> 4) * 16 + t] = sum;
        }
    };
    // NVFP4 with bf16 inputs: p of the staged rows t0 .. t0 + 3 (those below
    // m) from their largest magnitude, so that it stays below 2^15 in fp16
    // (m is uniform over the work group: every thread takes the barrier)
    auto f4_exps = [&](int t0) {
        if constexpr (kF4 && ACT == MOE_BF16) {
            float mx[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                mx[q] = 0.0f;
                if (t0 + q < m) {
#pragma unroll
                    for (int i = 0; i < SPT; ++i) {
                        const u32x4_t v = xv[q][i];      // past the row: its unit 0
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            mx[q] = fmaxf(mx[q], fmaxf(fabsf(bf16_bits_to_f32(v[c] & 0xFFFFu)),
                                                       fabsf(bf16_bits_to_f32(v[c] >> 16))));
                    }
                }
#pragma unroll
                for (int o = 1; o < kWave; o <<= 1) mx[q] = fmaxf(mx[q], shfl_xor_f(mx[q], o));
            }
            if (lane == 0) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (t0 + q < m) f4m[(t0 + q) * kMxWaves + wave] = mx[q];
            }
            lds_barrier();
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                pe[q] = 0;
                if (t0 + q < m) {
                    float v = 0.0f;
#pragma unroll
                    for (int w2 = 0; w2 < kMxWaves; ++w2) v = fmaxf(v, f4m[(t0 + q) * kMxWaves + w2]);
                    // largest in [2^E, 2^(E+1)) -> p = E - 14; a zero row keeps p = 0
                    const int eb = (int)((__float_as_uint(v) >> 23) & 0xFFu);
                    pe[q] = v > 0.0f ? eb - 127 - 14 : 0;
                    if (threadIdx.x == 0) f4e[t0 + q] = pe[q];
                }
            }
        }
    };
    f4_exps(0);
#pragma unroll
    for (int q = 0; q < 4 && q < TM; ++q)
        if (q < m) xstage(q, q);
    for (int t0 = 4; t0 < m; t0 += 4) {          // tiles of more than 4 rows
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (t0 + q < m) xload(t0 + q, q);
        f4_exps(t0);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (t0 + q < m) xstage(t0 + q, q);
    }
    lds_barrier();

    // ---- main loop ----------------------------------------------------------
    const uint32_t kv = in_vgpr(int4_key<ACT, FMT>());
    const uint32_t kv1 = in_vgpr(X16 ? 0x64806480u : 0u);
    // the A operand's slot: lanes past the tile's rows read a staged row's
    // copy (their outputs are not stored)
    const int xa0 = (r16 & (TM - 1)) * UPAD + 4 * g;
    // the weight tile: chunk c of row r at unit 4 r + (c ^ (r / 4 % 4)); the
    // load lanes' stores and the MFMA lanes' reads then both touch every bank
    // once per 16 lanes
    uint4 *const wt_st = wt + 4 * lr + (lc ^ ((lr >> 2) & 3));
    const uint4 *const wt_ld = wt + 4 * r16 + (g ^ ((r16 >> 2) & 3));
    f32x4_t acc[NM];
#pragma unroll
    for (int k = 0; k < NM; ++k) acc[k] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    auto finish = [&](int p) {
        if constexpr (KS > 1) {
            // the row block's other parts add to part 0 in the order of
            // their inputs
            if (kp != 0) {
#pragma unroll
                for (int k = 0; k < NM; ++k) red[(wave * NM + k) * kWave + lane] = acc[k];
            }
            lds_barrier();
            if (kp == 0) {
#pragma unroll
                for (int q = 1; q < KS; ++q) {
#pragma unroll
                    for (int k = 0; k < NM; ++k) {
                        const f32x4_t o = red[((wave + q) * NM + k) * kWave + lane];
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[k][i] += o[i];
                    }
                }
            }
        }
        const int row = block_of(p) + r16;
        if (kp == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int s = 4 * g + i;
                if (s < m) {
                    const size_t r = (size_t)tile * TM + s;
                    float v0 = acc[0][i], v1 = acc[NM - 1][i];
                    if constexpr (kF4) {
                        // global and input scales first, then 2^p: a sum of
                        // staged (< 2^15) inputs may exceed float32 once
                        // shifted back, the scaled value may not
                        const int pp = ACT == MOE_BF16 ? f4e[s] : 0;
                        v0 = __builtin_amdgcn_ldexpf(v0 * ca, pp);
                        v1 = __builtin_amdgcn_ldexpf(v1 * cb, pp);
                    }
                    if constexpr (GATEUP)
                        hout[r * n_rows + row] = f32_to_act<ACT>(silu_mul(v0, v1));
                    else
                        yout[r * n_rows + row] = v0;
                }
            }
        }
#pragma unroll
        for (int k = 0; k < NM; ++k) acc[k] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        if (KS > 1 && p + 1 < RP) lds_barrier();   // the partial sums' area is reused
    };
    constexpr float kBias = X16 ? 1.0f : Int4Bias<ACT>::kBias;
    const int src_s = 4 * (4 * r16);             // bpermute byte address of lane 4 r16
    // consume ring slot `slot` (step j of the current pass); REFILL: then
    // load step jr of pass pr into it (kPair: odd slots refill themselves and
    // the slot before, with step jr2 of pass pr2)
    auto step = [&](int slot, int j, bool refill, int pr, int jr, int pr2, int jr2) {
        uint4 d[NM][4];
        float sc[NM], bi[NM];
#pragma unroll
        for (int k = 0; k < NM; ++k) {
            // through the wave's tile into the MFMA layout: row r16, chunk g
            *wt_st = __builtin_bit_cast(uint4, w[slot][k]);
            const uint4 wv = *wt_ld;
            if constexpr (kF4) {
                // words 0, 1: block 2 g of the step; words 2, 3: block 2 g + 1,
                // loaded by lane 4 r16 + g
                const uint32_t sb =
                    (uint32_t)__builtin_amdgcn_ds_bpermute(src_s + 4 * g, (int)wsc[slot][k]);
                const uint32_t s0p = e4m3_f16_pair(sb & 0xFFu), s1p = e4m3_f16_pair(sb >> 8);
#pragma unroll
                for (int q = 0; q < 4; ++q) d[k][q] = mx_decode_f4((&wv.x)[q], q < 2 ? s0p : s1p);
                sc[k] = 1.0f;
                bi[k] = 0.0f;
                continue;
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) d[k][q] = mx_decode<X16>((&wv.x)[q], kv, kv1);
            // scale of (row r16, group j): bytes 2j of the row, held by lane
            // 4 r16 + (j % 8) / 2, dword j / 8
            const uint32_t sv = (uint32_t)__builtin_amdgcn_ds_bpermute(
                src_s + 4 * ((j % 8) >> 1), (int)sreg[k][j / 8]);
            sc[k] = __uint_as_float((j & 1) ? (sv & 0xFFFF0000u) : (sv << 16));
            if constexpr (kZ) {
                const uint32_t zv = (uint32_t)__builtin_amdgcn_ds_bpermute(
                    src_s + 4 * ((j % 16) >> 2), (int)zreg[k][j / 16]);
                bi[k] = Int4Bias<ACT>::kMagicValue + (float)((zv >> (8 * (j & 3))) & 0xFFu);
            } else {
                bi[k] = kBias;
            }
        }
        // slot consumed: refill it in place (the barrier keeps the refill
        // below the last use, so it reuses the same registers)
        __builtin_amdgcn_sched_barrier(0);
        if (refill) {
            if constexpr (kPair) {
                if (slot & 1) {
                    load(slot - 1, pr2, jr2);
                    load(slot, pr, jr);
                }
            } else {
                load(slot, pr, jr);
            }
        }
        const uint4 *xa = xs + xa0 + 16 * j;
        if constexpr (kF4) {                     // no group rescale: into the accumulators
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint4 x = xa[q];
#pragma unroll
                for (int k = 0; k < NM; ++k) acc[k] = mfma16<MOE_F16>(x, d[k][q], acc[k]);
            }
            return;
        }
        const f32x4_t xsum = *(const f32x4_t *)(xb + j * 16 + 4 * g);
        f32x4_t t[NM];
#pragma unroll
        for (int k = 0; k < NM; ++k) t[k] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 x = xa[q];
#pragma unroll
            for (int k = 0; k < NM; ++k) t[k] = mfma16<ACT>(x, d[k][q], t[k]);
        }
#pragma unroll
        for (int k = 0; k < NM; ++k) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[k][i] = __builtin_fmaf(sc[k], __builtin_fmaf(-bi[k], xsum[i], t[k][i]), acc[k][i]);
            // the rescale happens here, not sunk to the end of the unrolled
            // loop (that keeps every step's MFMA result and sums alive)
            asm volatile("" : "+v"(acc[k]));
        }
    };
    // Per pass the ring trips whose every step refills its slot, the last
    // pass's last trip (peeled) refilling nothing; a pass's stores, and the
    // next pass's scale loads, sit between them. i: the wave's step index.
#pragma unroll
    for (int p = 0; p < RP; ++p) {
        const bool last = p == RP - 1;
        const int trips = NSW / R - (last ? 1 : 0);
#pragma unroll
        for (int i0 = 0; i0 < trips * R; i0 += R) {
#pragma unroll
            for (int slot = 0; slot < R; ++slot) {
                const int i = i0 + slot;
                const bool next = i + R >= NSW;          // the refill starts the next pass
                const bool next2 = i - 1 + R >= NSW;
                step(slot, j_lo + i, true, next ? p + 1 : p,
                     j_lo + (next ? i + R - NSW : i + R), next2 ? p + 1 : p,
                     j_lo + (next2 ? i - 1 + R - NSW : i - 1 + R));
            }
        }
        if (last) {
#pragma unroll
            for (int slot = 0; slot < R; ++slot)
                step(slot, j_lo + NSW - R + slot, false, 0, 0, 0, 0);
        }
        finish(p);
        if (!last) load_scales(p + 1);
    }
}

// The layer's shapes only (4096 inputs to the gate/up pass, 1536 to the
// down pass, both row counts multiples of the work group's rows), with the
// weights 16-byte and the scales and zero points 4-byte aligned (the
// kernel's loads); other shapes, formats and layouts run the dot2 GEMV.
static bool mx_layout_ok(const moe_weight_desc_t &d) {
    auto al = [](const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; };
    if (d.fmt == MOE_W_NVFP4_G16)                // 2-byte scale loads, a global scale
        return al(d.qweight, 16) && d.qweight_row_stride % 16 == 0 &&
               d.qweight_expert_stride % 16 == 0 && al(d.scale, 2) && d.scale_row_stride % 2 == 0 &&
               d.scale_expert_stride % 2 == 0 && d.global_scale &&
               (int64_t)d.n * d.qweight_row_stride < INT32_MAX &&
               (int64_t)d.n * d.scale_row_stride < INT32_MAX;
    const bool z = d.fmt != MOE_W_INT4_G128_ASYM ||
                   (al(d.zero_point, 4) && d.zero_point_row_stride % 4 == 0 &&
                    d.zero_point_expert_stride % 4 == 0 &&
                    (int64_t)d.n * d.zero_point_row_stride < INT32_MAX);
    return al(d.qweight, 16) && d.qweight_row_stride % 16 == 0 &&
           d.qweight_expert_stride % 16 == 0 && al(d.scale, 4) && d.scale_row_stride % 4 == 0 &&
           d.scale_expert_stride % 4 == 0 && (int64_t)d.n * d.qweight_row_stride < INT32_MAX &&
           (int64_t)d.n * d.scale_row_stride < INT32_MAX && z;
}

// NVFP4 banks take this kernel only for T*K in [4E, 8E) (176 to 351 tokens
// at top-8 of 352), with 8-slot tiles. Below, the dot2 GEMV is faster: its
// decode is one conversion per pair, where exact fp16 operands need a
// conversion and a multiply, and that makes this kernel's gate/up pass
// issue-bound (same host: T=1 40.5 against 39.5 us per step, T=8 170 against
// 142, T=64 617 against 578). From 4E slots the dot2 GEMV's 4-slot tiles
// re-read experts and the 64-row GEMM tiles run mostly empty: at T=256 this
// kernel took 0.960 ms per step against the GEMM's 1.125 (16-slot tiles:
// 1.096), at T=512 1.376 against 1.148.
// int4-g128 (both forms) takes it at every batch below T*K = 7E, the band
// from 4E included: at T=200 / 256 0.741 / 0.795 ms per step against the
// GEMM's 0.876 / 0.887 (fp16; bf16 T=256 0.826 against 0.898, asymmetric
// 0.823 against 0.968), at T=336 (7.6E) 0.936 against 0.915.
bool gemv_mx_supported(const moe_ffn_desc_t &ex, int act, int T, int K) {
    const int f = ex.gate.fmt;
    const int64_t n = (int64_t)T * K, E = ex.gate.num_experts;
    if (f == MOE_W_NVFP4_G16 && n < 4 * E) return false;
    if (n >= (f == MOE_W_NVFP4_G16 ? 8 : 7) * E) return false;
    return (act == MOE_F16 || act == MOE_BF16) &&
           (f == MOE_W_INT4_G128 || f == MOE_W_INT4_G128_ASYM || f == MOE_W_NVFP4_G16) &&
           ex.gate.k == 4096 &&
           ex.gate.n == 1536 && ex.down.k == 1536 && ex.down.n == 4096 &&
           mx_layout_ok(ex.gate) && mx_layout_ok(ex.up) && mx_layout_ok(ex.down);
}

// Slots per tile: 8 for 5 to 32 tokens and from T*K = 4E, else
// 4. The plan sees the batch
// size but not the routing. Measured (bench, graph replay, same host):
// 8-slot tiles took the Zipf-routed 8-layer stack at T=32 from 1.33-1.35
// to 1.22-1.25 ms per step (a hot expert re-streams its weights once per
// tile), and uniform decode at T=8, 16 and 32 within 1 % either way; but
// uniform decode at T=64 from 488 to 508 us (twice the staged activations
// halve the work groups per CU) and at T=1 from 34.3 to 36.5 us. Up to 4
// tokens no expert holds more than 4 slots unless a token repeats an id.
// 16 slots were slower for both.
int gemv_mx_tile_m(int T, int K, int E) {
    return (T > 4 && T <= 32) || (int64_t)T * K >= 4 * (int64_t)E ? 8 : 4;
}
constexpr int kMxDeepTiles = 300;

template <int ACT, int FMT, int TM, bool GATEUP, int NS, int RP, int KS, int R>
moe_status_t launch_mx(const GemvMat &a, const GemvMat &b, int n_rows, const uint16_t *x,
                       int K, const moe_perm_t &p, int max_tiles, uint16_t *h, float *y,
                       hipStream_t s) {
    const size_t lds = gemv_mx_lds_bytes(TM, NS * 128, KS, GATEUP ? 2 : 1, FMT == MOE_W_NVFP4_G16);
    auto k = gemv_mx_kernel<ACT, FMT, TM, GATEUP, NS, RP, KS, R>;
    allow_lds(k, lds);
    const int rows_per_group = 16 * (kMxWaves / KS) * RP;
    hipLaunchKernelGGL(k, dim3(n_rows / rows_per_group, max_tiles), dim3(kMxThreads), lds, s, a, b,
                       n_rows, x, GATEUP ? 1 : 0, K, p.sorted_slots, p.tile_expert, p.num_tiles,
                       h, y);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

// Few tiles (small batches) split each row block's inputs over more waves;
// the thresholds keep at least ~2 work groups per CU. Past kMxDeepTiles
// tiles (T = 64 at top-8 of 352) a wave keeps 8 gate/up steps and all 12
// down steps in flight, the down pass one row block per wave: decode T=64
// 0.470 -> 0.460 ms (down 160 -> 153 us). At 256 tiles (the Zipf-routed
// stack at T=32) that form measured slower (down 40 -> 44 us per layer),
// so smaller batches keep the 4-step rings and two row passes.
template <int ACT, int FMT, int TM>
moe_status_t gemv_mx_forward_t(const moe_ffn_desc_t &ex, const uint16_t *x, int K,
                               const moe_perm_t &p, int max_tiles, uint16_t *h, float *y,
                               hipStream_t s, const std::function<moe_status_t(int)> &mark) {
    const int F = ex.gate.n, H = ex.gate.k;
    const GemvMat g = gemv_mat(ex.gate), u = gemv_mat(ex.up), d = gemv_mat(ex.down);
    moe_status_t st;
    if (max_tiles <= 16)
        st = launch_mx<ACT, FMT, TM, true, 32, 1, 4, 4>(g, u, F, x, K, p, max_tiles, h, nullptr, s);
    else if (max_tiles <= 48)
        st = launch_mx<ACT, FMT, TM, true, 32, 1, 2, 4>(g, u, F, x, K, p, max_tiles, h, nullptr, s);
    else if (max_tiles <= kMxDeepTiles)
        st = launch_mx<ACT, FMT, TM, true, 32, 1, 1, 4>(g, u, F, x, K, p, max_tiles, h, nullptr, s);
    else
        st = launch_mx<ACT, FMT, TM, true, 32, 1, 1, 8>(g, u, F, x, K, p, max_tiles, h, nullptr, s);
    if (st != MOE_OK) return st;
    if (mark && mark(1) != MOE_OK) return MOE_ERR_HIP;
    if (max_tiles <= 16)
        st = launch_mx<ACT, FMT, TM, false, 12, 1, 2, 3>(d, d, H, h, K, p, max_tiles, nullptr, y, s);
    else if (max_tiles <= 48)
        st = launch_mx<ACT, FMT, TM, false, 12, 1, 1, 4>(d, d, H, h, K, p, max_tiles, nullptr, y, s);
    else if (max_tiles <= kMxDeepTiles)
        st = launch_mx<ACT, FMT, TM, false, 12, 2, 1, 4>(d, d, H, h, K, p, max_tiles, nullptr, y, s);
    else
        st = launch_mx<ACT, FMT, TM, false, 12, 1, 1, 12>(d, d, H, h, K, p, max_tiles, nullptr, y, s);
    if (st != MOE_OK) return st;
    if (mark && mark(2) != MOE_OK) return MOE_ERR_HIP;
    return MOE_OK;
}

moe_status_t launch_gemv_mx_forward(const moe_ffn_desc_t &ex, const void *x, int act, int K,
                                    const moe_perm_t &p, int max_tiles, void *h, float *y,
                                    hipStream_t s, const std::function<moe_status_t(int)> &mark) {
    const uint16_t *xx = (const uint16_t *)x;
    uint16_t *hh = (uint16_t *)h;
#define MOE_MX_FMT(A, F)                                                                   \
    if (act == A && ex.gate.fmt == F)                                                      \
        return p.tile_m == 8 ? gemv_mx_forward_t<A, F, 8>(ex, xx, K, p, max_tiles, hh, y, s, mark) \
                             : gemv_mx_forward_t<A, F, 4>(ex, xx, K, p, max_tiles, hh, y, s, mark);
    MOE_MX_FMT(MOE_F16, MOE_W_INT4_G128)
    MOE_MX_FMT(MOE_F16, MOE_W_INT4_G128_ASYM)
    MOE_MX_FMT(MOE_BF16, MOE_W_INT4_G128)
    MOE_MX_FMT(MOE_BF16, MOE_W_INT4_G128_ASYM)
    MOE_MX_FMT(MOE_F16, MOE_W_NVFP4_G16)
    MOE_MX_FMT(MOE_BF16, MOE_W_NVFP4_G16)
#undef MOE_MX_FMT
    return MOE_ERR_UNSUPPORTED;
}

}  // namespace moe
