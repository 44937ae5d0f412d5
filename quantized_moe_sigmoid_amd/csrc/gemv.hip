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
//   in float32 (every chunk lies inside one group: 128 inputs, or 32 for
//   g32). The asymmetric form decodes MAGIC + q and removes MAGIC + z, its
//   group's zero point: acc += s_g * (dot - (MAGIC + z) * sum x).
// int8: a 16-byte chunk holds 16 inputs; each byte pair becomes the exact
//   16-bit pair BIAS + q (decode.h) and the chunk's sum(x) removes BIAS the
//   same way: acc += s_g * (dot - BIAS * sum x).
// NVFP4: the hardware pair conversion gives exact E2M1 values; the E4M3
//   block scale applies per 16 inputs in float32, the global scale once at
//   the end. With compressed scales (NVFP4_CSF) a chunk's two scale bytes
//   are its row's base plus the two 4-bit codes of one byte, unless one of
//   the row's exceptions holds that position: each lane keeps the (at most
//   two) exceptions that fall in its own chunks in registers; a lane with
//   more recomputes its partial sums at the end of the pass through the
//   exact per-chunk lookup, in the same order, so every result is the one
//   the expanded scales give.
#include <functional>

#include "decode.h"
#include "stream.h"

namespace moe {

constexpr int kGemvThreads = 256;
constexpr int kGemvWaves = kGemvThreads / kWave;

// NVFP4_CSF: the two scale bytes of chunk c (blocks p0 = r*C + 2c, p0 + 1
// of its row): base + code, or an exception's byte. ex0 / ex1: exceptions
// held in registers (0xFFFFFFFF: none; a 24-bit position never reaches
// 0xFFFFFF).
__device__ __forceinline__ uint32_t csf_scale_pair(uint32_t code, uint32_t base, uint32_t ex0,
                                                   uint32_t ex1, uint32_t p0) {
    uint32_t b0 = base + (code & 15u), b1 = base + (code >> 4);
    const uint32_t q0 = ex0 & 0xFFFFFFu, q1 = ex1 & 0xFFFFFFu;
    b0 = q0 == p0 ? ex0 >> 24 : b0;
    b1 = q0 == p0 + 1 ? ex0 >> 24 : b1;
    b0 = q1 == p0 ? ex1 >> 24 : b0;
    b1 = q1 == p0 + 1 ? ex1 >> 24 : b1;
    return b0 | (b1 << 8);
}
// The same pair by walking all of the row's exceptions [xl, xh).
__device__ __forceinline__ uint32_t csf_scale_pair_walk(uint32_t code, uint32_t base, int xl,
                                                        int xh, const uint32_t *xc, uint32_t p0) {
    uint32_t b0 = base + (code & 15u), b1 = base + (code >> 4);
    for (int x = xl; x < xh; ++x) {
        const uint32_t v = xc[x], q = v & 0xFFFFFFu;
        b0 = q == p0 ? v >> 24 : b0;
        b1 = q == p0 + 1 ? v >> 24 : b1;
    }
    return b0 | (b1 << 8);
}

// LDS unit (16 bytes = 4 pair dwords = 8 inputs) j of input chunk c (UPC
// units: 4 for 32-input chunks, 2 for int8's 16). For a fixed j the LPR
// chunks read together by one row's lanes are 16-byte neighbours, so one
// wave-wide 16-byte read touches all banks once.
template <int LPR, int UPC>
__device__ __forceinline__ int xs_unit(int c, int j) {
    return ((c / LPR) * UPC + j) * LPR + (c % LPR);
}
// LDS units per token row: chunks rounded up to a multiple of LPR.
template <int LPR, int CI>
__host__ __device__ __forceinline__ int xs_units_pad(int kin) {
    return (kin / CI + LPR - 1) / LPR * LPR * (CI / 8);
}

// Partial dot products of one 16-byte weight chunk against token t's x.
// KIND: 0 NVFP4, 1 the int4 family, 2 int8.
template <int ACT, int FMT, int KIND = is_int4(FMT) ? 1 : is_int8(FMT) ? 2 : 0>
struct ChunkDot;

// Signed int4 with fp16 activations (gate/up pass) decodes the odd pairs
// in place: the
// nibbles at bits 4..7 and 20..23 of a word (inputs 8w+1, 8w+5; after the
// 8-bit shift 8w+3, 8w+7) land in mantissa bits 4..7 of fp16 1024.0, the
// exact value 1024 + 16 (q + 8) = 1152 + 16 q (below 2048, ulp 1), so a word
// costs one shift and four bit operations instead of three shifts and four.
// The staged x of those inputs is pre-scaled by 1/16 (exact in fp16 down
// to |x| ~ 2^-10, far below what moves a sum), and the chunk's bias sum
// becomes 1032 sum(x even) + 72 sum(x odd). (Measured: 3 % off the decode
// gate/up pass; the down pass, with its row passes, gained nothing.)
template <int ACT, int FMT, bool GATEUP>
__host__ __device__ constexpr bool odd_x16() {
    return GATEUP && ACT == MOE_F16 && is_int4(FMT) && !int4_asym(FMT);
}

// The int4 family. kv = int4_key<ACT, FMT>() in a VGPR: each pair is then
// one shift and one v_bitop3 ((w >> 4i) & 0x000F000F) ^ kv, the exact
// 16-bit value BIAS + q (signed forms) or MAGIC + q (unsigned form).
template <int ACT, int FMT>
struct ChunkDot<ACT, FMT, 1> {
    uint32_t p[16];
    // X16: odd pairs in place (odd_x16), kv1 their key 0x64806480
    template <bool X16>
    __device__ __forceinline__ void decode(uint4 w, uint32_t kv, uint32_t kv1) {
        const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if constexpr (X16) {
                const uint32_t d8 = d[q] >> 8;
                p[4 * q + 0] = (d[q] & 0x000F000Fu) ^ kv;
                p[4 * q + 1] = (d[q] & 0x00F000F0u) ^ kv1;
                p[4 * q + 2] = (d8 & 0x000F000Fu) ^ kv;
                p[4 * q + 3] = (d8 & 0x00F000F0u) ^ kv1;
            } else {
                p[4 * q + 0] = (d[q] & 0x000F000Fu) ^ kv;
                p[4 * q + 1] = ((d[q] >> 4) & 0x000F000Fu) ^ kv;
                p[4 * q + 2] = ((d[q] >> 8) & 0x000F000Fu) ^ kv;
                p[4 * q + 3] = ((d[q] >> 12) & 0x000F000Fu) ^ kv;
            }
        }
    }
    // scale: the chunk's bf16 scale; bias: the 16-bit values' offset from
    // q (signed forms), or from q - z (asymmetric: MAGIC + z).
    __device__ __forceinline__ float apply(const uint4 *xu, int stride_j, float xs_sum,
                                           float scale, float bias, float acc) const {
        float d = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint4 x = xu[j * stride_j];
            d = dot2<ACT>(p[4 * j + 0], x.x, d);
            d = dot2<ACT>(p[4 * j + 1], x.y, d);
            d = dot2<ACT>(p[4 * j + 2], x.z, d);
            d = dot2<ACT>(p[4 * j + 3], x.w, d);
        }
        return __builtin_fmaf(scale, d - bias * xs_sum, acc);
    }
};

// int8: 16 inputs, natural pair order (2i, 2i+1), two LDS units.
template <int ACT, int FMT>
struct ChunkDot<ACT, FMT, 2> {
    uint32_t p[8];
    template <bool>
    __device__ __forceinline__ void decode(uint4 w, uint32_t, uint32_t) {
        const uint32_t d[4] = {w.x ^ 0x80808080u, w.y ^ 0x80808080u, w.z ^ 0x80808080u,
                               w.w ^ 0x80808080u};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            p[2 * q + 0] = int8_pair<ACT, 0>(d[q]);
            p[2 * q + 1] = int8_pair<ACT, 1>(d[q]);
        }
    }
    __device__ __forceinline__ float apply(const uint4 *xu, int stride_j, float xs_sum,
                                           float scale, float bias, float acc) const {
        float d = 0.0f;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint4 x = xu[j * stride_j];
            d = dot2<ACT>(p[4 * j + 0], x.x, d);
            d = dot2<ACT>(p[4 * j + 1], x.y, d);
            d = dot2<ACT>(p[4 * j + 2], x.z, d);
            d = dot2<ACT>(p[4 * j + 3], x.w, d);
        }
        return __builtin_fmaf(scale, d - bias * xs_sum, acc);
    }
};

template <int ACT, int FMT>
struct ChunkDot<ACT, FMT, 0> {
    uint32_t p[16];
    template <bool>
    __device__ __forceinline__ void decode(uint4 w, uint32_t, uint32_t) {
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

// The two scale bytes of chunk c of a row: int4, the bf16 scale of its
// group (one per 4 chunks at g128, one per chunk at g32) and (asymmetric)
// its zero point z; int8, the bf16 scale of its group (one per 8 chunks);
// NVFP4, its two E4M3 block scales. For the integer formats the second
// output is the bias apply() removes.
template <int ACT, int FMT, bool X16>
__device__ __forceinline__ void chunk_scales(uint32_t two, uint32_t z, float &a, float &b) {
    if constexpr (is_int4(FMT)) {
        a = bf16_bits_to_f32(two);
        // odd_x16: the chunk sum already carries the biases
        b = X16 ? 1.0f
            : int4_asym(FMT)    ? Int4Bias<ACT>::kMagicValue + (float)z
                                : Int4Bias<ACT>::kBias;
    } else if constexpr (is_int8(FMT)) {
        (void)z;
        a = bf16_bits_to_f32(two);
        b = Int8Bias<ACT>::kBias;
    } else {
        (void)z;
        a = e4m3_to_f32(two & 0xFF);
        b = e4m3_to_f32(two >> 8);
    }
}
template <int FMT>
__device__ __forceinline__ int scale_offset(int c) {
    return is_int4(FMT) ? 2 * (c / (int4_group(FMT) / 32)) : is_int8(FMT) ? 2 * (c / 8) : 2 * c;
}
// Formats whose chunks carry the sum of their inputs (the integer ones).
__host__ __device__ constexpr bool needs_xsum(int fmt) { return is_int4(fmt) || is_int8(fmt); }


// Chunks in flight per lane and matrix.
constexpr int kGemvRing = 4;
// Activation loads per thread issued together while staging.
constexpr int kGemvStage = 8;

// GATEUP: mats a = gate, b = up, output h (16-bit). Otherwise a = down,
// output y (float32).
//
// Per work group: the tile's slots, then up to kGemvStage 16-byte loads of
// activations per thread, then the first kGemvRing weight chunks of every
// lane (issued before the activations are needed, so the staging latency
// overlaps the weight stream), then the activations are written to LDS in
// the decoders' pair order together with (int4) each 32-input chunk's sum,
// reduced across the four lanes that hold its four 8-input units. The main
// loop consumes ring slot j and immediately refills it with the chunk
// kGemvRing iterations ahead.
template <int ACT, int FMT, int LPR, int TM, bool GATEUP, int NIT, int RPW>
__global__ void __launch_bounds__(kGemvThreads) gemv_kernel(
    GemvMat A, GemvMat B, int n_rows, int kin, const uint16_t *xin,
    int x_from_slots, int topk, const int32_t *__restrict__ sorted_slots,
    const int32_t *__restrict__ tile_expert, const int32_t *__restrict__ num_tiles,
    uint16_t *__restrict__ hout, float *__restrict__ yout) {
    extern __shared__ uint4 smem[];
    const int tile = blockIdx.y;
    if (tile >= num_tiles[0]) return;
    const int e = tile_expert[tile];

    static_assert(TM == kGemvWaves, "wave w stages the activation row of slot w");
    constexpr int CI = chunk_inputs(FMT), UPC = CI / 8, UPC_LOG = UPC == 4 ? 2 : 1;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
    // the tile's number of real rows (slots are -1 past them)
    int m = 0;
#pragma unroll
    for (int t = 0; t < TM; ++t)
        if (sorted_slots[tile * TM + t] >= 0) m = t + 1;

    // activation staging, first batch: loads only. Wave w stages the row of
    // the tile's slot w (a padding slot reads token 0; it is never used).
    const int units = kin / 8;                   // 8 inputs per unit
    const uint16_t *xrow;
    {
        const int sl = sorted_slots[tile * TM + wave];
        xrow = x_from_slots ? xin + (size_t)(sl >= 0 ? sl / topk : 0) * kin
                            : xin + (size_t)(tile * TM + wave) * kin;
    }
    u32x4_t xv[kGemvStage];
#pragma unroll
    for (int i = 0; i < kGemvStage; ++i) {
        const int g = lane + i * kWave;
        xv[i] = *(const u32x4_t *)(xrow + 8 * (g < units ? g : 0));  // past the end: unused
    }

    // weight ring: chunk c = sub + LPR * i of the lane's row
    // RPW passes of 32 rows per work group (a wave owns LPR-lane groups of
    // 8 rows per pass); the staged activations serve every pass
    static_assert(NIT > 0 || RPW == 1, "row passes need the unrolled kernel");
    const int sub = lane % LPR;
    auto row_of = [&](int pass) {
        return ((blockIdx.x * RPW + pass) * kGemvWaves + wave) * (kWave / LPR) + lane / LPR;
    };
    // chunks per row and iterations per lane and pass: NIT when the shape is
    // known at compile time (kin == CI * LPR * NIT; the main loop then
    // unrolls completely and every load offset is a constant), else computed
    const int nch = NIT > 0 ? NIT * LPR : kin / CI;
    const int nit = NIT > 0 ? NIT : (nch + LPR - 1) / LPR;
    const __amdgpu_buffer_rsrc_t rqa = buffer_rsrc(A.q + e * A.qe, (int64_t)n_rows * A.qr);
    constexpr bool kCsf = is_csf(FMT);
    // NVFP4_CSF: an expert's fixed tensor is n_rows * (1 + C/2) bytes, C = kin/16
    const int64_t csf_row_bytes = 1 + kin / 32;
    const __amdgpu_buffer_rsrc_t rsa =
        buffer_rsrc(A.s + e * A.se, (int64_t)n_rows * (kCsf ? csf_row_bytes : A.sr));
    const __amdgpu_buffer_rsrc_t rqb = buffer_rsrc(B.q + e * B.qe, (int64_t)n_rows * B.qr);
    const __amdgpu_buffer_rsrc_t rsb =
        buffer_rsrc(B.s + e * B.se, (int64_t)n_rows * (kCsf ? csf_row_bytes : B.sr));
    // per pass: byte offsets of the lane's row (rows past the matrix, never
    // stored, read its last row)
    int qra[RPW], sra[RPW], qrb[RPW], srb[RPW], zra[RPW], zrb[RPW];
#pragma unroll
    for (int ps = 0; ps < RPW; ++ps) {
        const int r = row_of(ps) < n_rows ? row_of(ps) : n_rows - 1;
        qra[ps] = r * (int)A.qr;
        qrb[ps] = r * (int)B.qr;
        if (kCsf) {                              // the row's codes in its 16-row slab
            sra[ps] = srb[ps] = (r >> 4) * 16 * (int)csf_row_bytes + 16 + (r & 15) * (kin / 32);
        } else {
            sra[ps] = r * (int)A.sr;
            srb[ps] = r * (int)B.sr;
        }
        zra[ps] = r * (int)A.zr;
        zrb[ps] = r * (int)B.zr;
    }
    // NVFP4_CSF: per pass and matrix the row's base byte (bit 31: the lane
    // has more than two exceptions in its chunks), the lane's first two
    // exceptions and the row's exception range
    uint32_t bsa[kCsf ? RPW : 1], bsb[kCsf ? RPW : 1], e0a[kCsf ? RPW : 1], e1a[kCsf ? RPW : 1],
        e0b[kCsf ? RPW : 1], e1b[kCsf ? RPW : 1];
    int xla[kCsf ? RPW : 1], xha[kCsf ? RPW : 1], xlb[kCsf ? RPW : 1], xhb[kCsf ? RPW : 1];
    if constexpr (kCsf) {
        auto row_state = [&](const GemvMat &M, int r, uint32_t &bs, uint32_t &e0, uint32_t &e1,
                             int &xl, int &xh) {
            const uint8_t *fx = M.s + e * M.se;
            bs = fx[(size_t)(r >> 4) * 16 * csf_row_bytes + (r & 15)];
            const int32_t *ri = M.ri + (size_t)e * (n_rows + 1) + r;
            xl = ri[0];
            xh = ri[1];
            e0 = e1 = 0xFFFFFFFFu;
            int cnt = 0;
            const uint32_t rC = (uint32_t)r * (uint32_t)(kin / 16);
            auto take = [&](uint32_t v) {
                if ((int)((((v & 0xFFFFFFu) - rC) >> 1) % LPR) == sub) {   // one of my chunks
                    e0 = cnt == 0 ? v : e0;
                    e1 = cnt == 1 ? v : e1;
                    ++cnt;
                }
            };
            // the row's first four exceptions loaded together, the rest (rows
            // with more: rare) one by one
            uint32_t v4[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) v4[q] = xl + q < xh ? M.xc[xl + q] : 0u;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (xl + q < xh) take(v4[q]);
            for (int x = xl + 4; x < xh; ++x) take(M.xc[x]);
            bs |= cnt > 2 ? 0x80000000u : 0u;
        };
#pragma unroll
        for (int ps = 0; ps < RPW; ++ps) {
            const int r = row_of(ps) < n_rows ? row_of(ps) : n_rows - 1;
            row_state(A, r, bsa[ps], e0a[ps], e1a[ps], xla[ps], xha[ps]);
            if (GATEUP) row_state(B, r, bsb[ps], e0b[ps], e1b[ps], xlb[ps], xhb[ps]);
        }
    }
    // asymmetric int4: one zero-point byte per 128 inputs, streamed with the scales
    constexpr bool kZ = int4_asym(FMT);
    const __amdgpu_buffer_rsrc_t rza = buffer_rsrc(kZ ? A.z + e * A.ze : A.q, (int64_t)n_rows * A.zr);
    const __amdgpu_buffer_rsrc_t rzb = buffer_rsrc(kZ ? B.z + e * B.ze : B.q, (int64_t)n_rows * B.zr);
    const uint32_t kv = in_vgpr(is_int4(FMT) ? int4_key<ACT, FMT>() : 0u);
    constexpr bool X16 = odd_x16<ACT, FMT, GATEUP>();
    const uint32_t kv1 = in_vgpr(X16 ? 0x64806480u : 0u);
    u32x4_t wa[kGemvRing], wb[kGemvRing];
    uint16_t sa[kGemvRing], sb[kGemvRing];
    uint8_t za[kGemvRing], zb[kGemvRing];
    // iteration I = pass * nit + i streams chunk c = sub + LPR * i of the pass's row
    auto load = [&](int j, int I) {
        const int ps = NIT > 0 ? I / NIT : 0, i = NIT > 0 ? I % NIT : I;
        const int c = sub + LPR * i;
        const bool ok = NIT > 0 ? ps < RPW : c < nch;   // past the work: read nothing
        const int pq = ok ? ps : 0;
        wa[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                   rqa, ok ? qra[pq] + 16 * c : kOutOfRange, 0, 0));
        if constexpr (kCsf)                      // one code byte: the chunk's two blocks
            sa[j] = __builtin_amdgcn_raw_buffer_load_b8(rsa, ok ? sra[pq] + c : kOutOfRange, 0, 0);
        else
            sa[j] = __builtin_amdgcn_raw_buffer_load_b16(
                rsa, ok ? sra[pq] + scale_offset<FMT>(c) : kOutOfRange, 0, 0);
        if constexpr (kZ)
            za[j] = __builtin_amdgcn_raw_buffer_load_b8(rza, ok ? zra[pq] + (c >> 2) : kOutOfRange,
                                                        0, 0);
        if (GATEUP) {
            wb[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                       rqb, ok ? qrb[pq] + 16 * c : kOutOfRange, 0, 0));
            if constexpr (kCsf)
                sb[j] = __builtin_amdgcn_raw_buffer_load_b8(rsb, ok ? srb[pq] + c : kOutOfRange, 0,
                                                            0);
            else
                sb[j] = __builtin_amdgcn_raw_buffer_load_b16(
                    rsb, ok ? srb[pq] + scale_offset<FMT>(c) : kOutOfRange, 0, 0);
            if constexpr (kZ)
                zb[j] = __builtin_amdgcn_raw_buffer_load_b8(
                    rzb, ok ? zrb[pq] + (c >> 2) : kOutOfRange, 0, 0);
        }
    };
#pragma unroll
    for (int j = 0; j < kGemvRing; ++j) load(j, j);
    // keep every load above in flight before the staging arithmetic starts
    __builtin_amdgcn_sched_barrier(0);

    // activations into LDS (pair order of the decoders) and chunk sums
    uint4 *xs = smem;
    const int upad = xs_units_pad<LPR, CI>(kin);
    float *xsum = (float *)(smem + TM * upad);
    // lanes past the end of the row write to a dummy area instead of
    // branching (a branch would let the compiler sink the staging loads
    // below the weight loads and wait for those too)
    uint4 *xdummy = xs + TM * upad + (TM * nch + 3) / 4;
    float *sdummy = (float *)(xdummy + kWave);
    auto stage = [&](const u32x4_t &v, int g) {
        const bool valid = g < units;            // the UPC lanes of a chunk agree (units % UPC == 0)
        uint4 p;
        if (is_int4(FMT)) {                      // pairs (i, i+4) of the 8 inputs
            p.x = (v.x & 0xFFFFu) | (v.z << 16);
            p.y = (v.x >> 16) | (v.z & 0xFFFF0000u);
            p.z = (v.y & 0xFFFFu) | (v.w << 16);
            p.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
            if constexpr (X16) {                 // the odd inputs' pairs, times 1/16
                const half2_t r16 = {(_Float16)0.0625f, (_Float16)0.0625f};
                p.y = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, p.y) * r16);
                p.w = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, p.w) * r16);
            }
        } else {                                 // pairs (2i, 2i+1): natural order
            p = make_uint4(v.x, v.y, v.z, v.w);
        }
        *(valid ? xs + wave * upad + xs_unit<LPR, UPC>(g >> UPC_LOG, g & (UPC - 1)) : xdummy + lane) = p;
        if (needs_xsum(FMT)) {
            const uint32_t d[4] = {v.x, v.y, v.z, v.w};
            float sum = 0.0f;
            if constexpr (X16) {                 // 1032 sum(x even) + 72 sum(x odd)
                float se = 0.0f, so = 0.0f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    se += act_to_f32<ACT>(d[q] & 0xFFFF);
                    so += act_to_f32<ACT>(d[q] >> 16);
                }
                sum = __builtin_fmaf(1032.0f, se, 72.0f * so);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    sum += act_to_f32<ACT>(d[q] & 0xFFFF) + act_to_f32<ACT>(d[q] >> 16);
            }
            // the UPC units of a chunk sit in UPC consecutive lanes
            sum += shfl_xor_f(sum, 1);
            if (UPC == 4) sum += shfl_xor_f(sum, 2);
            *(valid && (g & (UPC - 1)) == 0 ? xsum + wave * nch + (g >> UPC_LOG) : sdummy + lane) = sum;
        }
    };
#pragma unroll
    for (int i = 0; i < kGemvStage; ++i) stage(xv[i], lane + i * kWave);
    for (int g0 = kGemvStage * kWave; g0 < units; g0 += kWave) {   // rows over 4096 inputs
        const int g = g0 + lane;
        stage(*(const u32x4_t *)(xrow + 8 * (g < units ? g : 0)), g);
    }
    lds_barrier();

    float acc_a[TM], acc_b[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) acc_a[t] = acc_b[t] = 0.0f;
    float ga = 1.0f, gb = 1.0f;
    if (is_nvfp4(FMT)) {
        ga = A.gs[e] * A.xs;
        if (GATEUP) gb = B.gs[e] * B.xs;
    }
    // end of a pass: reduce the LPR partial sums of each row, store, reset
    auto finish = [&](int ps) {
#pragma unroll
        for (int t = 0; t < TM; ++t) {
#pragma unroll
            for (int msk = LPR / 2; msk >= 1; msk >>= 1) {
                acc_a[t] += shfl_xor_f(acc_a[t], msk);
                if (GATEUP) acc_b[t] += shfl_xor_f(acc_b[t], msk);
            }
        }
        const int row = row_of(ps);
        if (row < n_rows && sub == 0) {
#pragma unroll
            for (int t = 0; t < TM; ++t) {
                if (t < m) {
                    const size_t r = (size_t)tile * TM + t;
                    if (GATEUP)
                        hout[r * n_rows + row] =
                            f32_to_act<ACT>(silu_mul(acc_a[t] * ga, acc_b[t] * gb));
                    else
                        yout[r * n_rows + row] = acc_a[t] * ga;
                }
            }
        }
#pragma unroll
        for (int t = 0; t < TM; ++t) acc_a[t] = acc_b[t] = 0.0f;
    };
    // NVFP4_CSF: a lane with more than two exceptions in its chunks redoes
    // its pass with the full per-chunk lookup (the same operations in the
    // same order, so its sums equal those of the expanded scales)
    auto repair = [&](int ps) {
        if constexpr (kCsf) {
            if (((bsa[ps] | (GATEUP ? bsb[ps] : 0u)) >> 31) != 0) {
                const int r = row_of(ps) < n_rows ? row_of(ps) : n_rows - 1;
                const uint32_t rC = (uint32_t)r * (uint32_t)(kin / 16);
#pragma unroll
                for (int t = 0; t < TM; ++t) acc_a[t] = acc_b[t] = 0.0f;
                for (int i = 0; i < nit; ++i) {
                    const int c = sub + LPR * i;
                    if (c >= nch) break;
                    const uint32_t p0 = rC + 2u * (uint32_t)c;
                    ChunkDot<ACT, FMT> da, db;
                    float a0, a1, b0 = 0.0f, b1 = 0.0f;
                    const u32x4_t w = __builtin_bit_cast(
                        u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rqa, qra[ps] + 16 * c, 0, 0));
                    const uint32_t code = __builtin_amdgcn_raw_buffer_load_b8(rsa, sra[ps] + c, 0, 0);
                    da.template decode<X16>(make_uint4(w.x, w.y, w.z, w.w), kv, kv1);
                    chunk_scales<ACT, FMT, X16>(
                        csf_scale_pair_walk(code, bsa[ps] & 0xFFu, xla[ps], xha[ps], A.xc, p0), 0u,
                        a0, a1);
                    if (GATEUP) {
                        const u32x4_t wv = __builtin_bit_cast(
                            u32x4_t,
                            __builtin_amdgcn_raw_buffer_load_b128(rqb, qrb[ps] + 16 * c, 0, 0));
                        const uint32_t cb =
                            __builtin_amdgcn_raw_buffer_load_b8(rsb, srb[ps] + c, 0, 0);
                        db.template decode<X16>(make_uint4(wv.x, wv.y, wv.z, wv.w), kv, kv1);
                        chunk_scales<ACT, FMT, X16>(
                            csf_scale_pair_walk(cb, bsb[ps] & 0xFFu, xlb[ps], xhb[ps], B.xc, p0), 0u,
                            b0, b1);
                    }
                    const int u0 = xs_unit<LPR, UPC>(c, 0);
#pragma unroll
                    for (int t = 0; t < TM; ++t) {
                        if (t < m) {
                            const uint4 *xu = xs + t * upad + u0;
                            acc_a[t] = da.apply(xu, LPR, 0.0f, a0, a1, acc_a[t]);
                            if (GATEUP) acc_b[t] = db.apply(xu, LPR, 0.0f, b0, b1, acc_b[t]);
                        }
                    }
                }
            }
        }
    };
    const int total_it = RPW * nit;
    // every trip runs all kGemvRing slots (slots past the last iteration hold
    // zeros and are not computed)
    auto trip = [&](int I0) {
#pragma unroll
        for (int j = 0; j < kGemvRing; ++j) {
            const int I = I0 + j;
            const int i = NIT > 0 ? I % NIT : I;
            const int c = sub + LPR * i;
            ChunkDot<ACT, FMT> da, db;
            da.template decode<X16>(make_uint4(wa[j].x, wa[j].y, wa[j].z, wa[j].w), kv, kv1);
            float a0, a1, b0 = 0.0f, b1 = 0.0f;
            uint32_t two_a = sa[j], two_b = sb[j];
            if constexpr (kCsf) {
                const int ps = NIT > 0 ? I / NIT : 0;
                const int pp = ps < RPW ? ps : 0;
                const int r = row_of(pp) < n_rows ? row_of(pp) : n_rows - 1;
                const uint32_t p0 = (uint32_t)r * (uint32_t)(kin / 16) + 2u * (uint32_t)c;
                two_a = csf_scale_pair(sa[j], bsa[pp] & 0xFFu, e0a[pp], e1a[pp], p0);
                if (GATEUP) two_b = csf_scale_pair(sb[j], bsb[pp] & 0xFFu, e0b[pp], e1b[pp], p0);
            }
            chunk_scales<ACT, FMT, X16>(two_a, kZ ? za[j] : 0u, a0, a1);
            if (GATEUP) {
                db.template decode<X16>(make_uint4(wb[j].x, wb[j].y, wb[j].z, wb[j].w), kv, kv1);
                chunk_scales<ACT, FMT, X16>(two_b, kZ ? zb[j] : 0u, b0, b1);
            }
            // slot j is consumed: refill it in place (the barrier keeps the
            // refill below the last use, so it reuses the same registers)
            __builtin_amdgcn_sched_barrier(0);
            load(j, I + kGemvRing);
            if (I < total_it && c < nch) {
                const int u0 = xs_unit<LPR, UPC>(c, 0);
#pragma unroll
                for (int t = 0; t < TM; ++t) {
                    if (t < m) {
                        const uint4 *xu = xs + t * upad + u0;
                        const float xsm = needs_xsum(FMT) ? xsum[t * nch + c] : 0.0f;
                        acc_a[t] = da.apply(xu, LPR, xsm, a0, a1, acc_a[t]);
                        if (GATEUP) acc_b[t] = db.apply(xu, LPR, xsm, b0, b1, acc_b[t]);
                    }
                }
            }
            if (NIT > 0 && I < total_it && i == NIT - 1) {
                repair(I / NIT);
                finish(I / NIT);
            }
        }
    };
    if constexpr (NIT > 0) {
#pragma unroll
        for (int I0 = 0; I0 < RPW * NIT; I0 += kGemvRing) trip(I0);
    } else {
        for (int I0 = 0; I0 < nit; I0 += kGemvRing) trip(I0);
        repair(0);
        finish(0);
    }
}

constexpr int kGemvLPR = 8;
constexpr int kGemvTM = 4;

// Activation units, chunk sums (rounded up to 16 bytes) and the staging
// dummy area (64 units + 64 floats).
template <int LPR, int TM, int CI>
inline size_t gemv_lds_bytes(int kin) {
    return (size_t)TM * xs_units_pad<LPR, CI>(kin) * 16 + ((size_t)TM * (kin / CI) + 3) / 4 * 16 +
           (size_t)kWave * 16 + (size_t)kWave * 4;
}

template <int ACT, int FMT>
moe_status_t gemv_forward_t(const moe_ffn_desc_t &ex, const uint16_t *x, int K,
                            const moe_perm_t &p, int max_tiles, uint16_t *h, float *y,
                            hipStream_t s, const std::function<moe_status_t(int)> &mark) {
    constexpr int LPR = kGemvLPR, TM = kGemvTM, CI = chunk_inputs(FMT);
    const int F = ex.gate.n, H = ex.gate.k;
    const int rows_per_block = kGemvWaves * (kWave / LPR);
    // the layer's own shapes get fully unrolled kernels: 4096 inputs -> 16
    // iterations per lane (32 for int8), 1536 -> 6 (12); other shapes run
    // the generic loop
    constexpr int NIT_H = 4096 / (CI * LPR), NIT_F = 1536 / (CI * LPR);
    {
        const size_t lds = gemv_lds_bytes<LPR, TM, CI>(H);
        constexpr int RP = 1;                   // row passes per work group (more cost VGPRs)
        const bool fast = H == CI * LPR * NIT_H && F % (RP * rows_per_block) == 0;
        auto k = fast ? gemv_kernel<ACT, FMT, LPR, TM, true, NIT_H, RP>
                      : gemv_kernel<ACT, FMT, LPR, TM, true, 0, 1>;
        dim3 grid(fast ? F / (RP * rows_per_block) : (F + rows_per_block - 1) / rows_per_block,
                  max_tiles);
        allow_lds(k, lds);
        hipLaunchKernelGGL(k, grid, dim3(kGemvThreads), lds, s, gemv_mat(ex.gate),
                           gemv_mat(ex.up), F, H, x, 1, K, p.sorted_slots, p.tile_expert,
                           p.num_tiles, h, nullptr);
        MOE_LAUNCH_CHECK();
    }
    if (mark && mark(1) != MOE_OK) return MOE_ERR_HIP;
    {
        const size_t lds = gemv_lds_bytes<LPR, TM, CI>(F);
        // row passes: the staged h rows serve RP * 32 output rows
        constexpr int RP = is_int8(FMT) ? 2 : 4;
        const bool fast = F == CI * LPR * NIT_F && H % (RP * rows_per_block) == 0;
        auto k = fast ? gemv_kernel<ACT, FMT, LPR, TM, false, NIT_F, RP>
                      : gemv_kernel<ACT, FMT, LPR, TM, false, 0, 1>;
        dim3 grid(fast ? H / (RP * rows_per_block) : (H + rows_per_block - 1) / rows_per_block,
                  max_tiles);
        allow_lds(k, lds);
        hipLaunchKernelGGL(k, grid, dim3(kGemvThreads), lds, s, gemv_mat(ex.down),
                           gemv_mat(ex.down), H, F, h, 0, K, p.sorted_slots, p.tile_expert,
                           p.num_tiles, nullptr, y);
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
#define MOE_GEMV_FMT(A, F)                                                               \
    case F: return gemv_forward_t<A, F>(ex, xx, K, p, max_tiles, hh, y, s, mark)
    if (act == MOE_BF16) {
        switch (ex.gate.fmt) {
            MOE_GEMV_FMT(MOE_BF16, MOE_W_INT4_G128);
            MOE_GEMV_FMT(MOE_BF16, MOE_W_NVFP4_G16);
            MOE_GEMV_FMT(MOE_BF16, MOE_W_INT4_G32);
            MOE_GEMV_FMT(MOE_BF16, MOE_W_INT4_G128_ASYM);
            MOE_GEMV_FMT(MOE_BF16, MOE_W_INT8_G128);
            MOE_GEMV_FMT(MOE_BF16, MOE_W_NVFP4_CSF);
        }
    } else {
        switch (ex.gate.fmt) {
            MOE_GEMV_FMT(MOE_F16, MOE_W_INT4_G128);
            MOE_GEMV_FMT(MOE_F16, MOE_W_NVFP4_G16);
            MOE_GEMV_FMT(MOE_F16, MOE_W_INT4_G32);
            MOE_GEMV_FMT(MOE_F16, MOE_W_INT4_G128_ASYM);
            MOE_GEMV_FMT(MOE_F16, MOE_W_INT8_G128);
            MOE_GEMV_FMT(MOE_F16, MOE_W_NVFP4_CSF);
        }
    }
#undef MOE_GEMV_FMT
    return MOE_ERR_UNSUPPORTED;
}

}  // namespace moe
