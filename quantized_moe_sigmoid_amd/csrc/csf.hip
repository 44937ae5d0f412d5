// Expansion of CSF-compressed NVFP4 block scales (page
// "Step-5-Preview-NVFP4-Local", "Format"): every byte is rebuilt as the row
// base plus the 4-bit code at its position, and the positions the expert's
// exception list names are then overwritten with the bytes stored there.
//
// One kernel per scale tensor; work group = (expert, range of kCsfRows
// rows). The group first writes its rows from the fixed tensor (each
// thread: a row base and 8 code bytes in, one 16-byte store out), then,
// after a work-group barrier, the exceptions of its expert whose position
// falls in its rows (it scans the expert's exception list: a few hundred
// entries at the rates the page implies), so an exception always lands
// after the fixed byte it replaces. With expert_offsets (the moe_permute
// output) groups of experts no slot is routed to exit at once, so a layer
// expands only the scales its batch reads; with a bound on the number of
// routed experts the grid has only that many expert rows, row y expanding
// the y-th routed expert.
#include "common.h"

namespace moe {

// 8 code bytes (16 nibbles, low nibble first) + base -> 16 scale bytes.
// base + code <= 240 + 15, so the per-byte adds never carry.
__device__ __forceinline__ uint4 csf_expand16(uint2 codes, uint32_t base) {
    const uint32_t b4 = base * 0x01010101u;
    const uint32_t lo0 = codes.x & 0x0F0F0F0Fu, hi0 = (codes.x >> 4) & 0x0F0F0F0Fu;
    const uint32_t lo1 = codes.y & 0x0F0F0F0Fu, hi1 = (codes.y >> 4) & 0x0F0F0F0Fu;
    // output byte 2m = low nibble of code byte m, byte 2m + 1 = its high nibble
    uint4 o;
    o.x = __builtin_amdgcn_perm(hi0, lo0, 0x05010400u) + b4;
    o.y = __builtin_amdgcn_perm(hi0, lo0, 0x07030602u) + b4;
    o.z = __builtin_amdgcn_perm(hi1, lo1, 0x05010400u) + b4;
    o.w = __builtin_amdgcn_perm(hi1, lo1, 0x07030602u) + b4;
    return o;
}

__device__ __forceinline__ bool csf_expert_skipped(const int32_t *offsets, int e) {
    return offsets && offsets[e + 1] == offsets[e];
}

constexpr int kCsfRows = 256;

// The y-th expert (in index order) with a routed slot, or -1: wave 0 counts
// the non-empty experts 64 at a time with a ballot.
__device__ int csf_routed_expert(const int32_t *offsets, int E, int y) {
    __shared__ int found;
    if (threadIdx.x < kWave) {
        const int lane = threadIdx.x;
        int seen = 0, e_y = -1;
        for (int e0 = 0; e0 < E && e_y < 0; e0 += kWave) {
            const int e = e0 + lane;
            const bool nz = e < E && offsets[e + 1] != offsets[e];
            const uint64_t m = __ballot(nz);
            const int cnt = __popcll(m);
            if (y < seen + cnt) {
                // the (y - seen)-th set bit of m
                uint64_t mm = m;
                for (int k = 0; k < y - seen; ++k) mm &= mm - 1;
                e_y = e0 + __ffsll((unsigned long long)mm) - 1;
            }
            seen += cnt;
        }
        if (lane == 0) found = e_y;
    }
    __syncthreads();
    return found;
}

__global__ void __launch_bounds__(256) csf_expand_kernel(
    const uint8_t *__restrict__ fixed, const uint32_t *__restrict__ exceptions, int64_t n,
    const int64_t *__restrict__ starts, int E, int R, int C,
    const int32_t *__restrict__ expert_offsets, int compact, uint8_t *__restrict__ out) {
    // compact grids give row y of the grid the y-th routed expert
    const int e = compact ? csf_routed_expert(expert_offsets, E, blockIdx.y) : (int)blockIdx.y;
    if (e < 0 || csf_expert_skipped(expert_offsets, e)) return;
    const int r0 = blockIdx.x * kCsfRows;
    const int r1 = min(R, r0 + kCsfRows);
    const int per_row = C / 16;
    const int slab_bytes = 16 * (1 + C / 2);
    const uint8_t *fx = fixed + (int64_t)e * (R / 16) * slab_bytes;
    uint8_t *dst = out + (int64_t)e * R * C;
    for (int u = threadIdx.x; u < (r1 - r0) * per_row; u += blockDim.x) {
        const int r = r0 + u / per_row, j = u % per_row;
        const uint8_t *slab = fx + (r / 16) * slab_bytes;
        const uint32_t base = slab[r % 16];
        const uint2 codes = *(const uint2 *)(slab + 16 + (r % 16) * (C / 2) + 8 * j);
        *(uint4 *)(dst + (int64_t)r * C + 16 * j) = csf_expand16(codes, base);
    }
    if (n == 0) return;
    // the fixed bytes of these rows are written before any exception here
    __threadfence_block();
    __syncthreads();
    // the expert's range, clamped to the array (malformed starts never read past it)
    int64_t a = starts[e], b = starts[e + 1];
    a = a < 0 ? 0 : (a > n ? n : a);
    b = b < a ? a : (b > n ? n : b);
    const uint32_t lo = (uint32_t)r0 * C, hi = (uint32_t)r1 * C;
    for (int64_t i = a + threadIdx.x; i < b; i += blockDim.x) {
        const uint32_t x = exceptions[i];
        const uint32_t pos = x & 0xFFFFFFu;
        if (pos >= lo && pos < hi) dst[pos] = (uint8_t)(x >> 24);   // positions past R*C: ignored
    }
}

// Row ranges of the exceptions: one work group per expert walks its
// exceptions (stored in ascending position); exception x, in row r_x, is
// the first exception of every row after the previous exception's row up
// to r_x, so it fills those entries; the rows after the last exception get
// the expert's end. Every entry is written exactly once.
__global__ void __launch_bounds__(256) csf_row_index_kernel(
    const uint32_t *__restrict__ exceptions, int64_t n, const int64_t *__restrict__ starts, int E,
    int R, int C, const int32_t *__restrict__ expert_offsets, int compact,
    int32_t *__restrict__ row_index) {
    const int e = compact ? csf_routed_expert(expert_offsets, E, blockIdx.y) : (int)blockIdx.y;
    if (e < 0 || csf_expert_skipped(expert_offsets, e)) return;
    int64_t lo = starts[e], hi = starts[e + 1];
    lo = lo < 0 ? 0 : (lo > n ? n : lo);
    hi = hi < lo ? lo : (hi > n ? n : hi);
    int32_t *ri = row_index + (size_t)e * (R + 1);
    // positions past the matrix belong to no row (row R stands for them all)
    auto row = [&](int64_t x) {
        const uint32_t q = (exceptions[x] & 0xFFFFFFu) / (uint32_t)C;
        return q < (uint32_t)R ? (int)q : R;
    };
    for (int64_t x = lo + threadIdx.x; x < hi; x += 256) {
        const int rx = row(x), rp = x > lo ? row(x - 1) : -1;
        for (int r = rp + 1; r <= rx; ++r) ri[r] = (int32_t)x;
    }
    const int rl = hi > lo ? row(hi - 1) : -1;           // after the last row with one
    for (int r = rl + 1 + threadIdx.x; r <= R; r += 256) ri[r] = (int32_t)hi;
}

moe_status_t launch_csf_row_index(const uint32_t *exceptions, int64_t n, const int64_t *starts,
                                  int E, int R, int C, const int32_t *expert_offsets,
                                  int max_routed, int32_t *row_index, hipStream_t s) {
    const bool compact = expert_offsets && max_routed > 0 && max_routed < E;
    const dim3 grid(1, compact ? max_routed : E);
    hipLaunchKernelGGL(csf_row_index_kernel, grid, dim3(256), 0, s, exceptions, n, starts, E, R,
                       C, expert_offsets, compact ? 1 : 0, row_index);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

// Expansion from the per-row exception ranges (the row index the in-place
// kernels read), for the forward pass at prefill sizes: one thread per
// (row, 16 scale bytes), so no barrier is needed; the thread applies the
// row's exceptions whose column falls in its 16 bytes. Experts with no
// routed slot exit at once.
__global__ void __launch_bounds__(256) csf_expand_rows_kernel(
    const uint8_t *__restrict__ fixed, int64_t fixed_expert_stride,
    const uint32_t *__restrict__ xc, const int32_t *__restrict__ ri,
    const int32_t *__restrict__ expert_offsets, int R, int C, uint8_t *__restrict__ out) {
    const int e = blockIdx.y;
    if (expert_offsets[e + 1] == expert_offsets[e]) return;
    const int chunks = C / 16;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)R * chunks) return;
    const int r = (int)(idx / chunks), j = (int)(idx % chunks);
    const uint8_t *slab =
        fixed + e * fixed_expert_stride + (size_t)(r >> 4) * 16 * (1 + C / 2);
    const uint2 codes = *(const uint2 *)(slab + 16 + (r & 15) * (C / 2) + 8 * j);
    uint4 o = csf_expand16(codes, slab[r & 15]);
    const int32_t *rix = ri + (size_t)e * (R + 1);
    const uint32_t p0 = (uint32_t)r * (uint32_t)C + 16u * (uint32_t)j;
    for (int x = rix[r]; x < rix[r + 1]; ++x) {
        const uint32_t v = xc[x], d = (v & 0xFFFFFFu) - p0;
        if (d < 16) {
            const uint32_t sh = 8 * (d & 3), m = ~(0xFFu << sh), b = (v >> 24) << sh;
            if (d < 4) o.x = (o.x & m) | b;
            else if (d < 8) o.y = (o.y & m) | b;
            else if (d < 12) o.z = (o.z & m) | b;
            else o.w = (o.w & m) | b;
        }
    }
    *(uint4 *)(out + ((size_t)e * R + r) * C + 16 * j) = o;
}

moe_status_t launch_csf_expand_rows(const moe_weight_desc_t &d, const int32_t *expert_offsets,
                                    uint8_t *out, hipStream_t s) {
    const int R = d.n, C = d.k / 16;
    const dim3 grid((unsigned)(((int64_t)R * (C / 16) + 255) / 256), d.num_experts);
    hipLaunchKernelGGL(csf_expand_rows_kernel, grid, dim3(256), 0, s, (const uint8_t *)d.scale,
                       d.scale_expert_stride, d.csf_exceptions, d.csf_row_index, expert_offsets, R,
                       C, out);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

moe_status_t launch_csf_expand(const uint8_t *fixed, const uint32_t *exceptions, int64_t n,
                               const int64_t *starts, int E, int R, int C,
                               const int32_t *expert_offsets, int max_routed, uint8_t *out,
                               hipStream_t s) {
    const bool compact = expert_offsets && max_routed > 0 && max_routed < E;
    const dim3 grid((R + kCsfRows - 1) / kCsfRows, compact ? max_routed : E);
    hipLaunchKernelGGL(csf_expand_kernel, grid, dim3(256), 0, s, fixed, exceptions, n, starts, E,
                       R, C, expert_offsets, compact ? 1 : 0, out);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

}  // namespace moe
