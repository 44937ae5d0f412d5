// C ABI of the MoE library: host-side validation, workspace planning and
// dispatch to the kernels. Every check runs before the first launch, so an
// invalid call enqueues nothing.
#include <string.h>

#include <functional>
#include <mutex>

#include "common.h"

namespace moe {
moe_status_t launch_router_logits(const void *x, int x_dtype, const float *wT, const float *bias,
                                  int T, int H, int E, float *logits, hipStream_t s);
moe_status_t launch_topk(const float *logits, const float *bias, int T, int E, int K, int renorm,
                         int32_t *ids, float *wts, hipStream_t s, int P = 1);
moe_status_t launch_router_scores(const void *x, int x_dtype, const float *wT, int T, int H,
                                  int E, float *part, int *P, hipStream_t s);
size_t router_ws_floats(int T, int H, int E, int x_dtype);
size_t router_ws_floats_max(int T, int E);
int router_blocks(int H);
moe_status_t launch_permute(const int32_t *ids, int T, int K, int E, const moe_perm_t &p,
                            hipStream_t s);
bool route_perm_fused(int T, int K);
moe_status_t launch_route_perm_small(const float *scores, const float *bias, int T, int E, int K,
                                     int renorm, int P, int32_t *ids, float *wts,
                                     const moe_perm_t &p, hipStream_t s);
moe_status_t launch_dequant(const moe_weight_desc_t &d, int e, float *out, hipStream_t s);
moe_status_t launch_csf_expand(const uint8_t *fixed, const uint32_t *exceptions, int64_t n,
                               const int64_t *starts, int E, int R, int C,
                               const int32_t *expert_offsets, int max_routed, uint8_t *out,
                               hipStream_t s);
moe_status_t launch_csf_row_index(const uint32_t *exceptions, int64_t n, const int64_t *starts,
                                  int E, int R, int C, const int32_t *expert_offsets,
                                  int max_routed, int32_t *row_index, hipStream_t s);
moe_status_t launch_gemv_forward(const moe_ffn_desc_t &ex, const void *x, int act, int K,
                                 const moe_perm_t &p, int max_tiles, void *h, float *y,
                                 hipStream_t s, const std::function<moe_status_t(int)> &mark);
bool gemv_mx_supported(const moe_ffn_desc_t &ex, int act, int T, int K);
moe_status_t launch_gemv_mx_forward(const moe_ffn_desc_t &ex, const void *x, int act, int K,
                                    const moe_perm_t &p, int max_tiles, void *h, float *y,
                                    hipStream_t s, const std::function<moe_status_t(int)> &mark);
moe_status_t launch_combine(const float *y, const uint16_t *y16, const int8_t *yexp,
                            const int32_t *slot_to_row, const float *w, int T, int K, int H,
                            const float *shared, const float *residual, void *out, int out_dtype,
                            hipStream_t s);
moe_status_t launch_gemm_forward(const moe_ffn_desc_t &ex, const void *x, int act, int T, int K,
                                 const moe_perm_t &p, int max_tiles, void *h, float *y,
                                 uint16_t *y16, int8_t *yexp, void *xperm, float *xsum,
                                 float *hsum, hipStream_t s,
                                 const std::function<moe_status_t(int)> &mark);
bool gemm_stores_y16(int fmt);
moe_status_t launch_dense_swiglu(const moe_ffn_desc_t &sh, const void *x, int T, void *h,
                                 float *y, float *part, hipStream_t s);
moe_status_t launch_round(const float *in, size_t n, int dtype, void *out, hipStream_t s);
bool norm_route_fused(int T, int H, int E);
moe_status_t launch_csf_expand_rows(const moe_weight_desc_t &d, const int32_t *expert_offsets,
                                    uint8_t *out, hipStream_t s);
moe_status_t launch_norm_router_scores(const float *res, const float *gain, float eps, int T,
                                       int H, const float *wT, int E, void *a_out, float *part,
                                       hipStream_t s);
moe_status_t launch_rmsnorm(const float *x, const float *w, float eps, int T, int H, int dtype,
                            void *out, hipStream_t s);
moe_status_t launch_act_quant(const void *in, int dtype, int64_t rows, int k, float g,
                              void *out, const int32_t *row_slot, hipStream_t s);
DenseSplit dense_plan(int T, int H, int F);
bool dense_shape_ok(int H, int F);
int gemv_tile_m();
int gemv_mx_tile_m(int T, int K, int E);
int gemm_tile_m();
int gemm_group();
int gemm_bn();
}  // namespace moe

using namespace moe;

namespace {

constexpr int kMaxExperts = 512;
constexpr int kMaxTopK = 16;
constexpr int kMaxDim = 16384;
// Bytes a 32-bit buffer offset reaches, with room for a step past a row.
constexpr int64_t kMaxBufferBytes = ((int64_t)1 << 31) - ((int64_t)1 << 20);

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
inline bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int64_t perm_max_rows(int T, int K, int E, int tile_m) {
    const int64_t n = (int64_t)T * K;
    return n + (n < E ? n : E) * (int64_t)(tile_m - 1);
}

// An input scale of the NVFP4-activation forms: 0 (16-bit inputs) or a
// finite float32 in [2^-100, 2^100] (so 6 g and every bs g stay normal).
bool input_scale_ok(float g) { return g == 0.0f || (g >= 0x1p-100f && g <= 0x1p100f); }

// A quantized bank of E matrices [n][k]: format rules and alignment.
moe_status_t check_bank(const moe_weight_desc_t &d, int E, int n, int k) {
    if (d.num_experts != E || d.n != n || d.k != k) return MOE_ERR_INVALID_ARG;
    if (!input_scale_ok(d.input_scale)) return MOE_ERR_INVALID_ARG;
    if (d.input_scale != 0.0f && d.fmt != MOE_W_NVFP4_G16 && d.fmt != MOE_W_NVFP4_CSF)
        return MOE_ERR_INVALID_ARG;
    if (!d.qweight || !d.scale) return MOE_ERR_INVALID_ARG;
    if (n <= 0 || k <= 0 || n > kMaxDim || k > kMaxDim) return MOE_ERR_INVALID_ARG;
    if (!aligned(d.qweight, 16) || d.qweight_row_stride % 16 || d.qweight_expert_stride % 16)
        return MOE_ERR_INVALID_ARG;
    if (!aligned(d.scale, 2) || d.scale_row_stride % 2 || d.scale_expert_stride % 2)
        return MOE_ERR_INVALID_ARG;
    if (d.fmt == MOE_W_INT4_G128 || d.fmt == MOE_W_INT4_G128_ASYM) {
        if (k % 128) return MOE_ERR_INVALID_ARG;
        if (d.qweight_row_stride < k / 2 || d.scale_row_stride < (k / 128) * 2)
            return MOE_ERR_INVALID_ARG;
        if (d.fmt == MOE_W_INT4_G128_ASYM &&
            (!d.zero_point || d.zero_point_row_stride < k / 128 || d.zero_point_expert_stride < 0))
            return MOE_ERR_INVALID_ARG;
    } else if (d.fmt == MOE_W_INT8_G128) {
        if (k % 128) return MOE_ERR_INVALID_ARG;
        if (d.qweight_row_stride < k || d.scale_row_stride < (k / 128) * 2)
            return MOE_ERR_INVALID_ARG;
    } else if (d.fmt == MOE_W_INT4_G32) {
        if (k % 32) return MOE_ERR_INVALID_ARG;
        if (d.qweight_row_stride < k / 2 || d.scale_row_stride < (k / 32) * 2)
            return MOE_ERR_INVALID_ARG;
    } else if (d.fmt == MOE_W_NVFP4_CSF) {
        // codes as NVFP4; scales: the CSF fixed tensor, 16-row slabs
        if (k % 16 || n % 16) return MOE_ERR_INVALID_ARG;
        if (k % 32) return MOE_ERR_UNSUPPORTED;
        if ((int64_t)n * (k / 16) >= ((int64_t)1 << 24)) return MOE_ERR_UNSUPPORTED;
        if (!d.global_scale || !aligned(d.global_scale, 4) || !d.csf_row_index ||
            !aligned(d.csf_row_index, 4) || (d.csf_exceptions && !aligned(d.csf_exceptions, 4)))
            return MOE_ERR_INVALID_ARG;
        if (d.qweight_row_stride < k / 2 ||
            d.scale_expert_stride < (int64_t)n * (1 + k / 32))
            return MOE_ERR_INVALID_ARG;
    } else if (d.fmt == MOE_W_NVFP4_G16) {
        if (k % 16) return MOE_ERR_INVALID_ARG;
        if (k % 32) return MOE_ERR_UNSUPPORTED;     // kernels read 32 inputs per 16 bytes
        if (!d.global_scale || !aligned(d.global_scale, 4)) return MOE_ERR_INVALID_ARG;
        if (d.qweight_row_stride < k / 2 || d.scale_row_stride < k / 16)
            return MOE_ERR_INVALID_ARG;
    } else {
        return MOE_ERR_INVALID_ARG;
    }
    return MOE_OK;
}

moe_status_t check_experts(const moe_ffn_desc_t *ex, int *E, int *H, int *F) {
    if (!ex) return MOE_ERR_INVALID_ARG;
    const int e = ex->gate.num_experts, f = ex->gate.n, h = ex->gate.k;
    if (e < 1 || e > kMaxExperts) return MOE_ERR_INVALID_ARG;
    if (ex->up.fmt != ex->gate.fmt || ex->down.fmt != ex->gate.fmt) return MOE_ERR_INVALID_ARG;
    moe_status_t st;
    if ((st = check_bank(ex->gate, e, f, h)) != MOE_OK) return st;
    if ((st = check_bank(ex->up, e, f, h)) != MOE_OK) return st;
    if ((st = check_bank(ex->down, e, h, f)) != MOE_OK) return st;
    // quantized inputs: gate and up read the same x (one input scale), and
    // the down projection's input is quantized too
    if (ex->gate.input_scale != ex->up.input_scale ||
        (ex->gate.input_scale > 0.0f) != (ex->down.input_scale > 0.0f))
        return MOE_ERR_INVALID_ARG;
    *E = e; *H = h; *F = f;
    return MOE_OK;
}

bool is_act(int d) { return d == MOE_F16 || d == MOE_BF16; }

// The shared expert: one BF16 SwiGLU of any width Fs over the same H.
moe_status_t check_dense(const moe_weight_desc_t &d, int n, int k) {
    if (d.fmt != MOE_W_BF16 || d.num_experts != 1 || d.n != n || d.k != k || !d.qweight)
        return MOE_ERR_INVALID_ARG;
    if (n <= 0 || k <= 0 || n > kMaxDim || k > kMaxDim) return MOE_ERR_INVALID_ARG;
    if (!aligned(d.qweight, 16) || d.qweight_row_stride % 16 || d.qweight_row_stride < 2 * k)
        return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

moe_status_t check_shared(const moe_ffn_desc_t *sh, int H, int act, int *Fs) {
    if (!sh) { *Fs = 0; return MOE_OK; }
    const int f = sh->gate.n;
    moe_status_t st;
    if ((st = check_dense(sh->gate, f, H)) != MOE_OK) return st;
    if ((st = check_dense(sh->up, f, H)) != MOE_OK) return st;
    if ((st = check_dense(sh->down, H, f)) != MOE_OK) return st;
    if (act != MOE_BF16) return MOE_ERR_INVALID_ARG;      // bf16 x bf16 MFMA
    if (!dense_shape_ok(H, f)) return MOE_ERR_UNSUPPORTED;
    *Fs = f;
    return MOE_OK;
}

moe_status_t check_perm(const moe_perm_t *p) {
    if (!p || !p->counts || !p->expert_offsets || !p->padded_offsets || !p->sorted_slots ||
        !p->slot_to_row || !p->tile_expert || !p->num_tiles || !p->active_experts ||
        !p->num_active)
        return MOE_ERR_INVALID_ARG;
    if (p->tile_m < 1 || p->tile_m > 256) return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

struct FwdPlan {
    bool mfma;
    int tile_m;
    int64_t max_rows, max_tiles;
    size_t off_h, off_y, off_xperm, off_xsum, off_hsum;
    size_t off_sh_h, off_sh_y, off_sh_part, off_csf, off_xq, total;
};

// Kernel choice by batch shape: with few slots per expert the dequantizing
// GEMV streams each touched expert once per tile of 4 or 8 slots; once the
// average expert sees several tiles' worth of slots (T*K >= 4*E; at the
// layer's shape NVFP4 8*E and int4-g128 7*E, with the MFMA GEMV's 8-slot
// tiles in between) the
// MFMA grouped GEMM, which reads each weight once per tile of 64 slots,
// takes over. One code path per shape class.
bool mfma_layout_ok(const moe_weight_desc_t &d) {
    // compressed scales reach the GEMM expanded into the workspace (aligned
    // there); the expansion reads 8 code bytes at a time
    if (d.fmt == MOE_W_NVFP4_CSF)
        return aligned(d.scale, 8) && d.scale_expert_stride % 8 == 0;
    // the GEMM loads a step's scales as one 4-byte (int4) or 16-byte (NVFP4)
    // word, and an asymmetric bank's two zero points as one 2-byte word
    // (int4-g32: the step's eight bf16 scales, 16 bytes)
    const bool i4 = d.fmt == MOE_W_INT4_G128 || d.fmt == MOE_W_INT4_G128_ASYM ||
                    d.fmt == MOE_W_INT8_G128;
    const int64_t a = i4 ? 4 : 16;
    const bool zp = d.fmt != MOE_W_INT4_G128_ASYM ||
                    (aligned(d.zero_point, 2) && d.zero_point_row_stride % 2 == 0 &&
                     d.zero_point_expert_stride % 2 == 0 &&
                     (int64_t)d.n * d.zero_point_row_stride < INT32_MAX);
    return aligned(d.scale, a) && d.scale_row_stride % a == 0 && d.scale_expert_stride % a == 0 &&
           zp;
}

bool use_mfma(const moe_ffn_desc_t &ex, int T, int K) {
    const int E = ex.gate.num_experts, H = ex.gate.k, F = ex.gate.n;
    // the GEMM decodes every format (compressed NVFP4 scales after their
    // expansion into the workspace)
    const int f = ex.gate.fmt;
    if (f != MOE_W_INT4_G128 && f != MOE_W_INT4_G128_ASYM && f != MOE_W_INT4_G32 &&
        f != MOE_W_INT8_G128 && f != MOE_W_NVFP4_G16 && f != MOE_W_NVFP4_CSF)
        return false;
    // at the layer's shape from 4E slots to 8E (NVFP4) or 7E (int4-g128,
    // both forms): the MFMA GEMV with 8-slot tiles
    if ((f == MOE_W_NVFP4_G16 || f == MOE_W_INT4_G128 || f == MOE_W_INT4_G128_ASYM) &&
        gemv_mx_supported(ex, MOE_F16, T, K))
        return false;
    // 32-bit buffer offsets must reach every row of an expert matrix
    const bool fits = (int64_t)F * ex.gate.qweight_row_stride < INT32_MAX &&
                      (int64_t)F * ex.up.qweight_row_stride < INT32_MAX &&
                      (int64_t)H * ex.down.qweight_row_stride < INT32_MAX;
    // K steps of gemm_group() inputs; gate/up blocks of gemm_bn() columns,
    // down blocks of 2 * gemm_bn()
    return (int64_t)T * K >= 4 * (int64_t)E && H % gemm_group() == 0 &&
           F % gemm_group() == 0 && F % gemm_bn() == 0 && H % (2 * gemm_bn()) == 0 && fits &&
           mfma_layout_ok(ex.gate) && mfma_layout_ok(ex.up) && mfma_layout_ok(ex.down);
}

size_t csf_bytes(const moe_weight_desc_t &d) {
    return align256((size_t)d.num_experts * d.n * (d.k / 16));
}

FwdPlan plan_forward(const moe_ffn_desc_t &ex, int T, int K, int E, int H, int F, int Fs) {
    FwdPlan p;
    p.mfma = use_mfma(ex, T, K);
    p.tile_m = p.mfma ? gemm_tile_m()
               : gemv_mx_supported(ex, MOE_F16, T, K) ? gemv_mx_tile_m(T, K, E) : gemv_tile_m();
    p.max_rows = perm_max_rows(T, K, E, p.tile_m);
    p.max_tiles = p.max_rows / p.tile_m;
    p.off_h = 0;
    p.off_y = align256((size_t)p.max_rows * F * 2);
    // MFMA path, int4 (every form) and int8: x in the decoder's pair order,
    // and per-row sums of each 128-input group of x and of h (unused by
    // int4-g32)
    const bool sums = p.mfma && ex.gate.fmt != MOE_W_NVFP4_G16 && ex.gate.fmt != MOE_W_NVFP4_CSF;
    p.off_xperm = p.off_y + align256((size_t)p.max_rows * H * 4);
    p.off_xsum = p.off_xperm + (sums ? align256((size_t)T * H * 2) : 0);
    p.off_hsum = p.off_xsum + (sums ? align256((size_t)T * (H / 128) * 4) : 0);
    p.off_sh_h = p.off_hsum + (sums ? align256((size_t)p.max_rows * (F / 128) * 4) : 0);
    // shared expert: h [T][Fs] bf16, y [T][H] float32, split partial sums
    const size_t part = Fs ? dense_plan(T, H, Fs).part_floats : 0;
    p.off_sh_y = p.off_sh_h + (Fs ? align256((size_t)T * Fs * 2) : 0);
    p.off_sh_part = p.off_sh_y + (Fs ? align256((size_t)T * H * 4) : 0);
    p.off_csf = p.off_sh_part + align256(part * 4);
    // MFMA path, compressed NVFP4 scales: every routed expert's E4M3 block
    // scales of gate, up and down, expanded ([E][n][k/16] each)
    const bool csf = p.mfma && ex.gate.fmt == MOE_W_NVFP4_CSF;
    p.off_xq = p.off_csf + (csf ? csf_bytes(ex.gate) + csf_bytes(ex.up) + csf_bytes(ex.down) : 0);
    // quantized inputs: the quantized x [T][H] (16-bit values e2m1 x bs)
    const bool a4 = ex.gate.input_scale > 0.0f;
    p.total = p.off_xq + (a4 ? align256((size_t)T * H * 2) : 0);
    return p;
}

}  // namespace

extern "C" {

const char *moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
        case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
        case MOE_ERR_HIP: return "MOE_ERR_HIP";
        default: return "MOE_ERR_UNKNOWN";
    }
}

int moe_abi_version(void) { return 6; }

static moe_status_t check_router(const void *x, int x_dtype, const float *wT, int T, int H,
                                 int E) {
    if (T < 0 || E < 1 || E > kMaxExperts) return MOE_ERR_INVALID_ARG;
    if (!wT || !is_act(x_dtype) || H < 1) return MOE_ERR_INVALID_ARG;
    if (T > 0 && !x) return MOE_ERR_INVALID_ARG;
    if (H % 64 || E % 4) return MOE_ERR_UNSUPPORTED;
    if (!aligned(wT, 16) || (x && !aligned(x, 16))) return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

moe_status_t moe_router_logits(const void *x, int x_dtype, const float *router_wT,
                               const float *bias, int T, int H, int E, float *logits,
                               void *stream) {
    moe_status_t st = check_router(x, x_dtype, router_wT, T, H, E);
    if (st != MOE_OK) return st;
    if (T > 0 && !logits) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    return launch_router_logits(x, x_dtype, router_wT, bias, T, H, E, logits,
                                (hipStream_t)stream);
}

moe_status_t moe_route_workspace(int T, int E, int use_router_weight, size_t *bytes) {
    if (T < 0 || E < 1 || E > kMaxExperts || !bytes) return MOE_ERR_INVALID_ARG;
    *bytes = use_router_weight ? router_ws_floats_max(T, E) * 4 : 0;
    return MOE_OK;
}

moe_status_t moe_route_topk(const void *x, int x_dtype, const float *router_wT,
                            const float *logits_in, const float *bias, int T, int H, int E,
                            int K, int renormalize, int32_t *topk_ids, float *topk_w, void *ws,
                            size_t ws_bytes, void *stream) {
    if (T < 0 || E < 1 || E > kMaxExperts || K < 1 || K > E || K > kMaxTopK)
        return MOE_ERR_INVALID_ARG;
    if (!topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
    if ((router_wT == nullptr) == (logits_in == nullptr)) return MOE_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    if (router_wT) {
        moe_status_t st = check_router(x, x_dtype, router_wT, T, H, E);
        if (st != MOE_OK) return st;
        if (T > 0 && !ws) return MOE_ERR_INVALID_ARG;
        if (ws_bytes < router_ws_floats(T, H, E, x_dtype) * 4) return MOE_ERR_WORKSPACE_TOO_SMALL;
        if (ws && !aligned(ws, 16)) return MOE_ERR_INVALID_ARG;
        if (T == 0) return MOE_OK;
        float *part = (float *)ws;
        int P = 1;
        st = launch_router_scores(x, x_dtype, router_wT, T, H, E, part, &P, s);
        if (st != MOE_OK) return st;
        return launch_topk(part, bias, T, E, K, renormalize, topk_ids, topk_w, s, P);
    }
    if (T == 0) return MOE_OK;
    return launch_topk(logits_in, bias, T, E, K, renormalize, topk_ids, topk_w, s);
}

moe_status_t moe_route_permute(const void *x, int x_dtype, const float *router_wT,
                               const float *logits_in, const float *bias, int T, int H, int E,
                               int K, int renormalize, int32_t *topk_ids, float *topk_w,
                               const moe_perm_t *perm, void *ws, size_t ws_bytes,
                               void *stream) {
    if (T < 0 || E < 1 || E > kMaxExperts || K < 1 || K > E || K > kMaxTopK)
        return MOE_ERR_INVALID_ARG;
    if (!topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
    if ((router_wT == nullptr) == (logits_in == nullptr)) return MOE_ERR_INVALID_ARG;
    if ((int64_t)T * K > (1 << 24)) return MOE_ERR_UNSUPPORTED;
    moe_status_t st = check_perm(perm);
    if (st != MOE_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    const float *scores = logits_in;
    int P = 1;
    if (router_wT) {
        if ((st = check_router(x, x_dtype, router_wT, T, H, E)) != MOE_OK) return st;
        if (T > 0 && !ws) return MOE_ERR_INVALID_ARG;
        if (ws_bytes < router_ws_floats(T, H, E, x_dtype) * 4) return MOE_ERR_WORKSPACE_TOO_SMALL;
        if (ws && !aligned(ws, 16)) return MOE_ERR_INVALID_ARG;
        if (T == 0) return MOE_OK;
        st = launch_router_scores(x, x_dtype, router_wT, T, H, E, (float *)ws, &P, s);
        if (st != MOE_OK) return st;
        scores = (const float *)ws;
    }
    if (T == 0) return MOE_OK;
    if (route_perm_fused(T, K))
        return launch_route_perm_small(scores, bias, T, E, K, renormalize, P, topk_ids, topk_w,
                                       *perm, s);
    if ((st = launch_topk(scores, bias, T, E, K, renormalize, topk_ids, topk_w, s, P)) != MOE_OK)
        return st;
    return launch_permute(topk_ids, T, K, E, *perm, s);
}

moe_status_t moe_permute_sizes(int T, int K, int E, int tile_m, int64_t *max_rows,
                               int64_t *max_tiles) {
    if (T < 0 || K < 1 || E < 1 || E > kMaxExperts || tile_m < 1 || tile_m > 256 ||
        !max_rows || !max_tiles)
        return MOE_ERR_INVALID_ARG;
    *max_rows = perm_max_rows(T, K, E, tile_m);
    *max_tiles = *max_rows / tile_m;
    return MOE_OK;
}

moe_status_t moe_permute(const int32_t *topk_ids, int T, int K, int E, const moe_perm_t *perm,
                         void *stream) {
    if (T < 0 || K < 1 || E < 1 || E > kMaxExperts) return MOE_ERR_INVALID_ARG;
    if ((int64_t)T * K > (1 << 24)) return MOE_ERR_UNSUPPORTED;
    if (T > 0 && !topk_ids) return MOE_ERR_INVALID_ARG;
    moe_status_t st = check_perm(perm);
    if (st != MOE_OK) return st;
    return launch_permute(topk_ids, T, K, E, *perm, (hipStream_t)stream);
}

moe_status_t moe_forward_plan(const moe_ffn_desc_t *experts, const moe_ffn_desc_t *shared,
                              int T, int K, int act_dtype, int *tile_m, size_t *ws_bytes) {
    int E, H, F;
    moe_status_t st = check_experts(experts, &E, &H, &F);
    if (st != MOE_OK) return st;
    if (T < 0 || K < 1 || K > E || K > kMaxTopK || !is_act(act_dtype) || !tile_m || !ws_bytes)
        return MOE_ERR_INVALID_ARG;
    int Fs;
    if ((st = check_shared(shared, H, act_dtype, &Fs)) != MOE_OK) return st;
    const FwdPlan p = plan_forward(*experts, T, K, E, H, F, Fs);
    *tile_m = p.tile_m;
    *ws_bytes = p.total;
    return MOE_OK;
}

static moe_status_t forward_impl(const moe_ffn_desc_t *experts, const moe_ffn_desc_t *shared,
                                 const void *x, int act_dtype, int T, int K,
                                 const float *topk_w, const moe_perm_t *perm,
                                 const float *residual, void *out, int out_dtype, void *ws,
                                 size_t ws_bytes, void *stream, void *const *events,
                                 int n_events) {
    int E, H, F;
    moe_status_t st = check_experts(experts, &E, &H, &F);
    if (st != MOE_OK) return st;
    if (T < 0 || K < 1 || K > E || K > kMaxTopK || !is_act(act_dtype)) return MOE_ERR_INVALID_ARG;
    if (out_dtype != MOE_F32 && !is_act(out_dtype)) return MOE_ERR_INVALID_ARG;
    if ((st = check_perm(perm)) != MOE_OK) return st;
    int Fs;
    if ((st = check_shared(shared, H, act_dtype, &Fs)) != MOE_OK) return st;
    if (events && n_events != MOE_FORWARD_STAGES + 1) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if (!x || !topk_w || !out || !ws) return MOE_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(out, 16) || !aligned(ws, 256) ||
        (residual && !aligned(residual, 16)))
        return MOE_ERR_INVALID_ARG;
    const FwdPlan p = plan_forward(*experts, T, K, E, H, F, Fs);
    if (perm->tile_m != p.tile_m) return MOE_ERR_INVALID_ARG;
    if (ws_bytes < p.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
    if (!p.mfma && p.max_tiles > 65535) return MOE_ERR_UNSUPPORTED;     // grid.y
    if (p.mfma && p.max_tiles * ((H > F ? H : F) / 128 + 1) > (int64_t)1 << 30)
        return MOE_ERR_UNSUPPORTED;
    // the grouped GEMM reads x and h through 32-bit buffer offsets
    if (p.mfma && ((int64_t)T * H * 2 > kMaxBufferBytes || p.max_rows * F * 2 > kMaxBufferBytes))
        return MOE_ERR_UNSUPPORTED;

    hipStream_t s = (hipStream_t)stream;
    auto mark = [&](int i) -> moe_status_t {
        if (events && events[i] && hipEventRecord((hipEvent_t)events[i], s) != hipSuccess)
            return MOE_ERR_HIP;
        return MOE_OK;
    };
    char *w = (char *)ws;
    void *h = w + p.off_h;
    float *y = (float *)(w + p.off_y);
    // the grouped-GEMM path stores y (but for int4-g32) in fp16 with a
    // power-of-two scale per (row, 32-column group) in the same region:
    // [max_rows][H] fp16, then [max_rows][H / 32] signed bytes
    const bool y16_on = p.mfma && gemm_stores_y16(experts->gate.fmt);
    uint16_t *y16 = y16_on ? (uint16_t *)y : nullptr;
    int8_t *yexp = y16_on ? (int8_t *)(y16 + (size_t)p.max_rows * H) : nullptr;
    if ((st = mark(0)) != MOE_OK) return st;
    // quantized inputs (NVFP4 banks with input scales): x is quantized with
    // the gate/up input scale before the experts run, and h in place with
    // the down input scale between the two projections; the kernels
    // multiply their accumulators by the input scale with the global scale
    const bool a4 = experts->gate.input_scale > 0.0f;
    const void *xin = x;
    if (a4) {
        void *xq = w + p.off_xq;
        st = launch_act_quant(x, act_dtype, T, H, experts->gate.input_scale, xq, nullptr, s);
        if (st != MOE_OK) return st;
        xin = xq;
    }
    auto between = [&](int i) -> moe_status_t {
        moe_status_t r = mark(i);
        if (r == MOE_OK && i == 1 && a4)
            r = launch_act_quant(h, act_dtype, p.max_rows, F, experts->down.input_scale, h,
                                 perm->sorted_slots, s);
        return r;
    };
    const std::function<moe_status_t(int)> mk =
        events || a4 ? std::function<moe_status_t(int)>(between)
                     : std::function<moe_status_t(int)>();
    moe_ffn_desc_t ex = *experts;
    if (p.mfma && ex.gate.fmt == MOE_W_NVFP4_CSF) {
        // prefill sizes: the routed experts' compressed scales expanded into
        // the workspace, then the NVFP4 GEMM (the in-place GEMV rereads each
        // expert once per 4-slot tile)
        uint8_t *sc = (uint8_t *)(w + p.off_csf);
        moe_weight_desc_t *mats[3] = {&ex.gate, &ex.up, &ex.down};
        for (moe_weight_desc_t *d : mats) {
            st = launch_csf_expand_rows(*d, perm->expert_offsets, sc, s);
            if (st != MOE_OK) return st;
            d->fmt = MOE_W_NVFP4_G16;
            d->scale = sc;
            d->scale_row_stride = d->k / 16;
            d->scale_expert_stride = (int64_t)d->n * (d->k / 16);
            d->csf_exceptions = nullptr;
            d->csf_row_index = nullptr;
            sc += csf_bytes(*d);
        }
    }
    st = p.mfma ? launch_gemm_forward(ex, xin, act_dtype, T, K, *perm, (int)p.max_tiles, h, y,
                                      y16, yexp, w + p.off_xperm, (float *)(w + p.off_xsum),
                                      (float *)(w + p.off_hsum), s, mk)
         : gemv_mx_supported(*experts, act_dtype, T, K)
             ? launch_gemv_mx_forward(*experts, xin, act_dtype, K, *perm, (int)p.max_tiles, h, y,
                                      s, mk)
             : launch_gemv_forward(*experts, xin, act_dtype, K, *perm, (int)p.max_tiles, h, y, s,
                                   mk);
    if (st != MOE_OK) return st;
    float *ysh = shared ? (float *)(w + p.off_sh_y) : nullptr;
    if (shared) {
        st = launch_dense_swiglu(*shared, x, T, w + p.off_sh_h, ysh, (float *)(w + p.off_sh_part),
                                 s);
        if (st != MOE_OK) return st;
    }
    if ((st = mark(3)) != MOE_OK) return st;
    st = launch_combine(y, y16, yexp, perm->slot_to_row, topk_w, T, K, H, ysh, residual, out,
                        out_dtype, s);
    if (st != MOE_OK) return st;
    return mark(4);
}

moe_status_t moe_w4a16_forward(const moe_ffn_desc_t *experts, const moe_ffn_desc_t *shared,
                               const void *x, int act_dtype, int T, int K, const float *topk_w,
                               const moe_perm_t *perm, const float *residual, void *out,
                               int out_dtype, void *ws, size_t ws_bytes, void *stream) {
    return forward_impl(experts, shared, x, act_dtype, T, K, topk_w, perm, residual, out,
                        out_dtype, ws, ws_bytes, stream, nullptr, 0);
}

moe_status_t moe_w4a16_forward_profiled(const moe_ffn_desc_t *experts,
                                        const moe_ffn_desc_t *shared, const void *x,
                                        int act_dtype, int T, int K, const float *topk_w,
                                        const moe_perm_t *perm, const float *residual,
                                        void *out, int out_dtype, void *ws, size_t ws_bytes,
                                        void *stream, void *const *events, int n_events) {
    if (!events) return MOE_ERR_INVALID_ARG;
    return forward_impl(experts, shared, x, act_dtype, T, K, topk_w, perm, residual, out,
                        out_dtype, ws, ws_bytes, stream, events, n_events);
}

}  // extern "C"

// ---- the forward pass on library-owned device memory ----------------------
// For callers that cannot allocate device memory: one static device array,
// of which every GPU the library runs on holds its own copy until the
// process ends. Its device address is looked up once per device (host code
// must never pass the array's own name to a kernel: on the host that name
// is a stand-in, not a device address).
static __device__ __align__(256) uint8_t scratch[MOE_FORWARD_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

moe_status_t scratch_of_current_device(void **p) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return MOE_ERR_HIP;
        g_scratch_ptr[dev] = q;
    }
    *p = g_scratch_ptr[dev];
    return MOE_OK;
}
}  // namespace

extern "C" {

moe_status_t moe_w4a16_forward_scratch(const moe_ffn_desc_t *experts,
                                       const moe_ffn_desc_t *shared, const void *x,
                                       int act_dtype, int T, int K, const float *topk_w,
                                       const moe_perm_t *perm, const float *residual,
                                       void *out, int out_dtype, void *stream) {
    int tile_m = 0;
    size_t need = 0;
    moe_status_t st = moe_forward_plan(experts, shared, T, K, act_dtype, &tile_m, &need);
    if (st != MOE_OK) return st;
    if (need > (size_t)MOE_FORWARD_SCRATCH_BYTES) return MOE_ERR_WORKSPACE_TOO_SMALL;
    void *ws = nullptr;
    if ((st = scratch_of_current_device(&ws)) != MOE_OK) return st;
    return forward_impl(experts, shared, x, act_dtype, T, K, topk_w, perm, residual, out,
                        out_dtype, ws, (size_t)MOE_FORWARD_SCRATCH_BYTES, stream, nullptr, 0);
}

moe_status_t moe_round_activations(const float *in, int64_t n, int out_dtype, void *out,
                                   void *stream) {
    if (n < 0 || !is_act(out_dtype)) return MOE_ERR_INVALID_ARG;
    if (n == 0) return MOE_OK;
    if (!in || !out || !aligned(in, 16) || !aligned(out, 16)) return MOE_ERR_INVALID_ARG;
    return launch_round(in, (size_t)n, out_dtype, out, (hipStream_t)stream);
}

moe_status_t moe_rmsnorm(const float *x, const float *weight, float eps, int T, int H,
                         int out_dtype, void *out, void *stream) {
    if (T < 0 || H < 4 || H > kMaxDim || H % 4 || !is_act(out_dtype)) return MOE_ERR_INVALID_ARG;
    if (!(eps >= 0.0f) || eps > 1.0f) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if (!x || !out || !aligned(x, 16) || !aligned(out, 16) || (weight && !aligned(weight, 16)))
        return MOE_ERR_INVALID_ARG;
    return launch_rmsnorm(x, weight, eps, T, H, out_dtype, out, (hipStream_t)stream);
}

moe_status_t moe_norm_route(const float *residual, const float *norm_w, float eps, int T, int H,
                            const float *router_wT, const float *bias, int E, int K,
                            int renormalize, void *a_out, int32_t *topk_ids, float *topk_w,
                            void *ws, size_t ws_bytes, void *stream) {
    if (T < 0 || H < 4 || H > kMaxDim || E < 1 || E > kMaxExperts || K < 1 || K > E ||
        K > kMaxTopK)
        return MOE_ERR_INVALID_ARG;
    if (!(eps >= 0.0f) || eps > 1.0f || !router_wT) return MOE_ERR_INVALID_ARG;
    if (H % 64 || E % 4) return MOE_ERR_UNSUPPORTED;
    if (ws_bytes < router_ws_floats(T, H, E, MOE_BF16) * 4) return MOE_ERR_WORKSPACE_TOO_SMALL;
    if (T == 0) return MOE_OK;
    if (!residual || !a_out || !topk_ids || !topk_w || !ws) return MOE_ERR_INVALID_ARG;
    if (!aligned(residual, 16) || !aligned(a_out, 16) || !aligned(router_wT, 16) ||
        !aligned(ws, 16) || (norm_w && !aligned(norm_w, 16)))
        return MOE_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    float *part = (float *)ws;
    moe_status_t st;
    int P = 1;
    if (norm_route_fused(T, H, E)) {
        P = router_blocks(H);
        st = launch_norm_router_scores(residual, norm_w, eps, T, H, router_wT, E, a_out, part, s);
    } else {
        if ((st = launch_rmsnorm(residual, norm_w, eps, T, H, MOE_BF16, a_out, s)) != MOE_OK)
            return st;
        st = launch_router_scores(a_out, MOE_BF16, router_wT, T, H, E, part, &P, s);
    }
    if (st != MOE_OK) return st;
    return launch_topk(part, bias, T, E, K, renormalize, topk_ids, topk_w, s, P);
}

moe_status_t moe_dequant(const moe_weight_desc_t *w, int expert, float *out, void *stream) {
    if (!w || !out) return MOE_ERR_INVALID_ARG;
    const int E = w->num_experts;
    if (E < 1 || E > kMaxExperts || expert < 0 || expert >= E) return MOE_ERR_INVALID_ARG;
    moe_status_t st = check_bank(*w, E, w->n, w->k);
    if (st != MOE_OK) return st;
    if (!aligned(out, 16)) return MOE_ERR_INVALID_ARG;
    return launch_dequant(*w, expert, out, (hipStream_t)stream);
}

moe_status_t moe_quantize_nvfp4_act(const void *x, int dtype, int64_t rows, int k,
                                    float input_scale, void *out, void *stream) {
    if (rows < 0 || k < 16 || k % 16 || k > kMaxDim || !is_act(dtype)) return MOE_ERR_INVALID_ARG;
    if (!(input_scale > 0.0f) || !input_scale_ok(input_scale)) return MOE_ERR_INVALID_ARG;
    if (rows == 0) return MOE_OK;
    if (!x || !out || !aligned(x, 16) || !aligned(out, 16)) return MOE_ERR_INVALID_ARG;
    return launch_act_quant(x, dtype, rows, k, input_scale, out, nullptr, (hipStream_t)stream);
}

moe_status_t moe_csf_expand(const uint8_t *fixed, const uint32_t *exceptions,
                            int64_t n_exceptions, const int64_t *starts, int E, int R, int C,
                            const int32_t *expert_offsets, int max_routed_experts,
                            uint8_t *out, void *stream) {
    if (!fixed || !starts || !out || n_exceptions < 0 || (n_exceptions > 0 && !exceptions))
        return MOE_ERR_INVALID_ARG;
    if (E < 1 || E > kMaxExperts || R < 16 || R % 16 || C < 16 || C % 16)
        return MOE_ERR_INVALID_ARG;
    if ((int64_t)R * C >= ((int64_t)1 << 24)) return MOE_ERR_UNSUPPORTED;   // 24-bit positions
    if (max_routed_experts < 0) return MOE_ERR_INVALID_ARG;
    if (!aligned(fixed, 8) || !aligned(out, 16) || !aligned(starts, 8) ||
        (exceptions && !aligned(exceptions, 4)) || (expert_offsets && !aligned(expert_offsets, 4)))
        return MOE_ERR_INVALID_ARG;
    return launch_csf_expand(fixed, exceptions, n_exceptions, starts, E, R, C, expert_offsets,
                             max_routed_experts, out, (hipStream_t)stream);
}

moe_status_t moe_csf_row_index(const uint32_t *exceptions, int64_t n_exceptions,
                               const int64_t *starts, int E, int R, int C,
                               const int32_t *expert_offsets, int max_routed_experts,
                               int32_t *row_index, void *stream) {
    if (!starts || !row_index || n_exceptions < 0 || (n_exceptions > 0 && !exceptions))
        return MOE_ERR_INVALID_ARG;
    if (E < 1 || E > kMaxExperts || R < 16 || R % 16 || C < 16 || C % 16)
        return MOE_ERR_INVALID_ARG;
    if ((int64_t)R * C >= ((int64_t)1 << 24)) return MOE_ERR_UNSUPPORTED;   // 24-bit positions
    if (max_routed_experts < 0) return MOE_ERR_INVALID_ARG;
    if (!aligned(row_index, 4) || !aligned(starts, 8) || (exceptions && !aligned(exceptions, 4)) ||
        (expert_offsets && !aligned(expert_offsets, 4)))
        return MOE_ERR_INVALID_ARG;
    return launch_csf_row_index(exceptions, n_exceptions, starts, E, R, C, expert_offsets,
                                max_routed_experts, row_index, (hipStream_t)stream);
}

}  // extern "C"
