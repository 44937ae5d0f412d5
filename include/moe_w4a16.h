/*
 * moe_w4a16.h -- C ABI of the W4A16 routed-expert MoE layer for AMD MI355X
 * (CDNA4, gfx950).
 *
 * The layer (page "Step 5 Preview: 92 narrow layers, and a sparse indexer
 * that scores blocks of 8", section "The shape: narrow and deep"; page
 * "Step-5-Preview-Spark", "At a glance"): hidden size 4096, 352 routed
 * experts of which a sigmoid router picks 8 per token, plus one shared
 * expert; every expert is a SwiGLU of width 1536 made of gate, up and down
 * projections. Routed-expert weights are 4-bit and dequantized inside the
 * kernels; activations stay 16-bit (W4A16).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every pointer argument is a DEVICE pointer unless its comment says
 *   "host". The caller owns all memory, workspaces included; the library
 *   allocates nothing and keeps no mutable global state, apart from the
 *   static device buffer of moe_w4a16_forward_scratch and the per-device
 *   address of it that the first call on a device looks up.
 * - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *   Every call only enqueues work on it and returns; nothing synchronises.
 * - Arguments are validated on the host before anything is launched; an
 *   invalid call returns an error and enqueues nothing. A failed launch
 *   returns MOE_ERR_HIP. Faults inside kernels surface at the caller's next
 *   synchronisation.
 * - Inputs are assumed finite; NaN or Inf gives unspecified routing.
 * - Matrices are row-major. Slot s = t*K + k is the k-th expert choice of
 *   token t.
 */
#ifndef MOE_W4A16_H
#define MOE_W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,         /* null pointer, bad size or stride   */
    MOE_ERR_UNSUPPORTED = 2,         /* valid but not implemented shape    */
    MOE_ERR_WORKSPACE_TOO_SMALL = 3,
    MOE_ERR_HIP = 4                  /* a HIP launch or API call failed    */
} moe_status_t;

typedef enum { MOE_F16 = 1, MOE_BF16 = 2, MOE_F32 = 3 } moe_dtype_t;

/* Weight formats of one bank of expert matrices.
 *
 * MOE_W_INT4_G128 -- page "NeuroSenko/Step-5-Preview-Int4-g128", "Recipe"
 *   and "Tensor layout": symmetric int4, one bf16 scale per 128 input
 *   channels, routed experts fused as [experts, out, in].
 *   qweight: int32 [E][n][k/8]; nibble j (bits 4j..4j+3) of word w holds
 *            input 8w+j as a two's-complement value q in [-8, 7].
 *   scale:   bf16 [E][n][k/128].   weight = q * scale.
 *
 * MOE_W_NVFP4_G16 -- page "Step-5-Preview-NVFP4-Local", "Modifications"
 *   item 2 and "Format": weight U8 [E, R, K/2] of E2M1 pairs, F8_E4M3 block
 *   scale [E, R, K/16], F32 weight_scale_2 [E]; the W4A16 variant keeps
 *   activations in BF16.
 *   qweight: uint8 [E][n][k/2]; the low nibble is the even input index.
 *   scale:   uint8 E4M3FN [E][n][k/16].
 *   global_scale: float [E].   weight = e2m1 * e4m3 * global_scale.
 *
 * MOE_W_BF16 -- an unquantized bank (the shared expert stays BF16: page
 *   "NeuroSenko/Step-5-Preview-Int4-g128", "What stays in BF16").
 *   qweight: bf16 [E][n][k]; scale and global_scale NULL.
 *
 * MOE_W_INT4_G32 -- the same page, "Recipe" (its int4-g32 row, same clip
 *   search): as MOE_W_INT4_G128 with one bf16 scale per 32 inputs.
 *   scale:   bf16 [E][n][k/32].   weight = q * scale.
 *
 * MOE_W_INT4_G128_ASYM -- the same page, "Recipe" (its asymmetric
 *   int4-g128 row): unsigned nibbles q in [0, 15] (nibble j of word w =
 *   input 8w+j), one bf16 scale and one zero point per 128 inputs.
 *   scale:   bf16 [E][n][k/128];  zero_point: uint8 [E][n][k/128], values
 *   0..15.   weight = (q - zero_point) * scale.
 *
 * MOE_W_INT8_G128 -- the same page, "Recipe" (the 8-bit experts it
 *   compares against): symmetric int8 with one bf16 scale per 128 inputs.
 *   qweight: int8 [E][n][k], two's complement, input j at byte j.
 *   scale:   bf16 [E][n][k/128].   weight = q * scale.
 *
 * MOE_W_NVFP4_CSF -- MOE_W_NVFP4_G16 with the block scales left in the
 *   compressed scale format of page "Step-5-Preview-NVFP4-Local" ("Format",
 *   "Modifications" item 1; see moe_csf_expand), read directly by the
 *   kernels instead of being expanded first.
 *   qweight, global_scale: as MOE_W_NVFP4_G16;
 *   scale: the CSF `fixed` tensor U8 [E][n/16][16*(1 + C/2)], C = k/16,
 *            scale_expert_stride its expert stride in bytes (>= n*(1 + C/2)),
 *            scale_row_stride unused (0); n % 16 == 0;
 *   csf_exceptions: the exceptions U32 (row*C + col) | byte << 24, each
 *            expert's contiguous and in position order (NULL if none);
 *   csf_row_index: I32 [E][n+1] from moe_csf_row_index (the exceptions of
 *            row r of expert e are [row_index[e][r], row_index[e][r+1])).
 *
 * The decode kernels (the GEMV) serve every format, and so does the prefill
 * GEMM (batches with T*K >= 4E; at H = 4096, F = 1536 MOE_W_NVFP4_G16 banks
 * from 8E and int4-g128 banks, both forms, from 7E, with the MFMA GEMV's
 * 8-slot tiles from 4E up to there; for NVFP4 its fp16
 * arithmetic holds bf16 inputs exactly within 2^29 of each token's largest
 * magnitude and rounds smaller ones); for MOE_W_NVFP4_CSF banks the forward pass
 * first expands the routed experts' scales into its workspace (which
 * moe_forward_plan sizes for all E experts of the three matrices). The GEMM
 * needs 4-byte-aligned scale rows (int4-g128 forms, int8), 16-byte aligned
 * ones (int4-g32, NVFP4), 2-byte-aligned zero-point rows (asymmetric int4)
 * and an 8-byte-aligned CSF fixed tensor; a bank without them runs the GEMV
 * at every size. At
 * prefill sizes int4-g32 puts the group scale into the MFMA operand: with
 * bf16 activations q * s is rounded to bf16 (relative 2^-9 per weight);
 * with fp16 activations the scale is converted to fp16 and q * s formed in
 * fp16, which is exact while the scale lies in fp16's normal range
 * (2^-14 .. 65504) and rounds otherwise. Every other path decodes exactly.
 */
typedef enum {
    MOE_W_INT4_G128 = 1, MOE_W_NVFP4_G16 = 2, MOE_W_BF16 = 3,
    MOE_W_INT4_G32 = 4, MOE_W_INT4_G128_ASYM = 5, MOE_W_INT8_G128 = 6,
    MOE_W_NVFP4_CSF = 7
} moe_wfmt_t;

/* One bank of E matrices, each [n out][k in]. Strides are in bytes; the
 * row strides must be multiples of 16 and the base pointers 16-byte
 * aligned (the kernels load 128 bits at a time); scale pointers and strides
 * must be even. Per-expert tensors stored
 * at a constant distance are described by the expert stride. */
typedef struct {
    int32_t fmt;                 /* moe_wfmt_t                                  */
    int32_t num_experts, n, k;
    const void  *qweight;
    const void  *scale;          /* NULL for MOE_W_BF16                          */
    const float *global_scale;   /* NVFP4 only, else NULL                        */
    int64_t qweight_expert_stride, qweight_row_stride;
    int64_t scale_expert_stride, scale_row_stride;
    const uint8_t *zero_point;   /* MOE_W_INT4_G128_ASYM only, else NULL          */
    int64_t zero_point_expert_stride, zero_point_row_stride;
    const uint32_t *csf_exceptions;  /* MOE_W_NVFP4_CSF only, else NULL          */
    const int32_t *csf_row_index;    /* MOE_W_NVFP4_CSF only, else NULL          */
    float input_scale;           /* NVFP4 forms: 0 = 16-bit inputs (W4A16); > 0 =
                                    the inputs are NVFP4-quantized with this
                                    float32 global scale (see moe_w4a16_forward) */
} moe_weight_desc_t;

/* The three projections of a SwiGLU bank: gate and up are [F][H], down is
 * [H][F]; all three share one format and expert count. */
typedef struct { moe_weight_desc_t gate, up, down; } moe_ffn_desc_t;

/* Output of moe_permute (every pointer a device array the caller sized
 * with moe_permute_sizes). Definition:
 *   counts[e]            slots routed to expert e                     [E]
 *   expert_offsets[e]    exclusive prefix sum of counts               [E+1]
 *   padded_offsets[e]    exclusive prefix sum of counts rounded up to
 *                        a multiple of tile_m                         [E+1]
 *   sorted_slots[r]      row r of the expert-sorted order: each expert's
 *                        slots in ascending slot order, its segment
 *                        padded with -1 to its padded length; rows at and
 *                        beyond padded_offsets[E] are not written     [max_rows]
 *   slot_to_row[s]       row of slot s in sorted_slots                [T*K]
 *   tile_expert[i]       expert owning rows [i*tile_m, (i+1)*tile_m)  [max_tiles]
 *   num_tiles[0]         padded_offsets[E] / tile_m                   [1]
 *   active_experts[j]    experts with counts > 0, ascending           [E]
 *   num_active[0]        how many there are                           [1]
 */
typedef struct {
    int32_t *counts, *expert_offsets, *padded_offsets, *sorted_slots,
            *slot_to_row, *tile_expert, *num_tiles, *active_experts,
            *num_active;
    int32_t tile_m;
} moe_perm_t;

/* Human-readable name of a status code (host, static storage). */
const char *moe_status_string(int status);

/* ABI version of this header: 6 (moe_abi_version returns it). */
int moe_abi_version(void);

/*
 * moe_router_logits -- the router scores of every (token, expert) pair
 * (page "Step-5-Preview-Spark", "At a glance": a sigmoid router over 352
 * routed experts), as a float32 sum in one fixed order: the inputs in
 * blocks of 512 (the last may be shorter), each block a fused chain
 *     s_b = +0; for k in block b ascending: s_b = fma(float(x[t][k]), router_wT[k][e], s_b)
 *     logits[t][e] = ((s_0 + s_1) + s_2) + ...   (+ bias[e] if bias != NULL)
 * in float32 additions. This fixed order makes routing reproducible bit for
 * bit (page "Step-5-Preview-Spark", "Quality": top-8 choices flip under a
 * changed summation order); the blocks let small batches run a token's
 * chains side by side.
 * x [T][H] in x_dtype (MOE_F16 or MOE_BF16), router_wT [H][E] float (the
 * router weight transposed, 16-byte aligned), bias [E] float or NULL,
 * logits [T][E] float. Limits: H % 64 == 0, E % 4 == 0, E <= 512.
 */
moe_status_t moe_router_logits(const void *x, int x_dtype, const float *router_wT,
                               const float *bias, int T, int H, int E, float *logits,
                               void *stream);

/* Workspace bytes (host output) moe_route_topk and moe_norm_route need when
 * they compute the logits from a router weight (use_router_weight != 0),
 * else 0: one float32 per 512-input block, token and expert, 8*T*E*4
 * (a bf16 router input with H <= 4096 takes the block sums; f16 inputs and
 * larger H take the logits, T*E*4). */
moe_status_t moe_route_workspace(int T, int E, int use_router_weight, size_t *bytes);

/*
 * moe_route_topk -- sigmoid top-K routing (page "Step-5-Preview-Spark",
 * "At a glance": top-8 of 352 experts by a sigmoid router; ties go to the
 * lower index, as in the sparse indexer's region top-k on page "Step 5
 * Preview: ...", "Sparse GQA, read from the kernels", step 3).
 *
 * Logits come from exactly one of:
 *   router_wT: the moe_router_logits sum of x (x, x_dtype, H as there);
 *     its block sums (bf16 and H <= 4096) or the logits
 *     go to the workspace `ws` (moe_route_workspace bytes) and the top-K
 *     adds them up in block order;
 *   logits_in [T][E] float: given logits (x, router_wT, ws unused).
 * If bias [E] float is non-NULL, logit = logit + bias[e] in float32.
 * topk_ids [T][K] int32: the K largest logits by (logit descending, expert
 * index ascending), -0 equal to +0. topk_w [T][K] float: sigmoid of those
 * logits, divided by their sum over the K (summed in ascending k) when
 * renormalize != 0. Limits: 1 <= K <= min(E, 16), E <= 512. T == 0 is a
 * no-op.
 */
moe_status_t moe_route_topk(const void *x, int x_dtype, const float *router_wT,
                            const float *logits_in, const float *bias,
                            int T, int H, int E, int K, int renormalize,
                            int32_t *topk_ids, float *topk_w, void *ws, size_t ws_bytes,
                            void *stream);

/* Sizes (host outputs, in elements) of the moe_permute arrays for T tokens,
 * K choices, E experts and tile_m rows per tile:
 *   max_rows  = T*K + min(E, T*K)*(tile_m - 1)  (sorted_slots)
 *   max_tiles = max_rows / tile_m               (tile_expert)          */
moe_status_t moe_permute_sizes(int T, int K, int E, int tile_m,
                               int64_t *max_rows, int64_t *max_tiles);

/*
 * moe_norm_route -- the step before the routed experts, fused (the norm and
 * the router decide which experts a token reaches; page
 * "Step-5-Preview-Spark", "Quality": rounding the router input to bf16
 * flips about a third of the top-8 sets, so where it is rounded matters):
 *   a = bf16(residual / rms(residual) * (1 + norm_w))   (as moe_rmsnorm)
 *   topk_ids, topk_w = top-K routing of a from router_wT (+ bias)
 *                                                        (as moe_route_topk)
 * For batches of up to 192 tokens with H <= 4096 the norm, the cast and the
 * router chains run as one kernel (one work group per token pair or quad,
 * 64-expert block and 512-input block normalizes its token rows into LDS
 * and stores its chains' block sums; the first expert and input block
 * writes the rows to a_out), then
 * the top-K; otherwise the kernels of the separate calls run. Either way the
 * results are bitwise those of moe_rmsnorm followed by moe_route_topk.
 *   residual [T][H] float; norm_w [H] float or NULL (gain 1); eps in [0, 1];
 *   router_wT [H][E], bias [E] or NULL, K, renormalize: as moe_route_topk;
 *   a_out [T][H] bf16 (the layer input the experts read);
 *   topk_ids [T][K] int32, topk_w [T][K] float;
 *   ws: device workspace of moe_route_workspace(T, E, 1) bytes (the
 *   block sums or the logits), 16-byte aligned.
 * All pointers device memory, 16-byte aligned (ids and weights 4). Limits:
 * H % 64 == 0 and E % 4 == 0 (else MOE_ERR_UNSUPPORTED), H <= 16384,
 * 1 <= K <= min(E, 16), E <= 512. T == 0 is a no-op.
 */
moe_status_t moe_norm_route(const float *residual, const float *norm_w, float eps, int T, int H,
                            const float *router_wT, const float *bias, int E, int K,
                            int renormalize, void *a_out, int32_t *topk_ids, float *topk_w,
                            void *ws, size_t ws_bytes, void *stream);

/*
 * moe_permute -- expert histogram and stable expert-sorted permutation of
 * the T*K slots (see moe_perm_t). The pages do not describe this step; it
 * exists so that each touched expert's weights stream from HBM once
 * (on page "NeuroSenko/Step-5-Preview-Int4-g128", "Recipe", the routed
 * experts hold nearly all of the model's bytes).
 * topk_ids [T][K] int32, normally in [0, E); a slot whose id lies outside
 * is routed nowhere: it gets no row and slot_to_row[s] = -1, and the
 * forward pass adds nothing for it. Ids may repeat within a token.
 * tile_m in [1, 256].
 * Deterministic: no atomics decide any order (up to 1024 slots, one work
 * group combines per-expert slot masks with LDS ORs; beyond, each expert's
 * work group counts all slots with LDS integer adds; neither result depends
 * on arrival order).
 */
moe_status_t moe_permute(const int32_t *topk_ids, int T, int K, int E,
                         const moe_perm_t *perm, void *stream);

/*
 * moe_route_permute -- moe_route_topk followed by moe_permute on its ids,
 * in one call (the routing of page "Step-5-Preview-Spark", "At a glance",
 * and the expert-sorted permutation that lets each expert stream once).
 * Arguments as moe_route_topk (x, x_dtype, router_wT, logits_in, bias, T,
 * H, E, K, renormalize, topk_ids, topk_w, ws, ws_bytes) plus perm, the
 * moe_permute outputs (tile_m from moe_forward_plan). For batches of up to
 * 16 tokens (T*K <= 1024) the top-K and the permutation run as one kernel:
 * one wave per token selects, then the work group permutes the ids from
 * LDS; larger batches run the two calls' kernels. Either way every output
 * is bitwise that of moe_route_topk followed by moe_permute. Errors: as
 * those two calls (T*K > 2^24: MOE_ERR_UNSUPPORTED).
 */
moe_status_t moe_route_permute(const void *x, int x_dtype, const float *router_wT,
                               const float *logits_in, const float *bias, int T, int H, int E,
                               int K, int renormalize, int32_t *topk_ids, float *topk_w,
                               const moe_perm_t *perm, void *ws, size_t ws_bytes, void *stream);

/* The tile_m the forward pass needs for T tokens (host output), and the
 * workspace bytes it needs (host output), with or without the shared expert
 * (same argument rules as moe_w4a16_forward). Pass that tile_m to
 * moe_permute. The workspace holds h [max_rows][F] in the activation dtype
 * and y [max_rows][H] float32 (max_rows from moe_permute_sizes; on the
 * prefill GEMM path, but for int4-g32, the same bytes hold y in fp16 with a
 * power-of-two scale per row and 32 columns), plus, on
 * the prefill GEMM path, per-group sums of x and h; with a shared expert its
 * h, y and split partial sums; and for a MOE_W_NVFP4_CSF bank on the GEMM
 * path the expanded E4M3 scales of all E experts of gate, up and down (E *
 * (2 F H + H F) / 16 bytes, 415 MB at E = 352, H = 4096, F = 1536: the GEMM
 * path needs T*K >= 4E, so every expert may be routed). */
moe_status_t moe_forward_plan(const moe_ffn_desc_t *experts,
                              const moe_ffn_desc_t *shared, int T, int K,
                              int act_dtype, int *tile_m, size_t *ws_bytes);

/*
 * moe_w4a16_forward -- the routed experts, the optional shared expert and
 * the weighted combine (page "Step 5 Preview: ...", "The shape: narrow and
 * deep": each token reaches its 8 chosen routed experts and the one shared
 * expert, all SwiGLUs of width 1536; the residual stream is fp32 per the same page's paragraph on
 * fp32_residual_connection):
 *
 *   for each slot s = (t, k) routed to expert e:
 *     h_s = silu(Wg_e x_t) * (Wu_e x_t),   y_s = Wd_e h_s
 *   out_t = sum_{k ascending} topk_w[t][k] * y_(t,k)
 *           [+ Wd_sh (silu(Wg_sh x_t) * (Wu_sh x_t))]  [+ residual_t]
 *
 * x [T][H] in act_dtype (MOE_F16 or MOE_BF16); experts: a bank of any
 * quantized moe_wfmt_t with gate/up [F][H] and down [H][F]; shared: NULL or a MOE_W_BF16
 * bank with num_experts == 1, gate/up [Fs][H], down [H][Fs] (act_dtype must
 * then be MOE_BF16; Fs % 128 == 0 and H % 256 == 0, else
 * MOE_ERR_UNSUPPORTED); the shared expert's h is rounded to bf16 like the
 * routed experts' h, and its output is added unweighted;
 * topk_w [T][K] float; perm: moe_permute output for this routing with the
 * tile_m from moe_forward_plan; residual: NULL or [T][H] float;
 * out [T][H] in out_dtype (MOE_F32, MOE_F16 or MOE_BF16); ws: device
 * workspace of at least moe_forward_plan's ws_bytes, 256-byte aligned.
 * On the grouped-GEMM path (T*K >= 4*E) x and h are read through 32-bit
 * byte offsets: T*H*2 and max_rows*F*2 must stay below 2^31 - 2^20 bytes
 * (else MOE_ERR_UNSUPPORTED; about 85 K tokens at top-8, F = 1536).
 * Accumulation is float32; h is rounded to act_dtype before the down
 * projection.
 *
 * Quantized inputs (page "Step-5-Preview-NVFP4-Local", "Modifications"
 * items 2-3: the NVFP4 layers that keep an input scale quantize their
 * activations, the W4A16 ones keep 16-bit inputs): when the experts are an
 * NVFP4 bank (plain or CSF scales) whose input_scale is > 0, x is quantized
 * with gate.input_scale (which must equal up.input_scale) as
 * moe_quantize_nvfp4_act does, and h, after its rounding to act_dtype,
 * with down.input_scale (which must then be > 0 too); each projection's
 * accumulators are multiplied by its input scale with the global scale.
 * The shared expert reads x unquantized (it stays BF16). Input scales are
 * 0 or in [2^-100, 2^100]; any other combination is MOE_ERR_INVALID_ARG.
 * Limits: 1 <= K <= min(E, 16); H and F multiples of the
 * format's group (128; 32 for MOE_W_INT4_G32 and NVFP4), at most 16384;
 * E <= 512.
 */
moe_status_t moe_w4a16_forward(const moe_ffn_desc_t *experts,
                               const moe_ffn_desc_t *shared,
                               const void *x, int act_dtype, int T, int K,
                               const float *topk_w, const moe_perm_t *perm,
                               const float *residual, void *out, int out_dtype,
                               void *ws, size_t ws_bytes, void *stream);

/* Bytes of the library-owned device buffer of moe_w4a16_forward_scratch. */
#define MOE_FORWARD_SCRATCH_BYTES (64u << 20)

/*
 * moe_w4a16_forward_scratch -- for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): moe_w4a16_forward with its workspace replaced by one
 * library-owned device buffer of MOE_FORWARD_SCRATCH_BYTES (64 MiB), a
 * static device array of which each GPU the library runs on holds its own
 * copy until the process ends. Same arguments (minus ws, ws_bytes), same
 * kernels, same results. The device is the current HIP device of the
 * calling thread, which must own `stream`; the first call on a device looks
 * the buffer's address up (hipGetSymbolAddress, no allocation), later calls
 * reuse it. Nothing here allocates: no hipMalloc, hipFree or allocating
 * library routine. The buffer keeps the last call's contents; no step of
 * the forward pass reads workspace memory it has not written in the same
 * call, so nothing needs clearing. Calls that overlap on one GPU (other
 * streams, other threads) share the buffer and race: serialise them.
 * Errors: as moe_w4a16_forward, plus MOE_ERR_WORKSPACE_TOO_SMALL when
 * moe_forward_plan's ws_bytes for the call exceeds the buffer (at the
 * Step-5 shape every batch below T*K = 4E fits, i.e. up to 175 tokens at
 * K = 8 and E = 352, with or without the shared expert; the workspaces of
 * the prefill GEMM and of NVFP4 banks from 4E slots do not), MOE_ERR_HIP if the device or
 * the buffer's address cannot be had.
 */
moe_status_t moe_w4a16_forward_scratch(const moe_ffn_desc_t *experts,
                                       const moe_ffn_desc_t *shared,
                                       const void *x, int act_dtype, int T, int K,
                                       const float *topk_w, const moe_perm_t *perm,
                                       const float *residual, void *out, int out_dtype,
                                       void *stream);

/* Number of timed stages of moe_w4a16_forward_profiled. */
#define MOE_FORWARD_STAGES 4

/*
 * moe_w4a16_forward_profiled -- moe_w4a16_forward, additionally recording
 * the caller's HIP events on `stream` at the stage boundaries, so the
 * caller can time each kernel stage with hipEventElapsedTime:
 *   events[0] | routed gate/up + SwiGLU | events[1] | routed down |
 *   events[2] | shared expert (empty without one) | events[3] | combine |
 *   events[4]
 * events: host array of n_events == MOE_FORWARD_STAGES + 1 hipEvent_t
 * handles (passed as void*), created by the caller; an entry may be NULL,
 * and then nothing is recorded at that boundary. Each recorded event makes
 * the stream drain the previous kernel before the next one starts (a few
 * microseconds), so a caller timing one stage records only its two
 * boundaries. Same results, same kernels, same validation as
 * moe_w4a16_forward; MOE_ERR_INVALID_ARG if events is NULL or n_events is
 * not MOE_FORWARD_STAGES + 1.
 */
moe_status_t moe_w4a16_forward_profiled(const moe_ffn_desc_t *experts,
                                        const moe_ffn_desc_t *shared,
                                        const void *x, int act_dtype, int T, int K,
                                        const float *topk_w, const moe_perm_t *perm,
                                        const float *residual, void *out, int out_dtype,
                                        void *ws, size_t ws_bytes, void *stream,
                                        void *const *events, int n_events);

/*
 * moe_round_activations -- out[i] = in[i] rounded to out_dtype (MOE_F16 or
 * MOE_BF16) to nearest, ties to even, for 0 <= i < n: the next layer's
 * 16-bit input from the float32 residual stream when layers are stacked
 * (page "Step 5 Preview: ...", "The shape: narrow and deep", on
 * fp32_residual_connection). in float [n] and out [n] 16-byte aligned.
 * n == 0 is a no-op.
 */
moe_status_t moe_round_activations(const float *in, int64_t n, int out_dtype, void *out,
                                   void *stream);

/*
 * moe_rmsnorm -- the normalised 16-bit input of a layer from the float32
 * residual stream (page "Step 5 Preview: ...", the paragraph on training the
 * deep stack: Step5RMSNorm scales x / rms(x) by the zero-centred gain
 * (1 + w), computed in fp32; the gain is stored in FP32):
 *   out[t][h] = (x[t][h] / sqrt(mean_h x[t][h]^2 + eps)) * (1 + weight[h])
 * with every operation in float32, rounded to nearest even (IEEE division
 * and square root, no fused multiply-adds), then rounded to out_dtype
 * (MOE_F16 or MOE_BF16), ties to even. The pages do not fix the order of
 * the sum of squares; it is this one: partial p (p = 0..255) adds the
 * squares of columns 4p..4p+3, 1024+4p..1024+4p+3, ... in ascending column
 * order; each run of 64 consecutive partials is folded in halves (partial i
 * gets partial i + m added, m = 32, 16, .., 1); the four run sums are added
 * left to right. x [T][H] float and weight [H] float (NULL = all zero, a
 * gain of 1) 16-byte aligned; out [T][H] 16-byte aligned.
 * Limits: H % 4 == 0, 4 <= H <= 16384, 0 <= eps <= 1. T == 0 is a no-op.
 */
moe_status_t moe_rmsnorm(const float *x, const float *weight, float eps, int T, int H,
                         int out_dtype, void *out, void *stream);

/*
 * moe_dequant -- the exact dequantized matrix of one expert, as float32
 * [n][k]. int4 forms and int8 (page "NeuroSenko/Step-5-Preview-Int4-g128",
 * "Recipe" and "Tensor layout"): q * scale, or (q - zero_point) * scale for
 * the asymmetric form, exact in float32. NVFP4 (page
 * "Step-5-Preview-NVFP4-Local", "Format" and "Modifications" item 2): the
 * E2M1 value times its E4M3 block scale (exact), times the expert's float32
 * global scale with one float32 rounding; MOE_W_NVFP4_CSF banks decode their
 * compressed scales first. The export has decoders of its own (the biased
 * 16-bit int4 pair decode, the hardware E2M1 pair conversion); it checks the
 * format interpretation, not the forward kernels' decoders, which are
 * checked through the layer's outputs. w: a quantized bank (not
 * MOE_W_BF16); expert in [0, E); out [n][k] float, 16-byte aligned.
 */
moe_status_t moe_dequant(const moe_weight_desc_t *w, int expert, float *out,
                         void *stream);

/*
 * moe_quantize_nvfp4_act -- NVFP4 quantization of 16-bit activations with a
 * per-tensor float32 global scale g = input_scale, as the quantized-input
 * layers apply it (page "Step-5-Preview-NVFP4-Local", "Modifications" items
 * 2-3; the rule for activations is not on the pages: it is the weights'
 * two-level rule of the page's "Format" section, with every decision in
 * float32). For each block of 16 consecutive elements of a row:
 *   t  = max|x| / (6 g)                  (float32; 6 g rounded to float32)
 *   bs = E4M3(t): nearest, ties to even, saturating at 448
 *   code_i = E2M1(x_i / (bs g)): nearest, ties to even, saturating at 6;
 *            0 when bs = 0; a magnitude that rounds to 0 gives +0
 *   out_i  = e2m1(code_i) * bs           (exact in both 16-bit formats)
 * so the quantized value of x_i is out_i * g.
 * x [rows][k] and out [rows][k] in dtype (MOE_F16 or MOE_BF16), 16-byte
 * aligned (out may equal x); k % 16 == 0, 16 <= k <= 16384; input_scale in
 * [2^-100, 2^100]. rows == 0 is a no-op. Enqueues one kernel.
 */
moe_status_t moe_quantize_nvfp4_act(const void *x, int dtype, int64_t rows, int k,
                                    float input_scale, void *out, void *stream);

/*
 * moe_csf_expand -- the E4M3 block-scale bytes of an NVFP4 bank from their
 * compressed scale format (page "Step-5-Preview-NVFP4-Local", "Format" and
 * "Modifications" item 1): each byte is rebuilt as its row's base plus the
 * 4-bit code at its position, except at the positions its expert's
 * exception list names, which take the byte stored there. The expanded bytes are the `scale` array of an NVFP4
 * moe_weight_desc_t with scale_row_stride C and scale_expert_stride R*C
 * (the page's loader expands one layer's scales into scratch before the
 * layer runs).
 *   fixed          U8  [E][R/16][16*(1 + C/2)], 8-byte aligned: rows in
 *                  slabs of 16, each slab its 16 bases followed by the C
 *                  4-bit codes of each of its rows, packed in pairs with
 *                  the even column in the low bits;
 *   exceptions     U32 [n_exceptions], 4-byte aligned (NULL if none):
 *                  (row*C + col) | byte << 24, contiguous per expert, row and
 *                  col counted within the expert, positions distinct within
 *                  an expert; entries past R*C are ignored;
 *   starts         I64 [E+1], 8-byte aligned: the exceptions of expert e are
 *                  entries starts[e] .. starts[e+1]-1 (clamped to
 *                  [0, n_exceptions]);
 *   expert_offsets I32 [E+1] or NULL: the moe_permute expert offsets; experts
 *                  with no routed slot are skipped (their bytes in `out` are
 *                  left unchanged);
 *   max_routed_experts  with expert_offsets: an upper bound on the number of
 *                  experts with routed slots (min(E, T*K) for a batch of T
 *                  tokens and K choices), which sizes the grid to the routed
 *                  experts only; 0 = E. A bound below the true count leaves
 *                  the experts past it unexpanded;
 *   out            U8  [E][R][C], 16-byte aligned, caller-owned.
 * All arrays are device memory; the call enqueues one kernel on `stream`.
 * Limits: R and C positive multiples of 16, E <= 512, max_routed_experts >= 0
 * (MOE_ERR_INVALID_ARG), R*C < 2^24 (MOE_ERR_UNSUPPORTED): positions are
 * 24-bit.
 */
moe_status_t moe_csf_expand(const uint8_t *fixed, const uint32_t *exceptions,
                            int64_t n_exceptions, const int64_t *starts, int E, int R, int C,
                            const int32_t *expert_offsets, int max_routed_experts,
                            uint8_t *out, void *stream);

/*
 * moe_csf_row_index -- the per-row exception ranges of a compressed scale
 * tensor (same tensors as moe_csf_expand), which let the kernels read a
 * MOE_W_NVFP4_CSF bank's scales without expanding them:
 *   row_index[e][r] = the first x in [starts[e], starts[e+1]) whose
 *   position (low 24 bits) is >= r*C, for r = 0..R,
 * so the exceptions of row r are [row_index[e][r], row_index[e][r+1]).
 * Each expert's exceptions must be sorted by position (the order the
 * format's exceptions are stored in). exceptions, n_exceptions, starts, E,
 * R, C, expert_offsets, max_routed_experts: as in moe_csf_expand (only
 * routed experts are indexed when expert_offsets is given; the rows of the
 * others are left unchanged); row_index I32 [E][R+1], 4-byte aligned,
 * caller-owned. Enqueues one kernel. Errors as moe_csf_expand.
 */
moe_status_t moe_csf_row_index(const uint32_t *exceptions, int64_t n_exceptions,
                               const int64_t *starts, int E, int R, int C,
                               const int32_t *expert_offsets, int max_routed_experts,
                               int32_t *row_index, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_W4A16_H */
