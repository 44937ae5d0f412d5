/*
 * Canonical float32 router logits for the sigmoid top-K router.
 *
 * TEST INFRASTRUCTURE ONLY: part of the CPU oracle; the product library
 * never links it.
 *
 * The router scores every expert by the dot product of the token's hidden
 * state with that expert's router row (pages "Step-5-Preview-Spark",
 * "At a glance": a sigmoid router picks 8 of the 352 routed experts). The pages fix no
 * summation order, but they show that routing flips under a changed
 * summation order ("Step-5-Preview-Spark", "Quality", the noise-floor
 * paragraph). Bit-exact routing therefore needs one order; this file is its
 * definition. The inputs are taken in blocks of ROUTER_BLOCK = 512
 * consecutive positions; each block is one fused chain, and the blocks'
 * sums are added in ascending block order:
 *
 *   for each block b (inputs k0 = 512 b .. min(512 b + 512, H) - 1):
 *     s_b = +0.0f;  for k = k0 .. ascending:  s_b = fmaf(x[t][k], wT[k][e], s_b)
 *   logit = s_0;  for b = 1 .. ascending:  logit = logit + s_b
 *   if bias: logit = logit + bias[e]              (float32 additions)
 *
 * (with H <= 512 this is the single chain over all inputs). Blocks let a
 * kernel run a token's chains side by side instead of one 4096-step chain.
 * x is the 16-bit activation widened exactly to float32; wT is the router
 * weight stored transposed, [H][E] float32. fmaf is libm's correctly rounded
 * fused multiply-add. Build with -ffp-contract=off and without fast-math so
 * the compiler neither fuses an addition nor reorders anything.
 * The loops run e innermost for cache locality; each (t, e) chain still
 * visits k in ascending order.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>

#define ROUTER_BLOCK 512

void oracle_router_logits(const float *x, const float *wT, const float *bias,
                          int T, int H, int E, float *out)
{
    float *part = (float *)malloc((size_t)E * sizeof(float));
    for (int t = 0; t < T; ++t) {
        float *acc = out + (size_t)t * E;
        for (int k0 = 0; k0 < H; k0 += ROUTER_BLOCK) {
            const int k1 = k0 + ROUTER_BLOCK < H ? k0 + ROUTER_BLOCK : H;
            for (int e = 0; e < E; ++e)
                part[e] = 0.0f;
            for (int k = k0; k < k1; ++k) {
                const float xv = x[(size_t)t * H + k];
                const float *w = wT + (size_t)k * E;
                for (int e = 0; e < E; ++e)
                    part[e] = fmaf(xv, w[e], part[e]);
            }
            for (int e = 0; e < E; ++e)
                acc[e] = k0 == 0 ? part[e] : acc[e] + part[e];
        }
        if (H == 0)
            for (int e = 0; e < E; ++e)
                acc[e] = 0.0f;
        if (bias)
            for (int e = 0; e < E; ++e)
                acc[e] = acc[e] + bias[e];
    }
    free(part);
}
