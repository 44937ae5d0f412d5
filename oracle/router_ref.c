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
 * definition:
 *
 *   acc = +0.0f;  for k = 0 .. H-1 ascending:  acc = fmaf(x[t][k], wT[k][e], acc)
 *   logit = acc;  if bias: logit = logit + bias[e]   (one float32 addition)
 *
 * x is the 16-bit activation widened exactly to float32; wT is the router
 * weight stored transposed, [H][E] float32. fmaf is libm's correctly rounded
 * fused multiply-add. Build with -ffp-contract=off and without fast-math so
 * the compiler neither fuses the bias addition nor reorders anything.
 * The loops run e innermost for cache locality; each (t, e) chain still
 * visits k in ascending order.
 */
#include <math.h>
#include <stddef.h>

void oracle_router_logits(const float *x, const float *wT, const float *bias,
                          int T, int H, int E, float *out)
{
    for (int t = 0; t < T; ++t) {
        float *acc = out + (size_t)t * E;
        for (int e = 0; e < E; ++e)
            acc[e] = 0.0f;
        for (int k = 0; k < H; ++k) {
            const float xv = x[(size_t)t * H + k];
            const float *w = wT + (size_t)k * E;
            for (int e = 0; e < E; ++e)
                acc[e] = fmaf(xv, w[e], acc[e]);
        }
        if (bias)
            for (int e = 0; e < E; ++e)
                acc[e] = acc[e] + bias[e];
    }
}
