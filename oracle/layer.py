"""The routed-expert MoE layer in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Statement of the layer (page "Step 5 Preview: 92 narrow layers, and a sparse
indexer that scores blocks of 8", "The shape: narrow and deep"; page
"Step-5-Preview-Spark", "At a glance"): each MoE layer has 352 routed experts
of which 8 are chosen per token by a sigmoid router, plus one shared expert;
every expert is a SwiGLU of width 1536 on the hidden size 4096, built from
gate, up and down projections (page "NeuroSenko/Step-5-Preview-Int4-g128",
"Tensor layout"). The residual stream is kept in fp32 (page "Step 5
Preview: ...", the paragraph on training the deep stack:
fp32_residual_connection).

Per slot s = (t, k) routed to expert e:
    g = Wg_e x_t,  u = Wu_e x_t,  h = silu(g) * u = g u / (1 + exp(-g)),
    y_s = Wd_e h
and   out_t = sum_k w[t, k] y_(t,k)  (k ascending)
            [+ shared SwiGLU(x_t)] [+ residual_t].

Everything is float64 with no intermediate rounding; the weights are the
exact dequantized values and x is the 16-bit activation widened exactly.

NVFP4 layers with quantized activations (page "Step-5-Preview-NVFP4-Local",
"Modifications" items 2-3: the layers that keep an input scale) feed the
routed experts x quantized with the input scale of gate/up, and their down
projections h rounded to the activation dtype and quantized with the input
scale of down (quant.quantize_nvfp4_act; the rounding of h to 16 bits is a
reading: h is a 16-bit activation on every path here); a4_h_fn builds that
map.

Readings: silu applies to the gate and multiplies the up projection; there is
no clamp (the NVFP4 page names a "SwiGLU limit" but gives neither formula nor
value); the shared expert's output is added unweighted. The chained stack
(see norm.py) feeds each layer the RMSNorm of the fp32 residual rounded to
the activation dtype and adds the layer's output back to the residual.
"""
import numpy as np


def silu(g):
    return g / (1.0 + np.exp(-g))


def swiglu_ffn(x, Wg, Wu, Wd, h_fn=None):
    """x [m, H] -> [m, H] for one expert with float64 weights Wg, Wu [F, H]
    and Wd [H, F]. h_fn, if given, maps h to the down projection's input
    (the NVFP4 activation quantization of the quantized layers)."""
    g = x @ Wg.T
    u = x @ Wu.T
    h = silu(g) * u
    if h_fn is not None:
        h = h_fn(h)
    return h @ Wd.T


def routed_outputs(x, ids, expert_weights, h_fn=None):
    """y [T, K, H]: the output of the chosen expert for every slot.

    expert_weights(e) -> (Wg, Wu, Wd) float64. Slots routed to the same
    expert are evaluated together (one matrix product per expert); each
    slot's value depends only on its own token and expert.
    """
    x = np.asarray(x, dtype=np.float64)
    ids = np.asarray(ids)
    T, K = ids.shape
    y = np.zeros((T, K, x.shape[1]))
    for e in np.unique(ids):
        t_idx, k_idx = np.nonzero(ids == e)
        Wg, Wu, Wd = expert_weights(int(e))
        y[t_idx, k_idx] = swiglu_ffn(x[t_idx], Wg, Wu, Wd, h_fn)
    return y


def combine(y, w, shared=None, residual=None):
    """out[t] = sum over k ascending of w[t, k] * y[t, k]  (+ shared) (+ residual)."""
    T, K, H = y.shape
    out = np.zeros((T, H))
    for k in range(K):
        out += w[:, k:k + 1] * y[:, k, :]
    if shared is not None:
        out = out + shared
    if residual is not None:
        out = out + residual
    return out


def moe_layer(x, ids, w, expert_weights, shared_weights=None, residual=None, h_fn=None):
    """One layer: routed experts + optional shared expert + optional residual.
    h_fn as in swiglu_ffn (routed experts only)."""
    y = routed_outputs(x, ids, expert_weights, h_fn)
    sh = None
    if shared_weights is not None:
        sh = swiglu_ffn(np.asarray(x, dtype=np.float64), *shared_weights)
    return combine(y, w, sh, residual)


def a4_h_fn(g_h, act="bf16"):
    """The map h -> quantized h of the NVFP4-activation layers: h rounded to
    the activation dtype, quantized with input scale g_h, times g_h."""
    from .formats import to_bf16, to_fp16
    from .quant import quantize_nvfp4_act

    def fn(h):
        h16 = to_bf16(h) if act == "bf16" else to_fp16(h)
        return quantize_nvfp4_act(h16, g_h)[2] * float(np.float32(g_h))
    return fn
