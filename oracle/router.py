"""Sigmoid top-K router.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it computes (pages "Step-5-Preview-Spark", "At a glance": a sigmoid
router picks 8 of the 352 routed experts; "Step 5 Preview: 92 narrow layers, and a
sparse indexer that scores blocks of 8", "The shape: narrow and deep"):

1. logits[t, e] = x[t] . Wr[e] in the canonical float32 order of
   router_ref.c (one fused chain per block of 512 inputs, the blocks' sums
   added in ascending order; plus an optional per-expert bias), or given
   logits;
2. the K experts with the largest logits, ties broken by the lower expert
   index (the same convention the sparse indexer's region top-k uses, page
   "Step 5 Preview: ...", "Sparse GQA, read from the kernels", step 3);
3. routing weights p = sigmoid(logit) of the chosen experts, renormalised to
   sum to one.

Readings: ranking is on the float32 logit (sigmoid is strictly increasing,
so this equals ranking by the exact sigmoid); -0 ranks equal to +0; the
weights are sigmoid of the selected logits divided by their sum, with no
extra scaling factor (the pages name none).
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "router_ref.c")
_LIB = os.path.join(_HERE, "_router_ref.so")
_lib = None


def build(force=False):
    """Compile router_ref.c with gcc (no fusing of separate operations, no
    fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math",
                               "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        fp = ctypes.POINTER(ctypes.c_float)
        lib.oracle_router_logits.argtypes = [fp, fp, fp, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, fp]
        lib.oracle_router_logits.restype = None
        _lib = lib
    return _lib


def router_logits(x, wT, bias=None):
    """x [T, H] (values exactly float32, e.g. widened fp16/bf16), wT [H, E]
    float32, bias [E] float32 or None -> logits [T, E] float32."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    wT = np.ascontiguousarray(wT, dtype=np.float32)
    T, H = x.shape
    H2, E = wT.shape
    assert H == H2
    out = np.empty((T, E), dtype=np.float32)
    fp = ctypes.POINTER(ctypes.c_float)
    b = None
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        assert bias.shape == (E,)
        b = bias.ctypes.data_as(fp)
    lib.oracle_router_logits(x.ctypes.data_as(fp), wT.ctypes.data_as(fp), b,
                             T, H, E, out.ctypes.data_as(fp))
    return out


def topk_ids(logits, K):
    """Indices of the K largest logits per row, by (logit descending, expert
    index ascending). -0.0 and +0.0 rank equal."""
    lg = np.asarray(logits, dtype=np.float64) + 0.0        # -0 -> +0
    T, E = lg.shape
    assert 1 <= K <= E
    e = np.broadcast_to(np.arange(E), lg.shape)
    out = np.empty((T, K), dtype=np.int32)
    for t in range(T):
        order = np.lexsort((e[t], -lg[t]))                 # primary: -logit
        out[t] = order[:K]
    return out


def routing_weights(logits, ids, renormalize=True):
    """sigmoid of the selected logits (float64), optionally divided by their
    sum over the K selected experts."""
    lg = np.asarray(logits, dtype=np.float64)
    sel = np.take_along_axis(lg, np.asarray(ids, dtype=np.int64), axis=1)
    p = 1.0 / (1.0 + np.exp(-sel))
    if renormalize:
        p = p / np.sum(p, axis=1, keepdims=True)
    return p


def route(x=None, wT=None, logits=None, bias=None, K=8, renormalize=True):
    """Full routing step: logits (computed, or given and then biased), top-K
    ids, weights. Returns (logits_used float32, ids int32, weights float64)."""
    if logits is None:
        lg = router_logits(x, wT, bias)
    else:
        lg = np.asarray(logits, dtype=np.float32)
        if bias is not None:
            lg = (lg + np.asarray(bias, dtype=np.float32)).astype(np.float32)
    ids = topk_ids(lg, K)
    return lg, ids, routing_weights(lg, ids, renormalize)
