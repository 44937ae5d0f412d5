"""The layer-input normalisation of the stacked layers, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Page "Step 5 Preview: 92 narrow layers, and a sparse indexer that scores
blocks of 8", the paragraph on training the deep stack: the residual stream
is kept in fp32, and Step5RMSNorm scales x / rms(x) by a zero-centred gain,
i.e. multiplies by (1 + w) rather than by w (reading w as a plain scale would
multiply every activation by about zero). Here

    rmsnorm(x)[h] = x[h] / sqrt(mean_h x[h]^2 + eps) * (1 + w[h])

over the last axis. The pages give no eps; it is an argument (the stack uses
1e-5, a common choice, as a reading). The page computes the norm in fp32;
this restatement is float64 and the caller rounds the result once to the
activation format.
"""
import numpy as np


def rmsnorm(x, w=None, eps=1e-5):
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    y = x / np.sqrt(ms + eps)
    if w is not None:
        y = y * (1.0 + np.asarray(w, dtype=np.float64))
    return y
