"""The layer-input normalisation of the stacked layers, in float32.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Page "Step 5 Preview: 92 narrow layers, and a sparse indexer that scores
blocks of 8", the paragraph on training the deep stack: the residual stream
is kept in fp32, and Step5RMSNorm computes x / rms(x) times a zero-centred
gain (1 + w), in fp32, with the gain stored in FP32. Reading w as a plain
scale would multiply every activation by about zero, hence the (1 + w).

    rmsnorm(x)[h] = (x[h] / sqrt(mean_h x[h]^2 + eps)) * (1 + w[h])

over the last axis, every operation a float32 operation rounded to nearest
even. The pages give no eps; it is an argument (the stack uses 1e-5, a
common choice, as a reading). They do not give the order of the sum of
squares either, and in float32 the order changes the result, so one order is
fixed here (a reading; it is the one a 256-lane reduction produces):

1. every square x[h] * x[h] is rounded to float32;
2. partial p (p = 0 .. 255) adds, from +0 and one float32 addition at a time,
   the squares of the columns h with (h // 4) % 256 == p in ascending h
   (columns 4p .. 4p+3, then 1024 + 4p .. 1024 + 4p+3, and so on);
3. each run of 64 consecutive partials is folded in halves: partial i gets
   partial i + m added for m = 32, 16, 8, 4, 2, 1 (i < m), leaving the run's
   sum in its first partial;
4. the four run sums s0 .. s3 are added left to right, ((s0 + s1) + s2) + s3
   (a row shorter than 1024 columns leaves the later partials at +0);
5. mean = sum / H, r = sqrt(mean + eps), then x[h] / r and (1 + w[h]) and
   their product, each rounded to float32.

Division and square root are IEEE's correctly rounded ones (numpy's float32
operations are). The caller rounds the float32 result to the activation
format.
"""
import numpy as np

_LANES, _RUN = 256, 64


def sum_of_squares(x):
    """The float32 sum of squares of each row of x [..., H] (H % 4 == 0) in
    the order above."""
    x = np.asarray(x, dtype=np.float32)
    H = x.shape[-1]
    if H % 4:
        raise ValueError("H must be a multiple of 4")
    sq = x * x                                               # float32 products
    span = 4 * _LANES
    pad = (-H) % span
    if pad:
        # a column that does not exist adds nothing: +0 added to a partial
        # that started at +0 and only ever added squares leaves it unchanged
        sq = np.concatenate([sq, np.zeros(sq.shape[:-1] + (pad,), np.float32)], axis=-1)
    sq = sq.reshape(sq.shape[:-1] + (sq.shape[-1] // span, _LANES, 4))
    part = np.zeros(sq.shape[:-3] + (_LANES,), np.float32)
    for j in range(sq.shape[-3]):                            # ascending column order
        for i in range(4):
            part = part + sq[..., j, :, i]
    runs = part.reshape(part.shape[:-1] + (_LANES // _RUN, _RUN)).copy()
    m = _RUN // 2
    while m >= 1:
        runs[..., :m] = runs[..., :m] + runs[..., m:2 * m]
        m //= 2
    s = runs[..., 0]
    tot = s[..., 0]
    for g in range(1, _LANES // _RUN):
        tot = tot + s[..., g]
    return tot


def rmsnorm(x, w=None, eps=1e-5):
    """float32 RMSNorm of the rows of x [..., H] with gain (1 + w)."""
    x = np.asarray(x, dtype=np.float32)
    H = x.shape[-1]
    ss = sum_of_squares(x)
    mean = ss / np.float32(H)
    r = np.sqrt(mean + np.float32(eps))
    y = x / r[..., None]
    if w is not None:
        y = y * (np.float32(1.0) + np.asarray(w, dtype=np.float32))
    return y.astype(np.float32)
