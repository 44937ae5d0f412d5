"""Weight formats of the routed experts: quantizers, packing, dequantization.

TEST INFRASTRUCTURE ONLY (see the package docstring).

int4-g128 (page "NeuroSenko/Step-5-Preview-Int4-g128", sections "Recipe" and
"Tensor layout"): symmetric int4, one scale per 128 input channels, the scale
stored in bf16; each group tries 17 clipping ratios between 0.60 and 1.00
and keeps the one with the smallest squared rounding error, the search done in the scale's own precision so
that quantizing and dequantizing agree exactly. Routed experts only; the
fused source tensors are [experts, out, in].

NVFP4 (page "Step-5-Preview-NVFP4-Local", "Modifications" item 2 and
"Format"): bytes [E, R, K/2], each holding two E2M1 codes; an E4M3 block
scale for every 16 weights [E, R, K/16]; one float32 global scale
(weight_scale_2) per expert [E]. A weight's value is the product of its E2M1
value, its block scale and its expert's global scale. The page's last three
layers were BF16 at the source and were brought to NVFP4 by the page's
author with the same recipe as the others.

Readings where the pages are silent (each also listed in the design notes):
* int4 scale = clip_ratio * max|w| / 7 (divisor 7), q = clamp(rne(w/s), -8, 7).
  The divisor is not printed; 7 is the one that reproduces the page's error
  table (max-abs 11.74 %, clip search 10.11 %) on Gaussian weights.
* the 17 ratios are 1.00, 0.975, ..., 0.60 (evenly spaced, step 0.025); the
  candidate scale is bf16(fl64((40 - i) * a / 280)), rounded once to bf16;
  the MSE of a candidate is accumulated in float64 in ascending input order;
  the first minimum in ratio order wins (ties go to the larger ratio).
* nibble j of int32 word w along K holds input 8w+j (low nibble first, as the
  NVFP4 page's scale codes are stored), as a two's-complement 4-bit integer.
* int4 g32 (the error table's int4-g32 row, searched like g128): the same quantizer
  with one scale per 32 inputs.
* asymmetric int4 (the error table's asymmetric int4-g128 row): min-max range
  widened to contain 0, scale bf16((hi - lo) / 15), zero point
  clamp(rne(-lo / s), 0, 15) stored as one byte per group, unsigned nibbles
  q in [0, 15], w = (q - z) * s; no clip search. This reading gives 10.04 %
  on Gaussian weights and inputs against the page's 10.05 % (a clip search
  would give 9.5 %).
* int8 (the page compares against 8-bit experts but gives no format): the int4-g128 recipe
  on the 8-bit grid: candidate scale bf16(ratio * max|w| / 127) over the
  same 17 ratios, q = clamp(rne(w / s), -128, 127), one byte per weight
  [n, k] (two's complement), bf16 scales [n, k/128]. On Gaussian weights
  this gives 0.65 % against the page's 0.73 %, and per-row scales 0.86 %;
  neither reproduces the page's figure, so it is not a pin.
* NVFP4 global scale = fp32(max|W| / (6 * 448)) per expert matrix (1 for an
  all-zero matrix); block scale = E4M3(max|block| / (6 * gs)), saturating,
  ties to even; element code = E2M1(w / (bs * gs)), saturating, ties to
  even, a value that rounds to zero gets code 0 (+0). Within a byte the low
  nibble is the even input index.
"""
import numpy as np

from .formats import (E2M1, E2M1_TABLE, E4M3, E4M3_TABLE, bf16_from_bits, round_to_format,
                      to_bf16, to_fp32, e2m1_decode, e2m1_encode, e4m3_decode,
                      e4m3_encode_nonneg)

INT4_GROUP = 128
NVFP4_GROUP = 16
N_CLIP = 17


# ------------------------------------------------------------------ int4 ---
def int4_candidate_scale(a, i, qmax=7):
    """Scale of clip ratio i (ratio (40 - i)/40) for a group with max|w| = a
    on the grid [-qmax - 1, qmax]."""
    return to_bf16(((40 - i) * np.asarray(a, dtype=np.float64)) / (40.0 * qmax))


def quantize_int4(W, clip_search=True, group=INT4_GROUP):
    """Quantize W [n, k] (bf16-representable values, float64 array).

    Returns q [n, k] int8 in [-8, 7] and s [n, k/group] float64 (bf16 values).
    With clip_search=False only ratio 1.00 is tried (the max-abs comparator).
    """
    return _quantize_symmetric(W, clip_search, group, 7)


def quantize_int8(W, clip_search=True, group=INT4_GROUP):
    """The same recipe on the 8-bit grid: q [n, k] int8 in [-128, 127] and s
    [n, k/group] float64 (bf16 values)."""
    return _quantize_symmetric(W, clip_search, group, 127)


def _quantize_symmetric(W, clip_search, group, qmax):
    W = np.asarray(W, dtype=np.float64)
    n, k = W.shape
    assert k % group == 0
    Wg = W.reshape(n, k // group, group)
    a = np.max(np.abs(Wg), axis=-1)
    best_mse = np.full(a.shape, np.inf)
    best_s = np.zeros(a.shape)
    best_q = np.zeros(Wg.shape, dtype=np.int8)
    for i in range(N_CLIP if clip_search else 1):
        s = int4_candidate_scale(a, i, qmax)
        sg = s[..., None]
        with np.errstate(divide="ignore", invalid="ignore"):
            q = np.where(sg > 0, np.clip(np.rint(Wg / sg), -qmax - 1, qmax), 0.0)
        err = q * sg - Wg
        mse = np.cumsum(err * err, axis=-1)[..., -1]    # ascending k, fp64
        better = mse < best_mse                          # first minimum wins
        best_mse = np.where(better, mse, best_mse)
        best_s = np.where(better, s, best_s)
        best_q = np.where(better[..., None], q.astype(np.int8), best_q)
    return best_q.reshape(n, k), best_s


def pack_int4(q):
    """q [n, k] int in [-8, 7] -> int32 words [n, k/8]; nibble j of word w is
    input 8w+j, stored as its two's-complement low 4 bits."""
    q = np.asarray(q, dtype=np.int64)
    n, k = q.shape
    assert k % 8 == 0 and q.min(initial=0) >= -8 and q.max(initial=0) <= 7
    nib = (q & 0xF).astype(np.uint64).reshape(n, k // 8, 8)
    shifts = (4 * np.arange(8)).astype(np.uint64)
    words = np.bitwise_or.reduce(nib << shifts, axis=-1).astype(np.uint32)
    return words.view(np.int32)


def unpack_int4(words):
    """int32 words [n, k/8] -> q [n, k] int8: nibble j of a word, read as a
    4-bit two's-complement number (8..15 stand for -8..-1)."""
    w = np.asarray(words).view(np.uint32)
    n, kw = w.shape
    nib = ((w[..., None] >> (4 * np.arange(8, dtype=np.uint32))) & 0xF).astype(np.int8)
    q = nib - np.int8(16) * (nib >= 8)
    return q.reshape(n, kw * 8)


def _group_scale(q, s, group):
    """q [n, k] times the scale of its group, s [n, k/group] (float64)."""
    n, k = q.shape
    return (q.reshape(n, k // group, group) * s[..., None]).reshape(n, k)


def dequant_int4(words, scales_bf16_bits, group=INT4_GROUP):
    """Exact dequantized values q * s (float64) from packed words [n, k/8]
    and bf16 scale bit patterns [n, k/group] (uint16)."""
    return _group_scale(unpack_int4(words), bf16_from_bits(scales_bf16_bits), group)


def dequant_int8(q, scales_bf16_bits, group=INT4_GROUP):
    """Exact q * s (float64) from int8 weights [n, k] and bf16 scale bit
    patterns [n, k/group]."""
    return _group_scale(np.asarray(q, dtype=np.int8), bf16_from_bits(scales_bf16_bits), group)


def rel_error(W, Wq, X):
    """||(Wq - W) X|| / ||W X|| (Frobenius norm over the columns of X), the
    error measure of the int4 page's table."""
    return np.linalg.norm((Wq - W) @ X) / np.linalg.norm(W @ X)


# ------------------------------------------------------- int4 asymmetric ---
def quantize_int4_asym(W, group=INT4_GROUP):
    """Asymmetric int4 with one bf16 scale and one zero point per group (the
    int4 page's error table, its asymmetric g128 row). Min-max range that
    always contains 0: lo = min(min w, 0), hi = max(max w, 0);
    s = bf16((hi - lo) / 15); z = clamp(rne(-lo / s), 0, 15);
    q = clamp(rne(w / s) + z, 0, 15); w ~ (q - z) * s. An all-zero group
    gets s = 0, z = 0, q = 0. Returns q [n, k] uint8, s [n, k/group] float64
    (bf16 values), z [n, k/group] uint8."""
    W = np.asarray(W, dtype=np.float64)
    n, k = W.shape
    assert k % group == 0
    Wg = W.reshape(n, k // group, group)
    lo = np.minimum(Wg.min(axis=-1), 0.0)
    hi = np.maximum(Wg.max(axis=-1), 0.0)
    s = to_bf16((hi - lo) / 15.0)
    safe = np.where(s > 0, s, 1.0)
    z = np.where(s > 0, np.clip(np.rint(-lo / safe), 0, 15), 0.0)
    q = np.where(s[..., None] > 0, np.clip(np.rint(Wg / safe[..., None]) + z[..., None], 0, 15),
                 0.0)
    return q.reshape(n, k).astype(np.uint8), s, z.astype(np.uint8)


def pack_uint4(q):
    """q [n, k] in [0, 15] -> int32 words [n, k/8]; nibble j of word w is input 8w+j."""
    q = np.asarray(q, dtype=np.int64)
    assert q.min(initial=0) >= 0 and q.max(initial=0) <= 15
    return pack_int4(q - 16 * (q >= 8))      # the same nibble bits, read as unsigned


def unpack_uint4(words):
    """int32 words [n, k/8] -> q [n, k] uint8 in [0, 15]."""
    return (unpack_int4(words).astype(np.int64) & 0xF).astype(np.uint8)


def dequant_int4_asym(words, scales_bf16_bits, zeros, group=INT4_GROUP):
    """Exact (q - z) * s (float64) from packed unsigned nibbles [n, k/8], bf16
    scale bit patterns [n, k/group] and zero points uint8 [n, k/group]."""
    q = unpack_uint4(words).astype(np.float64)
    n, k = q.shape
    d = q.reshape(n, k // group, group) - np.asarray(zeros, dtype=np.float64)[..., None]
    return _group_scale(d.reshape(n, k), bf16_from_bits(scales_bf16_bits), group)


# ----------------------------------------------------------------- NVFP4 ---
def nvfp4_global_scale(W):
    A = float(np.max(np.abs(W))) if np.size(W) else 0.0
    if A == 0.0:
        return 1.0
    return float(to_fp32(A / (6.0 * 448.0)))


def quantize_nvfp4(W, group=NVFP4_GROUP):
    """Quantize one expert matrix W [n, k] (float64, bf16-representable).

    Returns codes [n, k] uint8 (E2M1 codes), block-scale values bs [n, k/16]
    (float64, E4M3-representable, >= 0) and the global scale gs (float,
    fp32-representable).
    """
    W = np.asarray(W, dtype=np.float64)
    n, k = W.shape
    assert k % group == 0
    gs = nvfp4_global_scale(W)
    Wb = W.reshape(n, k // group, group)
    amax = np.max(np.abs(Wb), axis=-1)
    bs = round_to_format(amax / (6.0 * gs), E4M3, saturate=True)
    denom = (bs * gs)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(denom > 0, Wb / denom, 0.0)
    vq = round_to_format(v, E2M1, saturate=True)
    codes = e2m1_encode(vq.reshape(n, k))
    return codes, bs, gs


def quantize_nvfp4_act(x, g, group=NVFP4_GROUP):
    """NVFP4 quantization of activations (rows of x [..., k], 16-bit values
    widened to float32) with the tensor's float32 global scale g > 0.

    The pages give no rule for activations; the reading taken is the
    weights' two-level rule (page "Step-5-Preview-NVFP4-Local", "Format":
    E2M1 value x E4M3 block scale per 16 x a float32 scale, here the input
    scale of the quantized layers, "Modifications" items 2-3), with every
    decision taken in float32, the precision of the kernels:
        D = 6 g;  per 16-block t = max|x| / D;  bs = E4M3(t), nearest,
        ties to even, saturating at 448;  den = bs g;  v = x / den;
        code = E2M1(v), nearest, ties to even, saturating at 6 (a zero
        block scale gives code 0, a magnitude rounding to 0 gives +0),
    each arithmetic step one float32 operation rounded to nearest even.
    Returns (codes uint8 [..., k], bs float64 [..., k/16] E4M3 values,
    xhat float64 [..., k] = e2m1 x bs, exact); the quantized activation is
    xhat * g.
    """
    x32 = np.asarray(x, dtype=np.float32)
    g32 = np.float32(g)
    k = x32.shape[-1]
    assert k % group == 0 and g32 > 0
    xb = x32.reshape(x32.shape[:-1] + (k // group, group))
    D = np.float32(6.0) * g32
    with np.errstate(over="ignore", under="ignore"):
        t = np.max(np.abs(xb), axis=-1) / D                       # float32
        bs = round_to_format(t.astype(np.float64), E4M3, saturate=True)
        den = bs.astype(np.float32) * g32                         # float32
        safe = np.where(den > 0, den, np.float32(1.0))
        v = np.where(den[..., None] > 0, xb / safe[..., None], np.float32(0.0))
    vq = round_to_format(v.astype(np.float64), E2M1, saturate=True)
    codes = e2m1_encode(vq).reshape(x32.shape)
    xhat = (vq * bs[..., None]).reshape(x32.shape) + 0.0       # -0 -> +0
    return codes, bs, xhat


def pack_nvfp4(codes):
    """codes [n, k] -> bytes [n, k/2]; the low nibble is the even input."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] & 0xF) | ((c[:, 1::2] & 0xF) << 4)


def unpack_nvfp4(packed):
    p = np.asarray(packed, dtype=np.uint8)
    n, kh = p.shape
    out = np.empty((n, 2 * kh), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def e4m3_bytes(bs):
    return e4m3_encode_nonneg(bs)


def dequant_nvfp4(packed, scale_bytes, gs, group=NVFP4_GROUP):
    """The product of the E2M1 value, its E4M3 block scale and the expert's
    global scale, exact in float64."""
    v = E2M1_TABLE[unpack_nvfp4(packed)]          # value of every code
    b = E4M3_TABLE[np.asarray(scale_bytes, dtype=np.uint8)]
    return _group_scale(v, b, group) * float(gs)


def dequant_nvfp4_fp32(packed, scale_bytes, gs, group=NVFP4_GROUP):
    """The dequantized weight rounded once to float32 (the exact float64
    product has at most 2 + 4 + 24 significant bits)."""
    return to_fp32(dequant_nvfp4(packed, scale_bytes, gs, group))


def nmse(W, Wq):
    """Weight normalised MSE ||Wq - W||^2 / ||W||^2."""
    return float(np.sum((Wq - W) ** 2) / np.sum(W ** 2))
