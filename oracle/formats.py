"""Number formats used by the layer, restated from their bit-field definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources
-------
* bf16 / fp16 / fp32: IEEE 754 binary formats (bf16 = the top half of an
  fp32 word); rounding is round-to-nearest, ties-to-even.
* E2M1 (FP4) and E4M3FN (FP8): the OCP Microscaling and OCP 8-bit
  floating-point specifications. The NVFP4 page (Step-5-Preview-NVFP4-Local,
  "Modifications" item 2 and "Format") names the weight as E2M1 pairs with
  F8_E4M3 block scales; the bit layouts themselves come from those specs.

Everything here works on float64 numpy arrays. One generic rounding routine
serves every format: a value is rounded to `p` significant bits, with the
exponent of the smallest normal number `emin` bounding the precision of the
subnormal range, ties to even.
"""
import numpy as np

# (significant bits incl. the implicit one, min normal exponent, max finite)
BF16 = (8, -126, float.fromhex("0x1.fe00000000000p+127"))
FP16 = (11, -14, 65504.0)
FP32 = (24, -126, float.fromhex("0x1.fffffe0000000p+127"))
E4M3 = (4, -6, 448.0)          # OCP E4M3FN: no infinities, 0x7F/0xFF are NaN
E2M1 = (2, 0, 6.0)             # OCP FP4 E2M1: no infinities, no NaN


def round_to_format(x, fmt, saturate=False):
    """Round float64 values to the nearest value of `fmt`, ties to even.

    Overflow goes to +-inf, or to +-max when `saturate` (the FP8 / FP4
    conversions used by the NVFP4 quantizer saturate). Zero keeps its sign.
    """
    p, emin, vmax = fmt
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                       # x = m * 2**e, 0.5 <= |m| < 1
    exp = np.maximum(e - 1, emin)            # exponent of the leading bit
    ulp = np.ldexp(1.0, exp - (p - 1))
    r = np.rint(x / ulp) * ulp               # np.rint: ties to even
    r = np.where(x == 0, x, r)
    big = np.abs(r) > vmax
    if saturate:
        r = np.where(big, np.copysign(vmax, x), r)
    else:
        r = np.where(big, np.copysign(np.inf, x), r)
    return r


def to_bf16(x):
    return round_to_format(x, BF16)


def to_fp16(x):
    return round_to_format(x, FP16)


def to_fp32(x):
    return round_to_format(x, FP32)


def bf16_bits(v):
    """uint16 bit patterns of values already representable in bf16."""
    v = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def bf16_from_bits(b):
    b = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- E2M1 ---
def e2m1_decode(code):
    """Value of a 4-bit E2M1 code: sign | 2 exponent bits | 1 mantissa bit,
    exponent bias 1; exponent field 0 is subnormal (0 or 0.5)."""
    c = np.asarray(code, dtype=np.int64) & 0xF
    sign = np.where(c & 8, -1.0, 1.0)
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return sign * mag


E2M1_TABLE = e2m1_decode(np.arange(16))          # index = code


def e2m1_encode(v):
    """Code of a value that is exactly representable in E2M1. Zero (of
    either sign) maps to code 0."""
    v = np.asarray(v, dtype=np.float64)
    mags = E2M1_TABLE[:8]
    idx = np.searchsorted(mags, np.abs(v))
    if not np.all(mags[np.minimum(idx, 7)] == np.abs(v)):
        raise ValueError("value not representable in E2M1")
    return np.where((v < 0) & (idx != 0), idx | 8, idx).astype(np.uint8)


# ---------------------------------------------------------------- E4M3 ---
def e4m3_decode(byte):
    """Value of an E4M3FN byte: sign | 4 exponent bits (bias 7) | 3 mantissa
    bits; exponent field 0 is subnormal; S.1111.111 is NaN."""
    b = np.asarray(byte, dtype=np.int64) & 0xFF
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


E4M3_TABLE = e4m3_decode(np.arange(256))         # index = byte


def e4m3_encode_nonneg(v):
    """Byte of a non-negative value exactly representable in E4M3FN."""
    v = np.asarray(v, dtype=np.float64)
    pos = E4M3_TABLE[:0x7F]                     # 0x00..0x7E, ascending
    idx = np.searchsorted(pos, v)
    if not np.all(pos[np.minimum(idx, 0x7E)] == v):
        raise ValueError("value not representable in E4M3")
    return idx.astype(np.uint8)
