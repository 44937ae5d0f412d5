"""Pins of the oracle's number formats against library routines and the OCP
specification tables (tests/golden/ocp_e2m1_e4m3.txt)."""
import math
import os

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLD = os.path.join(os.path.dirname(__file__), "golden", "ocp_e2m1_e4m3.txt")


def _golden():
    rows = {"e2m1": {}, "e4m3": {}}
    for line in open(GOLD):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        kind, code, val = line.split()
        rows[kind][int(code, 16)] = float(val)
    return rows


def _same(a, b):
    if math.isnan(b):
        return math.isnan(a)
    return a == b and math.copysign(1, a) == math.copysign(1, b)


def test_e2m1_table_matches_spec():
    g = _golden()["e2m1"]
    assert len(g) == 16
    for code, val in g.items():
        assert _same(float(F.E2M1_TABLE[code]), val), code


def test_e4m3_table_matches_spec_points():
    g = _golden()["e4m3"]
    for b, val in g.items():
        assert _same(float(F.E4M3_TABLE[b]), val), hex(b)
    finite = F.E4M3_TABLE[~np.isnan(F.E4M3_TABLE)]
    assert finite.size == 254
    pos = F.E4M3_TABLE[:0x7F]
    assert np.all(np.diff(pos) > 0)


def test_fp32_and_fp16_rounding_match_numpy_casts():
    r = np.random.default_rng(1)
    x = np.concatenate([r.standard_normal(20000) * 10.0 ** r.integers(-9, 6, 20000),
                        [0.0, -0.0, 1.0, 65504.0, 65520.0, 1e-8, 3e-5]])
    assert np.array_equal(F.to_fp32(x), x.astype(np.float32).astype(np.float64))
    with np.errstate(over="ignore"):
        ref16 = x.astype(np.float16).astype(np.float64)
    assert np.array_equal(F.to_fp16(x), ref16)
    # exact ties of fp16: 1 + 2^-11 lies halfway between 1 and 1 + 2^-10
    assert F.to_fp16(1.0 + 2.0 ** -11) == 1.0
    assert F.to_fp16(1.0 + 3 * 2.0 ** -11) == 1.0 + 2.0 ** -9


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(2)
    x = (r.standard_normal(50000) * 10.0 ** r.integers(-30, 30, 50000)).astype(np.float32)
    # plus exact halfway cases: low 16 bits 0x8000 with both parities above
    bits = r.integers(0, 2 ** 31, 2000).astype(np.uint32) & np.uint32(0x7F7F0000)
    halves = (bits | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, halves, -halves])
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy().astype(np.float64)
    assert np.array_equal(F.to_bf16(x.astype(np.float64)), ref)


def test_small_format_rounding_is_nearest_ties_even_by_brute_force():
    """E4M3 / E2M1 rounding equals the nearest table entry, ties to the entry
    with an even mantissa (even code), saturating at the maximum."""
    r = np.random.default_rng(3)
    for fmt, table, vmax in ((F.E4M3, F.E4M3_TABLE[:0x7F], 448.0),
                             (F.E2M1, F.E2M1_TABLE[:8], 6.0)):
        mids = (table[1:] + table[:-1]) / 2
        x = np.concatenate([r.uniform(0, vmax * 1.2, 5000), mids, table])
        got = F.round_to_format(x, fmt, saturate=True)
        for xi, gi in zip(x, got):
            d = np.abs(table - xi)
            cand = np.nonzero(d == d.min())[0]
            if xi > vmax:
                want = vmax
            elif cand.size == 1:
                want = table[cand[0]]
            else:
                want = table[[c for c in cand if c % 2 == 0][0]]
            assert gi == want, (xi, gi, want)


@pytest.mark.parametrize("v,want", [(0.25, 0.0), (0.75, 1.0), (1.25, 1.0), (1.75, 2.0),
                                    (2.5, 2.0), (3.5, 4.0), (5.0, 4.0), (7.0, 6.0),
                                    (100.0, 6.0), (-0.2, -0.0), (-2.9, -3.0)])
def test_e2m1_worked_ties(v, want):
    assert _same(float(F.round_to_format(v, F.E2M1, saturate=True)), want)


def test_e2m1_encode_decode_roundtrip():
    for c in range(16):
        v = F.E2M1_TABLE[c]
        enc = int(F.e2m1_encode(v))
        assert enc == (0 if c == 8 else c)     # -0 encodes as +0
    for b in range(0x7F):
        assert int(F.e4m3_encode_nonneg(F.E4M3_TABLE[b])) == b
