"""Pins of the CSF scale codec (oracle/csf.py) against the page's format
description, its size table, brute force and hand-worked rows."""
import json
import os

import numpy as np

from oracle import csf as OC
from oracle import quant as OQ

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def _brute_base(row):
    best, best_n = 0, -1
    for b in range(0, 241):
        n = sum(1 for v in row if b <= v <= b + 15)
        if n > best_n:
            best, best_n = b, n
    return best


def test_base_rule_against_brute_force():
    rng = np.random.default_rng(11)
    rows = [rng.integers(0, 256, 12), rng.integers(100, 130, 12), rng.integers(0, 8, 12) * 32,
            np.full(12, 255), np.array([0x10, 0x30, 0x50, 0x70] * 3), rng.integers(0x30, 0x7F, 12)]
    rows += [rng.integers(0, 256, 12) for _ in range(40)]
    rows = np.array(rows, dtype=np.uint8)
    got = OC.row_bases(rows)
    assert [int(g) for g in got] == [_brute_base(list(map(int, r))) for r in rows]


def test_hand_worked_rows():
    s = np.zeros((1, 16, 4), dtype=np.uint8)
    s[0, 0] = [0x30, 0x31, 0x3F, 0x40]     # windows at 0x30 and 0x31 both hold 3: the lower wins
    s[0, 2] = [0x10, 0x30, 0x50, 0x70]     # every window holds at most 1: base 1 (covers 0x10)
    s[0, 3] = [0xFF, 0xFF, 0xF0, 0x00]     # the top window [240, 255]
    fixed, exc, starts = OC.encode(s)
    bases = [0x30, 0, 1, 0xF0] + [0] * 12
    codes = [[0x10, 0x0F], [0, 0], [0x0F, 0x00], [0xFF, 0x00]] + [[0, 0]] * 12
    want = np.array([bases + sum(codes, [])], dtype=np.uint8).reshape(1, 1, 16 * 3)
    assert np.array_equal(fixed, want)
    want_exc = [(0 * 4 + 3) | (0x40 << 24),
                (2 * 4 + 1) | (0x30 << 24), (2 * 4 + 2) | (0x50 << 24), (2 * 4 + 3) | (0x70 << 24),
                (3 * 4 + 3) | (0x00 << 24)]
    assert exc.tolist() == want_exc
    assert starts.tolist() == [0, 5]
    assert np.array_equal(OC.decode(fixed, exc, starts, 16, 4), s)


def test_round_trip_random_and_grouped_by_expert():
    rng = np.random.default_rng(5)
    E, R, C = 3, 32, 10
    s = (0x38 + rng.integers(0, 16, (E, R, C))).astype(np.uint8)
    out = rng.random((E, R, C)) < 0.07
    s[out] = rng.integers(0, 256, out.sum())
    fixed, exc, starts = OC.encode(s)
    assert fixed.shape == (E, R // 16, 16 * (1 + C // 2))
    assert starts[0] == 0 and starts[-1] == exc.size and np.all(np.diff(starts) >= 0)
    for e in range(E):     # row-major within an expert
        pos = exc[starts[e]:starts[e + 1]] & 0xFFFFFF
        assert np.all(np.diff(pos.astype(np.int64)) > 0)
    assert np.array_equal(OC.decode(fixed, exc, starts, R, C), s)


def test_round_trip_of_quantizer_scales():
    """Block scales of the NVFP4 quantizer on N(0, 0.02) weights."""
    rng = np.random.default_rng(3)
    W = (rng.standard_normal((2, 32, 256)) * 0.02)
    scales = np.stack([OQ.e4m3_bytes(OQ.quantize_nvfp4(W[e])[1]) for e in range(2)]).astype(np.uint8)
    fixed, exc, starts = OC.encode(scales)
    assert np.array_equal(OC.decode(fixed, exc, starts, 32, 16), scales)


def test_sizes_reproduce_the_page_table():
    """fixed = E * R * (1 + C/2) per tensor; with the starts tensors, the
    page's CSF totals leave a whole number of 4-byte exceptions, and the
    ratio to the raw scales is the page's 51.44 %."""
    g = GOLD["csf_sizes_bytes"]
    sz = GOLD["nvfp4_sizes_bytes"]
    E = 352
    per_layer_fixed = (2 * OC.fixed_bytes(E, sz["gate_up_R"], sz["gate_up_C"]) +
                       OC.fixed_bytes(E, sz["down_R"], sz["down_C"]))
    assert per_layer_fixed == 2 * 352 * 1536 * 129 + 352 * 4096 * 49
    starts = 3 * (E + 1) * 8
    for layers, total in ((g["layers_3_87"], g["layers_3_87_csf_scales"]),
                          (g["layers_88_90"], g["layers_88_90_csf_scales"])):
        rest = total - layers * (per_layer_fixed + starts)
        assert rest > 0 and rest % 4 == 0
    raw = g["layers_3_87"] * (2 * E * sz["gate_up_R"] * sz["gate_up_C"] + E * sz["down_R"] * sz["down_C"])
    assert raw == g["layers_3_87_raw_scales"]
    assert round(100 * g["layers_3_87_csf_scales"] / raw, 2) == g["csf_percent"]


def test_row_starts_by_brute_force_and_partition():
    """Every row's range holds exactly the exceptions whose position falls
    in that row (brute force over all positions), the ranges tile each
    expert's list in order, and decoding a row from its range alone
    reproduces the row."""
    rng = np.random.default_rng(5)
    E, R, C = 3, 32, 48
    base = rng.integers(0x30, 0x60, (E, R, 1))
    s = (base + rng.integers(0, 16, (E, R, C))).astype(np.uint8)
    out = rng.random((E, R, C)) < 0.15
    s[out] = rng.integers(0, 0x7F, int(out.sum()))
    s[1, 7, :] = 0x7E                     # a row made only of one value
    s[2] = s[2, :, :1]                    # an expert without exceptions
    fixed, exc, starts = OC.encode(s)
    rs = OC.row_starts(exc, starts, E, R, C)
    assert rs.shape == (E, R + 1) and rs.dtype == np.int32
    for e in range(E):
        assert rs[e, 0] == starts[e] and rs[e, R] == starts[e + 1]
        assert np.all(np.diff(rs[e]) >= 0)
        for r in range(R):
            mine = [x for x in range(int(starts[e]), int(starts[e + 1]))
                    if r * C <= (int(exc[x]) & 0xFFFFFF) < (r + 1) * C]
            assert list(range(rs[e, r], rs[e, r + 1])) == mine, (e, r)
            row = (fixed[e, r // 16, r % 16] + np.concatenate(
                [[b & 15, b >> 4] for b in fixed[e, r // 16, 16 + (r % 16) * (C // 2):
                                                 16 + (r % 16 + 1) * (C // 2)]])).astype(np.uint8)
            for x in range(rs[e, r], rs[e, r + 1]):
                row[(int(exc[x]) & 0xFFFFFF) - r * C] = int(exc[x]) >> 24
            assert np.array_equal(row, s[e, r]), (e, r)
