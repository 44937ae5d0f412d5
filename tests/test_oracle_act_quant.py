"""Pins of the oracle's NVFP4 activation quantizer (the quantized-activation
layers) and of the layer map that quantizes h: values worked by hand, the
E2M1 and E4M3 tie rules, saturation, zero blocks, brute force over both
grids, an exact round trip, the error bound, and the layer's reduction to
plain NVFP4 weights when every activation is already on the grid."""
import numpy as np
import pytest

from oracle import formats as OF
from oracle import layer as OL
from oracle import quant as OQ

F32 = np.float32


def test_hand_worked_block():
    # g = fl32(1/6): D = fl32(6 g) = 1 exactly (6 * 0.1666666716... =
    # 1.00000003, nearest float32 1.0); amax 6 -> t = 6 -> block scale 6
    # (E4M3 1.5 * 2^2); den = fl32(6 g) = 1, so v = x: 3 -> 3 (code 5),
    # -1.5 -> code 0b1011, 0.25 ties to 0, 0.75 ties to 1.0 (even mantissa),
    # 2.5 ties to 2, 5 ties to 4, 6 and -6 stay
    x = np.array([3, -1.5, 0.25, 0.75, 2.5, 5, 6, -6] + [0] * 8, np.float32)
    codes, bs, xhat = OQ.quantize_nvfp4_act(x, F32(1 / 6))
    assert bs.tolist() == [6.0]
    assert codes.tolist() == [5, 11, 0, 2, 4, 6, 7, 15] + [0] * 8
    assert xhat.tolist() == [18, -9, 0, 6, 12, 24, 36, -36] + [0] * 8


def test_block_scale_rounding_and_saturation():
    # g = 1/24 (power-of-two fraction free: 24 g = 1): D = fl32(6 g) = 0.25
    g = F32(1 / 24)
    assert F32(6) * g == F32(0.25)
    # amax 1.375 -> t = 5.5: E4M3 grid at 4..8 has step 0.5: 5.5 exact
    _, bs, _ = OQ.quantize_nvfp4_act(np.r_[F32(1.375), np.zeros(15, F32)], g)
    assert bs.tolist() == [5.5]
    # amax 1.40625 -> t = 5.625: neighbours 5.5 and 6.0 at 0.125 and 0.375
    # -> 5.5; amax 1.4375 -> t = 5.75, halfway: 5.5 has an odd mantissa
    # (0b011), 6.0 an even one (0b100) -> 6.0
    _, bs, _ = OQ.quantize_nvfp4_act(np.r_[F32(1.40625), np.zeros(15, F32)], g)
    assert bs.tolist() == [5.5]
    _, bs, _ = OQ.quantize_nvfp4_act(np.r_[F32(1.4375), np.zeros(15, F32)], g)
    assert bs.tolist() == [6.0]
    # t = 1000 -> saturates at 448; values beyond 6 * 448 * g saturate at 6
    x = np.r_[F32(250.0), F32(-300.0), F32(1.0), np.zeros(13, F32)]
    codes, bs, xhat = OQ.quantize_nvfp4_act(x, g)
    assert bs.tolist() == [448.0]
    assert codes[:2].tolist() == [7, 15]                  # 250/(448/24) = 13.4 -> 6
    assert xhat[:2].tolist() == [6 * 448.0, -6 * 448.0]
    # 1 / (448 / 24) = 0.0536 -> rounds to 0: code +0
    assert codes[2] == 0 and xhat[2] == 0.0 and not np.signbit(xhat[2])


def test_zero_block_and_negative_zero():
    x = np.zeros((2, 32), np.float32)
    x[1, 16:] = -0.0
    codes, bs, xhat = OQ.quantize_nvfp4_act(x, F32(0.5))
    assert np.all(codes == 0) and np.all(bs == 0) and not np.any(np.signbit(xhat))


def test_brute_force_nearest():
    """Every block scale is the nearest finite E4M3 value to t (ties to the
    even byte, whose mantissa is even), capped at 448; every code is the nearest of the 8 E2M1
    magnitudes to |v| (ties to the even code), with the sign of x unless
    it rounds to 0."""
    r = np.random.default_rng(3)
    g = F32(0.0123)
    x = (r.standard_normal((40, 64)) * np.exp(r.uniform(-6, 6, (40, 1)))).astype(np.float32)
    x[:, ::7] = x[:, ::7] * 8                                  # force ties of amax scales
    codes, bs, xhat = OQ.quantize_nvfp4_act(x, g)
    e4 = OF.E4M3_TABLE[:0x7F]
    e2 = OF.E2M1_TABLE[:8]
    D = F32(6) * g
    for row in range(x.shape[0]):
        for blk in range(4):
            xb = x[row, 16 * blk:16 * blk + 16]
            t = float(np.max(np.abs(xb)) / D)
            d = np.abs(e4 - t)
            best = np.flatnonzero(d == d.min())
            want = e4[best[0]] if len(best) == 1 else e4[best[best % 2 == 0][0]]
            want = min(want, 448.0) if t <= 448.0 else 448.0
            assert bs[row, blk] == want, (row, blk, t)
            den = F32(bs[row, blk]) * g
            for i in range(16):
                if bs[row, blk] == 0:
                    assert codes[row, 16 * blk + i] == 0
                    continue
                v = float(xb[i] / den)
                dd = np.abs(e2 - abs(v))
                b = np.flatnonzero(dd == dd.min())
                m = b[0] if len(b) == 1 else b[b % 2 == 0][0]
                if abs(v) > 6:
                    m = 7
                c = codes[row, 16 * blk + i]
                assert (c & 7) == m, (row, blk, i, v)
                assert (c >> 3) == (1 if (v < 0 and m != 0) else 0)


def test_round_trip_on_the_grid():
    """Activations that already are e2m1 x bs x g, with a full-scale value in
    every block (so that max / (6 g) = bs exactly, g a power of two),
    quantize to themselves."""
    r = np.random.default_rng(5)
    g = F32(2.0 ** -7)
    codes = r.integers(0, 16, (8, 128)).astype(np.uint8)
    codes[:, ::16] = 7                                         # +6 in every block
    bs = OF.E4M3_TABLE[r.integers(0x08, 0x7F, (8, 8))]
    x = (OF.E2M1_TABLE[codes] * np.repeat(bs, 16, axis=1) * float(g)).astype(np.float32)
    c2, bs2, xhat = OQ.quantize_nvfp4_act(x, g)
    assert np.array_equal(bs2, bs)
    assert np.array_equal(xhat * float(g), x.astype(np.float64) + 0.0)
    assert np.array_equal(OF.E2M1_TABLE[c2], OF.E2M1_TABLE[codes] + 0.0)


def test_error_bound():
    """Unsaturated values land within half an E2M1 step of x / (bs g): the
    step is 0.5 below 2, 1 below 4 and 2 above, so |xhat g - x| <= bs g
    times 0.25, 0.5 or 1; a block's max is never clipped when t < 448."""
    r = np.random.default_rng(7)
    g = F32(0.031)
    x = (r.standard_normal((16, 256)) * 3).astype(np.float32)
    codes, bs, xhat = OQ.quantize_nvfp4_act(x, g)
    assert np.all(bs < 448)
    den = np.repeat(bs, 16, axis=1) * float(g)
    v = x.astype(np.float64) / den
    half_step = np.where(np.abs(v) < 2, 0.25, np.where(np.abs(v) < 4, 0.5, 1.0))
    assert np.all(np.abs(xhat * float(g) - x) <= half_step * den * (1 + 1e-6))
    # each block's largest magnitude maps to at most 6 (no clipping)
    assert np.all(np.abs(v).reshape(16, 16, 16).max(axis=-1) <= 6.0 * (1 + 2 ** -3))


def test_h_map_idempotent_and_close():
    """The layer's map of h (round to bf16, quantize with g_h, times g_h) is
    idempotent once h is on its grid (g_h a power of two), and stays
    within a third of each block's range of h."""
    g_h = F32(2.0 ** -6)
    fn = OL.a4_h_fn(g_h)
    r = np.random.default_rng(9)
    h = r.standard_normal((3, 64))
    q1 = fn(h)
    q2 = fn(q1)
    assert np.array_equal(q1, q2)                              # idempotent on its grid
    assert np.max(np.abs(q1 - h)) < 0.35 * np.max(np.abs(h))   # and close to h
