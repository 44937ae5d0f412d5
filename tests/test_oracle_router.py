"""Pins of the oracle router: the canonical float32 logit chain, top-K
selection with lower-index ties, and the sigmoid weights."""
import math

import numpy as np
import pytest

from oracle import router as R
from quantized_moe_sigmoid_amd import synth


def test_logits_within_fp32_error_bound_of_exact_sum():
    """|chain - exact| <= H * 2^-24 * sum|x w| (the sequential summation
    bound, which also covers block chains added in order), on the tiny
    layer; a transposed or mis-indexed weight fails this."""
    cfg = synth.CONFIGS["tiny"]
    T, H, E = cfg["T"][0], cfg["H"], cfg["E"]
    x = synth.activations(T, H, "f16", 0).float().numpy()
    wT = synth.router_weight_T(H, E, 0)
    lg = R.router_logits(x, wT)
    x64, w64 = x.astype(np.float64), wT.astype(np.float64)
    for t in range(T):
        for e in range(E):
            exact = math.fsum(float(x64[t, k] * w64[k, e]) for k in range(H))
            bound = H * 2.0 ** -24 * sum(abs(x64[t, k] * w64[k, e]) for k in range(H))
            assert abs(float(lg[t, e]) - exact) <= bound


def test_logits_exact_when_every_partial_sum_is_exact():
    r = np.random.default_rng(0)
    x = r.integers(-8, 8, (3, 64)).astype(np.float32)
    wT = (r.integers(-16, 16, (64, 5)) * 0.25).astype(np.float32)
    lg = R.router_logits(x, wT)
    assert np.array_equal(lg, (x.astype(np.float64) @ wT.astype(np.float64)).astype(np.float32))


def test_chain_uses_fused_multiply_add_in_ascending_order():
    """x = [-1, 1+2^-12], w = [1, 1+2^-12]: the exact dot product is
    2^-11 + 2^-24. The ascending fma chain keeps it; a separate multiply and
    add, or the descending order, rounds 1 + 2^-11 + 2^-24 first and
    returns 2^-11."""
    a = 1.0 + 2.0 ** -12
    x = np.array([[-1.0, a]], dtype=np.float32)
    wT = np.array([[1.0], [a]], dtype=np.float32)
    lg = R.router_logits(x, wT)
    assert float(lg[0, 0]) == 2.0 ** -11 + 2.0 ** -24
    lg_rev = R.router_logits(x[:, ::-1], wT[::-1])
    assert float(lg_rev[0, 0]) == 2.0 ** -11


def _boundary_case(H, k_one, k_minus, k_tiny):
    """x w = 1 at k_one, -1 at k_minus, 2^-30 at k_tiny (in that order): a
    chain holding all three returns 2^-30; one whose -1 and 2^-30 start a
    fresh chain after the 1 returns 0 (-1 + 2^-30 rounds to -1)."""
    x = np.zeros((1, H), dtype=np.float32)
    wT = np.zeros((H, 1), dtype=np.float32)
    x[0, [k_one, k_minus, k_tiny]] = [1.0, -1.0, 1.0]
    wT[[k_one, k_minus, k_tiny], 0] = [1.0, 1.0, 2.0 ** -30]
    return float(R.router_logits(x, wT)[0, 0])


def test_chain_restarts_at_every_512_input_block():
    """Blocks of exactly 512: a fresh chain starts at input 512 (the 1 at
    511 and the -1 at 512 fall in different blocks) but not at 256."""
    assert _boundary_case(1024, 511, 512, 513) == 0.0
    assert _boundary_case(1024, 255, 256, 257) == 2.0 ** -30
    assert _boundary_case(1024, 0, 300, 301) == 2.0 ** -30
    # a short last block (H = 576): its chain also starts fresh
    assert _boundary_case(576, 100, 512, 575) == 0.0


def test_block_sums_added_in_ascending_order():
    """Block sums 1, 2^-24, 2^-24: ((1 + 2^-24) + 2^-24) rounds to 1 twice
    (ties to even); the other grouping would give 1 + 2^-23."""
    H = 1536
    x = np.zeros((1, H), dtype=np.float32)
    wT = np.zeros((H, 1), dtype=np.float32)
    x[0, [0, 512, 1024]] = 1.0
    wT[[0, 512, 1024], 0] = [1.0, 2.0 ** -24, 2.0 ** -24]
    assert float(R.router_logits(x, wT)[0, 0]) == 1.0


def test_bias_added_after_the_chain_in_float32():
    x = np.ones((1, 4), dtype=np.float32)
    wT = np.full((4, 2), 0.25, dtype=np.float32)
    b = np.array([2.0 ** -30, -1.0], dtype=np.float32)
    lg = R.router_logits(x, wT, b)
    assert lg[0, 0] == np.float32(1.0) + np.float32(2.0 ** -30) == 1.0
    assert lg[0, 1] == 0.0


def _textbook_topk(key, K):
    return sorted(range(len(key)), key=lambda e: (-key[e], e))[:K]


def test_topk_matches_textbook_sort():
    r = np.random.default_rng(1)
    lg = r.standard_normal((50, 352)).astype(np.float32)
    lg[:, 100] = lg[:, 7]          # exact duplicates: lower index first
    ids = R.topk_ids(lg, 8)
    for t in range(50):
        assert list(ids[t]) == _textbook_topk([float(v) for v in lg[t]], 8)


def test_topk_ties_and_signed_zero():
    lg = np.zeros((3, 16), dtype=np.float32)
    lg[1, :8] = -0.0
    lg[1, 8:] = 0.0
    lg[2, 3] = 1.0
    lg[2, 9] = 1.0
    ids = R.topk_ids(lg, 4)
    assert list(ids[0]) == [0, 1, 2, 3]
    assert list(ids[1]) == [0, 1, 2, 3]          # -0 ranks equal to +0
    assert list(ids[2]) == [3, 9, 0, 1]


def test_topk_full_sort_when_k_equals_e():
    r = np.random.default_rng(2)
    lg = r.standard_normal((4, 16)).astype(np.float32)
    ids = R.topk_ids(lg, 16)
    for t in range(4):
        assert list(ids[t]) == list(np.argsort(-lg[t].astype(np.float64), kind="stable"))


def test_weights_sigmoid_and_renormalised():
    lg = np.array([[0.0, 1.0, -2.0, 3.0]], dtype=np.float32)
    ids = np.array([[3, 1]])
    w = R.routing_weights(lg, ids, renormalize=False)
    assert w[0, 0] == pytest.approx(1 / (1 + math.exp(-3.0)), rel=1e-15)
    assert w[0, 1] == pytest.approx(1 / (1 + math.exp(-1.0)), rel=1e-15)
    wn = R.routing_weights(lg, ids)
    assert wn.sum() == pytest.approx(1.0, abs=1e-15)
    assert wn[0, 0] / wn[0, 1] == pytest.approx(w[0, 0] / w[0, 1], rel=1e-14)


def test_route_given_logits_plus_bias():
    r = np.random.default_rng(3)
    lg = r.standard_normal((5, 32)).astype(np.float32)
    b = synth.zipf_bias(32, 5)
    used, ids, w = R.route(logits=lg, bias=b, K=4)
    assert np.array_equal(used, lg + b)
    assert np.allclose(w.sum(1), 1.0)
