"""Pins of the oracle permutation and layer: brute force on tiny inputs,
reductions to a dense SwiGLU, and invariants."""
import math

import numpy as np

from oracle import layer as L
from oracle import permute as P
from oracle import router as R
from quantized_moe_sigmoid_amd import synth


# ---------------------------------------------------------- permutation ---
def _brute_permute(ids, E, tile_m):
    flat = [int(v) for v in np.asarray(ids).ravel()]
    segs = {e: [s for s, v in enumerate(flat) if v == e] for e in range(E)}
    rows, s2r, tiles = [], {}, []
    for e in range(E):
        if not segs[e]:
            continue
        start = len(rows)
        for s in segs[e]:
            s2r[s] = len(rows)
            rows.append(s)
        while (len(rows) - start) % tile_m:
            rows.append(-1)
        tiles += [e] * ((len(rows) - start) // tile_m)
    return rows, [s2r[s] for s in range(len(flat))], tiles


def test_permute_matches_brute_force():
    r = np.random.default_rng(0)
    for (T, K, E, tm) in ((8, 2, 16, 4), (5, 3, 7, 1), (33, 8, 40, 16), (1, 8, 352, 64)):
        ids = np.stack([r.choice(E, K, replace=False) for _ in range(T)])
        p = P.permute(ids, E, tm)
        rows, s2r, tiles = _brute_permute(ids, E, tm)
        assert list(p["sorted_slots"]) == rows
        assert list(p["slot_to_row"]) == s2r
        assert list(p["tile_expert"]) == tiles
        assert p["num_tiles"] == len(tiles)
        assert p["expert_offsets"][-1] == T * K
        assert p["padded_offsets"][-1] <= P.max_rows(T, K, E, tm)
        counts = np.bincount(ids.ravel(), minlength=E)
        assert list(p["active_experts"]) == [e for e in range(E) if counts[e]]


def test_permute_skewed_single_expert():
    ids = np.zeros((10, 1), dtype=np.int32)
    p = P.permute(ids, 4, 4)
    assert list(p["sorted_slots"]) == list(range(10)) + [-1, -1]
    assert list(p["tile_expert"]) == [0, 0, 0]


# ---------------------------------------------------------------- layer ---
def _brute_ffn(x, Wg, Wu, Wd):
    F, H = Wg.shape
    h = []
    for n in range(F):
        g = sum(Wg[n, k] * x[k] for k in range(H))
        u = sum(Wu[n, k] * x[k] for k in range(H))
        h.append(g / (1.0 + math.exp(-g)) * u)
    return np.array([sum(Wd[m, n] * h[n] for n in range(F)) for m in range(H)])


def _rand_experts(E, F, H, seed):
    r = np.random.default_rng(seed)
    return [(r.standard_normal((F, H)) * 0.3, r.standard_normal((F, H)) * 0.3,
             r.standard_normal((H, F)) * 0.3) for _ in range(E)]


def test_layer_matches_brute_force_on_tiny_shapes():
    T, H, F, E, K = 3, 6, 5, 4, 2
    r = np.random.default_rng(1)
    x = r.standard_normal((T, H))
    ex = _rand_experts(E, F, H, 2)
    ids = np.array([[1, 3], [0, 1], [2, 0]])
    w = np.array([[0.7, 0.3], [0.25, 0.75], [0.5, 0.5]])
    out = L.moe_layer(x, ids, w, lambda e: ex[e])
    for t in range(T):
        want = sum(w[t, k] * _brute_ffn(x[t], *ex[ids[t, k]]) for k in range(K))
        assert np.allclose(out[t], want, rtol=1e-12, atol=1e-12)


def test_identical_experts_reduce_to_dense_swiglu():
    """With every expert equal and the weights renormalised to one, the
    layer is one dense SwiGLU, whatever the routing."""
    T, H, F, E, K = 7, 16, 12, 9, 3
    r = np.random.default_rng(3)
    x = r.standard_normal((T, H))
    Wg, Wu, Wd = _rand_experts(1, F, H, 4)[0]
    lg = r.standard_normal((T, E)).astype(np.float32)
    _, ids, w = R.route(logits=lg, K=K)
    out = L.moe_layer(x, ids, w, lambda e: (Wg, Wu, Wd))
    g = x @ Wg.T
    dense = ((g * (1 / (1 + np.exp(-g)))) * (x @ Wu.T)) @ Wd.T
    assert np.allclose(out, dense, rtol=1e-12, atol=1e-12)


def test_single_expert_single_choice_is_one_ffn():
    H, F = 8, 4
    r = np.random.default_rng(5)
    x = r.standard_normal((2, H))
    ex = _rand_experts(1, F, H, 6)
    out = L.moe_layer(x, np.zeros((2, 1), int), np.ones((2, 1)), lambda e: ex[0])
    for t in range(2):
        assert np.allclose(out[t], _brute_ffn(x[t], *ex[0]), rtol=1e-12)


def test_zero_input_and_zero_experts_give_residual():
    T, H, F, E = 4, 8, 4, 3
    ex = _rand_experts(E, F, H, 7)
    ids = np.array([[0, 1]] * T)
    w = np.full((T, 2), 0.5)
    res = np.random.default_rng(8).standard_normal((T, H))
    out = L.moe_layer(np.zeros((T, H)), ids, w, lambda e: ex[e], residual=res)
    assert np.array_equal(out, res)
    z = (np.zeros((F, H)), np.zeros((F, H)), np.zeros((H, F)))
    x = np.random.default_rng(9).standard_normal((T, H))
    out = L.moe_layer(x, ids, w, lambda e: z, residual=res)
    assert np.array_equal(out, res)


def test_shared_expert_is_added_unweighted():
    T, H, F = 3, 6, 4
    r = np.random.default_rng(10)
    x = r.standard_normal((T, H))
    ex = _rand_experts(2, F, H, 11)
    sh = _rand_experts(1, F, H, 12)[0]
    ids = np.array([[0], [1], [0]])
    w = np.ones((T, 1))
    a = L.moe_layer(x, ids, w, lambda e: ex[e], shared_weights=sh)
    b = L.moe_layer(x, ids, w, lambda e: ex[e])
    for t in range(T):
        assert np.allclose(a[t] - b[t], _brute_ffn(x[t], *sh), rtol=1e-10, atol=1e-12)
