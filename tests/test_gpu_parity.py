"""GPU parity of every step of the layer against the CPU oracle, through the
C ABI: dequant and routing bit for bit, permutation bit for bit, layer
outputs within |gpu - oracle| <= 1e-2 (|oracle| + rms(oracle))."""
import numpy as np
import pytest
import torch

from oracle import formats as OF
from oracle import layer as OL
from oracle import norm as ON
from oracle import permute as OP
from oracle import quant as OQ
from oracle import router as OR
from quantized_moe_sigmoid_amd import binding as B
from quantized_moe_sigmoid_amd import synth
from tests import fixtures as FX

pytestmark = pytest.mark.gpu

H, F, E, K = 4096, 1536, 352, 8


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    return torch.device("cuda:0")


def _bits_equal(a, b):
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    return a.shape == b.shape and np.array_equal(a.view(np.uint32), b.view(np.uint32))


# ------------------------------------------------------------------ dequant ---
def test_dequant_int4_bitwise_tiny(dev):
    cfg = synth.CONFIGS["tiny"]
    for which, (n, k) in (("gate", (cfg["F"], cfg["H"])), ("down", (cfg["H"], cfg["F"]))):
        q, s = FX.int4_bank_oracle(cfg["E"], n, k, 0, 0, which)
        qt, st = FX.int4_to_device(q, s, dev)
        d = B.bank_int4(qt, st)
        for e in range(cfg["E"]):
            got = B.moe_dequant(d, e, device=dev).cpu().numpy()
            assert _bits_equal(got, FX.oracle_int4_expert(q, s, e)), (which, e)


def test_dequant_int4_bitwise_full_shape_sampled(dev):
    qt, st = synth.packed_int4_random(E, F, H, 11, dev)
    d = B.bank_int4(qt, st)
    for e in (0, 177, 351):
        got = B.moe_dequant(d, e, device=dev).cpu().numpy()
        q = qt[e].cpu().numpy()
        sb = st[e].view(torch.int16).cpu().numpy().view(np.uint16)
        assert _bits_equal(got, OQ.dequant_int4(q, sb)), e


def test_dequant_nvfp4_bitwise(dev):
    q, s, gs = FX.nvfp4_bank_oracle(3, 64, 512, 4, 0, "up")
    d = B.bank_nvfp4(torch.from_numpy(q).to(dev), torch.from_numpy(s).to(dev),
                     torch.from_numpy(gs).to(dev))
    for e in range(3):
        got = B.moe_dequant(d, e, device=dev).cpu().numpy()
        want = OQ.dequant_nvfp4_fp32(q[e], s[e], gs[e])
        assert _bits_equal(got, want), e
    qt, st, gt = synth.packed_nvfp4_random(E, H, F, 12, dev)
    d = B.bank_nvfp4(qt, st, gt)
    for e in (5, 300):
        got = B.moe_dequant(d, e, device=dev).cpu().numpy()
        want = OQ.dequant_nvfp4_fp32(qt[e].cpu().numpy(), st[e].cpu().numpy(),
                                     float(gt[e].cpu()))
        assert _bits_equal(got, want), e


# ------------------------------------------------------------------ routing ---
def _check_route(ids, w, lg_used, K):
    want_ids = OR.topk_ids(lg_used, K)
    assert np.array_equal(ids.cpu().numpy(), want_ids)
    want_w = OR.routing_weights(lg_used, want_ids)
    np.testing.assert_allclose(w.cpu().numpy(), want_w, rtol=1e-5, atol=0)


@pytest.mark.parametrize("T", [1, 8, 64, 256, 2048])
def test_route_given_logits(dev, T):
    lg = synth.router_logits(T, E, 2)
    ids, w = B.moe_route_topk(K, logits=torch.from_numpy(lg).to(dev))
    _check_route(ids, w, lg, K)
    b = synth.zipf_bias(E, 2)
    ids, w = B.moe_route_topk(K, logits=torch.from_numpy(lg).to(dev),
                              bias=torch.from_numpy(b).to(dev))
    _check_route(ids, w, (lg + b).astype(np.float32), K)


def test_route_adversarial_ties(dev):
    T = 6
    lg = np.zeros((T, E), dtype=np.float32)
    lg[1, :] = -0.0
    lg[1, 100:] = 0.0
    lg[2, [5, 70, 300, 7]] = 1.5                 # four-way tie inside the top-8
    lg[3, :] = np.repeat(np.arange(44, dtype=np.float32), 8)   # ties across the K boundary
    lg[4, 351] = 3.0
    lg[5, :] = -50.0                             # all equal and tiny sigmoid
    ids, w = B.moe_route_topk(K, logits=torch.from_numpy(lg).to(dev))
    _check_route(ids, w, lg, K)
    ids, w = B.moe_route_topk(3, logits=torch.from_numpy(lg).to(dev), renormalize=False)
    got = ids.cpu().numpy()
    assert np.array_equal(got, OR.topk_ids(lg, 3))
    np.testing.assert_allclose(w.cpu().numpy(), OR.routing_weights(lg, got, False), rtol=1e-5)


@pytest.mark.parametrize("act", ["f16", "bf16"])
def test_route_from_router_weight_tiny(dev, act):
    cfg = synth.CONFIGS["tiny"]
    x = synth.activations(8, cfg["H"], act, 0)
    wT = synth.router_weight_T(cfg["H"], cfg["E"], 0)
    lg = OR.router_logits(x.float().numpy(), wT)
    ids, w = B.moe_route_topk(cfg["K"], x=x.to(dev), router_wT=torch.from_numpy(wT).to(dev))
    _check_route(ids, w, lg, cfg["K"])


@pytest.mark.parametrize("T,Hh,Ee,act", [(37, 4096, 352, "bf16"), (2048, 4096, 352, "bf16"),
                                         (4099, 4096, 352, "bf16"), (200, 4096, 352, "bf16"),
                                         (9, 576, 20, "bf16"),
                                         (3, 64, 8, "bf16"), (600, 320, 24, "bf16"),
                                         (8, 256, 16, "f16"), (70, 192, 20, "f16")])
def test_router_logits_bitwise(dev, T, Hh, Ee, act):
    """The canonical float32 block sum, bit for bit against the C oracle
    (partial token and expert tiles included; bf16 inputs whose 64-input
    chunk count is below or not a multiple of the weight prefetch depth)."""
    x = synth.activations(T, Hh, act, 5)
    wT = synth.router_weight_T(Hh, Ee, 5)
    b = synth.zipf_bias(Ee, 5)
    for bias in (None, b):
        got = B.moe_router_logits(x.to(dev), torch.from_numpy(wT).to(dev),
                                  None if bias is None else torch.from_numpy(bias).to(dev))
        want = OR.router_logits(x.float().numpy(), wT, bias)
        assert _bits_equal(got.cpu().numpy(), want)


@pytest.mark.parametrize("T", [3, 200])
def test_router_block_order_every_path(dev, T):
    """Inputs whose logit depends on where the canonical sum starts a fresh
    chain: x w = 1 at input 511, -1 at 512 and 2^-30 at 513 give 2^-30 in
    one 1024-step chain but 0 in the two 512-input blocks (-1 + 2^-30
    rounds to -1), against a lone 2^-31 for expert 1. Every router path
    returns the blocks' answer, so expert 1 is the top-1: the bf16 rows
    kernel (T = 3: logits in turn, block sums side by side for the top-K),
    the tiled kernel (T = 200: logits in turn, one block per work group for
    the top-K), the f16 kernel, and the fused norm (the
    +-1 rows normalise to +-16 exactly with eps = 0)."""
    Hh, Ee = 1024, 8
    xv = np.zeros((T, Hh), np.float32)
    xv[:, [511, 512, 513, 700]] = [1.0, -1.0, 1.0, 1.0]
    wT = np.zeros((Hh, Ee), np.float32)
    wT[[511, 512, 513], 0] = [1.0, 1.0, 2.0 ** -30]
    wT[700, 1] = 2.0 ** -31
    want = OR.router_logits(xv, wT)
    assert want[0, 0] == 0.0 and want[0, 1] == 2.0 ** -31
    wd = torch.from_numpy(wT).to(dev)
    for dt in (torch.bfloat16, torch.float16):
        x = torch.from_numpy(xv).to(dt).to(dev)
        got = B.moe_router_logits(x, wd)
        assert _bits_equal(got.cpu().numpy(), want)
        ids, w = B.moe_route_topk(1, x=x, router_wT=wd)
        assert (ids.cpu().numpy() == 1).all()
    a, ids, w = B.moe_norm_route(torch.from_numpy(xv).to(dev), wd, 1, eps=0.0)
    assert (a.float().cpu().numpy()[:, [511, 512, 513, 700]] == [16.0, -16.0, 16.0, 16.0]).all()
    assert (ids.cpu().numpy() == 1).all()


@pytest.mark.parametrize("T,Hh,Ee,Kk", [(5, 576, 20, 3), (70, 576, 24, 4), (3, 1088, 352, 8),
                                         (300, 1088, 352, 8), (600, 576, 40, 8)])
def test_block_sum_routing_short_last_block(dev, T, Hh, Ee, Kk):
    """The block-sum paths with a last block shorter than 512 inputs (H = 576:
    512 + 64; H = 1088: 2 x 512 + 64): moe_route_topk from a bf16 router
    input and moe_norm_route (fused) give the oracle's ids bit for bit and
    its weights within 1e-5; T = 70 runs two tokens per wave; T = 300 takes
    the tiled kernel's block sums with 4 tokens per wave (and the unfused
    norm), T = 600 with 8 and a last 32-token tile of 24."""
    x = synth.activations(T, Hh, "bf16", 60 + T)
    wT = synth.router_weight_T(Hh, Ee, 60 + T)
    b = synth.zipf_bias(Ee, 60 + T)
    lg = OR.router_logits(x.float().numpy(), wT, b)
    ids, w = B.moe_route_topk(Kk, x=x.to(dev), router_wT=torch.from_numpy(wT).to(dev),
                              bias=torch.from_numpy(b).to(dev))
    oids = OR.topk_ids(lg, Kk)
    assert np.array_equal(ids.cpu().numpy(), oids)
    np.testing.assert_allclose(w.cpu().numpy(), OR.routing_weights(lg, oids), rtol=1e-5, atol=0)
    r = synth.normal((T, Hh), 1.0, 61, 0, synth.T_X, T)
    a, ids2, w2 = B.moe_norm_route(torch.from_numpy(r).to(dev), torch.from_numpy(wT).to(dev), Kk,
                                   eps=1e-5, bias=torch.from_numpy(b).to(dev))
    oa = OF.round_to_format(ON.rmsnorm(r, None, 1e-5), OF.BF16)
    assert np.array_equal(a.view(torch.int16).cpu().numpy().view(np.uint16), OF.bf16_bits(oa))
    lg2 = OR.router_logits(oa.astype(np.float32), wT, b)
    oids2 = OR.topk_ids(lg2, Kk)
    assert np.array_equal(ids2.cpu().numpy(), oids2)
    np.testing.assert_allclose(w2.cpu().numpy(), OR.routing_weights(lg2, oids2), rtol=1e-5,
                               atol=0)


@pytest.mark.parametrize("T,zipf", [(37, False), (2048, False), (300, True)])
def test_route_from_router_weight_full(dev, T, zipf):
    x = synth.activations(T, H, "bf16", 3)
    wT = synth.router_weight_T(H, E, 3)
    b = synth.zipf_bias(E, 3) if zipf else None
    lg = OR.router_logits(x.float().numpy(), wT, b)
    ids, w = B.moe_route_topk(K, x=x.to(dev), router_wT=torch.from_numpy(wT).to(dev),
                              bias=None if b is None else torch.from_numpy(b).to(dev))
    _check_route(ids, w, lg, K)


@pytest.mark.parametrize("T,Kk,Ee,src", [(1, 8, 352, "logits"), (5, 8, 352, "bias"),
                                         (16, 8, 352, "logits"), (17, 8, 352, "bias"),
                                         (64, 8, 352, "logits"), (16, 16, 512, "bias"),
                                         (3, 2, 16, "logits"), (3, 8, 352, "weight"),
                                         (32, 8, 352, "weight"), (2, 4, 64, "weight_f16")])
def test_route_permute_matches_separate_calls(dev, T, Kk, Ee, src):
    """moe_route_permute (one kernel up to 16 tokens, the two calls' kernels
    beyond) is bitwise moe_route_topk followed by moe_permute: ids, weights
    and every permutation array; given logits with or without a bias, and
    a router weight (bf16 block sums, f16 logits)."""
    tm = 8 if 5 <= T <= 32 else 4
    kw = {}
    if src in ("logits", "bias"):
        kw["logits"] = torch.from_numpy(synth.router_logits(T, Ee, 40 + T)).to(dev)
        if src == "bias":
            kw["bias"] = torch.from_numpy(synth.zipf_bias(Ee, 40 + T)).to(dev)
    else:
        Hh = 1024
        act = "f16" if src == "weight_f16" else "bf16"
        kw["x"] = synth.activations(T, Hh, act, 40 + T).to(dev)
        kw["router_wT"] = torch.from_numpy(synth.router_weight_T(Hh, Ee, 40 + T)).to(dev)
    perm = B.Perm(T, Kk, Ee, tm, dev)
    ids, w = B.moe_route_permute(Kk, perm, **kw)
    ids2, w2 = B.moe_route_topk(Kk, **kw)
    perm2 = B.moe_permute(ids2, Ee, tm)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2)
    assert torch.equal(w.view(torch.int32), w2.view(torch.int32))
    n_rows = int(perm2.padded_offsets[Ee])
    n_tiles = int(perm2.num_tiles[0])
    n_act = int(perm2.num_active[0])
    for f, m in (("counts", None), ("expert_offsets", None), ("padded_offsets", None),
                 ("slot_to_row", None), ("num_tiles", None), ("num_active", None),
                 ("sorted_slots", n_rows), ("tile_expert", n_tiles), ("active_experts", n_act)):
        a, b = getattr(perm, f), getattr(perm2, f)
        if m is not None:
            a, b = a[:m], b[:m]
        assert torch.equal(a, b), f


# -------------------------------------------------------------- permutation ---
@pytest.mark.parametrize("T,Kk,Ee,tm,skew", [(1, 8, 352, 4, False), (64, 8, 352, 4, False),
                                             (2048, 8, 352, 64, False), (2048, 8, 352, 64, True),
                                             (4096, 8, 352, 128, True), (8, 2, 16, 4, False),
                                             (3, 3, 5, 1, False), (0, 8, 352, 4, False),
                                             (128, 8, 352, 4, True), (129, 8, 352, 4, False),
                                             (128, 8, 512, 4, True), (5, 16, 512, 16, False),
                                             (1000, 3, 352, 16, True), (700, 8, 512, 32, False)])
def test_permute_bitwise(dev, T, Kk, Ee, tm, skew):
    """Batches of up to 1024 slots take the one-work-group kernel, larger
    ones the one-work-group-per-expert form (ragged last passes included);
    both must match the oracle bit for bit."""
    r = np.random.default_rng(T * 7 + Kk)
    if skew:
        p = 1.0 / np.arange(1, Ee + 1) ** 1.1
        p = p / p.sum()
        ids = np.stack([r.choice(Ee, Kk, replace=False, p=p) for _ in range(T)]) if T else \
            np.zeros((0, Kk), dtype=np.int64)
    else:
        ids = np.stack([r.choice(Ee, Kk, replace=False) for _ in range(T)]) if T else \
            np.zeros((0, Kk), dtype=np.int64)
    ids = ids.astype(np.int32)
    perm = B.moe_permute(torch.from_numpy(ids).reshape(T, Kk).to(dev), Ee, tm)
    torch.cuda.synchronize()
    want = OP.permute(ids.reshape(T, Kk), Ee, tm)
    tot = int(want["padded_offsets"][-1])
    assert np.array_equal(perm.counts.cpu().numpy(), want["counts"])
    assert np.array_equal(perm.expert_offsets.cpu().numpy(), want["expert_offsets"])
    assert np.array_equal(perm.padded_offsets.cpu().numpy(), want["padded_offsets"])
    assert np.array_equal(perm.sorted_slots.cpu().numpy()[:tot], want["sorted_slots"])
    if T:
        assert np.array_equal(perm.slot_to_row.cpu().numpy(), want["slot_to_row"])
    assert int(perm.num_tiles.cpu()[0]) == want["num_tiles"]
    assert np.array_equal(perm.tile_expert.cpu().numpy()[:want["num_tiles"]], want["tile_expert"])
    na = want["num_active"]
    assert int(perm.num_active.cpu()[0]) == na
    assert np.array_equal(perm.active_experts.cpu().numpy()[:na], want["active_experts"])


@pytest.mark.parametrize("T,Kk,Ee,tm", [(40, 8, 16, 4), (300, 8, 16, 8), (1100, 4, 352, 64)])
def test_permute_repeated_and_foreign_ids(dev, T, Kk, Ee, tm):
    """Ids need not be distinct within a token, and ids outside [0, E) are
    routed nowhere; slots keep their order inside an expert either way."""
    r = np.random.default_rng(T + 11)
    ids = r.integers(-2, Ee + 2, (T, Kk)).astype(np.int32)
    perm = B.moe_permute(torch.from_numpy(ids).to(dev), Ee, tm)
    torch.cuda.synchronize()
    ok = (ids >= 0) & (ids < Ee)
    # the oracle with the foreign slots sent to an extra, last expert: the
    # first Ee experts' rows are then exactly the expected ones
    want = OP.permute(np.where(ok, ids, Ee), Ee + 1, tm)
    tot = int(want["padded_offsets"][Ee])
    assert np.array_equal(perm.counts.cpu().numpy(), want["counts"][:Ee])
    assert np.array_equal(perm.padded_offsets.cpu().numpy(), want["padded_offsets"][:Ee + 1])
    assert np.array_equal(perm.sorted_slots.cpu().numpy()[:tot], want["sorted_slots"][:tot])
    assert int(perm.num_tiles.cpu()[0]) == tot // tm
    s2r = perm.slot_to_row.cpu().numpy()
    assert np.array_equal(s2r[ok.ravel()], want["slot_to_row"][ok.ravel()])


# ------------------------------------------------------------------ forward ---
def _int4_ffn_from_oracle(E_, H_, F_, root, dev):
    banks, host = [], []
    for which, (n, k) in (("gate", (F_, H_)), ("up", (F_, H_)), ("down", (H_, F_))):
        q, s = FX.int4_bank_oracle(E_, n, k, root, 0, which)
        qt, st = FX.int4_to_device(q, s, dev)
        banks.append(B.bank_int4(qt, st))
        host.append((q, s))
    return B.ffn(*banks), host


_int4_ffn_random = FX.int4_ffn_random
_experts_fn_int4 = FX.experts_fn_int4


def _run_layer(dev, ffn, x, ids, w, Ee, residual=None, out_dtype=torch.float32):
    tm, _ = B.moe_forward_plan(ffn, x.shape[0], ids.shape[1], x.dtype)
    perm = B.moe_permute(ids, Ee, tm)
    return B.moe_w4a16_forward(ffn, x, w, perm, residual=residual, out_dtype=out_dtype)


def test_forward_tiny_end_to_end(dev):
    """The tiny layer: router from weights, clip-search int4 experts."""
    cfg = synth.CONFIGS["tiny"]
    T, Hh, Ee, Kk, Ff = 8, cfg["H"], cfg["E"], cfg["K"], cfg["F"]
    ffn, host = _int4_ffn_from_oracle(Ee, Hh, Ff, 0, dev)
    x = synth.activations(T, Hh, "f16", 0)
    wT = synth.router_weight_T(Hh, Ee, 0)
    ids, w = B.moe_route_topk(Kk, x=x.to(dev), router_wT=torch.from_numpy(wT).to(dev))
    out = _run_layer(dev, ffn, x.to(dev), ids, w, Ee).cpu().numpy()
    lg, oids, ow = OR.route(x=x.float().numpy(), wT=wT, K=Kk)
    assert np.array_equal(ids.cpu().numpy(), oids)
    ref = FX.oracle_layer(x, oids, ow, _experts_fn_int4(host))
    ok, ratio = FX.within_tolerance(out, ref)
    assert ok, ratio


def _host_int4(host):
    return [FX.host_bank(q, s) for (q, s) in host]


@pytest.mark.parametrize("T", [1, 8, 64])
def test_forward_decode_full_shape(dev, T):
    """Decode shape: 352 int4 experts, hidden 4096, width 1536, fp16 x,
    given logits. Every token against the oracle (streamed per expert)."""
    ffn, host = _int4_ffn_random(E, H, F, 100 + T, dev)
    x = synth.activations(T, H, "f16", 2)
    lg = synth.router_logits(T, E, 2)
    ids, w = B.moe_route_topk(K, logits=torch.from_numpy(lg).to(dev))
    out = _run_layer(dev, ffn, x.to(dev), ids, w, E).cpu().numpy()
    oids = OR.topk_ids(lg, K)
    assert np.array_equal(ids.cpu().numpy(), oids)
    ow = OR.routing_weights(lg, oids)
    ref = FX.oracle_layer_streamed(x, oids, ow, FX.dequant_fn(_host_int4(host)))
    ok, ratio = FX.within_tolerance(out, ref)
    assert ok, ratio


@pytest.mark.parametrize("T", [8, 256])
def test_forward_profiled_matches_plain(dev, T):
    """The profiled entry point runs the same kernels: bitwise the same output
    as the plain forward, with every boundary recorded and with only the
    gate/up boundaries (NULL entries elsewhere); the recorded stages have
    positive durations. T = 8 runs the decode kernels, T = 256 the GEMMs."""
    ffn, _ = _int4_ffn_random(E, H, F, 300 + T, dev)
    x = synth.activations(T, H, "bf16", 4).to(dev)
    lg = synth.router_logits(T, E, 4)
    ids, w = B.moe_route_topk(K, logits=torch.from_numpy(lg).to(dev))
    tm, _ = B.moe_forward_plan(ffn, T, K, x.dtype)
    perm = B.moe_permute(ids, E, tm)
    plain = B.moe_w4a16_forward(ffn, x, w, perm).cpu().numpy()
    hip = FX.HipEvents()
    n = B.MOE_FORWARD_STAGES + 1
    full = [hip.create() for _ in range(n)]
    gu = [hip.create(), hip.create()]
    try:
        a = B.moe_w4a16_forward(ffn, x, w, perm, events=full).cpu().numpy()
        b = B.moe_w4a16_forward(ffn, x, w, perm, events=gu + [None] * (n - 2)).cpu().numpy()
        torch.cuda.synchronize()
        assert _bits_equal(a, plain) and _bits_equal(b, plain)
        assert hip.elapsed_ms(full[0], full[1]) > 0 and hip.elapsed_ms(full[1], full[2]) > 0
        assert hip.elapsed_ms(gu[0], gu[1]) > 0
    finally:
        for e in full + gu:
            hip.destroy(e)


def test_forward_nvfp4_small(dev):
    Ee, Hh, Ff, T, Kk = 6, 512, 256, 5, 3
    banks, host = [], []
    for which, (n, k) in (("gate", (Ff, Hh)), ("up", (Ff, Hh)), ("down", (Hh, Ff))):
        q, s, gs = FX.nvfp4_bank_oracle(Ee, n, k, 4, 0, which)
        banks.append(B.bank_nvfp4(torch.from_numpy(q).to(dev), torch.from_numpy(s).to(dev),
                                  torch.from_numpy(gs).to(dev)))
        host.append((q, s, gs))
    ffn = B.ffn(*banks)
    x = synth.activations(T, Hh, "bf16", 4)
    lg = synth.router_logits(T, Ee, 4)
    ids, w = B.moe_route_topk(Kk, logits=torch.from_numpy(lg).to(dev))
    out = _run_layer(dev, ffn, x.to(dev), ids, w, Ee).cpu().numpy()
    oids = OR.topk_ids(lg, Kk)
    ow = OR.routing_weights(lg, oids)

    def efn(e):
        return tuple(FX.oracle_nvfp4_expert(q, s, gs, e) for (q, s, gs) in host)
    ref = FX.oracle_layer(x, oids, ow, efn)
    ok, ratio = FX.within_tolerance(out, ref)
    assert ok, ratio


def test_forward_nvfp4_decode_full_shape(dev):
    T = 1
    banks, host = [], []
    for i, (n, k) in enumerate(((F, H), (F, H), (H, F))):
        qt, st, gt = synth.packed_nvfp4_random(E, n, k, 40 + i, dev)
        banks.append(B.bank_nvfp4(qt, st, gt))
        host.append((qt, st, gt))
    ffn = B.ffn(*banks)
    x = synth.activations(T, H, "bf16", 4)
    lg = synth.router_logits(T, E, 4)
    ids, w = B.moe_route_topk(K, logits=torch.from_numpy(lg).to(dev))
    out = _run_layer(dev, ffn, x.to(dev), ids, w, E).cpu().numpy()
    oids = OR.topk_ids(lg, K)
    ow = OR.routing_weights(lg, oids)

    def efn(e):
        return tuple(OQ.dequant_nvfp4(q[e].cpu().numpy(), s[e].cpu().numpy(), float(g[e].cpu()))
                     for (q, s, g) in host)
    ref = FX.oracle_layer(x, oids, ow, efn)
    ok, ratio = FX.within_tolerance(out, ref)
    assert ok, ratio


_NV_DECODE = {}


def _nvfp4_decode_banks(dev):
    """One full-shape NVFP4 bank set for the decode-range tests (built once)."""
    if "ffn" not in _NV_DECODE:
        banks, host = [], []
        for i, (n, k) in enumerate(((F, H), (F, H), (H, F))):
            qt, st, gt = synth.packed_nvfp4_random(E, n, k, 90 + i, dev)
            banks.append(B.bank_nvfp4(qt, st, gt))
            host.append(FX.host_bank(qt, st, gs=gt.cpu().numpy()))
        _NV_DECODE["ffn"], _NV_DECODE["host"] = B.ffn(*banks), host
    return _NV_DECODE["ffn"], _NV_DECODE["host"]


@pytest.mark.parametrize("T,act,shift", [
    (176, "bf16", 0), (351, "bf16", 0), (200, "f16", 0), (256, "bf16", 60),
    (256, "bf16", -60), (176, "bf16", "split"), (180, "bf16", "zero")])
def test_forward_nvfp4_band_activation_range(dev, T, act, shift):
    """NVFP4 at the layer shape for T*K in [4E, 8E), the batches the MFMA
    GEMV serves with 8-slot tiles (T = 176 and 351 its ends), against the
    oracle on tile-probing tokens (the last rows of full and partial 8-slot
    tiles, and spread tokens): fp16 and bf16 inputs, bf16 inputs far outside
    fp16's range (whole batches scaled by 2^60 or 2^-60; tokens whose halves
    differ by 2^40, where the staged fp16 values of the small half lose bits
    below the tolerance), which the per-row staging exponent has to bring
    into range, and all-zero tokens among ordinary ones (exactly zero out)."""
    ffn, hb = _nvfp4_decode_banks(dev)
    x = synth.activations(T, H, act, 11 + T).float()
    if shift == "split":
        x[:, : H // 2] *= 2.0 ** 20
        x[:, H // 2:] *= 2.0 ** -20
    elif shift == "zero":
        x[::3] = 0.0
    else:
        x *= 2.0 ** shift
    x = x.to(torch.bfloat16 if act == "bf16" else torch.float16)
    assert torch.isfinite(x.float()).all()
    lg = synth.router_logits(T, E, 11 + T)
    ids, w = B.moe_route_topk(K, logits=torch.from_numpy(lg).to(dev))
    tm, _ = B.moe_forward_plan(ffn, T, K, x.dtype)
    assert tm == 8
    out = _run_layer(dev, ffn, x.to(dev), ids, w, E).cpu().numpy()
    oids = OR.topk_ids(lg, K)
    toks = FX.tile_probe_tokens(oids, E, 8, min_tokens=48, max_tokens=64)
    if shift == "zero":
        toks = sorted(set(toks) | {0, 3, 6})
        assert not out[::3].any()
    ref = FX.oracle_layer_streamed(x[toks], oids[toks], OR.routing_weights(lg, oids)[toks],
                                   FX.dequant_fn(hb, "nvfp4"))
    assert np.isfinite(out).all()
    ok, ratio = FX.within_tolerance(out[toks], ref)
    assert ok, ratio


@pytest.mark.parametrize("T,act", [(176, "f16"), (256, "bf16"), (307, "f16")])
def test_forward_int4_band_full_shape(dev, T, act):
    """int4-g128 at the layer shape for T*K in [4E, 7E) (the MFMA GEMV with
    8-slot tiles; T = 176 and 307 the band's ends) against the oracle on
    tile-probing tokens."""
    ffn, host = _int4_ffn_random(E, H, F, 300 + T, dev)
    x = synth.activations(T, H, act, 5 + T)
    lg = synth.router_logits(T, E, 5 + T)
    ids, w = B.moe_route_topk(K, logits=torch.from_numpy(lg).to(dev))
    tm, _ = B.moe_forward_plan(ffn, T, K, x.dtype)
    assert tm == 8
    out = _run_layer(dev, ffn, x.to(dev), ids, w, E).cpu().numpy()
    oids = OR.topk_ids(lg, K)
    toks = FX.tile_probe_tokens(oids, E, 8, min_tokens=48, max_tokens=64)
    ref = FX.oracle_layer_streamed(x[toks], oids[toks], OR.routing_weights(lg, oids)[toks],
                                   FX.dequant_fn(_host_int4(host)))
    ok, ratio = FX.within_tolerance(out[toks], ref)
    assert ok, ratio


# --------------------------------------------------------------- properties ---
@pytest.mark.parametrize("T", [1, 3, 37])
def test_forward_single_expert(dev, T):
    """E = K = 1: every token goes to the one expert with weight exactly 1,
    so the layer is one SwiGLU FFN (T = 37 takes the MFMA path)."""
    Ee, Kk, Hh, Ff = 1, 1, 512, 256
    ffn, host = _int4_ffn_from_oracle(Ee, Hh, Ff, 12, dev)
    x = synth.activations(T, Hh, "bf16", 12)
    lg = synth.router_logits(T, Ee, 12)
    ids, w = B.moe_route_topk(Kk, logits=torch.from_numpy(lg).to(dev))
    assert torch.all(ids == 0) and torch.all(w == 1.0)
    out = _run_layer(dev, ffn, x.to(dev), ids, w, Ee).cpu().numpy()
    ref = OL.swiglu_ffn(x.float().numpy().astype(np.float64), *_experts_fn_int4(host)(0))
    ok, ratio = FX.within_tolerance(out, ref)
    assert ok, ratio


def test_forward_empty_batch(dev):
    """T = 0: plan, permutation and forward pass all succeed and write
    nothing."""
    Ee, Kk, Hh, Ff = 8, 2, 512, 256
    ffn, _ = _int4_ffn_from_oracle(Ee, Hh, Ff, 13, dev)
    ids = torch.empty((0, Kk), dtype=torch.int32, device=dev)
    w = torch.empty((0, Kk), dtype=torch.float32, device=dev)
    tm, _ = B.moe_forward_plan(ffn, 0, Kk, torch.bfloat16)
    perm = B.moe_permute(ids, Ee, tm)
    torch.cuda.synchronize()
    assert int(perm.num_tiles.cpu()[0]) == 0
    x = torch.empty((0, Hh), dtype=torch.bfloat16, device=dev)
    out = B.moe_w4a16_forward(ffn, x, w, perm)
    torch.cuda.synchronize()
    assert out.shape == (0, Hh)


def test_forward_properties(dev):
    """Determinism, zero input, residual pass-through, and exact doubling of
    the output when every down-projection scale doubles."""
    Ee, Hh, Ff, T, Kk = 16, 512, 256, 12, 4
    ffn, host = _int4_ffn_random(Ee, Hh, Ff, 7, dev)
    x = synth.activations(T, Hh, "bf16", 9).to(dev)
    lg = torch.from_numpy(synth.router_logits(T, Ee, 9)).to(dev)
    ids, w = B.moe_route_topk(Kk, logits=lg)
    a = _run_layer(dev, ffn, x, ids, w, Ee)
    b = _run_layer(dev, ffn, x, ids, w, Ee)
    assert torch.equal(a, b)
    z = _run_layer(dev, ffn, torch.zeros_like(x), ids, w, Ee)
    assert torch.count_nonzero(z) == 0
    res = torch.randn(T, Hh, device=dev)
    r = _run_layer(dev, ffn, torch.zeros_like(x), ids, w, Ee, residual=res)
    assert torch.equal(r, res)
    qd, sd = host[2]
    ffn2 = B.ffn(ffn.gate, ffn.up, B.bank_int4(qd, (sd.float() * 2).to(torch.bfloat16)))
    c = _run_layer(dev, ffn2, x, ids, w, Ee)
    assert torch.equal(c, 2 * a)


# ------------------------------------------------- prefill (MFMA) forward ---
def _nvfp4_ffn_from_oracle(E_, H_, F_, root, dev):
    banks, host = [], []
    for which, (n, k) in (("gate", (F_, H_)), ("up", (F_, H_)), ("down", (H_, F_))):
        q, s, gs = FX.nvfp4_bank_oracle(E_, n, k, root, 0, which)
        banks.append(B.bank_nvfp4(torch.from_numpy(q).to(dev), torch.from_numpy(s).to(dev),
                                  torch.from_numpy(gs).to(dev)))
        host.append((q, s, gs))
    return B.ffn(*banks), host


def _efn_nvfp4(host):
    cache = {}

    def fn(e):
        if e not in cache:
            mats = []
            for (q, s, g) in host:
                if isinstance(q, torch.Tensor):
                    mats.append(OQ.dequant_nvfp4(q[e].cpu().numpy(), s[e].cpu().numpy(),
                                                 float(g[e].cpu())))
                else:
                    mats.append(FX.oracle_nvfp4_expert(q, s, g, e))
            cache[e] = tuple(mats)
        return cache[e]
    return fn


@pytest.mark.parametrize("act,Ee,Kk,T", [("bf16", 8, 4, 40), ("bf16", 4, 2, 150),
                                         ("f16", 8, 4, 40), ("f16", 5, 3, 97)])
def test_forward_mfma_int4_small(dev, act, Ee, Kk, T):
    """MFMA grouped-GEMM path (T*K >= 4E) on clip-search int4 experts:
    partial tiles, one and two 32-row blocks, several tiles per expert."""
    Hh, Ff = 512, 256
    assert T * Kk >= 4 * Ee
    ffn, host = _int4_ffn_from_oracle(Ee, Hh, Ff, 6, dev)
    x = synth.activations(T, Hh, act, 6)
    lg = synth.router_logits(T, Ee, 6)
    ids, w = B.moe_route_topk(Kk, logits=torch.from_numpy(lg).to(dev))
    tm, _ = B.moe_forward_plan(ffn, T, Kk, x.dtype)
    assert tm == 64
    out = _run_layer(dev, ffn, x.to(dev), ids, w, Ee).cpu().numpy()
    oids = OR.topk_ids(lg, Kk)
    ref = FX.oracle_layer(x, oids, OR.routing_weights(lg, oids), _experts_fn_int4(host))
    ok, ratio = FX.within_tolerance(out, ref)
    assert ok, ratio


@pytest.mark.parametrize("act,shift", [("bf16", 22), ("f16", -20)])
def test_forward_mfma_y_far_outside_fp16(dev, act, shift):
    """The grouped-GEMM path hands y to the combine in fp16 with a
    power-of-two scale per (row, 32 columns): with the down projection's
    scales multiplied by 2^22 (y far above fp16's largest value) or 2^-20
    (far below its normal range) the layer still meets the tolerance."""
    Ee, Hh, Ff, T, Kk = 8, 512, 256, 40, 4
    banks, host = [], []
    for which, (n, k) in (("gate", (Ff, Hh)), ("up", (Ff, Hh)), ("down", (Hh, Ff))):
        q, sbits = FX.int4_bank_oracle(Ee, n, k, 6, 0, which)
        if which == "down":   # a power of two: add to the bf16 exponent field
            sbits = (sbits.astype(np.int32) + (shift << 7)).astype(np.uint16)
        qt, st = FX.int4_to_device(q, sbits, dev)
        banks.append(B.bank_int4(qt, st))
        host.append((q, sbits))
    ffn = B.ffn(*banks)
    x = synth.activations(T, Hh, act, 6)
    lg = synth.router_logits(T, Ee, 6)
    ids, w = B.moe_route_topk(Kk, logits=torch.from_numpy(lg).to(dev))
    tm, _ = B.moe_forward_plan(ffn, T, Kk, x.dtype)
    assert tm == 64
    out = _run_layer(dev, ffn, x.to(dev), ids, w, Ee).cpu().numpy()
    oids = OR.topk_ids(lg, Kk)
    ref = FX.oracle_layer(x, oids, OR.routing_weights(lg, oids), _experts_fn_int4(host))
    big = np.max(np.abs(ref))
    assert (big > 6.6e4) if shift > 0 else (big < 6.1e-5)
    ok, ratio = FX.within_tolerance(out, ref)
    assert ok, ratio


def test_forward_mfma_nvfp4_small(dev):
    Ee, Hh, Ff, T, Kk = 6, 512, 256, 64, 3
    ffn, host = _nvfp4_ffn_from_oracle(Ee, Hh, Ff, 8, dev)
    x = synth.activations(T, Hh, "bf16", 8)
    lg = synth.router_logits(T, Ee, 8)
    ids, w = B.moe_route_topk(Kk, logits=torch.from_numpy(lg).to(dev))
    out = _run_layer(dev, ffn, x.to(dev), ids, w, Ee).cpu().numpy()
    oids = OR.topk_ids(lg, Kk)
    ref = FX.oracle_layer(x, oids, OR.routing_weights(lg, oids), _efn_nvfp4(host))
    ok, ratio = FX.within_tolerance(out, ref)
    assert ok, ratio


@pytest.mark.parametrize("zipf", [False, True])
def test_forward_prefill_full_shape(dev, zipf):
    """Prefill shape T=2048, bf16 x, router from a N(0, 0.02) weight (plus
    Zipf expert biases when skewed), 352 int4 experts; outputs of sampled
    tokens against the oracle, routing of every token bit for bit."""
    T = 2048
    ffn, host = _int4_ffn_random(E, H, F, 300 + int(zipf), dev)
    x = synth.activations(T, H, "bf16", 3)
    wT = synth.router_weight_T(H, E, 3)
    b = synth.zipf_bias(E, 3) if zipf else None
    ids, w = B.moe_route_topk(K, x=x.to(dev), router_wT=torch.from_numpy(wT).to(dev),
                              bias=None if b is None else torch.from_numpy(b).to(dev))
    out = _run_layer(dev, ffn, x.to(dev), ids, w, E).cpu().numpy()
    lg = OR.router_logits(x.float().numpy(), wT, b)
    oids = OR.topk_ids(lg, K)
    assert np.array_equal(ids.cpu().numpy(), oids)
    # tokens on rows 0, 31, 32, 63 of full tiles and the last rows of
    # partial ones (tile_m 64), and evenly spaced ones
    toks = FX.tile_probe_tokens(oids, E, 64)
    assert len(toks) >= 64
    ow = OR.routing_weights(lg, oids)
    ref = FX.oracle_layer_streamed(x[toks], oids[toks], ow[toks],
                                   FX.dequant_fn(_host_int4(host)))
    ok, ratio = FX.within_tolerance(out[toks], ref)
    assert ok, ratio


def test_forward_nvfp4_prefill_full_shape(dev):
    T = 256
    banks, host = [], []
    for i, (n, k) in enumerate(((F, H), (F, H), (H, F))):
        qt, st, gt = synth.packed_nvfp4_random(E, n, k, 60 + i, dev)
        banks.append(B.bank_nvfp4(qt, st, gt))
        host.append((qt, st, gt))
    ffn = B.ffn(*banks)
    x = synth.activations(T, H, "bf16", 4)
    lg = synth.router_logits(T, E, 4)
    ids, w = B.moe_route_topk(K, logits=torch.from_numpy(lg).to(dev))
    out = _run_layer(dev, ffn, x.to(dev), ids, w, E).cpu().numpy()
    oids = OR.topk_ids(lg, K)
    toks = FX.tile_probe_tokens(oids, E, 64)
    assert len(toks) >= 64
    hb = [FX.host_bank(q, s, gs=g) for (q, s, g) in host]
    ref = FX.oracle_layer_streamed(x[toks], oids[toks], OR.routing_weights(lg, oids)[toks],
                                   FX.dequant_fn(hb, "nvfp4"))
    ok, ratio = FX.within_tolerance(out[toks], ref)
    assert ok, ratio


@pytest.mark.parametrize("T", [64, 256])
def test_forward_nvfp4_every_scale_byte(dev, T):
    """NVFP4 at the layer shape with block-scale bytes spanning every finite
    non-negative E4M3 value: each expert draws its bytes from its own window
    of 8 (zero and subnormal scales included) and its global scale brings
    its weights back to a common magnitude, so a mis-decoded scale byte
    shows in the outputs. T = 64 runs the decode kernels, T = 256 the
    grouped GEMM; every token (T = 64) or tile-probing tokens."""
    banks, hb = [], []
    for i, (n, k) in enumerate(((F, H), (F, H), (H, F))):
        qt, st, _ = synth.packed_nvfp4_random(E, n, k, 80 + i, dev, scale_window=8)
        mid = st.amin(dim=(1, 2)).cpu().numpy().astype(np.int64) + 4
        gs = (2.0e-5 * 320.0 / OF.E4M3_TABLE[mid]).astype(np.float32)
        gt = torch.from_numpy(gs).to(dev)
        banks.append(B.bank_nvfp4(qt, st, gt))
        hb.append(FX.host_bank(qt, st, gs=gs))
    bytes_seen = np.unique(np.concatenate([np.unique(h[1]) for h in hb]))
    assert bytes_seen.min() == 0 and bytes_seen.max() == 0x7E
    ffn = B.ffn(*banks)
    x = synth.activations(T, H, "bf16", 8)
    lg = synth.router_logits(T, E, 8)
    ids, w = B.moe_route_topk(K, logits=torch.from_numpy(lg).to(dev))
    out = _run_layer(dev, ffn, x.to(dev), ids, w, E).cpu().numpy()
    oids = OR.topk_ids(lg, K)
    toks = list(range(T)) if T <= 64 else FX.tile_probe_tokens(oids, E, 64)
    ref = FX.oracle_layer_streamed(x[toks], oids[toks], OR.routing_weights(lg, oids)[toks],
                                   FX.dequant_fn(hb, "nvfp4"))
    ok, ratio = FX.within_tolerance(out[toks], ref)
    assert ok, ratio


# -------------------------------------------- fused norm + router + top-K ---
@pytest.mark.parametrize("T,Hh,Ee,Kk,with_bias,with_gain", [
    (1, 4096, 352, 8, True, True), (5, 4096, 352, 8, False, True), (32, 4096, 352, 8, True, True),
    (65, 4096, 352, 8, True, True), (192, 4096, 352, 8, True, False), (193, 4096, 352, 8, True, True),
    (9, 256, 16, 2, True, True), (4, 1024, 512, 16, False, False), (3, 192, 20, 3, True, True),
    (6, 8192, 64, 4, True, True)])
def test_norm_route_matches_separate_calls(dev, T, Hh, Ee, Kk, with_bias, with_gain):
    """moe_norm_route (norm fused into the block-sum router up to 192 tokens
    and H = 4096, one token per wave up to 64, two beyond; separate kernels
    past that: T = 193, H = 8192) is bitwise moe_rmsnorm + moe_route_topk,
    which the tests above pin to the oracle."""
    r = torch.from_numpy(synth.normal((T, Hh), 1.0, 14, 0, synth.T_X, T)).to(dev)
    gain = torch.from_numpy(synth.norm_weight(Hh, 14, 0)).to(dev) if with_gain else None
    wT = torch.from_numpy(synth.router_weight_T(Hh, Ee, 14)).to(dev)
    bias = torch.from_numpy(synth.zipf_bias(Ee, 14, 0)).to(dev) if with_bias else None
    a, ids, w = B.moe_norm_route(r, wT, Kk, norm_w=gain, eps=1e-5, bias=bias)
    a2 = B.moe_rmsnorm(r, gain, 1e-5, torch.bfloat16)
    ids2, w2 = B.moe_route_topk(Kk, x=a2, router_wT=wT, bias=bias)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), a2.view(torch.int16))
    assert torch.equal(ids, ids2)
    assert torch.equal(w.view(torch.int32), w2.view(torch.int32))


@pytest.mark.parametrize("T,Hh,Ee,Kk,with_bias,with_gain", [
    (1, 4096, 352, 8, True, True), (32, 4096, 352, 8, True, True),
    (192, 4096, 352, 8, True, True), (193, 4096, 352, 8, True, True),
    (6, 8192, 64, 4, True, False)])
def test_norm_route_against_oracle(dev, T, Hh, Ee, Kk, with_bias, with_gain):
    """moe_norm_route against the oracle directly: the layer input a is the
    oracle's float32 RMSNorm rounded to bf16, bit for bit; the expert ids are
    the oracle's top-K of its router chain on that a, bit for bit; weights
    within 1e-5. T <= 192 runs the fused block-sum kernel (one and two
    tokens per wave), T = 193 and H = 8192 the separate kernels."""
    r = synth.normal((T, Hh), 1.0, 15, 0, synth.T_X, T)
    r[0] *= 300.0                                          # rows of other scales
    if T > 2:
        r[2] *= 1e-3
    gain = synth.norm_weight(Hh, 15, 0) if with_gain else None
    wT = synth.router_weight_T(Hh, Ee, 15)
    bias = synth.zipf_bias(Ee, 15, 0) if with_bias else None
    a, ids, w = B.moe_norm_route(torch.from_numpy(r).to(dev), torch.from_numpy(wT).to(dev), Kk,
                                 norm_w=None if gain is None else torch.from_numpy(gain).to(dev),
                                 eps=1e-5,
                                 bias=None if bias is None else torch.from_numpy(bias).to(dev))
    oa = OF.round_to_format(ON.rmsnorm(r, gain, 1e-5), OF.BF16)
    a16 = a.view(torch.int16).cpu().numpy().view(np.uint16)
    bad = np.argwhere(a16 != OF.bf16_bits(oa))
    assert bad.size == 0, bad[:5]
    lg = OR.router_logits(oa.astype(np.float32), wT, bias)
    oids = OR.topk_ids(lg, Kk)
    assert np.array_equal(ids.cpu().numpy(), oids)
    np.testing.assert_allclose(w.cpu().numpy(), OR.routing_weights(lg, oids), rtol=1e-5, atol=0)


@pytest.mark.parametrize("T,Kk,Ee", [(9, 4, 16), (300, 4, 16)])
def test_forward_foreign_ids(dev, T, Kk, Ee):
    """Slots whose expert id lies outside [0, E) are routed nowhere: the
    layer equals the oracle's layer with those slots dropped (their weight
    set to zero). T = 9 runs the decode kernels and the one-group
    permutation, T = 300 the GEMM and the two-launch permutation."""
    Hh, Ff = 512, 256
    ffn, host = FX.int4_ffn_random(Ee, Hh, Ff, 90 + T, dev)
    r = np.random.default_rng(T)
    ids = np.stack([r.choice(Ee, Kk, replace=False) for _ in range(T)]).astype(np.int32)
    foreign = r.random((T, Kk)) < 0.2
    ids[foreign] = r.choice([-3, -1, Ee, Ee + 5], int(foreign.sum()))
    w = r.random((T, Kk)).astype(np.float32)
    x = synth.activations(T, Hh, "bf16", 16)
    tm, _ = B.moe_forward_plan(ffn, T, Kk, x.dtype)
    perm = B.moe_permute(torch.from_numpy(ids).to(dev), Ee, tm)
    out = B.moe_w4a16_forward(ffn, x.to(dev), torch.from_numpy(w).to(dev), perm).cpu().numpy()
    s2r = perm.slot_to_row.cpu().numpy().reshape(T, Kk)
    assert np.all(s2r[foreign] == -1) and np.all(s2r[~foreign] >= 0)
    ref = FX.oracle_layer(x, np.where(foreign, 0, ids), np.where(foreign, 0.0, w),
                          FX.experts_fn_int4(host))
    ok, ratio = FX.within_tolerance(out, ref)
    assert ok, ratio


@pytest.mark.parametrize("T,fmt", [(1, "int4"), (8, "int4"), (64, "int4"), (300, "int4"),
                                   (5, "nvfp4"), (300, "nvfp4")])
def test_forward_workspace_nan_canary(dev, T, fmt):
    """Workspace contents never reach the output: the forward pass run on a
    workspace filled with NaN gives bitwise the output it gives on a
    zero-filled one (padded tile rows stage uninitialised h and y rows; the
    kernels must keep them out of every result). Decode (T <= 64, E = 16,
    K = 4) and GEMM (T = 300) paths, with the shared expert at T = 300."""
    Ee, Kk, Hh, Ff = 16, 4, 512, 256
    if fmt == "int4":
        ffn, _ = FX.int4_ffn_random(Ee, Hh, Ff, 95, dev)
    else:
        ffn, _ = _nvfp4_ffn_from_oracle(Ee, Hh, Ff, 9, dev)
    sh = FX.shared_bf16(256, Hh, 4, 0, dev)[0] if T == 300 else None
    x = synth.activations(T, Hh, "bf16", 17).to(dev)
    lg = synth.router_logits(T, Ee, 17)
    ids, w = B.moe_route_topk(Kk, logits=torch.from_numpy(lg).to(dev))
    tm, need = B.moe_forward_plan(ffn, T, Kk, x.dtype, sh)
    perm = B.moe_permute(ids, Ee, tm)
    outs = []
    for fill in (0.0, float("nan")):
        ws = torch.full(((need + 3) // 4,), fill, dtype=torch.float32, device=dev)
        o = B.moe_w4a16_forward(ffn, x, w, perm, shared=sh, ws=ws.view(torch.uint8))
        outs.append(o.cpu().numpy())
    assert not np.isnan(outs[1]).any()
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
