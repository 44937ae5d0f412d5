"""GPU parity of the CSF scale expansion (moe_csf_expand) against the oracle's
CSF codec: the expanded bytes are bitwise the bytes the tensors encode, at
small and at the layer's own shapes, with and without the routed-experts
restriction; an NVFP4 forward pass on expanded scales is bitwise the one on
the raw scales."""
import numpy as np
import pytest
import torch

from oracle import csf as OC
from oracle import quant as OQ
from oracle import router as OR
from quantized_moe_sigmoid_amd import binding as B
from quantized_moe_sigmoid_amd import synth
from tests import fixtures as FX

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    return torch.device("cuda:0")


def _scales(E, R, C, seed, outlier_rate, near=False):
    """E4M3 scale bytes with the structure CSF targets: each row clustered in
    a window (its base drawn per row, in [0x20, 0x6E], or with near in
    [0x50, 0x5F]), a fraction of outliers (exceptions) anywhere in the
    finite non-negative range 0x00..0x7E, or, with near, within 16 bytes
    below or above the row's window (at most 4x from the row's own scales,
    and rows within 4x of each other)."""
    rng = np.random.default_rng(seed)
    base = rng.integers(0x50, 0x60, (E, R, 1)) if near else rng.integers(0x20, 0x6F, (E, R, 1))
    s = base + rng.integers(0, 16, (E, R, C))
    out = rng.random((E, R, C)) < outlier_rate
    if near:
        b = np.broadcast_to(base, s.shape)[out]
        d = rng.integers(0, 32, int(out.sum()))
        s[out] = np.where(d < 16, b - 1 - d, b + d)          # below or above the window
    else:
        s[out] = rng.integers(0, 0x7F, int(out.sum()))
    return np.clip(s, 0, 0x7E).astype(np.uint8)


def _to_dev(fixed, exc, starts, dev):
    return (torch.from_numpy(fixed).to(dev),
            torch.from_numpy(exc.view(np.int32)).to(dev),
            torch.from_numpy(starts).to(dev))


@pytest.mark.parametrize("E,R,C,rate", [(3, 32, 16, 0.05), (5, 48, 96, 0.2), (2, 16, 256, 0.0),
                                        (4, 64, 32, 1.0)])
def test_csf_expand_small(dev, E, R, C, rate):
    s = _scales(E, R, C, 10 + E, rate)
    fixed, exc, starts = OC.encode(s)
    want = OC.decode(fixed, exc, starts, R, C)
    assert np.array_equal(want, s)
    got = B.moe_csf_expand(*_to_dev(fixed, exc, starts, dev), R, C).cpu().numpy()
    assert np.array_equal(got, want)


@pytest.mark.parametrize("R,C", [(1536, 256), (4096, 96)])
def test_csf_expand_layer_shapes(dev, R, C):
    """The gate/up and down scale tensors of one layer (352 experts), with
    0.2 % exceptions (the page's CSF totals imply about that rate)."""
    s = _scales(352, R, C, R + C, 0.002)
    fixed, exc, starts = OC.encode(s)
    assert exc.size > 0
    got = B.moe_csf_expand(*_to_dev(fixed, exc, starts, dev), R, C).cpu().numpy()
    assert np.array_equal(got, s)


def test_csf_expand_routed_experts_only(dev):
    """With the permutation's expert offsets, experts with no routed slot are
    left untouched and every routed expert is expanded exactly."""
    E, R, C, T, K = 16, 32, 32, 3, 2
    s = _scales(E, R, C, 7, 0.1)
    fixed, exc, starts = OC.encode(s)
    lg = synth.router_logits(T, E, 7)
    ids, _ = B.moe_route_topk(K, logits=torch.from_numpy(lg).to(dev))
    perm = B.moe_permute(ids, E, 4)
    routed = set(OR.topk_ids(lg, K).ravel().tolist())
    assert 0 < len(routed) < E
    # full grid with skipped experts, and the compact grid sized by T*K
    for max_routed in (0, min(E, T * K)):
        out = torch.full((E, R, C), 0xAB, dtype=torch.uint8, device=dev)
        B.moe_csf_expand(*_to_dev(fixed, exc, starts, dev), R, C, out=out,
                         expert_offsets=perm.expert_offsets, max_routed=max_routed)
        got = out.cpu().numpy()
        for e in range(E):
            if e in routed:
                assert np.array_equal(got[e], s[e]), (max_routed, e)
            else:
                assert np.all(got[e] == 0xAB), (max_routed, e)


def test_nvfp4_forward_on_expanded_scales(dev):
    """NVFP4 experts whose block scales come from moe_csf_expand give
    bitwise the output of the same experts on their raw scale bytes, and
    the oracle's output on the bytes its own CSF decoder returns."""
    Ee, Hh, Ff, T, Kk = 6, 512, 256, 5, 3
    raw, csf, hb = [], [], []
    for which, (n, k) in (("gate", (Ff, Hh)), ("up", (Ff, Hh)), ("down", (Hh, Ff))):
        q, s, gs = FX.nvfp4_bank_oracle(Ee, n, k, 4, 0, which)
        qd, gsd = torch.from_numpy(q).to(dev), torch.from_numpy(gs).to(dev)
        raw.append(B.bank_nvfp4(qd, torch.from_numpy(s).to(dev), gsd))
        fixed, exc, starts = OC.encode(s)
        sx = B.moe_csf_expand(*_to_dev(fixed, exc, starts, dev), n, k // 16)
        csf.append(B.bank_nvfp4(qd, sx, gsd))
        hb.append((q, OC.decode(fixed, exc, starts, n, k // 16), None, gs))
    x = synth.activations(T, Hh, "bf16", 4).to(dev)
    lg = synth.router_logits(T, Ee, 4)
    ids, w = B.moe_route_topk(Kk, logits=torch.from_numpy(lg).to(dev))
    outs = []
    for banks in (raw, csf):
        ffn = B.ffn(*banks)
        tm, _ = B.moe_forward_plan(ffn, T, Kk, x.dtype)
        perm = B.moe_permute(ids, Ee, tm)
        outs.append(B.moe_w4a16_forward(ffn, x, w, perm).cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    oids = OR.topk_ids(lg, Kk)
    assert np.array_equal(ids.cpu().numpy(), oids)
    toks = list(range(T)) if T <= 64 else FX.tile_probe_tokens(oids, Ee, 64)
    ref = FX.oracle_layer_streamed(x.cpu()[toks], oids[toks],
                                   OR.routing_weights(lg, oids)[toks], FX.dequant_fn(hb, "nvfp4"))
    ok, ratio = FX.within_tolerance(outs[1][toks], ref)
    assert ok, ratio


# ------------------------------------- compressed scales read in place ---
def _row_index(exc, starts, R, C, dev, offsets=None, max_routed=0):
    ex, st = (torch.from_numpy(exc.view(np.int32)).to(dev), torch.from_numpy(starts).to(dev))
    return B.moe_csf_row_index(ex, st, R, C, expert_offsets=offsets, max_routed=max_routed)


@pytest.mark.parametrize("E,R,C,rate", [(3, 32, 16, 0.05), (5, 48, 96, 0.3), (2, 16, 256, 0.0),
                                        (352, 1536, 256, 0.002), (352, 4096, 96, 0.002)])
def test_csf_row_index_bitwise(dev, E, R, C, rate):
    s = _scales(E, R, C, 30 + R + C, rate)
    fixed, exc, starts = OC.encode(s)
    got = _row_index(exc, starts, R, C, dev).cpu().numpy()
    assert np.array_equal(got, OC.row_starts(exc, starts, E, R, C))


def test_csf_row_index_routed_experts_only(dev):
    E, R, C, T, K = 16, 32, 32, 3, 2
    s = _scales(E, R, C, 8, 0.2)
    fixed, exc, starts = OC.encode(s)
    lg = synth.router_logits(T, E, 8)
    ids, _ = B.moe_route_topk(K, logits=torch.from_numpy(lg).to(dev))
    perm = B.moe_permute(ids, E, 4)
    routed = set(OR.topk_ids(lg, K).ravel().tolist())
    want = OC.row_starts(exc, starts, E, R, C)
    for max_routed in (0, min(E, T * K)):
        out = torch.full((E, R + 1), -7, dtype=torch.int32, device=dev)
        ex, st = torch.from_numpy(exc.view(np.int32)).to(dev), torch.from_numpy(starts).to(dev)
        B.moe_csf_row_index(ex, st, R, C, out=out, expert_offsets=perm.expert_offsets,
                            max_routed=max_routed)
        got = out.cpu().numpy()
        for e in range(E):
            if e in routed:
                assert np.array_equal(got[e], want[e]), (max_routed, e)
            else:
                assert np.all(got[e] == -7), (max_routed, e)


def _csf_bank(q, s, gs, dev):
    """An NVFP4_CSF bank of codes q, scale bytes s (host uint8 [E, n, k/16],
    encoded by the oracle) and global scales gs (device)."""
    E, n, C = s.shape
    fixed, exc, starts = OC.encode(s)
    ri = _row_index(exc, starts, n, C, dev)
    ex = torch.from_numpy(exc.view(np.int32)).to(dev) if exc.size else None
    return B.bank_nvfp4_csf(q, torch.from_numpy(fixed).to(dev), ex, ri, gs)


def test_nvfp4_csf_dequant_bitwise(dev):
    E, n, k = 3, 64, 512
    q, _, gs = synth.packed_nvfp4_random(E, n, k, 31, dev)
    s = _scales(E, n, k // 16, 31, 0.25)
    bank = _csf_bank(q, s, gs, dev)
    qh, gh = q.cpu().numpy(), gs.cpu().numpy()
    for e in range(E):
        got = B.moe_dequant(bank, e, device=dev).cpu().numpy()
        want = OQ.dequant_nvfp4_fp32(qh[e], s[e], gh[e]).astype(np.float32)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), e


@pytest.mark.parametrize("Ee,Hh,Ff,T,Kk,rate,act", [(6, 512, 256, 5, 3, 0.3, "bf16"),
                                                    (6, 512, 256, 7, 2, 0.0, "f16"),
                                                    (352, 4096, 1536, 64, 8, 0.002, "bf16"),
                                                    (6, 512, 256, 40, 3, 0.3, "f16"),
                                                    (352, 4096, 1536, 256, 8, 0.002, "bf16")])
def test_nvfp4_csf_forward_equals_raw_scales(dev, Ee, Hh, Ff, T, Kk, rate, act):
    """The layer on compressed scales, read in place by the decode kernels
    (small batches) or expanded into the workspace for the grouped GEMM
    (T*K >= 4E), is bitwise the layer on the same scale bytes stored plainly
    where both run the same kernel, and within tolerance of the oracle, whose
    scale bytes come from its own CSF decoder (every token up to T = 64,
    tile-probing tokens beyond). At the layer's shape and T*K in [4E, 8E)
    the plain bytes take the MFMA GEMV and the compressed ones the grouped
    GEMM, so there both are held to the oracle."""
    raw, csf, hb = [], [], []
    for i, (n, k) in enumerate(((Ff, Hh), (Ff, Hh), (Hh, Ff))):
        q, _, gs = synth.packed_nvfp4_random(Ee, n, k, 40 + i, dev)
        # rows of similar scale and exceptions near their row's window:
        # scales spread over three decades make h heavy-tailed (its channel
        # magnitudes follow the product of a gate and an up row scale), and
        # rounding h to the activation dtype, as the kernels do before the
        # down projection, then moves outputs by about the tolerance even
        # with every other step exact (checked on the CPU)
        s = _scales(Ee, n, k // 16, 40 + i, rate, near=True)
        raw.append(B.bank_nvfp4(q, torch.from_numpy(s).to(dev), gs))
        csf.append(_csf_bank(q, s, gs, dev))
        fixed, exc, starts = OC.encode(s)
        hb.append(FX.host_bank(q, OC.decode(fixed, exc, starts, n, k // 16), gs=gs))
    x = synth.activations(T, Hh, act, 41).to(dev)
    lg = synth.router_logits(T, Ee, 41)
    ids, w = B.moe_route_topk(Kk, logits=torch.from_numpy(lg).to(dev))
    outs = []
    for banks in (raw, csf):
        ffn = B.ffn(*banks)
        tm, _ = B.moe_forward_plan(ffn, T, Kk, x.dtype)
        perm = B.moe_permute(ids, Ee, tm)
        outs.append(B.moe_w4a16_forward(ffn, x, w, perm).cpu().numpy())
    same_kernel = not (Hh == 4096 and Ff == 1536 and 4 * Ee <= T * Kk < 8 * Ee)
    if same_kernel:
        assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    oids = OR.topk_ids(lg, Kk)
    assert np.array_equal(ids.cpu().numpy(), oids)
    toks = list(range(T)) if T <= 64 else FX.tile_probe_tokens(oids, Ee, 64)
    ref = FX.oracle_layer_streamed(x.cpu()[toks], oids[toks],
                                   OR.routing_weights(lg, oids)[toks], FX.dequant_fn(hb, "nvfp4"))
    for o in (outs if not same_kernel else outs[1:]):
        ok, ratio = FX.within_tolerance(o[toks], ref)
        assert ok, ratio
