"""GPU parity of the weight-format variants of the int4 page's error table
(int4-g32, asymmetric int4-g128, int8-g128) against the oracle: dequant
bit for bit, the layer within |gpu - oracle| <= 1e-2 (|oracle| +
rms(oracle)) at small, decode and prefill sizes."""
import numpy as np
import pytest
import torch

from oracle import router as OR
from quantized_moe_sigmoid_amd import binding as B
from quantized_moe_sigmoid_amd import synth
from tests import fixtures as FX

pytestmark = pytest.mark.gpu

H, F, E, K = 4096, 1536, 352, 8
FORMATS = [B.MOE_W_INT4_G32, B.MOE_W_INT4_G128_ASYM, B.MOE_W_INT8_G128]


def _bank(q, s, z):
    return B.bank_int8(q, s) if q.dtype == torch.int8 else B.bank_int4(q, s, z)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    return torch.device("cuda:0")


def _oracle_ffn(fmt, Ee, Hh, Ff, root, dev):
    banks, host = [], []
    for which, (n, k) in (("gate", (Ff, Hh)), ("up", (Ff, Hh)), ("down", (Hh, Ff))):
        q, s, z = FX.variant_bank_oracle(Ee, n, k, root, 0, which, fmt)
        banks.append(_bank(*FX.variant_to_device(q, s, z, dev)))
        host.append((q, s, z))
    assert banks[0].fmt == fmt
    return B.ffn(*banks), host


def _random_ffn(fmt, seed, dev):
    banks, host = [], []
    for i, (n, k) in enumerate(((F, H), (F, H), (H, F))):
        if fmt == B.MOE_W_INT8_G128:
            (q, s), z = synth.int8_random(E, n, k, seed + i, dev), None
        else:
            q, s, z = synth.packed_int4_variant_random(
                E, n, k, seed + i, dev, group=32 if fmt == B.MOE_W_INT4_G32 else 128,
                asym=fmt == B.MOE_W_INT4_G128_ASYM)
        banks.append(_bank(q, s, z))
        host.append((q, s, z))
    assert banks[0].fmt == fmt
    return B.ffn(*banks), host


def _experts_fn(host):
    cache = {}

    def fn(e):
        if e not in cache:
            cache[e] = tuple(FX.oracle_variant_expert(q, s, z, e) for (q, s, z) in host)
        return cache[e]
    return fn


def _layer(ffn, x, lg, Ee, Kk, dev):
    ids, w = B.moe_route_topk(Kk, logits=torch.from_numpy(lg).to(dev))
    tm, _ = B.moe_forward_plan(ffn, x.shape[0], Kk, x.dtype)
    perm = B.moe_permute(ids, Ee, tm)
    return B.moe_w4a16_forward(ffn, x, w, perm).cpu().numpy()


@pytest.mark.parametrize("fmt", FORMATS)
def test_dequant_bitwise(dev, fmt):
    q, s, z = FX.variant_bank_oracle(3, 64, 256, 21, 0, "gate", fmt)
    bank = _bank(*FX.variant_to_device(q, s, z, dev))
    for e in range(3):
        got = B.moe_dequant(bank, e, device=dev).cpu().numpy()
        want = FX.oracle_variant_expert(q, s, z, e).astype(np.float32)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), e


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("act", ["f16", "bf16"])
def test_forward_small(dev, fmt, act):
    Ee, Hh, Ff, T, Kk = 8, 512, 256, 5, 3
    ffn, host = _oracle_ffn(fmt, Ee, Hh, Ff, 22, dev)
    x = synth.activations(T, Hh, act, 22)
    lg = synth.router_logits(T, Ee, 22)
    out = _layer(ffn, x.to(dev), lg, Ee, Kk, dev)
    oids = OR.topk_ids(lg, Kk)
    ref = FX.oracle_layer(x, oids, OR.routing_weights(lg, oids), _experts_fn(host))
    ok, ratio = FX.within_tolerance(out, ref)
    assert ok, ratio


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("act", ["f16", "bf16"])
@pytest.mark.parametrize("zero_groups", [False, True])
def test_forward_small_grouped_gemm(dev, fmt, act, zero_groups):
    """The variants on the grouped MFMA GEMM (T*K >= 4E): 4 experts, hidden
    512, width 256, 40 tokens, top-2, several tiles per expert; with
    zero_groups, some groups of every matrix get a zero scale (the g128
    forms drop such a group), which the oracle dequantizes to zeros."""
    Ee, Hh, Ff, T, Kk = 4, 512, 256, 40, 2
    banks, host = [], []
    for which, (n, k) in (("gate", (Ff, Hh)), ("up", (Ff, Hh)), ("down", (Hh, Ff))):
        q, s, z = FX.variant_bank_oracle(Ee, n, k, 24, 0, which, fmt)
        if zero_groups:
            s = s.copy()
            s[:, ::7, 1] = 0
            s[1, 3, :] = 0
        banks.append(_bank(*FX.variant_to_device(q, s, z, dev)))
        host.append((q, s, z))
    ffn = B.ffn(*banks)
    x = synth.activations(T, Hh, act, 24)
    lg = synth.router_logits(T, Ee, 24)
    out = _layer(ffn, x.to(dev), lg, Ee, Kk, dev)
    oids = OR.topk_ids(lg, Kk)
    ref = FX.oracle_layer(x, oids, OR.routing_weights(lg, oids), _experts_fn(host))
    ok, ratio = FX.within_tolerance(out, ref)
    assert ok, ratio


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("T,act,toks", [(8, "f16", list(range(8))), (64, "f16", [0, 17, 40, 63]),
                                        (256, "bf16", [0, 101, 255]), (2048, "f16", [0, 1000, 2047])])
def test_forward_layer_shape(dev, fmt, T, act, toks):
    """352 experts, hidden 4096, width 1536: decode batches (decode GEMV) and
    prefill-sized ones (grouped MFMA GEMM)."""
    ffn, host = _random_ffn(fmt, 600 + T, dev)
    x = synth.activations(T, H, act, 23)
    lg = synth.router_logits(T, E, 23)
    out = _layer(ffn, x.to(dev), lg, E, K, dev)
    oids = OR.topk_ids(lg, K)
    ow = OR.routing_weights(lg, oids)
    ref = FX.oracle_layer(x[toks], oids[toks], ow[toks], _experts_fn(host))
    ok, ratio = FX.within_tolerance(out[toks], ref)
    assert ok, ratio
