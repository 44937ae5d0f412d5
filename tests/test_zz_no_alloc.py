"""The forward entry point that allocates nothing (moe_w4a16_forward_scratch,
for callers that cannot allocate device memory) against the workspace entry
point moe_w4a16_forward, through the C ABI: the same kernels, so the same
bits, on consecutive calls whose second is smaller (the library's buffer
keeps the first call's contents), with and without the shared expert, and
the error for a call whose workspace would not fit the buffer."""
import numpy as np
import pytest
import torch

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


def _pair(dev, ffn, T, Ee, Kk, act, seed, shared=None, residual=None):
    x = synth.activations(T, ffn.gate.k, act, seed).to(dev)
    lg = synth.router_logits(T, Ee, seed)
    ids, w = B.moe_route_topk(Kk, logits=torch.from_numpy(lg).to(dev))
    tm, _ = B.moe_forward_plan(ffn, T, Kk, x.dtype, shared)
    perm = B.moe_permute(ids, Ee, tm)
    ref = B.moe_w4a16_forward(ffn, x, w, perm, shared=shared, residual=residual)
    got = B.moe_w4a16_forward_scratch(ffn, x, w, perm, shared=shared, residual=residual)
    torch.cuda.synchronize()
    return got.cpu().numpy(), ref.cpu().numpy()


def _same_bits(a, b):
    return a.shape == b.shape and np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_scratch_forward_two_calls_second_smaller(dev):
    """Layer shape, int4 experts, fp16 x: T = 64, then T = 5 on the same
    buffer."""
    ffn, _ = FX.int4_ffn_random(E, H, F, 500, dev)
    for T in (64, 5):
        got, ref = _pair(dev, ffn, T, E, K, "f16", 60 + T)
        assert not np.isnan(got).any()
        assert _same_bits(got, ref), T


def test_scratch_forward_shared_expert_and_nvfp4(dev):
    """With the BF16 shared expert and a residual (T = 32, then 3), and an
    NVFP4 bank (T = 16, then 1), one after the other on the same buffer."""
    ffn, _ = FX.int4_ffn_random(E, H, F, 501, dev)
    sh, _ = FX.shared_bf16(F, H, 5, 0, dev)
    for T in (32, 3):
        r = torch.from_numpy(synth.normal((T, H), 1.0, 9, 0, synth.T_X, T)).to(dev)
        got, ref = _pair(dev, ffn, T, E, K, "bf16", 70 + T, shared=sh, residual=r)
        assert _same_bits(got, ref), T
    banks = []
    for i, (n, k) in enumerate(((F, H), (F, H), (H, F))):
        banks.append(B.bank_nvfp4(*synth.packed_nvfp4_random(E, n, k, 510 + i, dev)))
    nv = B.ffn(*banks)
    for T in (16, 1):
        got, ref = _pair(dev, nv, T, E, K, "bf16", 80 + T)
        assert _same_bits(got, ref), T


def test_scratch_forward_refuses_workspace_over_the_buffer(dev):
    """T = 256 takes the prefill GEMM, whose workspace exceeds the buffer:
    the call fails with MOE_ERR_WORKSPACE_TOO_SMALL and launches nothing
    (the output keeps its contents); a decode batch after it still works."""
    ffn, _ = FX.int4_ffn_random(E, H, F, 502, dev)
    T = 256
    x = synth.activations(T, H, "bf16", 90).to(dev)
    ids, w = B.moe_route_topk(K, logits=torch.from_numpy(synth.router_logits(T, E, 90)).to(dev))
    tm, need = B.moe_forward_plan(ffn, T, K, x.dtype)
    assert need > B.MOE_FORWARD_SCRATCH_BYTES
    perm = B.moe_permute(ids, E, tm)
    out = torch.full((T, H), 7.0, device=dev)
    with pytest.raises(B.MoeError) as e:
        B.moe_w4a16_forward_scratch(ffn, x, w, perm, out=out)
    assert e.value.status == B.MOE_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
    got, ref = _pair(dev, ffn, 8, E, K, "bf16", 91)
    assert _same_bits(got, ref)
