"""HIP-graph replay of the library's calls: a stacked-layer step (RMSNorm,
router, top-K, permutation, routed + shared experts, combine with the
residual) and a decode step (top-K on given logits, permutation, routed
experts, combine) captured once and replayed give bitwise the eager result
on every replay, with eager work and synchronisations between the replays.
Every call only enqueues kernels on the caller's stream and allocates
nothing, which is what makes the capture possible."""
import pytest
import torch

from quantized_moe_sigmoid_amd import binding as B
from quantized_moe_sigmoid_amd import synth
from tests import fixtures as FX

pytestmark = pytest.mark.gpu

H, F, E, K = 4096, 1536, 352, 8
ROOT = 9


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    return torch.device("cuda:0")


def test_stack_step_graph_replays_match_eager(dev):
    T, L = 32, 2
    layers = []
    for l in range(L):
        ffn, _ = FX.int4_ffn_random(E, H, F, 9000 + 10 * l, dev)
        sh, _ = FX.shared_bf16(F, H, ROOT, l, dev)
        wT = torch.from_numpy(synth.router_weight_T(H, E, ROOT, l)).to(dev)
        bias = torch.from_numpy(synth.zipf_bias(E, ROOT, l)).to(dev)
        nw = torch.from_numpy(synth.norm_weight(H, ROOT, l)).to(dev)
        layers.append((ffn, sh, wT, bias, nw))
    r0 = synth.activations(T, H, "bf16", ROOT).float().to(dev)
    res = [torch.empty_like(r0), torch.empty_like(r0)]
    a = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    tm, wsb = B.moe_forward_plan(layers[0][0], T, K, torch.bfloat16, layers[0][1])
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    ids = torch.empty((T, K), dtype=torch.int32, device=dev)
    w = torch.empty((T, K), dtype=torch.float32, device=dev)
    perm = B.Perm(T, K, E, tm, dev)
    rws = torch.empty(B.moe_route_workspace(T, E, True), dtype=torch.uint8, device=dev)

    def step():
        res[0].copy_(r0)
        for l, (ffn, sh, wT, bias, nw) in enumerate(layers):
            src, dst = res[l % 2], res[(l + 1) % 2]
            if l % 2 == 0:                      # the fused call and the separate ones
                B.moe_norm_route(src, wT, K, norm_w=nw, eps=1e-5, bias=bias, a=a, ids=ids, w=w,
                                 ws=rws)
            else:
                B.moe_rmsnorm(src, nw, 1e-5, out=a)
                B.moe_route_topk(K, x=a, router_wT=wT, bias=bias, ids=ids, w=w, ws=rws)
            B.moe_permute(ids, E, tm, perm=perm)
            B.moe_w4a16_forward(ffn, a, w, perm, residual=src, out=dst, ws=ws, shared=sh)

    step()
    torch.cuda.synchronize()
    ref = res[L % 2].clone()
    ref_ids = ids.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        res[L % 2].zero_()                      # eager work between the replays
        ids.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(res[L % 2], ref), rep
        assert torch.equal(ids, ref_ids), rep
        step()                                  # an eager step in between
        torch.cuda.synchronize()
        assert torch.equal(res[L % 2], ref), rep


def test_decode_step_graph_replays_match_eager(dev):
    """Fresh logits are copied into the captured input before each replay."""
    T = 64
    ffn, _ = FX.int4_ffn_random(E, H, F, 9100, dev)
    x = synth.activations(T, H, "f16", ROOT).to(dev)
    lg_in = torch.empty((T, E), dtype=torch.float32, device=dev)
    tm, wsb = B.moe_forward_plan(ffn, T, K, torch.float16)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    ids = torch.empty((T, K), dtype=torch.int32, device=dev)
    w = torch.empty((T, K), dtype=torch.float32, device=dev)
    perm = B.Perm(T, K, E, tm, dev)
    out = torch.empty((T, H), dtype=torch.float32, device=dev)

    def step():
        B.moe_route_topk(K, logits=lg_in, ids=ids, w=w)
        B.moe_permute(ids, E, tm, perm=perm)
        B.moe_w4a16_forward(ffn, x, w, perm, out=out, ws=ws)

    logits = [torch.from_numpy(synth.router_logits(T, E, 3000 + i)).to(dev) for i in range(3)]
    refs = []
    for lg in logits:
        lg_in.copy_(lg)
        step()
        torch.cuda.synchronize()
        refs.append(out.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(2):
        for i, lg in enumerate(logits):
            out.zero_()
            lg_in.copy_(lg)
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, refs[i]), (rep, i)
        lg_in.copy_(logits[0])                  # eager work between the rounds
        step()
        torch.cuda.synchronize()
        assert torch.equal(out, refs[0]), rep
