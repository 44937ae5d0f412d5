"""The C-ABI library loads, exports every declared entry point, and rejects
invalid arguments on the host before any HIP call (runs without a GPU)."""
import ctypes
import os
import re

import pytest

from quantized_moe_sigmoid_amd import binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "moe_w4a16.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.library_path()):
        pytest.skip("library not built")
    return B.lib()


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert set(names) == set(B.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version(L):
    assert L.moe_abi_version() == 6
    assert B.status_string(0) == "MOE_OK"
    assert B.status_string(3) == "MOE_ERR_WORKSPACE_TOO_SMALL"
    assert B.status_string(99) == "MOE_ERR_UNKNOWN"


FAKE = 0x10000          # an aligned non-null address; validation never dereferences it


def _bank(fmt, E, n, k, qrow=None, srow=None):
    if fmt == B.MOE_W_INT4_G128:
        qr = qrow if qrow is not None else k // 2
        sr = srow if srow is not None else (k // 128) * 2
        return B.WeightDesc(fmt, E, n, k, FAKE, FAKE, None, qr * n, qr, sr * n, sr)
    qr = qrow if qrow is not None else k // 2
    sr = srow if srow is not None else k // 16
    return B.WeightDesc(fmt, E, n, k, FAKE, FAKE, FAKE, qr * n, qr, sr * n, sr)


def _ffn(fmt=B.MOE_W_INT4_G128, E=352, H=4096, F=1536):
    return B.FfnDesc(_bank(fmt, E, F, H), _bank(fmt, E, F, H), _bank(fmt, E, H, F))


def _plan(ex, T=8, K=8, act=B.MOE_F16, shared=None):
    tm, ws = ctypes.c_int(), ctypes.c_size_t()
    st = B.lib().moe_forward_plan(ctypes.byref(ex), shared, T, K, act, ctypes.byref(tm),
                                  ctypes.byref(ws))
    return st, tm.value, ws.value


def test_forward_plan_rejects_k_over_16(L):
    """The combine sums at most 16 routed slots per token."""
    assert _plan(_ffn(), T=8, K=16)[0] == B.MOE_OK
    assert _plan(_ffn(), T=8, K=17)[0] == B.MOE_ERR_INVALID_ARG


def test_forward_plan_sizes(L):
    st, tm, ws = _plan(_ffn(), T=64)
    assert st == B.MOE_OK and tm >= 1
    mr, mt = B.moe_permute_sizes(64, 8, 352, tm)
    assert mr == 512 + 352 * (tm - 1) and mt == mr // tm
    assert ws >= mr * 1536 * 2 + mr * 4096 * 4


@pytest.mark.parametrize("mutate,want", [
    (lambda f: setattr(f.gate, "k", 4000), B.MOE_ERR_INVALID_ARG),        # k % 128
    (lambda f: setattr(f.up, "num_experts", 351), B.MOE_ERR_INVALID_ARG),
    (lambda f: setattr(f.down, "n", 2048), B.MOE_ERR_INVALID_ARG),        # down must be [H][F]
    (lambda f: setattr(f.gate, "qweight", None), B.MOE_ERR_INVALID_ARG),
    (lambda f: setattr(f.gate, "qweight_row_stride", 2056), B.MOE_ERR_INVALID_ARG),  # %16
    (lambda f: setattr(f.gate, "fmt", 7), B.MOE_ERR_INVALID_ARG),
    (lambda f: setattr(f.gate, "qweight", FAKE + 8), B.MOE_ERR_INVALID_ARG),        # alignment
])
def test_forward_plan_rejects_bad_descriptors(L, mutate, want):
    f = _ffn()
    mutate(f)
    assert _plan(f)[0] == want


def test_nvfp4_rules(L):
    assert _plan(_ffn(B.MOE_W_NVFP4_G16), act=B.MOE_BF16)[0] == B.MOE_OK
    f = _ffn(B.MOE_W_NVFP4_G16)
    f.gate.global_scale = None
    assert _plan(f)[0] == B.MOE_ERR_INVALID_ARG
    nv = B.MOE_W_NVFP4_G16                        # 16 | k but not 32 | k (rows padded to 16 B)
    f = B.FfnDesc(_bank(nv, 352, 1536, 4112, qrow=2064, srow=258),
                  _bank(nv, 352, 1536, 4112, qrow=2064, srow=258),
                  _bank(nv, 352, 4112, 1536))
    assert _plan(f)[0] == B.MOE_ERR_UNSUPPORTED


def test_forward_plan_rejects_bad_sizes(L):
    assert _plan(_ffn(), K=0)[0] == B.MOE_ERR_INVALID_ARG
    assert _plan(_ffn(E=4), K=5)[0] == B.MOE_ERR_INVALID_ARG
    assert _plan(_ffn(), act=B.MOE_F32)[0] == B.MOE_ERR_INVALID_ARG
    assert _plan(_ffn(E=513))[0] == B.MOE_ERR_INVALID_ARG


def test_route_topk_validation(L):
    R = L.moe_route_topk
    p = ctypes.c_void_p(FAKE)
    n = None
    big = 1 << 30
    # K > E, K > 16, E > 512, both or neither logit source
    assert R(n, 0, n, p, n, 4, 0, 8, 9, 1, p, p, n, 0, n) == B.MOE_ERR_INVALID_ARG
    assert R(n, 0, n, p, n, 4, 0, 64, 17, 1, p, p, n, 0, n) == B.MOE_ERR_INVALID_ARG
    assert R(n, 0, n, p, n, 4, 0, 513, 8, 1, p, p, n, 0, n) == B.MOE_ERR_INVALID_ARG
    assert R(p, 1, p, p, n, 4, 64, 16, 2, 1, p, p, p, big, n) == B.MOE_ERR_INVALID_ARG
    assert R(n, 0, n, n, n, 4, 64, 16, 2, 1, p, p, p, big, n) == B.MOE_ERR_INVALID_ARG
    # router weight: missing x, bad dtype, H % 64, E % 4, workspace
    assert R(n, 1, p, n, n, 4, 64, 16, 2, 1, p, p, p, big, n) == B.MOE_ERR_INVALID_ARG
    assert R(p, 3, p, n, n, 4, 64, 16, 2, 1, p, p, p, big, n) == B.MOE_ERR_INVALID_ARG
    assert R(p, 1, p, n, n, 4, 96, 16, 2, 1, p, p, p, big, n) == B.MOE_ERR_UNSUPPORTED
    assert R(p, 1, p, n, n, 4, 64, 18, 2, 1, p, p, p, big, n) == B.MOE_ERR_UNSUPPORTED
    assert R(p, 1, p, n, n, 4, 64, 16, 2, 1, p, p, n, big, n) == B.MOE_ERR_INVALID_ARG
    assert R(p, 1, p, n, n, 4, 64, 16, 2, 1, p, p, p, 4 * 16 * 4 - 1, n) == \
        B.MOE_ERR_WORKSPACE_TOO_SMALL
    # bf16 up to 192 tokens: one float per 512-input block, token and expert
    assert R(p, 2, p, n, n, 4, 1024, 16, 2, 1, p, p, p, 2 * 4 * 16 * 4 - 1, n) == \
        B.MOE_ERR_WORKSPACE_TOO_SMALL
    assert R(n, 0, n, p, n, 4, 0, 16, 2, 1, n, p, n, 0, n) == B.MOE_ERR_INVALID_ARG
    # T == 0 is a no-op that touches nothing
    assert R(n, 0, n, p, n, 0, 0, 16, 2, 1, p, p, n, 0, n) == B.MOE_OK
    # the workspace holds one sum per 512-input block, token and expert (8
    # blocks for H <= 4096; wider f16 or bf16 inputs need only the logits)
    assert B.moe_route_workspace(2048, 352, True) == 8 * 2048 * 352 * 4
    assert B.moe_route_workspace(2048, 352, False) == 0
    assert B.moe_route_workspace(192, 352, True) == 8 * 192 * 352 * 4
    assert B.moe_route_workspace(193, 352, True) == 8 * 193 * 352 * 4
    # bf16 past 192 tokens still takes the block sums
    assert R(p, 2, p, n, n, 200, 1024, 16, 2, 1, p, p, p, 2 * 200 * 16 * 4 - 1, n) == \
        B.MOE_ERR_WORKSPACE_TOO_SMALL
    # f16 takes the logits: one float per token and expert
    assert R(p, 1, p, n, n, 200, 1024, 16, 2, 1, p, p, p, 200 * 16 * 4 - 1, n) == \
        B.MOE_ERR_WORKSPACE_TOO_SMALL


def test_router_logits_validation(L):
    G = L.moe_router_logits
    p = ctypes.c_void_p(FAKE)
    assert G(p, 2, None, None, 4, 4096, 352, p, None) == B.MOE_ERR_INVALID_ARG
    assert G(p, 2, p, None, 4, 4000, 352, p, None) == B.MOE_ERR_UNSUPPORTED
    assert G(p, 2, ctypes.c_void_p(FAKE + 4), None, 4, 4096, 352, p, None) == B.MOE_ERR_INVALID_ARG
    assert G(p, 2, p, None, 4, 4096, 352, None, None) == B.MOE_ERR_INVALID_ARG
    assert G(None, 2, p, None, 0, 4096, 352, None, None) == B.MOE_OK


def test_permute_validation(L):
    p = B.PermDesc(*([FAKE] * 9), 4)
    assert L.moe_permute(None, 2, 2, 16, ctypes.byref(p), None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_permute(ctypes.c_void_p(FAKE), 2, 0, 16, ctypes.byref(p), None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_permute(ctypes.c_void_p(FAKE), 2, 2, 600, ctypes.byref(p), None) == B.MOE_ERR_INVALID_ARG
    p.tile_m = 0
    assert L.moe_permute(ctypes.c_void_p(FAKE), 2, 2, 16, ctypes.byref(p), None) == B.MOE_ERR_INVALID_ARG
    p = B.PermDesc(*([FAKE] * 8), None, 4)
    assert L.moe_permute(ctypes.c_void_p(FAKE), 2, 2, 16, ctypes.byref(p), None) == B.MOE_ERR_INVALID_ARG


def test_route_permute_validation(L):
    """moe_route_permute checks moe_route_topk's and moe_permute's argument
    rules before any launch."""
    R = L.moe_route_permute
    p = ctypes.c_void_p(FAKE)
    n = None
    big = 1 << 30
    d = B.PermDesc(*([FAKE] * 9), 4)
    pd = ctypes.byref(d)
    # K > E, K > 16, E > 512, both or neither logit source, missing outputs
    assert R(n, 0, n, p, n, 4, 0, 8, 9, 1, p, p, pd, n, 0, n) == B.MOE_ERR_INVALID_ARG
    assert R(n, 0, n, p, n, 4, 0, 64, 17, 1, p, p, pd, n, 0, n) == B.MOE_ERR_INVALID_ARG
    assert R(n, 0, n, p, n, 4, 0, 513, 8, 1, p, p, pd, n, 0, n) == B.MOE_ERR_INVALID_ARG
    assert R(p, 2, p, p, n, 4, 64, 16, 2, 1, p, p, pd, p, big, n) == B.MOE_ERR_INVALID_ARG
    assert R(n, 0, n, n, n, 4, 64, 16, 2, 1, p, p, pd, p, big, n) == B.MOE_ERR_INVALID_ARG
    assert R(n, 0, n, p, n, 4, 0, 16, 2, 1, n, p, pd, n, 0, n) == B.MOE_ERR_INVALID_ARG
    # the permutation arrays: a missing array, tile_m out of range
    d2 = B.PermDesc(*([FAKE] * 8), None, 4)
    assert R(n, 0, n, p, n, 4, 0, 16, 2, 1, p, p, ctypes.byref(d2), n, 0, n) == \
        B.MOE_ERR_INVALID_ARG
    d3 = B.PermDesc(*([FAKE] * 9), 0)
    assert R(n, 0, n, p, n, 4, 0, 16, 2, 1, p, p, ctypes.byref(d3), n, 0, n) == \
        B.MOE_ERR_INVALID_ARG
    # router weight: H % 64, workspace (one float per 512-input block)
    assert R(p, 2, p, n, n, 4, 96, 16, 2, 1, p, p, pd, p, big, n) == B.MOE_ERR_UNSUPPORTED
    assert R(p, 2, p, n, n, 4, 1024, 16, 2, 1, p, p, pd, p, 2 * 4 * 16 * 4 - 1, n) == \
        B.MOE_ERR_WORKSPACE_TOO_SMALL
    # T == 0 is a no-op
    assert R(n, 0, n, p, n, 0, 0, 16, 2, 1, p, p, pd, n, 0, n) == B.MOE_OK


def test_forward_validation_before_launch(L):
    f = _ffn()
    st, tm, ws = _plan(f, T=8)
    p = B.PermDesc(*([FAKE] * 9), tm)
    F = L.moe_w4a16_forward
    x = ctypes.c_void_p(FAKE)
    # workspace too small
    assert F(ctypes.byref(f), None, x, B.MOE_F16, 8, 8, x, ctypes.byref(p), None, x, B.MOE_F32,
             x, ws - 1, None) == B.MOE_ERR_WORKSPACE_TOO_SMALL
    # tile_m not the planned one
    p.tile_m = tm + 1
    assert F(ctypes.byref(f), None, x, B.MOE_F16, 8, 8, x, ctypes.byref(p), None, x, B.MOE_F32,
             x, ws, None) == B.MOE_ERR_INVALID_ARG
    p.tile_m = tm
    # bad output dtype, null output, misaligned workspace
    assert F(ctypes.byref(f), None, x, B.MOE_F16, 8, 8, x, ctypes.byref(p), None, x, 9,
             x, ws, None) == B.MOE_ERR_INVALID_ARG
    assert F(ctypes.byref(f), None, x, B.MOE_F16, 8, 8, x, ctypes.byref(p), None, None, B.MOE_F32,
             x, ws, None) == B.MOE_ERR_INVALID_ARG
    assert F(ctypes.byref(f), None, x, B.MOE_F16, 8, 8, x, ctypes.byref(p), None, x, B.MOE_F32,
             ctypes.c_void_p(FAKE + 16), ws, None) == B.MOE_ERR_INVALID_ARG
    # T == 0 is a no-op
    assert F(ctypes.byref(f), None, None, B.MOE_F16, 0, 8, None, ctypes.byref(p), None, None,
             B.MOE_F32, None, 0, None) == B.MOE_OK


def test_forward_gemm_offsets_limit(L):
    """The grouped GEMM reads x and h through 32-bit byte offsets: a batch
    whose h would pass 2^31 - 2^20 bytes (T = 90000, top-8: about 720 K
    rows of 3 KB) is refused before any launch; T = 80000 passes that
    check (and stops at the workspace size)."""
    f = _ffn()
    F = L.moe_w4a16_forward
    x = ctypes.c_void_p(FAKE)
    for T, want in ((90000, B.MOE_ERR_UNSUPPORTED), (80000, B.MOE_ERR_WORKSPACE_TOO_SMALL)):
        st, tm, ws = _plan(f, T=T)
        assert st == B.MOE_OK
        p = B.PermDesc(*([FAKE] * 9), tm)
        big = ws if want == B.MOE_ERR_UNSUPPORTED else ws - 1
        assert F(ctypes.byref(f), None, x, B.MOE_F16, T, 8, x, ctypes.byref(p), None, x,
                 B.MOE_F32, x, big, None) == want


def test_forward_profiled_validation(L):
    """The profiled entry: events must be an array of MOE_FORWARD_STAGES + 1
    entries; NULL entries are boundaries that record nothing."""
    f = _ffn()
    st, tm, ws = _plan(f, T=8)
    p = B.PermDesc(*([FAKE] * 9), tm)
    F = L.moe_w4a16_forward_profiled
    x = ctypes.c_void_p(FAKE)
    n = B.MOE_FORWARD_STAGES + 1
    none = (ctypes.c_void_p * n)()
    args = (ctypes.byref(f), None, x, B.MOE_F16, 8, 8, x, ctypes.byref(p), None, x, B.MOE_F32,
            x, ws, None)
    assert F(*args, None, n) == B.MOE_ERR_INVALID_ARG
    assert F(*args, none, n - 1) == B.MOE_ERR_INVALID_ARG
    # the usual validation still runs first
    bad = args[:12] + (ws - 1, None)
    assert F(*bad, none, n) == B.MOE_ERR_WORKSPACE_TOO_SMALL
    # T == 0 with only NULL entries: a no-op that touches no device
    assert F(ctypes.byref(f), None, None, B.MOE_F16, 0, 8, None, ctypes.byref(p), None, None,
             B.MOE_F32, None, 0, None, none, n) == B.MOE_OK


def test_forward_scratch_validation(L):
    """The entry on the library's own buffer: argument errors as
    moe_w4a16_forward, and a call whose workspace would exceed the buffer is
    refused before any HIP call. Every decode-kernel batch of the Step-5
    shape below T*K = 4E fits (up to 175 tokens, with the shared expert
    too); the larger batches' workspaces do not."""
    F = L.moe_w4a16_forward_scratch
    x = ctypes.c_void_p(FAKE)
    f = _ffn()
    for T in (1, 64, 175):
        st, tm, ws = _plan(f, T=T, act=B.MOE_BF16)
        assert st == B.MOE_OK and tm == 4 and ws <= B.MOE_FORWARD_SCRATCH_BYTES, (T, ws)
        sh = _shared()
        st, tm, ws = _plan(f, T=T, act=B.MOE_BF16, shared=ctypes.byref(sh))
        assert st == B.MOE_OK and ws <= B.MOE_FORWARD_SCRATCH_BYTES, (T, ws)
    # from 4E slots the MFMA GEMV's 8-slot tiles (up to 7E), then the GEMM:
    # neither workspace fits
    st, tm, ws = _plan(f, T=308, act=B.MOE_BF16)
    assert st == B.MOE_OK and tm == 64 and ws > B.MOE_FORWARD_SCRATCH_BYTES
    st, tm, ws = _plan(f, T=176, act=B.MOE_BF16)
    assert tm == 8 and ws > B.MOE_FORWARD_SCRATCH_BYTES
    p = B.PermDesc(*([FAKE] * 9), tm)
    assert F(ctypes.byref(f), None, x, B.MOE_BF16, 176, 8, x, ctypes.byref(p), None, x,
             B.MOE_F32, None) == B.MOE_ERR_WORKSPACE_TOO_SMALL
    # invalid arguments are reported before the buffer is looked up
    assert F(None, None, x, B.MOE_BF16, 8, 8, x, ctypes.byref(p), None, x, B.MOE_F32,
             None) == B.MOE_ERR_INVALID_ARG
    assert F(ctypes.byref(f), None, x, 9, 8, 8, x, ctypes.byref(p), None, x, B.MOE_F32,
             None) == B.MOE_ERR_INVALID_ARG
    assert F(ctypes.byref(f), None, x, B.MOE_BF16, 8, 17, x, ctypes.byref(p), None, x,
             B.MOE_F32, None) == B.MOE_ERR_INVALID_ARG


def test_dequant_validation(L):
    b = _bank(B.MOE_W_INT4_G128, 4, 64, 256)
    out = ctypes.c_void_p(FAKE)
    assert L.moe_dequant(ctypes.byref(b), 4, out, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_dequant(ctypes.byref(b), -1, out, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_dequant(ctypes.byref(b), 0, None, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_dequant(ctypes.byref(b), 0, ctypes.c_void_p(FAKE + 4), None) == B.MOE_ERR_INVALID_ARG


def _dense(n, k, row=None):
    r = row if row is not None else 2 * k
    return B.WeightDesc(B.MOE_W_BF16, 1, n, k, FAKE, None, None, r * n, r, 0, 0)


def _shared(H=4096, Fs=1536):
    return B.FfnDesc(_dense(Fs, H), _dense(Fs, H), _dense(H, Fs))


def test_shared_expert_plan(L):
    ex = _ffn()
    st0, tm0, ws0 = _plan(ex, T=32, act=B.MOE_BF16)
    st, tm, ws = _plan(ex, T=32, act=B.MOE_BF16, shared=ctypes.byref(_shared()))
    assert st0 == st == B.MOE_OK and tm == tm0
    # at least h [T][Fs] bf16 and y [T][H] float32 more
    assert ws >= ws0 + 32 * 1536 * 2 + 32 * 4096 * 4


@pytest.mark.parametrize("mutate,act,want", [
    (lambda s: None, B.MOE_F16, B.MOE_ERR_INVALID_ARG),                # bf16 activations only
    (lambda s: setattr(s.gate, "fmt", B.MOE_W_INT4_G128), B.MOE_BF16, B.MOE_ERR_INVALID_ARG),
    (lambda s: setattr(s.up, "num_experts", 2), B.MOE_BF16, B.MOE_ERR_INVALID_ARG),
    (lambda s: setattr(s.down, "k", 1024), B.MOE_BF16, B.MOE_ERR_INVALID_ARG),    # Fs mismatch
    (lambda s: setattr(s.gate, "k", 2048), B.MOE_BF16, B.MOE_ERR_INVALID_ARG),    # H mismatch
    (lambda s: setattr(s.gate, "qweight_row_stride", 8200), B.MOE_BF16, B.MOE_ERR_INVALID_ARG),
    (lambda s: setattr(s.gate, "qweight_row_stride", 4096), B.MOE_BF16, B.MOE_ERR_INVALID_ARG),
    (lambda s: setattr(s.down, "qweight", None), B.MOE_BF16, B.MOE_ERR_INVALID_ARG),
])
def test_shared_expert_rejects_bad_descriptors(L, mutate, act, want):
    s = _shared()
    mutate(s)
    assert _plan(_ffn(), act=act, shared=ctypes.byref(s))[0] == want


def test_shared_expert_unsupported_width(L):
    s = _shared(Fs=1600)                      # not a multiple of the 128-column block
    assert _plan(_ffn(), act=B.MOE_BF16, shared=ctypes.byref(s))[0] == B.MOE_ERR_UNSUPPORTED


def test_round_activations_validation(L):
    R = L.moe_round_activations
    p = ctypes.c_void_p(FAKE)
    assert R(p, 16, B.MOE_F32, p, None) == B.MOE_ERR_INVALID_ARG
    assert R(p, -1, B.MOE_BF16, p, None) == B.MOE_ERR_INVALID_ARG
    assert R(None, 16, B.MOE_BF16, p, None) == B.MOE_ERR_INVALID_ARG
    assert R(ctypes.c_void_p(FAKE + 4), 16, B.MOE_BF16, p, None) == B.MOE_ERR_INVALID_ARG
    assert R(None, 0, B.MOE_BF16, None, None) == B.MOE_OK


def test_rmsnorm_validation(L):
    N = L.moe_rmsnorm
    p = ctypes.c_void_p(FAKE)
    assert N(p, None, 1e-5, 4, 4096, B.MOE_F32, p, None) == B.MOE_ERR_INVALID_ARG   # dtype
    assert N(p, None, 1e-5, 4, 4094, B.MOE_BF16, p, None) == B.MOE_ERR_INVALID_ARG  # H % 4
    assert N(p, None, -1.0, 4, 4096, B.MOE_BF16, p, None) == B.MOE_ERR_INVALID_ARG  # eps
    assert N(p, None, float("nan"), 4, 4096, B.MOE_BF16, p, None) == B.MOE_ERR_INVALID_ARG
    assert N(p, ctypes.c_void_p(FAKE + 4), 1e-5, 4, 4096, B.MOE_BF16, p, None) == \
        B.MOE_ERR_INVALID_ARG                                                      # alignment
    assert N(None, None, 1e-5, 4, 4096, B.MOE_BF16, p, None) == B.MOE_ERR_INVALID_ARG
    assert N(None, None, 1e-5, 0, 4096, B.MOE_BF16, None, None) == B.MOE_OK


def test_csf_expand_validation(L):
    """Argument errors of moe_csf_expand are found before any launch."""
    F = L.moe_csf_expand
    p = ctypes.c_void_p(FAKE)
    ok = (p, p, 4, p, 2, 32, 16, None, 0, p, None)
    bad = [
        ((None,) + ok[1:], B.MOE_ERR_INVALID_ARG),                     # fixed
        (ok[:1] + (None,) + ok[2:], B.MOE_ERR_INVALID_ARG),            # exceptions with n > 0
        (ok[:2] + (-1,) + ok[3:], B.MOE_ERR_INVALID_ARG),              # n < 0
        (ok[:3] + (None,) + ok[4:], B.MOE_ERR_INVALID_ARG),            # starts
        (ok[:4] + (0,) + ok[5:], B.MOE_ERR_INVALID_ARG),               # E
        (ok[:5] + (24,) + ok[6:], B.MOE_ERR_INVALID_ARG),              # R % 16
        (ok[:6] + (8,) + ok[7:], B.MOE_ERR_INVALID_ARG),               # C % 16
        (ok[:5] + (4096, 4096) + ok[7:], B.MOE_ERR_UNSUPPORTED),       # R*C >= 2^24
        (ok[:8] + (-1,) + ok[9:], B.MOE_ERR_INVALID_ARG),              # max_routed_experts
        (ok[:9] + (None,) + ok[10:], B.MOE_ERR_INVALID_ARG),           # out
        (ok[:9] + (ctypes.c_void_p(FAKE + 8),) + ok[10:], B.MOE_ERR_INVALID_ARG),  # out alignment
        ((ctypes.c_void_p(FAKE + 4),) + ok[1:], B.MOE_ERR_INVALID_ARG),            # fixed alignment
    ]
    for args, want in bad:
        assert F(*args) == want, args


def test_norm_route_validation(L):
    """Argument errors of moe_norm_route are found before any launch."""
    F = L.moe_norm_route
    p = ctypes.c_void_p(FAKE)
    # the workspace: one float per 512-input block, token and expert
    ok = (p, None, 1e-5, 8, 4096, p, None, 352, 8, 1, p, p, p, p, 8 * 8 * 352 * 4, None)
    bad = [
        ((None,) + ok[1:], B.MOE_ERR_INVALID_ARG),                     # residual
        (ok[:2] + (-1.0,) + ok[3:], B.MOE_ERR_INVALID_ARG),            # eps
        (ok[:3] + (-1,) + ok[4:], B.MOE_ERR_INVALID_ARG),              # T
        (ok[:4] + (4032 + 32,) + ok[5:], B.MOE_ERR_UNSUPPORTED),       # H % 64
        (ok[:5] + (None,) + ok[6:], B.MOE_ERR_INVALID_ARG),            # router weight
        (ok[:7] + (350,) + ok[8:], B.MOE_ERR_UNSUPPORTED),             # E % 4
        (ok[:8] + (17,) + ok[9:], B.MOE_ERR_INVALID_ARG),              # K > 16
        (ok[:10] + (None,) + ok[11:], B.MOE_ERR_INVALID_ARG),          # a_out
        (ok[:13] + (None,) + ok[14:], B.MOE_ERR_INVALID_ARG),          # ws
        (ok[:14] + (8 * 8 * 352 * 4 - 4,) + ok[15:], B.MOE_ERR_WORKSPACE_TOO_SMALL),
        (ok[:10] + (ctypes.c_void_p(FAKE + 8),) + ok[11:], B.MOE_ERR_INVALID_ARG),  # alignment
    ]
    for args, want in bad:
        assert F(*args) == want, args
    assert F(*(ok[:3] + (0,) + ok[4:])) == B.MOE_OK                   # T == 0: a no-op


def test_csf_row_index_validation(L):
    """Argument errors of moe_csf_row_index are found before any launch."""
    F = L.moe_csf_row_index
    p = ctypes.c_void_p(FAKE)
    ok = (p, 4, p, 2, 32, 16, None, 0, p, None)
    bad = [
        ((None,) + ok[1:], B.MOE_ERR_INVALID_ARG),                     # exceptions with n > 0
        (ok[:1] + (-1,) + ok[2:], B.MOE_ERR_INVALID_ARG),              # n < 0
        (ok[:2] + (None,) + ok[3:], B.MOE_ERR_INVALID_ARG),            # starts
        (ok[:3] + (0,) + ok[4:], B.MOE_ERR_INVALID_ARG),               # E
        (ok[:4] + (24,) + ok[5:], B.MOE_ERR_INVALID_ARG),              # R % 16
        (ok[:5] + (8,) + ok[6:], B.MOE_ERR_INVALID_ARG),               # C % 16
        (ok[:4] + (4096, 4096) + ok[6:], B.MOE_ERR_UNSUPPORTED),       # R*C >= 2^24
        (ok[:7] + (-1,) + ok[8:], B.MOE_ERR_INVALID_ARG),              # max_routed_experts
        (ok[:8] + (None,) + ok[9:], B.MOE_ERR_INVALID_ARG),            # row_index
        (ok[:8] + (ctypes.c_void_p(FAKE + 2),) + ok[9:], B.MOE_ERR_INVALID_ARG),  # alignment
    ]
    for args, want in bad:
        assert F(*args) == want, args


def _bank_csf(E, n, k, fstride=None, ri=True, gs=True):
    """A MOE_W_NVFP4_CSF bank descriptor (fake pointers; code rows padded to
    16 bytes)."""
    fs = fstride if fstride is not None else n * (1 + k // 32)
    qr = (k // 2 + 15) // 16 * 16
    return B.WeightDesc(B.MOE_W_NVFP4_CSF, E, n, k, FAKE, FAKE, FAKE if gs else None,
                        n * qr, qr, fs, 0, None, 0, 0, FAKE, FAKE if ri else None)


def test_nvfp4_csf_banks_plan_kernels_and_errors(L):
    """Decode sizes read the compressed scales in place (GEMV tile); prefill
    sizes expand them into the workspace for the grouped GEMM (its tile,
    and room for every expert's expanded scales); a fixed tensor whose
    experts are not 8 bytes apart cannot be expanded with 8-byte reads and
    keeps the GEMV."""
    f = B.FfnDesc(_bank_csf(352, 1536, 4096), _bank_csf(352, 1536, 4096),
                  _bank_csf(352, 4096, 1536))
    st, tm_small, _ = _plan(f, T=8, act=B.MOE_BF16)
    assert st == B.MOE_OK
    st, tm_big, ws_big = _plan(f, T=2048, act=B.MOE_BF16)
    st_g, tm_g128, _ = _plan(_ffn(), T=2048)
    assert st == B.MOE_OK and tm_big == tm_g128 != tm_small
    assert ws_big >= 352 * (2 * 1536 * 256 + 4096 * 96)
    odd = 1536 * (1 + 4096 // 32) + 4
    f = B.FfnDesc(_bank_csf(352, 1536, 4096, fstride=odd), _bank_csf(352, 1536, 4096),
                  _bank_csf(352, 4096, 1536))
    st, tm_odd, _ = _plan(f, T=2048, act=B.MOE_BF16)
    assert st == B.MOE_OK and tm_odd == tm_small
    for g in (_bank_csf(352, 1536, 4096, ri=False),         # no row index
              _bank_csf(352, 1536, 4096, gs=False),         # no global scale
              _bank_csf(352, 1536, 4096, fstride=1536 * 100),   # fixed tensor too small
              _bank_csf(352, 1528, 4096)):                  # rows not in 16-row slabs
        f = B.FfnDesc(g, _bank_csf(352, 1536, 4096), _bank_csf(352, 4096, 1536))
        assert _plan(f, act=B.MOE_BF16)[0] == B.MOE_ERR_INVALID_ARG, g.n
    f = B.FfnDesc(_bank_csf(4, 64, 48), _bank_csf(4, 64, 48), _bank_csf(4, 48, 64))
    assert _plan(f, act=B.MOE_BF16)[0] == B.MOE_ERR_UNSUPPORTED   # k % 32


def _bank_v(fmt, E, n, k, srow=None, zrow=None, zp=True, qrow=None):
    """An int4-g32, asymmetric int4-g128 or int8-g128 bank descriptor (fake
    pointers)."""
    g = 32 if fmt == B.MOE_W_INT4_G32 else 128
    qr = qrow if qrow is not None else (k if fmt == B.MOE_W_INT8_G128 else k // 2)
    sr = srow if srow is not None else (k // g) * 2
    zr = zrow if zrow is not None else k // 128
    z = FAKE if (fmt == B.MOE_W_INT4_G128_ASYM and zp) else None
    return B.WeightDesc(fmt, E, n, k, FAKE, FAKE, None, qr * n, qr, sr * n, sr,
                        z, zr * n if z else 0, zr if z else 0)


@pytest.mark.parametrize("fmt", [B.MOE_W_INT4_G32, B.MOE_W_INT4_G128_ASYM, B.MOE_W_INT8_G128])
def test_variant_banks_plan_kernels(L, fmt):
    """The variants are accepted, planned on the GEMV tile at decode size and
    on the grouped GEMM's tile at prefill size, like int4-g128."""
    f = B.FfnDesc(_bank_v(fmt, 352, 1536, 4096), _bank_v(fmt, 352, 1536, 4096),
                  _bank_v(fmt, 352, 4096, 1536))
    st, tm_small, _ = _plan(f, T=8)
    assert st == B.MOE_OK
    st, tm_big, _ = _plan(f, T=2048)
    assert st == B.MOE_OK
    st, tm_g128, _ = _plan(_ffn(), T=2048)
    assert tm_g128 != tm_small
    assert tm_big == tm_g128


def test_asym_bank_with_odd_zero_point_stride_plans_the_gemv(L):
    """The GEMM loads a step's two zero points as one 2-byte word; a bank
    whose zero-point rows are an odd number of bytes apart runs the GEMV at
    every size."""
    A = B.MOE_W_INT4_G128_ASYM
    f = B.FfnDesc(_bank_v(A, 352, 1536, 4096, zrow=33), _bank_v(A, 352, 1536, 4096, zrow=33),
                  _bank_v(A, 352, 4096, 1536, zrow=13))
    st, tm_small, _ = _plan(f, T=8)
    assert st == B.MOE_OK
    st, tm_big, _ = _plan(f, T=2048)
    assert st == B.MOE_OK and tm_big == tm_small


def test_g32_bank_with_unaligned_scale_rows_plans_the_gemv(L):
    """The GEMM loads a step's eight int4-g32 scales as one 16-byte word; a
    bank whose scale rows are not a multiple of 16 bytes apart runs the GEMV
    at every size."""
    G = B.MOE_W_INT4_G32
    f = B.FfnDesc(_bank_v(G, 352, 1536, 4096, srow=264), _bank_v(G, 352, 1536, 4096, srow=264),
                  _bank_v(G, 352, 4096, 1536, srow=104))
    st, tm_small, _ = _plan(f, T=8)
    assert st == B.MOE_OK
    st, tm_big, _ = _plan(f, T=2048)
    assert st == B.MOE_OK and tm_big == tm_small


def test_int4_variant_bank_errors(L):
    G32, ASYM = B.MOE_W_INT4_G32, B.MOE_W_INT4_G128_ASYM
    bad = [
        _bank_v(ASYM, 352, 1536, 4096, zp=False),            # no zero points
        _bank_v(ASYM, 352, 1536, 4096, zrow=31),             # zero-point rows too short
        _bank_v(G32, 352, 1536, 4096, srow=(4096 // 128) * 2),   # g128-sized scale rows
        _bank_v(B.MOE_W_INT8_G128, 352, 1536, 4096, qrow=2048),  # int4-sized weight rows
        _bank_v(B.MOE_W_INT8_G128, 352, 1536, 4096, srow=62),     # scale rows too short
    ]
    for g in bad:
        f = B.FfnDesc(g, _bank_v(g.fmt, 352, 1536, 4096), _bank_v(g.fmt, 352, 4096, 1536))
        assert _plan(f)[0] == B.MOE_ERR_INVALID_ARG
    # g32 needs k % 32; the variant formats mixed with another format are refused
    f = B.FfnDesc(_bank_v(G32, 4, 64, 48), _bank_v(G32, 4, 64, 48), _bank_v(G32, 4, 48, 64))
    assert _plan(f)[0] == B.MOE_ERR_INVALID_ARG
    I8 = B.MOE_W_INT8_G128        # int8 groups are 128 inputs: k % 128
    f = B.FfnDesc(_bank_v(I8, 4, 64, 192), _bank_v(I8, 4, 64, 192), _bank_v(I8, 4, 192, 64))
    assert _plan(f)[0] == B.MOE_ERR_INVALID_ARG
    f = B.FfnDesc(_bank_v(G32, 352, 1536, 4096), _bank(B.MOE_W_INT4_G128, 352, 1536, 4096),
                  _bank_v(G32, 352, 4096, 1536))
    assert _plan(f)[0] == B.MOE_ERR_INVALID_ARG


def test_input_scale_rules(L):
    """Quantized inputs: NVFP4 banks only, gate and up with one input scale,
    the down projection quantized too; scales 0 or in [2^-100, 2^100]; the
    plan holds the quantized x."""
    f = _ffn(B.MOE_W_NVFP4_G16)
    st, tm, ws0 = _plan(f, T=8, act=B.MOE_BF16)
    assert st == B.MOE_OK
    for b in (f.gate, f.up, f.down):
        b.input_scale = 0.01
    st, tm, ws1 = _plan(f, T=8, act=B.MOE_BF16)
    assert st == B.MOE_OK and ws1 >= ws0 + 8 * 4096 * 2
    f.up.input_scale = 0.02                                   # gate and up differ
    assert _plan(f, T=8, act=B.MOE_BF16)[0] == B.MOE_ERR_INVALID_ARG
    f.up.input_scale = 0.01
    f.down.input_scale = 0.0                                  # h left unquantized
    assert _plan(f, T=8, act=B.MOE_BF16)[0] == B.MOE_ERR_INVALID_ARG
    for bad in (-1.0, 2.0 ** -101, 2.0 ** 101, float("inf"), float("nan")):
        for b in (f.gate, f.up, f.down):
            b.input_scale = bad
        assert _plan(f, T=8, act=B.MOE_BF16)[0] == B.MOE_ERR_INVALID_ARG, bad
    g = _ffn(B.MOE_W_INT4_G128)                               # not an NVFP4 bank
    for b in (g.gate, g.up, g.down):
        b.input_scale = 0.01
    assert _plan(g, T=8)[0] == B.MOE_ERR_INVALID_ARG


def test_quantize_nvfp4_act_validation(L):
    Q = L.moe_quantize_nvfp4_act
    x = ctypes.c_void_p(FAKE)
    assert Q(x, B.MOE_BF16, 4, 24, 0.1, x, None) == B.MOE_ERR_INVALID_ARG     # k % 16
    assert Q(x, B.MOE_BF16, 4, 32, 0.0, x, None) == B.MOE_ERR_INVALID_ARG     # scale 0
    assert Q(x, B.MOE_BF16, 4, 32, 2.0 ** 101, x, None) == B.MOE_ERR_INVALID_ARG
    assert Q(x, B.MOE_F32, 4, 32, 0.1, x, None) == B.MOE_ERR_INVALID_ARG      # dtype
    assert Q(ctypes.c_void_p(FAKE + 8), B.MOE_BF16, 4, 32, 0.1, x, None) == B.MOE_ERR_INVALID_ARG
    assert Q(None, B.MOE_BF16, 0, 32, 0.1, None, None) == B.MOE_OK            # no-op
