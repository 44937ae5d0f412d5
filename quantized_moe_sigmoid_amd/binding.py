"""Thin Python binding of libmoe_w4a16.so (ctypes).

Argument marshalling only: torch supplies device memory and the current
stream; every step of the layer runs in the library's HIP kernels. The
function names are the C entry points' names. If the library is missing
the calls raise: there is no fallback.
"""
import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_w4a16.so")
_lib = None

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE_TOO_SMALL, MOE_ERR_HIP = range(5)
MOE_F16, MOE_BF16, MOE_F32 = 1, 2, 3
MOE_W_INT4_G128, MOE_W_NVFP4_G16, MOE_W_BF16, MOE_W_INT4_G32, MOE_W_INT4_G128_ASYM = 1, 2, 3, 4, 5
MOE_W_INT8_G128, MOE_W_NVFP4_CSF = 6, 7

EXPORTS = ("moe_status_string", "moe_abi_version", "moe_router_logits", "moe_route_workspace",
           "moe_route_topk", "moe_route_permute", "moe_permute_sizes",
           "moe_permute", "moe_forward_plan", "moe_w4a16_forward", "moe_w4a16_forward_profiled",
           "moe_round_activations", "moe_rmsnorm", "moe_dequant", "moe_csf_expand",
           "moe_csf_row_index", "moe_norm_route", "moe_w4a16_forward_scratch",
           "moe_quantize_nvfp4_act")
MOE_FORWARD_STAGES = 4
MOE_FORWARD_SCRATCH_BYTES = 64 << 20

_DT = {torch.float16: MOE_F16, torch.bfloat16: MOE_BF16, torch.float32: MOE_F32}
_TD = {v: k for k, v in _DT.items()}


class MoeError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s: %s" % (where, status_string(status)))


class WeightDesc(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("n", ctypes.c_int32), ("k", ctypes.c_int32),
                ("qweight", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("global_scale", ctypes.c_void_p),
                ("qweight_expert_stride", ctypes.c_int64), ("qweight_row_stride", ctypes.c_int64),
                ("scale_expert_stride", ctypes.c_int64), ("scale_row_stride", ctypes.c_int64),
                ("zero_point", ctypes.c_void_p),
                ("zero_point_expert_stride", ctypes.c_int64), ("zero_point_row_stride", ctypes.c_int64),
                ("csf_exceptions", ctypes.c_void_p), ("csf_row_index", ctypes.c_void_p),
                ("input_scale", ctypes.c_float)]


class FfnDesc(ctypes.Structure):
    _fields_ = [("gate", WeightDesc), ("up", WeightDesc), ("down", WeightDesc)]


class PermDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("counts", "expert_offsets", "padded_offsets", "sorted_slots", "slot_to_row",
                 "tile_expert", "num_tiles", "active_experts", "num_active")] + \
               [("tile_m", ctypes.c_int32)]


def library_path():
    return _LIB_PATH


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("libmoe_w4a16.so is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
        P = ctypes.POINTER
        L.moe_status_string.argtypes = [i32]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_abi_version.restype = i32
        L.moe_router_logits.argtypes = [vp, i32, vp, vp, i32, i32, i32, vp, vp]
        L.moe_route_workspace.argtypes = [i32, i32, i32, P(sz)]
        L.moe_route_topk.argtypes = [vp, i32, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, sz,
                                     vp]
        L.moe_permute_sizes.argtypes = [i32, i32, i32, i32, P(i64), P(i64)]
        L.moe_permute.argtypes = [vp, i32, i32, i32, P(PermDesc), vp]
        L.moe_route_permute.argtypes = [vp, i32, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp,
                                        P(PermDesc), vp, sz, vp]
        L.moe_forward_plan.argtypes = [P(FfnDesc), P(FfnDesc), i32, i32, i32, P(i32), P(sz)]
        L.moe_w4a16_forward.argtypes = [P(FfnDesc), P(FfnDesc), vp, i32, i32, i32, vp,
                                        P(PermDesc), vp, vp, i32, vp, sz, vp]
        L.moe_w4a16_forward_profiled.argtypes = L.moe_w4a16_forward.argtypes + [P(vp), i32]
        L.moe_w4a16_forward_scratch.argtypes = [P(FfnDesc), P(FfnDesc), vp, i32, i32, i32, vp,
                                                P(PermDesc), vp, vp, i32, vp]
        L.moe_quantize_nvfp4_act.argtypes = [vp, i32, i64, i32, ctypes.c_float, vp, vp]
        L.moe_round_activations.argtypes = [vp, i64, i32, vp, vp]
        L.moe_rmsnorm.argtypes = [vp, vp, ctypes.c_float, i32, i32, i32, vp, vp]
        L.moe_dequant.argtypes = [P(WeightDesc), i32, vp, vp]
        L.moe_csf_expand.argtypes = [vp, vp, i64, vp, i32, i32, i32, vp, i32, vp, vp]
        L.moe_csf_row_index.argtypes = [vp, i64, vp, i32, i32, i32, vp, i32, vp, vp]
        L.moe_norm_route.argtypes = [vp, vp, ctypes.c_float, i32, i32, vp, vp, i32, i32, i32, vp,
                                     vp, vp, vp, ctypes.c_size_t, vp]
        for name in ("moe_router_logits", "moe_route_workspace", "moe_route_topk",
                     "moe_route_permute",
                     "moe_permute_sizes", "moe_permute", "moe_forward_plan",
                     "moe_w4a16_forward", "moe_w4a16_forward_profiled",
                     "moe_round_activations", "moe_rmsnorm", "moe_dequant",
                     "moe_csf_expand", "moe_csf_row_index", "moe_norm_route",
                     "moe_w4a16_forward_scratch", "moe_quantize_nvfp4_act"):
            getattr(L, name).restype = i32
        _lib = L
    return _lib


def status_string(st):
    return lib().moe_status_string(int(st)).decode()


def _check(st, where):
    if st != MOE_OK:
        raise MoeError(st, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device=None):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


# ------------------------------------------------------------ descriptors ---
def bank_int4(qweight, scale, zero_point=None):
    """qweight int32 [E, n, k/8], scale bf16 [E, n, k/G] (device). G = 128 is
    MOE_W_INT4_G128, G = 32 MOE_W_INT4_G32; with zero_point (uint8 [E, n,
    k/128]) the nibbles are unsigned: MOE_W_INT4_G128_ASYM."""
    E, n, kw = qweight.shape
    k = kw * 8
    groups = scale.shape[2]
    if zero_point is not None:
        assert groups * 128 == k and zero_point.shape == (E, n, k // 128)
        fmt = MOE_W_INT4_G128_ASYM
    else:
        assert groups * 128 == k or groups * 32 == k
        fmt = MOE_W_INT4_G128 if groups * 128 == k else MOE_W_INT4_G32
    zp = zero_point.data_ptr() if zero_point is not None else None
    zs = (zero_point.stride(0), zero_point.stride(1)) if zero_point is not None else (0, 0)
    d = WeightDesc(fmt, E, n, k, qweight.data_ptr(), scale.data_ptr(), None,
                   qweight.stride(0) * 4, qweight.stride(1) * 4,
                   scale.stride(0) * 2, scale.stride(1) * 2, zp, zs[0], zs[1])
    d._keep = (qweight, scale, zero_point)
    return d


def bank_int8(qweight, scale):
    """qweight int8 [E, n, k], scale bf16 [E, n, k/128] (device): MOE_W_INT8_G128."""
    E, n, k = qweight.shape
    assert qweight.dtype == torch.int8 and scale.shape == (E, n, k // 128)
    d = WeightDesc(MOE_W_INT8_G128, E, n, k, qweight.data_ptr(), scale.data_ptr(), None,
                   qweight.stride(0), qweight.stride(1), scale.stride(0) * 2, scale.stride(1) * 2)
    d._keep = (qweight, scale)
    return d


def bank_nvfp4(qweight, scale, global_scale, input_scale=0.0):
    """qweight uint8 [E, n, k/2], scale uint8 (E4M3) [E, n, k/16], global_scale
    float [E]; input_scale > 0 quantizes the bank's inputs (NVFP4)."""
    E, n, kh = qweight.shape
    d = WeightDesc(MOE_W_NVFP4_G16, E, n, kh * 2, qweight.data_ptr(), scale.data_ptr(),
                   global_scale.data_ptr(), qweight.stride(0), qweight.stride(1),
                   scale.stride(0), scale.stride(1))
    d.input_scale = float(input_scale)
    d._keep = (qweight, scale, global_scale)
    return d


def bank_nvfp4_csf(qweight, fixed, exceptions, row_index, global_scale, input_scale=0.0):
    """MOE_W_NVFP4_CSF: qweight uint8 [E, n, k/2], the CSF fixed tensor uint8
    [E, n/16, 16*(1+k/32)], exceptions int32/uint32 [m] (or None), the row
    index int32 [E, n+1] from moe_csf_row_index, global_scale float [E]."""
    E, n, kh = qweight.shape
    m = exceptions.numel() if exceptions is not None else 0
    d = WeightDesc(MOE_W_NVFP4_CSF, E, n, kh * 2, qweight.data_ptr(), fixed.data_ptr(),
                   global_scale.data_ptr(), qweight.stride(0), qweight.stride(1),
                   fixed.stride(0), 0, None, 0, 0,
                   exceptions.data_ptr() if m else None, row_index.data_ptr())
    d.input_scale = float(input_scale)
    d._keep = (qweight, fixed, exceptions, row_index, global_scale)
    return d


def bank_bf16(weight):
    """weight bf16 [n, k] or [E, n, k] (device), rows contiguous."""
    w = weight if weight.dim() == 3 else weight.unsqueeze(0)
    E, n, k = w.shape
    d = WeightDesc(MOE_W_BF16, E, n, k, w.data_ptr(), None, None,
                   w.stride(0) * 2, w.stride(1) * 2, 0, 0)
    d._keep = (w,)
    return d


def ffn(gate, up, down):
    f = FfnDesc(gate, up, down)
    f._keep = (gate, up, down)
    return f


# ----------------------------------------------------------------- calls ---
def moe_router_logits(x, router_wT, bias=None, out=None):
    """Canonical float32 router logits [T, E]."""
    T, H = x.shape
    E = router_wT.shape[1]
    if out is None:
        out = torch.empty((T, E), dtype=torch.float32, device=x.device)
    _check(lib().moe_router_logits(_ptr(x), _DT[x.dtype], _ptr(router_wT), _ptr(bias), T, H, E,
                                   _ptr(out), _stream(x.device)), "moe_router_logits")
    return out


def moe_route_workspace(T, E, use_router_weight):
    b = ctypes.c_size_t()
    _check(lib().moe_route_workspace(T, E, int(bool(use_router_weight)), ctypes.byref(b)),
           "moe_route_workspace")
    return b.value


def moe_route_topk(K, x=None, router_wT=None, logits=None, bias=None, renormalize=True,
                   ids=None, w=None, ws=None):
    """Returns (topk_ids int32 [T, K], topk_w float32 [T, K])."""
    src = logits if logits is not None else x
    T = src.shape[0]
    E = logits.shape[1] if logits is not None else router_wT.shape[1]
    H = x.shape[1] if x is not None else 0
    dev = src.device
    if ids is None:
        ids = torch.empty((T, K), dtype=torch.int32, device=dev)
    if w is None:
        w = torch.empty((T, K), dtype=torch.float32, device=dev)
    need = moe_route_workspace(T, E, router_wT is not None)
    if need and (ws is None or ws.numel() < need):
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    xd = _DT.get(x.dtype, 0) if x is not None else 0
    st = lib().moe_route_topk(_ptr(x), xd, _ptr(router_wT), _ptr(logits), _ptr(bias), T, H, E,
                              K, int(bool(renormalize)), _ptr(ids), _ptr(w),
                              _ptr(ws) if need else None, need, _stream(dev))
    _check(st, "moe_route_topk")
    return ids, w


def moe_permute_sizes(T, K, E, tile_m):
    mr, mt = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().moe_permute_sizes(T, K, E, tile_m, ctypes.byref(mr), ctypes.byref(mt)),
           "moe_permute_sizes")
    return mr.value, mt.value


class Perm:
    """Device arrays of one permutation (see moe_perm_t)."""

    FIELDS = ("counts", "expert_offsets", "padded_offsets", "sorted_slots", "slot_to_row",
              "tile_expert", "num_tiles", "active_experts", "num_active")

    def __init__(self, T, K, E, tile_m, device):
        mr, mt = moe_permute_sizes(T, K, E, tile_m)
        i32 = dict(dtype=torch.int32, device=device)
        self.tile_m, self.E = tile_m, E
        self.counts = torch.zeros(E, **i32)
        self.expert_offsets = torch.zeros(E + 1, **i32)
        self.padded_offsets = torch.zeros(E + 1, **i32)
        self.sorted_slots = torch.full((max(mr, 1),), -2, **i32)
        self.slot_to_row = torch.zeros(max(T * K, 1), **i32)
        self.tile_expert = torch.full((max(mt, 1),), -2, **i32)
        self.num_tiles = torch.zeros(1, **i32)
        self.active_experts = torch.full((E,), -2, **i32)
        self.num_active = torch.zeros(1, **i32)

    def desc(self):
        d = PermDesc(*[getattr(self, f).data_ptr() for f in self.FIELDS], self.tile_m)
        return d


def moe_permute(topk_ids, E, tile_m, perm=None):
    T, K = topk_ids.shape
    if perm is None:
        perm = Perm(T, K, E, tile_m, topk_ids.device)
    d = perm.desc()
    _check(lib().moe_permute(_ptr(topk_ids), T, K, E, ctypes.byref(d), _stream(topk_ids.device)),
           "moe_permute")
    return perm


def moe_route_permute(K, perm, x=None, router_wT=None, logits=None, bias=None, renormalize=True,
                      ids=None, w=None, ws=None):
    """moe_route_topk then moe_permute into perm (a Perm of the batch's
    T, K, E and tile_m), in one call. Returns (topk_ids, topk_w)."""
    src = logits if logits is not None else x
    T = src.shape[0]
    E = logits.shape[1] if logits is not None else router_wT.shape[1]
    H = x.shape[1] if x is not None else 0
    dev = src.device
    if ids is None:
        ids = torch.empty((T, K), dtype=torch.int32, device=dev)
    if w is None:
        w = torch.empty((T, K), dtype=torch.float32, device=dev)
    need = moe_route_workspace(T, E, router_wT is not None)
    if need and (ws is None or ws.numel() < need):
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    xd = _DT.get(x.dtype, 0) if x is not None else 0
    d = perm.desc()
    st = lib().moe_route_permute(_ptr(x), xd, _ptr(router_wT), _ptr(logits), _ptr(bias), T, H, E,
                                 K, int(bool(renormalize)), _ptr(ids), _ptr(w), ctypes.byref(d),
                                 _ptr(ws) if need else None, need, _stream(dev))
    _check(st, "moe_route_permute")
    return ids, w


def moe_forward_plan(experts, T, K, act_dtype, shared=None):
    tm, ws = ctypes.c_int(), ctypes.c_size_t()
    st = lib().moe_forward_plan(ctypes.byref(experts),
                                ctypes.byref(shared) if shared is not None else None,
                                T, K, _DT[act_dtype], ctypes.byref(tm), ctypes.byref(ws))
    _check(st, "moe_forward_plan")
    return tm.value, ws.value


def moe_w4a16_forward(experts, x, topk_w, perm, residual=None, out_dtype=torch.float32,
                      shared=None, out=None, ws=None, events=None):
    """events: None, or a sequence of MOE_FORWARD_STAGES + 1 hipEvent_t
    handles (ints, or None for a boundary that records nothing) recorded at
    the stage boundaries (the profiled entry)."""
    T, H = x.shape
    K = topk_w.shape[1]
    dev = x.device
    _, need = moe_forward_plan(experts, T, K, x.dtype, shared)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=dev)
    pd = perm.desc()
    args = [ctypes.byref(experts), ctypes.byref(shared) if shared is not None else None, _ptr(x),
            _DT[x.dtype], T, K, _ptr(topk_w), ctypes.byref(pd), _ptr(residual), _ptr(out),
            _DT[out.dtype], _ptr(ws), ws.numel(), _stream(dev)]
    if events is None:
        _check(lib().moe_w4a16_forward(*args), "moe_w4a16_forward")
    else:
        arr = (ctypes.c_void_p * len(events))(*events)
        _check(lib().moe_w4a16_forward_profiled(*args, arr, len(events)),
               "moe_w4a16_forward_profiled")
    return out


def moe_w4a16_forward_scratch(experts, x, topk_w, perm, residual=None, out_dtype=torch.float32,
                              shared=None, out=None):
    """moe_w4a16_forward on the library's own device buffer (no workspace
    argument; the library allocates nothing). `out` is allocated here by
    torch unless given."""
    T, H = x.shape
    K = topk_w.shape[1]
    dev = x.device
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=dev)
    pd = perm.desc()
    _check(lib().moe_w4a16_forward_scratch(
        ctypes.byref(experts), ctypes.byref(shared) if shared is not None else None, _ptr(x),
        _DT[x.dtype], T, K, _ptr(topk_w), ctypes.byref(pd), _ptr(residual), _ptr(out),
        _DT[out.dtype], _stream(dev)), "moe_w4a16_forward_scratch")
    return out


def moe_quantize_nvfp4_act(x, input_scale, out=None):
    """x [rows, k] float16 / bfloat16 -> e2m1 x bs values [rows, k], same dtype
    (the quantized activation is that times input_scale)."""
    rows, k = x.shape
    if out is None:
        out = torch.empty_like(x)
    _check(lib().moe_quantize_nvfp4_act(_ptr(x), _DT[x.dtype], rows, k, float(input_scale),
                                        _ptr(out), _stream(x.device)), "moe_quantize_nvfp4_act")
    return out


def moe_round_activations(x, dtype=torch.bfloat16, out=None):
    """float32 tensor -> `dtype` (float16 / bfloat16), round to nearest even."""
    if out is None:
        out = torch.empty(x.shape, dtype=dtype, device=x.device)
    _check(lib().moe_round_activations(_ptr(x), x.numel(), _DT[out.dtype], _ptr(out),
                                       _stream(x.device)), "moe_round_activations")
    return out


def moe_rmsnorm(x, weight=None, eps=1e-5, dtype=torch.bfloat16, out=None):
    """float32 [T, H] -> x / sqrt(mean(x^2) + eps) * (1 + weight) in `dtype`."""
    T, H = x.shape
    if out is None:
        out = torch.empty((T, H), dtype=dtype, device=x.device)
    _check(lib().moe_rmsnorm(_ptr(x), _ptr(weight), float(eps), T, H, _DT[out.dtype], _ptr(out),
                             _stream(x.device)), "moe_rmsnorm")
    return out


def moe_norm_route(residual, router_wT, K, norm_w=None, eps=1e-5, bias=None, renormalize=True,
                   a=None, ids=None, w=None, ws=None):
    """Fused RMSNorm + bf16 cast + router + top-K of a float32 residual [T, H]:
    returns (a bf16 [T, H], ids int32 [T, K], weights float [T, K])."""
    T, H = residual.shape
    E = router_wT.shape[1]
    dev = residual.device
    if a is None:
        a = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    if ids is None:
        ids = torch.empty((T, K), dtype=torch.int32, device=dev)
    if w is None:
        w = torch.empty((T, K), dtype=torch.float32, device=dev)
    if ws is None:
        ws = torch.empty(max(moe_route_workspace(T, E, True), 16), dtype=torch.uint8, device=dev)
    _check(lib().moe_norm_route(_ptr(residual), _ptr(norm_w), float(eps), T, H, _ptr(router_wT),
                                _ptr(bias), E, K, 1 if renormalize else 0, _ptr(a), _ptr(ids),
                                _ptr(w), _ptr(ws), ws.numel(), _stream(dev)),
           "moe_norm_route")
    return a, ids, w


def moe_dequant(desc, expert, out=None, device=None):
    if out is None:
        out = torch.empty((desc.n, desc.k), dtype=torch.float32, device=device or "cuda")
    _check(lib().moe_dequant(ctypes.byref(desc), expert, _ptr(out), _stream(out.device)),
           "moe_dequant")
    return out


def moe_csf_row_index(exceptions, starts, R, C, out=None, expert_offsets=None, max_routed=0):
    """Per-row exception ranges int32 [E, R+1] of a CSF scale tensor (see
    moe_csf_expand for the arguments)."""
    E = starts.numel() - 1
    if out is None:
        out = torch.zeros((E, R + 1), dtype=torch.int32, device=starts.device)
    n = exceptions.numel() if exceptions is not None else 0
    _check(lib().moe_csf_row_index(_ptr(exceptions) if n else None, n, _ptr(starts), E, R, C,
                                   _ptr(expert_offsets), int(max_routed), _ptr(out),
                                   _stream(out.device)),
           "moe_csf_row_index")
    return out


def moe_csf_expand(fixed, exceptions, starts, R, C, out=None, expert_offsets=None,
                   max_routed=0):
    """NVFP4 block-scale bytes [E][R][C] (uint8) from the CSF tensors: fixed
    uint8 [E][R/16][16*(1+C/2)], exceptions int32/uint32 [n], starts int64
    [E+1]; expert_offsets (int32 [E+1], the permute output) limits the
    expansion to routed experts, max_routed (e.g. min(E, T*K)) bounds their
    number so the grid covers only them."""
    E = fixed.shape[0]
    if out is None:
        out = torch.empty((E, R, C), dtype=torch.uint8, device=fixed.device)
    n = exceptions.numel() if exceptions is not None else 0
    _check(lib().moe_csf_expand(_ptr(fixed), _ptr(exceptions) if n else None, n, _ptr(starts), E,
                                R, C, _ptr(expert_offsets), int(max_routed), _ptr(out),
                                _stream(out.device)),
           "moe_csf_expand")
    return out
