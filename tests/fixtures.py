"""Shared helpers of the test suite: seeded inputs quantized by the oracle,
conversion to device tensors, oracle references and the tolerance rule."""
import numpy as np
import torch

from oracle import formats as OF
from oracle import layer as OL
from oracle import quant as OQ
from quantized_moe_sigmoid_amd import binding as B
from quantized_moe_sigmoid_amd import synth

TENSOR_OF = {"gate": synth.T_GATE, "up": synth.T_UP, "down": synth.T_DOWN}


def int4_bank_oracle(E, n, k, root, layer, which):
    """Gaussian bf16 weights quantized by the oracle's clip search and packed.
    Returns (words int32 [E, n, k/8], scale bits uint16 [E, n, k/128])."""
    q = np.empty((E, n, k // 8), dtype=np.int32)
    s = np.empty((E, n, k // 128), dtype=np.uint16)
    for e in range(E):
        W = synth.expert_weight_bf16(n, k, root, layer, TENSOR_OF[which], e)
        qq, ss = OQ.quantize_int4(W.float().numpy().astype(np.float64))
        q[e] = OQ.pack_int4(qq)
        s[e] = OF.bf16_bits(ss)
    return q, s


def nvfp4_bank_oracle(E, n, k, root, layer, which):
    """Gaussian bf16 weights quantized by the oracle's NVFP4 rule and packed.
    Returns (bytes uint8 [E, n, k/2], E4M3 bytes uint8 [E, n, k/16], gs float32 [E])."""
    q = np.empty((E, n, k // 2), dtype=np.uint8)
    s = np.empty((E, n, k // 16), dtype=np.uint8)
    gs = np.empty((E,), dtype=np.float32)
    for e in range(E):
        W = synth.expert_weight_bf16(n, k, root, layer, TENSOR_OF[which], e)
        codes, bs, g = OQ.quantize_nvfp4(W.float().numpy().astype(np.float64))
        q[e] = OQ.pack_nvfp4(codes)
        s[e] = OQ.e4m3_bytes(bs)
        gs[e] = g
    return q, s, gs


def int4_to_device(q, s_bits, device="cuda"):
    qt = torch.from_numpy(np.ascontiguousarray(q)).to(device)
    st = torch.from_numpy(np.ascontiguousarray(s_bits).view(np.int16)).view(torch.bfloat16).to(device)
    return qt, st


def int4_from_device(qt, st):
    q = qt.cpu().numpy()
    s = st.view(torch.int16).cpu().numpy().view(np.uint16)
    return q, s


def oracle_int4_expert(q, s, e):
    return OQ.dequant_int4(q[e], s[e])


def oracle_nvfp4_expert(q, s, gs, e):
    return OQ.dequant_nvfp4(q[e], s[e], float(gs[e]))


def within_tolerance(gpu, ref, rel=1e-2):
    """|gpu - ref| <= rel * (|ref| + rms(ref)) elementwise, rms over the whole
    output. Returns (ok, worst ratio)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    bound = rel * (np.abs(ref) + rms)
    err = np.abs(gpu - ref)
    ratio = float(np.max(err / np.maximum(bound, 1e-300))) if ref.size else 0.0
    return bool(np.all(err <= bound)), ratio


def oracle_layer(x16, ids, w, experts_fn, shared=None, residual=None):
    x = x16.float().cpu().numpy().astype(np.float64)
    return OL.moe_layer(x, ids, np.asarray(w, dtype=np.float64), experts_fn, shared, residual)


def int4_ffn_random(E_, H_, F_, seed, dev):
    """Random packed int4 gate/up/down banks on `dev` (see
    synth.packed_int4_random); returns (ffn descriptor, device tensors)."""
    banks, host = [], []
    for i, (n, k) in enumerate(((F_, H_), (F_, H_), (H_, F_))):
        qt, st = synth.packed_int4_random(E_, n, k, seed + i, dev)
        banks.append(B.bank_int4(qt, st))
        host.append((qt, st))
    return B.ffn(*banks), host


def experts_fn_int4(host):
    """expert -> float64 (Wg, Wu, Wd) dequantized by the oracle, cached."""
    cache = {}

    def fn(e):
        if e not in cache:
            mats = []
            for (q, s) in host:
                if isinstance(q, torch.Tensor):
                    qq = q[e].cpu().numpy()
                    ss = s[e].view(torch.int16).cpu().numpy().view(np.uint16)
                else:
                    qq, ss = q[e], s[e]
                mats.append(OQ.dequant_int4(qq, ss))
            cache[e] = tuple(mats)
        return cache[e]
    return fn


def shared_bf16(Fs, H, root, layer, dev):
    """The BF16 shared expert: N(0, 0.02) weights rounded to bf16. Returns
    (ffn descriptor on `dev`, float64 (Wg, Wu, Wd) for the oracle)."""
    mats = (synth.expert_weight_bf16(Fs, H, root, layer, synth.T_SH_GATE, 0),
            synth.expert_weight_bf16(Fs, H, root, layer, synth.T_SH_UP, 0),
            synth.expert_weight_bf16(H, Fs, root, layer, synth.T_SH_DOWN, 0))
    desc = B.ffn(*[B.bank_bf16(W.to(dev)) for W in mats])
    return desc, tuple(W.float().numpy().astype(np.float64) for W in mats)


class HipEvents:
    """hipEvent_t handles through the HIP runtime (ctypes), for the profiled
    forward entry point."""

    def __init__(self):
        import ctypes
        self.c = ctypes
        self.L = ctypes.CDLL("libamdhip64.so")
        self.L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.L.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = self.c.c_void_p()
        assert self.L.hipEventCreate(self.c.byref(e)) == 0
        return e.value

    def elapsed_ms(self, a, b):
        ms = self.c.c_float()
        assert self.L.hipEventElapsedTime(self.c.byref(ms), self.c.c_void_p(a),
                                          self.c.c_void_p(b)) == 0
        return ms.value

    def destroy(self, e):
        self.L.hipEventDestroy(self.c.c_void_p(e))


def variant_bank_oracle(E, n, k, root, layer, which, fmt):
    """Gaussian bf16 weights quantized by the oracle as int4-g32, asymmetric
    int4-g128 or int8-g128. Returns (weights: int32 words [E, n, k/8], or
    int8 [E, n, k]; bf16 scale bits uint16 [E, n, k/G]; zero points uint8
    [E, n, k/128] or None)."""
    g = 32 if fmt == B.MOE_W_INT4_G32 else 128
    i8 = fmt == B.MOE_W_INT8_G128
    q = np.empty((E, n, k) if i8 else (E, n, k // 8), dtype=np.int8 if i8 else np.int32)
    s = np.empty((E, n, k // g), dtype=np.uint16)
    z = np.empty((E, n, k // 128), dtype=np.uint8) if fmt == B.MOE_W_INT4_G128_ASYM else None
    for e in range(E):
        W = synth.expert_weight_bf16(n, k, root, layer, TENSOR_OF[which], e)
        W = W.float().numpy().astype(np.float64)
        if i8:
            q[e], ss = OQ.quantize_int8(W)
        elif z is None:
            qq, ss = OQ.quantize_int4(W, group=32)
            q[e] = OQ.pack_int4(qq)
        else:
            qq, ss, zz = OQ.quantize_int4_asym(W)
            q[e] = OQ.pack_uint4(qq)
            z[e] = zz
        s[e] = OF.bf16_bits(ss)
    return q, s, z


def variant_to_device(q, s_bits, z, device="cuda"):
    qt, st = int4_to_device(q, s_bits, device)
    zt = torch.from_numpy(np.ascontiguousarray(z)).to(device) if z is not None else None
    return qt, st, zt


def oracle_variant_expert(q, s_bits, z, e):
    """Exact float64 dequantized expert e of an int4-g32, asymmetric or int8
    bank (host arrays or device tensors; int8 weights mark the int8 bank)."""
    if isinstance(q, torch.Tensor):
        q = q[e].cpu().numpy()
        s_bits = s_bits[e].view(torch.int16).cpu().numpy().view(np.uint16)
        z = z[e].cpu().numpy() if z is not None else None
    else:
        q, s_bits = q[e], s_bits[e]
        z = z[e] if z is not None else None
    if q.dtype == np.int8:
        return OQ.dequant_int8(q, s_bits)
    if z is not None:
        return OQ.dequant_int4_asym(q, s_bits, z)
    return OQ.dequant_int4(q, s_bits, group=32)


# ------------------------------------------------ streamed oracle layer ---
def host_bank(q, s, z=None, gs=None):
    """Host (numpy) copies of a bank's device tensors: codes, scale bits or
    bytes, zero points, global scales (None passes through)."""
    def h(t):
        if t is None or not isinstance(t, torch.Tensor):
            return t
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        return t.cpu().numpy()
    return h(q), h(s), h(z), h(gs)


def dequant_fn(host, fmt="int4"):
    """expert -> float64 (Wg, Wu, Wd) from host banks (see host_bank), no
    cache: each call dequantizes afresh."""
    def fn(e):
        mats = []
        for (q, s, z, gs) in host:
            if fmt == "int4":
                mats.append(OQ.dequant_int4(q[e], s[e]))
            elif fmt == "nvfp4":
                mats.append(OQ.dequant_nvfp4(q[e], s[e], float(gs[e])))
            else:
                raise ValueError(fmt)
        return tuple(mats)
    return fn


def oracle_layer_streamed(x16, ids, w, expert_fn, shared=None, residual=None, threads=16,
                          h_fn=None):
    """The oracle's layer (oracle.layer) on rows x16 [n, H] with routing ids
    [n, K] and weights w [n, K]: every expert the rows reach is dequantized
    once by expert_fn, its slots evaluated and its weights dropped, so the
    memory held stays a few experts'. Experts run on a thread pool (numpy
    releases the GIL in its array operations); h_fn as in oracle.layer.
    Each slot's value depends
    only on its own token and expert, so the order of the experts does not
    change any result."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    x = x16.float().cpu().numpy().astype(np.float64) if isinstance(x16, torch.Tensor) \
        else np.asarray(x16, dtype=np.float64)
    ids = np.asarray(ids)
    T, K = ids.shape
    y = np.zeros((T, K, x.shape[1]))

    def work(e):
        t_idx, k_idx = np.nonzero(ids == e)
        Wg, Wu, Wd = expert_fn(int(e))
        return t_idx, k_idx, OL.swiglu_ffn(x[t_idx], Wg, Wu, Wd, h_fn)

    with threadpool_limits(1), ThreadPoolExecutor(threads) as ex:
        for t_idx, k_idx, out in ex.map(work, np.unique(ids)):
            y[t_idx, k_idx] = out
    sh = OL.swiglu_ffn(x, *shared) if shared is not None else None
    return OL.combine(y, np.asarray(w, dtype=np.float64), sh, residual)


def tile_probe_tokens(ids, E, tile_m, min_tokens=64, max_tokens=96):
    """Tokens whose slots land on chosen rows of the expert-sorted tiles
    (the oracle's permutation): rows 0, 31, 32 and 63 of full tiles and the
    last filled row of partial tiles, over experts with several tiles first,
    then experts with one partial tile; topped up with evenly spaced tokens
    (the first and last included) to at least min_tokens. Sorted, at most
    max_tokens."""
    from oracle import permute as OP
    ids = np.asarray(ids)
    K = ids.shape[1]
    p = OP.permute(ids, E, tile_m)
    counts, po, ss = p["counts"], p["padded_offsets"], p["sorted_slots"]
    order = list(np.argsort(-counts, kind="stable"))
    big = [e for e in order if counts[e] > tile_m][:16]
    small = [e for e in order[::-1] if 0 < counts[e] < tile_m][:16]
    picks = []
    for e in big + small:
        c = int(counts[e])
        for t0 in range(0, c, tile_m):
            for r in (0, 31, 32, 63, min(c - t0, tile_m) - 1):
                if r < tile_m and t0 + r < c:
                    picks.append(int(ss[po[e] + t0 + r]) // K)
    T = ids.shape[0]
    toks = list(dict.fromkeys(picks + [0, T - 1]))[:max_tokens]
    for t in np.linspace(0, T - 1, min_tokens).astype(int):
        if len(toks) >= min_tokens:
            break
        if int(t) not in toks:
            toks.append(int(t))
    return sorted(toks)
