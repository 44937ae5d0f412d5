#!/usr/bin/env python3
"""Throughput of the W4A16 routed-expert MoE layer on one MI355X.

A step is one pass of the whole hot path over one batch: sigmoid top-8
routing, expert histogram + permutation, the int4 (or NVFP4) SwiGLU experts
and the weighted combine, all in the HIP library. Inputs are synthetic,
seeded and resident in HBM before the timed region; weights rotate over
several copies and every step routes a fresh batch of logits, so the 256 MB
Infinity Cache cannot serve a step from the previous one.

Prints one JSON line: tokens/s of the chosen workload, the roofline of its
dominant kernel (algorithmic bytes or FLOPs per launch over the launch's
HIP-event duration, against the MI355X peak), the CPU oracle timed on a
bounded sample, and a sweep over the other layer shapes. Inside the timed
steps HIP events are recorded only around the gate/up kernel (every recorded
event drains the stream); the other stages' durations come from a separate,
untimed pass over the same inputs with every stage boundary recorded.
The default workload, decode T=64, replays its timed steps as one HIP graph
(the way a serving loop launches a decode step); the sweep also times it
with every kernel launched from the host.

  python bench.py [--gpus 1] [--steps K] [--warmup W]
                  [--workload decode|decode-graph|prefill|prefill-zipf|nvfp4|nvfp4-csf|
                              nvfp4-csf-expand|nvfp4-a4|int4-g32|int4-asym|int8|stack]
                  [--tokens T] [--no-sweep] [--no-cpu-baseline]
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

from quantized_moe_sigmoid_amd import binding as B  # noqa: E402
from quantized_moe_sigmoid_amd import synth  # noqa: E402

HBM_PEAK = 8.0e12          # B/s, MI355X HBM3E
MFMA_BF16_PEAK = 2.5e15    # FLOP/s, dense bf16 / fp16
H, F, E, K = 4096, 1536, 352, 8
# Algorithmic bytes of one touched expert (packed weights + scales).
INT4_GATEUP_BYTES = 2 * (F * H // 2 + F * (H // 128) * 2)
INT4_DOWN_BYTES = H * F // 2 + H * (F // 128) * 2
NVFP4_GATEUP_BYTES = 2 * (F * H // 2 + F * (H // 16))
NVFP4_DOWN_BYTES = H * F // 2 + H * (F // 16) + 4
INT4_G32_GATEUP_BYTES = 2 * (F * H // 2 + F * (H // 32) * 2)
INT4_G32_DOWN_BYTES = H * F // 2 + H * (F // 32) * 2
INT4_ASYM_GATEUP_BYTES = 2 * (F * H // 2 + F * (H // 128) * 3)      # + one zero-point byte
INT4_ASYM_DOWN_BYTES = H * F // 2 + H * (F // 128) * 3
# NVFP4 with compressed scales read in place: codes, the CSF fixed bytes
# (a base per row and a 4-bit code per scale) and the global scale
NVFP4_CSF_GATEUP_BYTES = 2 * (F * H // 2 + F * (1 + H // 32))
NVFP4_CSF_DOWN_BYTES = H * F // 2 + H * (1 + F // 32) + 4
INT8_GATEUP_BYTES = 2 * (F * H + F * (H // 128) * 2)
INT8_DOWN_BYTES = H * F + H * (F // 128) * 2
EXPERT_BYTES = {"int4": (INT4_GATEUP_BYTES, INT4_DOWN_BYTES),
                "nvfp4": (NVFP4_GATEUP_BYTES, NVFP4_DOWN_BYTES),
                "int4-g32": (INT4_G32_GATEUP_BYTES, INT4_G32_DOWN_BYTES),
                "int4-asym": (INT4_ASYM_GATEUP_BYTES, INT4_ASYM_DOWN_BYTES),
                "int8": (INT8_GATEUP_BYTES, INT8_DOWN_BYTES),
                "nvfp4-csf": (NVFP4_CSF_GATEUP_BYTES, NVFP4_CSF_DOWN_BYTES),
                "nvfp4-a4": (NVFP4_GATEUP_BYTES, NVFP4_DOWN_BYTES)}
FLOP_PER_SLOT = 3 * 2 * H * F
# Timed steps that record the gate/up kernel's events: every recorded HIP
# event drains the stream for a few microseconds, so only every
# EVENT_EVERY-th timed step carries them (the kernel's duration is still
# measured inside the timed region).
EVENT_EVERY = 4


class Hip:
    """hipEvent_t handles through the HIP runtime (ctypes)."""

    def __init__(self):
        self.L = ctypes.CDLL("libamdhip64.so")
        self.L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.L.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.L.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def record(self, e, stream=None):
        s = torch.cuda.current_stream().cuda_stream if stream is None else stream
        assert self.L.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(s)) == 0

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.L.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a),
                                          ctypes.c_void_p(b)) == 0
        return ms.value

    def destroy(self, e):
        self.L.hipEventDestroy(ctypes.c_void_p(e))


def int4_banks(copies, dev, seed0):
    out = []
    for c in range(copies):
        mats = []
        for i, (n, k) in enumerate(((F, H), (F, H), (H, F))):
            q, s = synth.packed_int4_random(E, n, k, seed0 + 10 * c + i, dev)
            mats.append(B.bank_int4(q, s))
        out.append(B.ffn(*mats))
    return out


def variant_banks(copies, dev, seed0, fmt):
    out = []
    for c in range(copies):
        mats = []
        for i, (n, k) in enumerate(((F, H), (F, H), (H, F))):
            if fmt == "int8":
                mats.append(B.bank_int8(*synth.int8_random(E, n, k, seed0 + 10 * c + i, dev)))
                continue
            q, s, z = synth.packed_int4_variant_random(E, n, k, seed0 + 10 * c + i, dev,
                                                       group=32 if fmt == "int4-g32" else 128,
                                                       asym=fmt == "int4-asym")
            mats.append(B.bank_int4(q, s, z))
        out.append(B.ffn(*mats))
    return out


def csf_inputs(banks, dev, seed0):
    """Per bank copy and matrix: random CSF tensors whose expansion becomes
    that matrix's scale bytes, and the scale buffer to expand into."""
    out = []
    for c, bank in enumerate(banks):
        mats = []
        for i, scale in enumerate(bank.scale_tensors):
            R, C = scale.shape[1], scale.shape[2]
            mats.append((synth.csf_random(E, R, C, seed0 + 10 * c + i, dev), R, C, scale))
        out.append(mats)
    return out


def csf_bytes(R, C):
    """Algorithmic bytes of expanding one expert's scale matrix: the fixed
    codes and bases read, the bytes written (exceptions are ~0.2 % extra)."""
    return R * (1 + C // 2) + R * C


def nvfp4_banks(copies, dev, seed0):
    out = []
    for c in range(copies):
        mats = []
        for i, (n, k) in enumerate(((F, H), (F, H), (H, F))):
            q, s, g = synth.packed_nvfp4_random(E, n, k, seed0 + 10 * c + i, dev)
            mats.append(B.bank_nvfp4(q, s, g))
        f = B.ffn(*mats)
        f.scale_tensors = [m._keep[1] for m in mats]     # gate, up, down scale bytes
        f.code_tensors = [m._keep[0] for m in mats]
        f.gs_tensors = [m._keep[2] for m in mats]
        out.append(f)
    return out


def a4_banks(nv, g_x, g_h):
    """The NVFP4 banks `nv` with quantized inputs: input scale g_x for gate
    and up, g_h for down."""
    out = []
    for bank in nv:
        mats = [B.bank_nvfp4(q, s, g, input_scale=(g_h if i == 2 else g_x))
                for i, (q, s, g) in enumerate(zip(bank.code_tensors, bank.scale_tensors,
                                                   bank.gs_tensors))]
        out.append(B.ffn(*mats))
    return out


def csf_banks(nv, dev, seed0):
    """NVFP4 banks with random compressed scales read in place (the codes and
    global scales of `nv`): per copy the bank, and per matrix the inputs of
    its per-step row index (exceptions, starts, R, C, row index buffer)."""
    banks, idx = [], []
    for c, bank in enumerate(nv):
        mats, ins = [], []
        for i, scale in enumerate(bank.scale_tensors):
            R, C = scale.shape[1], scale.shape[2]
            fx, ex, st = synth.csf_random(E, R, C, seed0 + 10 * c + i, dev)
            ri = torch.zeros((E, R + 1), dtype=torch.int32, device=dev)
            mats.append(B.bank_nvfp4_csf(bank.code_tensors[i], fx, ex, ri, bank.gs_tensors[i]))
            ins.append((ex, st, R, C, ri))
        banks.append(B.ffn(*mats))
        idx.append(ins)
    return banks, idx


def touched_experts(logits_cpu):
    return int(torch.unique(torch.topk(logits_cpu, K, dim=1).indices).numel())


def run_layer(name, banks, T, act, route_mode, steps, warmup, hip, dev, fmt, csf=None,
              csf_mode="expand", use_graph=False):
    """Times `steps` layer passes. route_mode: 'logits' (fresh N(0,1) logits
    per step), 'weights' (router weight + fixed batch) or 'zipf' (router
    weight + Zipf(1.1) expert biases, fixed batch). csf: per bank copy, the
    compressed scales of its three matrices; each step then either expands
    the routed experts' scales before the forward pass (csf_mode 'expand')
    or builds their row index for the kernels that read them in place
    ('index'). use_graph: the timed steps are captured once as one HIP graph
    (each step its own logits and weight copy, as eagerly) and replayed.
    Returns a dict."""
    n_in = steps + warmup
    x = synth.activations(T, H, act, 2 if route_mode == "logits" else 3).to(dev)
    bias = None
    if route_mode == "logits":
        lg_cpu = [torch.from_numpy(synth.router_logits(T, E, 1000 + i)) for i in range(n_in)]
        logits = [t.to(dev) for t in lg_cpu]
        wT = None
    else:
        lg_cpu = None
        wT = torch.from_numpy(synth.router_weight_T(H, E, 3)).to(dev)
        if route_mode == "zipf":
            bias = torch.from_numpy(synth.zipf_bias(E, 3)).to(dev)
    tm, ws_bytes = B.moe_forward_plan(banks[0], T, K, x.dtype)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ids = torch.empty((T, K), dtype=torch.int32, device=dev)
    w = torch.empty((T, K), dtype=torch.float32, device=dev)
    perm = B.Perm(T, K, E, tm, dev)
    out = torch.empty((T, H), dtype=torch.float32, device=dev)
    rws = torch.empty(max(B.moe_route_workspace(T, E, route_mode != "logits"), 256),
                      dtype=torch.uint8, device=dev)
    NS = B.MOE_FORWARD_STAGES
    # timed loop: events only at the gate/up boundaries of every
    # EVENT_EVERY-th step; the other stages are timed in a separate pass
    ev_t = {i: [hip.event(), hip.event()] for i in range(0, steps, EVENT_EVERY)}
    nb = min(steps, 10)
    ev_b = [[hip.event() for _ in range(NS + 1)] for _ in range(nb)]

    ev_c = [[hip.event(), hip.event()] for _ in range(nb)] if csf else None

    def step(i, events=None, csf_events=None):
        # top-K and permutation in one call (one kernel up to 16 tokens)
        if route_mode == "logits":
            B.moe_route_permute(K, perm, logits=logits[i], ids=ids, w=w)
        else:
            B.moe_route_permute(K, perm, x=x, router_wT=wT, bias=bias, ids=ids, w=w, ws=rws)
        if csf:
            if csf_events:
                hip.record(csf_events[0])
            if csf_mode == "expand":
                for (fx, ex, st), R, C, scale in csf[i % len(csf)]:
                    B.moe_csf_expand(fx, ex, st, R, C, out=scale,
                                     expert_offsets=perm.expert_offsets, max_routed=min(E, T * K))
            else:
                for ex, st, R, C, ri in csf[i % len(csf)]:
                    B.moe_csf_row_index(ex, st, R, C, out=ri, expert_offsets=perm.expert_offsets,
                                        max_routed=min(E, T * K))
            if csf_events:
                hip.record(csf_events[1])
        B.moe_w4a16_forward(banks[i % len(banks)], x, w, perm, out=out, ws=ws, events=events)

    for i in range(warmup):
        step(steps + i)
    torch.cuda.synchronize()
    graph = None
    if use_graph:
        # the timed steps as one HIP graph, replayed once untimed first
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(steps):
                step(i)
        graph.replay()
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graph is not None:
        graph.replay()
    else:
        for i in range(steps):
            step(i, ev_t[i] + [None] * (NS - 1) if i in ev_t else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # per-step durations (events at step boundaries only), for the median
    ev_s = [hip.event() for _ in range(min(steps, 20) + 1)]
    hip.record(ev_s[0])
    for i in range(len(ev_s) - 1):
        step(i)
        hip.record(ev_s[i + 1])
    torch.cuda.synchronize()
    step_ms = np.array([hip.elapsed_ms(ev_s[i], ev_s[i + 1]) for i in range(len(ev_s) - 1)])
    for e in ev_s:
        hip.destroy(e)
    if graph is not None:
        # gate/up events from an eager pass over every step in order (a
        # graph replay records none; running only the evented steps would
        # leave the previous step's weight copy in the Infinity Cache)
        for i in range(steps):
            step(i, ev_t[i] + [None] * (NS - 1) if i in ev_t else None)
        torch.cuda.synchronize()
        del graph
    gu_idx = sorted(ev_t)
    gu_ms = np.array([hip.elapsed_ms(*ev_t[i]) for i in gu_idx])
    # stage breakdown: the first nb steps again, every boundary recorded
    for i in range(nb):
        step(i, ev_b[i], ev_c[i] if csf else None)
    torch.cuda.synchronize()
    stage_ms = np.array([[hip.elapsed_ms(e[j], e[j + 1]) for j in range(NS)] for e in ev_b])
    csf_ms = np.array([hip.elapsed_ms(e[0], e[1]) for e in ev_c]) if csf else None
    for e in list(ev_t.values()) + ev_b + (ev_c or []):
        for h in e:
            hip.destroy(h)
    if route_mode == "logits":
        U = np.array([touched_experts(lg_cpu[i]) for i in range(steps)], dtype=np.float64)
    else:
        U = np.full(steps, float(torch.unique(ids).numel()))
    gu_bytes, dn_bytes = EXPERT_BYTES[fmt]
    ms = wall / steps * 1e3
    r = dict(workload=name, tokens=T, graph=use_graph, ms_per_step=ms, tok_s=T / (ms * 1e-3),
             ms_per_step_median=float(np.median(step_ms)),
             touched_experts=float(U.mean()),
             layer_GBps=float((U * (gu_bytes + dn_bytes)).mean() / (ms * 1e-3) / 1e9),
             gateup_ms=float(gu_ms.mean()), down_ms=float(stage_ms[:, 1].mean()),
             combine_ms=float(stage_ms[:, 3].mean()),
             gateup_GBps=float(np.mean(U[gu_idx] * gu_bytes / (gu_ms * 1e-3)) / 1e9),
             down_GBps=float(np.mean(U[:nb] * dn_bytes / (stage_ms[:, 1] * 1e-3)) / 1e9),
             layer_TFLOPs=float(T * K * FLOP_PER_SLOT / (ms * 1e-3) / 1e12))
    r["gateup_frac_hbm"] = r["gateup_GBps"] * 1e9 / HBM_PEAK
    r["gateup_TFLOPs"] = float(T * K * 2 * 2 * H * F / (gu_ms.mean() * 1e-3) / 1e12)
    r["down_TFLOPs"] = float(T * K * 2 * H * F / (stage_ms[:, 1].mean() * 1e-3) / 1e12)
    if csf:
        r["csf_ms"] = float(csf_ms.mean())
        if csf_mode == "expand":
            cb = 2 * csf_bytes(F, H // 16) + csf_bytes(H, F // 16)
            r["csf_GBps"] = float(np.mean(U[:nb] * cb / (csf_ms * 1e-3)) / 1e9)
    return r


def run_tiny(steps, warmup, dev):
    """The tiny layer (8 tokens, hidden 256, 16 experts, top-2, SwiGLU width
    128, int4-g128, fp16 x, router from a N(0, 0.02) weight): a step is
    route + permute + forward. Launch-bound, so it is reported as latency,
    eager and as a HIP graph replay."""
    cfg = synth.CONFIGS["tiny"]
    T, h, e, k, f = cfg["T"][0], cfg["H"], cfg["E"], cfg["K"], cfg["F"]
    mats = []
    for i, (n, kk) in enumerate(((f, h), (f, h), (h, f))):
        mats.append(B.bank_int4(*synth.packed_int4_random(e, n, kk, 50 + i, dev)))
    ffn = B.ffn(*mats)
    x = synth.activations(T, h, "f16", 0).to(dev)
    wT = torch.from_numpy(synth.router_weight_T(h, e, 0)).to(dev)
    tm, ws_bytes = B.moe_forward_plan(ffn, T, k, x.dtype)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    rws = torch.empty(max(B.moe_route_workspace(T, e, True), 256), dtype=torch.uint8, device=dev)
    perm = B.Perm(T, k, e, tm, dev)
    out = torch.empty((T, h), dtype=torch.float32, device=dev)

    def step():
        B.moe_route_permute(k, perm, x=x, router_wT=wT, ids=ids, w=w, ws=rws)
        B.moe_w4a16_forward(ffn, x, w, perm, out=out, ws=ws)

    res = dict(workload="tiny T=8", tokens=T)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    res["us_per_step_eager"] = (time.perf_counter() - t0) / steps * 1e6
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(steps):
            step()
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    res["us_per_step_graph"] = (time.perf_counter() - t0) / steps * 1e6
    res["tok_s"] = T / (res["us_per_step_graph"] * 1e-6)
    return res


class StackLayer:
    """One layer of the stack: 352 random packed int4 experts, a BF16 shared
    expert N(0, 0.02), a router weight N(0, 0.02) and Zipf expert biases."""

    def __init__(self, l, dev):
        mats = []
        for i, (n, k) in enumerate(((F, H), (F, H), (H, F))):
            q, s = synth.packed_int4_random(E, n, k, 7000 + 10 * l + i, dev)
            mats.append(B.bank_int4(q, s))
        self.ffn = B.ffn(*mats)
        sh = [synth.device_normal(shape, 0.02, 7500 + 10 * l + i, dev, torch.bfloat16)
              for i, shape in enumerate(((F, H), (F, H), (H, F)))]
        self.shared = B.ffn(*[B.bank_bf16(w) for w in sh])
        self.wT = torch.from_numpy(synth.router_weight_T(H, E, 5, l)).to(dev)
        self.bias = torch.from_numpy(synth.zipf_bias(E, 5, l)).to(dev)
        self.norm_w = torch.from_numpy(synth.norm_weight(H, 5, l)).to(dev)


def run_stack(layers, T, steps, warmup, hip, dev, use_graph=True):
    """Times `steps` passes of the 8-layer stack: per layer, the RMSNorm of
    the fp32 residual rounded to bf16 and the routing from the router weight
    plus Zipf bias (one fused call), permutation, routed + shared experts and
    the combine with the residual."""
    r0 = synth.activations(T, H, "bf16", 5).float().to(dev)
    res = [r0.clone(), torch.empty_like(r0)]
    a = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    tm, ws_bytes = B.moe_forward_plan(layers[0].ffn, T, K, torch.bfloat16, layers[0].shared)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ids = torch.empty((T, K), dtype=torch.int32, device=dev)
    w = torch.empty((T, K), dtype=torch.float32, device=dev)
    perm = B.Perm(T, K, E, tm, dev)
    rws = torch.empty(B.moe_route_workspace(T, E, True), dtype=torch.uint8, device=dev)
    NS = B.MOE_FORWARD_STAGES
    # timed loop: events at each layer's gate/up boundaries of every
    # EVENT_EVERY-th step only (none when the step is a graph replay); the
    # other stages come from a separate eager pass with every boundary
    # recorded
    ev_t = ({} if use_graph else
            {i: [[hip.event(), hip.event()] for _ in layers] for i in range(0, steps, EVENT_EVERY)})
    nb = min(steps, 3)
    ev_b = [[[hip.event() for _ in range(NS + 1)] for _ in layers] for _ in range(nb)]

    def step(events=None, keep_ids=None):
        res[0].copy_(r0)
        for l, L in enumerate(layers):
            src, dst = res[l % 2], res[(l + 1) % 2]
            B.moe_norm_route(src, L.wT, K, norm_w=L.norm_w, eps=1e-5, bias=L.bias, a=a, ids=ids,
                             w=w, ws=rws)
            B.moe_permute(ids, E, tm, perm=perm)
            B.moe_w4a16_forward(L.ffn, a, w, perm, residual=src, out=dst, ws=ws,
                                shared=L.shared, events=None if events is None else events[l])
            if keep_ids is not None:
                keep_ids.append(int(torch.unique(ids).numel()))

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    graph = None
    if use_graph:
        # the whole 8-layer step as one HIP graph (the step launches ~10
        # kernels per layer; replaying them as a graph removes the host's
        # launch gaps); captured after the warm-up, replayed once untimed
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if graph is not None:
            graph.replay()
        else:
            step([e + [None] * (NS - 1) for e in ev_t[i]] if i in ev_t else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gu = (np.array([[hip.elapsed_ms(e[0], e[1]) for e in ev_t[i]] for i in sorted(ev_t)])
          if graph is None else None)                   # [step, layer]
    for i in range(nb):
        step(ev_b[i])
    torch.cuda.synchronize()
    st = np.array([[[hip.elapsed_ms(e[j], e[j + 1]) for j in range(NS)] for e in le]
                   for le in ev_b])                        # [step, layer, stage]
    for le in list(ev_t.values()) + ev_b:
        for e in le:
            for h in e:
                hip.destroy(h)
    U = []
    step(keep_ids=U)
    torch.cuda.synchronize()
    ms = wall / steps * 1e3
    per = st.sum(axis=1).mean(axis=0)                      # stage ms per step, all layers
    if gu is not None:
        per[0] = gu.sum(axis=1).mean()                     # gate/up from the timed loop
    flop = len(layers) * T * (K + 1) * FLOP_PER_SLOT
    gu_flop = len(layers) * T * K * 2 * 2 * H * F
    return dict(workload="stack T=%d" % T, tokens=T, layers=len(layers), graph=use_graph,
                ms_per_step=ms,
                tok_s=T / (ms * 1e-3), ms_per_layer=ms / len(layers),
                touched_experts=float(np.mean(U)),
                layer_GBps=float(np.sum(U) * (INT4_GATEUP_BYTES + INT4_DOWN_BYTES) /
                                 (ms * 1e-3) / 1e9),
                gateup_ms=float(per[0]), down_ms=float(per[1]), shared_ms=float(per[2]),
                combine_ms=float(per[3]),
                gateup_TFLOPs=float(gu_flop / (per[0] * 1e-3) / 1e12),
                layer_TFLOPs=float(flop / (ms * 1e-3) / 1e12))


def _oracle_tokens(x, lg, wT, bias, n_tok, efn, router=True):
    """The oracle on the first n_tok tokens: routing (the C router chain from
    the router weight, or the given logits), the 8 experts of each token
    dequantized by efn, SwiGLU and combine. Returns seconds."""
    from oracle import layer as OL
    from oracle import router as OR
    t0 = time.perf_counter()
    if router:
        _, ids, w = OR.route(x=x[:n_tok].float().numpy(), wT=wT, bias=bias, K=K)
    else:
        _, ids, w = OR.route(logits=lg[:n_tok], K=K)
    OL.moe_layer(x[:n_tok].float().numpy().astype(np.float64), ids, w, efn)
    return time.perf_counter() - t0


def _efn(mats, fmt):
    from oracle import quant as OQ

    def fn(e):
        if fmt == "int4":
            return tuple(OQ.dequant_int4(m._keep[0][e].cpu().numpy(),
                                         m._keep[1][e].view(torch.int16).cpu().numpy()
                                         .view(np.uint16)) for m in mats)
        return tuple(OQ.dequant_nvfp4(m._keep[0][e].cpu().numpy(), m._keep[1][e].cpu().numpy(),
                                      float(m._keep[2][e].cpu())) for m in mats)
    return fn


def cpu_baseline(int4, nv, n_tok=4):
    """The oracle, as it stands, on bounded samples: n_tok tokens of the
    decode T=64 batch (the headline), and n_tok tokens of the prefill batch
    (routing by the C router chain), of the NVFP4 batch, and the whole tiny
    layer. Each token's 8 experts are dequantized from the same packed bytes
    the GPU streams, in float64; threads as numpy's BLAS uses them."""
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        blas = 1
    cores = len(os.sched_getaffinity(0))
    lg = synth.router_logits(64, E, 1000)
    x = synth.activations(64, H, "f16", 2)
    dt = _oracle_tokens(x, lg, None, None, n_tok, _efn(int4[0]._keep, "int4"), router=False)
    per = []
    xp = synth.activations(n_tok, H, "bf16", 3)
    wT = synth.router_weight_T(H, E, 3)
    t = _oracle_tokens(xp, None, wT, None, n_tok, _efn(int4[0]._keep, "int4"))
    per.append(dict(workload="prefill T=2048", tokens=n_tok, seconds=round(t, 2),
                    tok_s=n_tok / t))
    if nv is not None:
        lgn = synth.router_logits(n_tok, E, 1000)
        xn = synth.activations(n_tok, H, "bf16", 2)
        t = _oracle_tokens(xn, lgn, None, None, n_tok, _efn(nv[0]._keep, "nvfp4"), router=False)
        per.append(dict(workload="nvfp4 T=256", tokens=n_tok, seconds=round(t, 2),
                        tok_s=n_tok / t))
    from tests import fixtures as FX       # the tiny layer's oracle-quantized experts
    cfg = synth.CONFIGS["tiny"]
    host = []
    for which, (n, k) in (("gate", (cfg["F"], cfg["H"])), ("up", (cfg["F"], cfg["H"])),
                          ("down", (cfg["H"], cfg["F"]))):
        host.append(FX.int4_bank_oracle(cfg["E"], n, k, 0, 0, which))
    from oracle import layer as OL
    from oracle import quant as OQ
    from oracle import router as OR
    xt = synth.activations(8, cfg["H"], "f16", 0)
    wTt = synth.router_weight_T(cfg["H"], cfg["E"], 0)
    t0 = time.perf_counter()
    _, ids, w = OR.route(x=xt.float().numpy(), wT=wTt, K=cfg["K"])
    OL.moe_layer(xt.float().numpy().astype(np.float64), ids, w,
                 lambda e: tuple(OQ.dequant_int4(q[e], sc[e]) for (q, sc) in host))
    t = time.perf_counter() - t0
    per.append(dict(workload="tiny T=8", tokens=8, seconds=round(t, 4), tok_s=8 / t))
    return dict(value=n_tok / dt, unit="tokens/s", cores=cores, blas_threads=int(blas),
                kind="oracle",
                sample="%d tokens of the decode T=64 batch (route on given logits, 8 int4 "
                       "experts per token dequantized to float64, SwiGLU, combine); %.1f s"
                       % (n_tok, dt),
                per_config=per)


# Sources a kernel is built from: its counters stay valid while these are
# unchanged.
GEMV_SOURCES = ("gemv.hip", "decode.h", "stream.h", "common.h")
GEMV_MFMA_SOURCES = ("gemv_mfma.hip", "decode.h", "stream.h", "common.h")
GEMM_SOURCES = ("gemm.hip", "decode.h", "stream.h", "common.h")


def decode_kernel(fmt, act, T):
    """The gate/up kernel a batch of T tokens runs at the layer's shape: the
    grouped GEMM from T * top-k >= 4 * experts slots on (NVFP4: 8 * experts,
    the MFMA GEMV from 4 to 8; int4-g128, both forms: 7 * experts, the MFMA
    GEMV below), below that the dot2 GEMV for the other formats."""
    if fmt == "nvfp4" and 4 * E <= T * K < 8 * E:
        return "gemv_mfma_gateup_nvfp4_%s" % act, GEMV_MFMA_SOURCES
    if fmt in ("int4", "int4-asym") and T * K < 7 * E:
        return "gemv_mfma_gateup_%s_%s" % (fmt, act), GEMV_MFMA_SOURCES
    if T * K >= 4 * E:
        return "gemm_gateup_%s_%s" % (fmt, act), GEMM_SOURCES
    if fmt in ("int4", "int4-asym"):
        return "gemv_mfma_gateup_%s_%s" % (fmt, act), GEMV_MFMA_SOURCES
    return "gemv_gateup_%s_%s" % (fmt, act), GEMV_SOURCES


def traffic_for(kernel, files=GEMV_SOURCES):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(kernel)
    except Exception:
        return None
    if not rec or rec.get("source_sha") != source_sha(files):
        return None
    return rec.get("bytes_per_launch")


def source_sha(files=GEMV_SOURCES):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_moe_sigmoid_amd", "csrc")
    for f in files:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode-graph",
                    choices=["decode", "decode-graph", "prefill", "prefill-zipf", "nvfp4",
                             "nvfp4-csf", "nvfp4-csf-expand", "nvfp4-a4", "int4-g32",
                             "int4-asym", "int8", "stack"])
    ap.add_argument("--tokens", type=int, default=None)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="run the stack's timed steps eagerly instead of as a HIP graph replay")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run a plain streaming kernel over MIB MiB (read once, written "
                         "once), the reference for scaling hardware byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the layer has no multi-GPU path in this build "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    hip = Hip()
    B.lib()

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)                    # reads n*4 bytes, writes n*4 bytes
        torch.cuda.synchronize()
        del src, dst

    int4 = int4_banks(2, dev, 500)
    jobs = []
    main_T = args.tokens or {"decode": 64, "decode-graph": 64, "prefill": 2048, "nvfp4-a4": 256,
                             "prefill-zipf": 2048, "nvfp4": 256, "nvfp4-csf": 64,
                             "nvfp4-csf-expand": 64,
                             "int4-g32": 64, "int4-asym": 64, "int8": 64,
                             "stack": 4096}[args.workload]
    spec = {"decode": ("f16", "logits", "int4"), "decode-graph": ("f16", "logits", "int4"),
            "prefill": ("bf16", "weights", "int4"), "prefill-zipf": ("bf16", "zipf", "int4"),
            "nvfp4": ("bf16", "logits", "nvfp4"), "nvfp4-csf": ("bf16", "logits", "nvfp4-csf"),
            "nvfp4-a4": ("bf16", "logits", "nvfp4-a4"),
            "nvfp4-csf-expand": ("bf16", "logits", "nvfp4"),
            "int4-g32": ("f16", "logits", "int4-g32"), "int4-asym": ("f16", "logits", "int4-asym"),
            "int8": ("f16", "logits", "int8"),
            "stack": ("bf16", "weights", "int4")}
    jobs.append((args.workload, main_T))
    if not args.no_sweep:
        for wl, T in (("tiny", 8), ("decode", 1), ("decode", 8), ("decode", 64),
                      ("decode-graph", 1), ("decode-graph", 8), ("decode-graph", 64),
                      ("prefill", 2048), ("prefill-zipf", 2048),
                      ("nvfp4", 1), ("nvfp4", 256), ("nvfp4-csf", 64), ("nvfp4-csf-expand", 64),
                      ("nvfp4-csf-expand", 256), ("nvfp4-a4", 1), ("nvfp4-a4", 256),
                      ("int4-g32", 64), ("int4-g32", 2048),
                      ("int4-asym", 64), ("int4-asym", 2048), ("int8", 64), ("int8", 2048),
                      ("stack", 32),
                      ("stack", 4096)):
            if (wl, T) != (args.workload, main_T):
                jobs.append((wl, T))
    nv = None
    nv_csf = None
    nv_csf_in = None
    variants = {}
    stack = None
    results = []
    for wl, T in jobs:
        steps = args.steps if (wl, T) == jobs[0] else max(10, args.steps // 2)
        if wl == "tiny":
            results.append(run_tiny(100, 10, dev))
            print("# %s" % json.dumps(results[-1]), file=sys.stderr, flush=True)
            continue
        act, rmode, fmt = spec[wl]
        if wl == "stack":
            if stack is None:
                stack = [StackLayer(l, dev) for l in range(8)]
            results.append(run_stack(stack, T, max(5, steps // 4), max(2, args.warmup // 4),
                                     hip, dev, use_graph=not args.no_graph))
        else:
            if fmt in ("nvfp4", "nvfp4-csf", "nvfp4-a4") and nv is None:
                nv = nvfp4_banks(2, dev, 900)
            if fmt in ("int4-g32", "int4-asym", "int8") and fmt not in variants:
                variants[fmt] = variant_banks(
                    2, dev, {"int4-g32": 2000, "int4-asym": 2100, "int8": 2200}[fmt], fmt)
            banks = int4 if fmt == "int4" else (nv if fmt == "nvfp4" else variants.get(fmt))
            if fmt == "nvfp4-a4":
                # input scales: x's from the largest activation of the decode
                # batches (N(0, 1) in bf16), h's 2^-7 (the h of these weights
                # stays below 6 x 448 x 2^-7 = 21)
                g_x = float(np.float32(5.5 / (6 * 448)))
                banks = a4_banks(nv, g_x, 2.0 ** -7)
            csf, csf_mode = None, "expand"
            if wl == "nvfp4-csf-expand":
                if nv_csf is None:
                    nv_csf = csf_inputs(nv, dev, 1900)
                csf = nv_csf
            if wl == "nvfp4-csf":
                if nv_csf_in is None:
                    nv_csf_in = csf_banks(nv, dev, 1900)
                banks, csf, csf_mode = nv_csf_in[0], nv_csf_in[1], "index"
            results.append(run_layer("%s T=%d" % (wl, T), banks, T, act, rmode, steps,
                                     args.warmup, hip, dev, fmt, csf, csf_mode,
                                     use_graph=wl == "decode-graph"))
        print("# %s" % json.dumps(results[-1]), file=sys.stderr, flush=True)

    head = results[0]
    if args.workload == "stack":
        print(json.dumps({"workload": "stack", "result": head}))
        return
    act, rmode, fmt = spec[args.workload]
    kern, kern_src = decode_kernel(fmt, act, main_T)
    traffic = traffic_for(kern, kern_src)
    roof = dict(bound="hbm", kernel=kern, achieved=round(head["gateup_GBps"], 1),
                peak=HBM_PEAK / 1e9, unit="GB/s", frac=round(head["gateup_frac_hbm"], 4),
                traffic=traffic,
                algorithmic_bytes_per_launch=round(head["touched_experts"] *
                                                   EXPERT_BYTES[fmt][0]))
    # the prefill grouped GEMM (gate/up at T = 2048, uniform routing):
    # MFMA fraction (the bound the pages' prefill figures are about) and the
    # HBM fraction of the same launch
    pre = next((r for r in results if r["workload"] == "prefill T=2048"), None)
    roof_pre = None
    if pre is not None:
        gu_b = EXPERT_BYTES["int4"][0]
        roof_pre = dict(bound="mfma", kernel="gemm_gateup_int4_bf16", unit="TFLOP/s",
                        achieved=round(pre["gateup_TFLOPs"], 1), peak=MFMA_BF16_PEAK / 1e12,
                        frac=round(pre["gateup_TFLOPs"] * 1e12 / MFMA_BF16_PEAK, 4),
                        hbm_GBps=round(pre["gateup_GBps"], 1),
                        hbm_frac=round(pre["gateup_frac_hbm"], 4),
                        traffic=traffic_for("gemm_gateup_int4_bf16", GEMM_SOURCES),
                        flop_per_launch=2048 * K * 2 * 2 * H * F,
                        algorithmic_bytes_per_launch=round(pre["touched_experts"] * gu_b))
    cpu = None if args.no_cpu_baseline else cpu_baseline(int4, nv)
    line = {
        "metric": "W4A16 MoE layer tok/s; decode HBM GB/s %peak; prefill TFLOP/s %peak",
        "value": round(head["tok_s"], 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": act, "data": "synthetic",
        "config": {"workload": "%s T=%d: 352 %s experts, top-8 sigmoid routing, hidden 4096, "
                               "SwiGLU width 1536, %s activations" % (args.workload, main_T,
                                                                      fmt, act),
                   "tokens": main_T, "experts": E, "top_k": K, "hidden": H, "width": F},
        "roofline": roof,
        "roofline_prefill": roof_pre,
        "cpu_baseline": cpu,
        "sweep": results,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
