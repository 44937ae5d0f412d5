"""Seeded synthetic inputs for the MoE layer workloads.

This module only draws random numbers and casts them to storage types; it
holds none of the layer's arithmetic (no routing, quantization, dequant or
FFN). Both the test oracle and the HIP library are fed from here.

Every stream is numpy's PCG64 seeded by SeedSequence([root, layer, tensor,
expert]), so one tensor never depends on the shapes or draw order of another.
Tensor ids: 0 activations, 1 router weight, 2 router logits, 3 Zipf
permutation, 10/11/12 gate/up/down expert weights, 20/21/22 shared expert.

Distributions (the layer's shapes are those of page "Step 5 Preview: 92
narrow layers, and a sparse indexer that scores blocks of 8", "The shape:
narrow and deep": hidden 4096, 352 experts, top-8, SwiGLU width 1536):
* activations N(0, 1), rounded to fp16 or bf16;
* expert weights N(0, 0.02), rounded to bf16 (the source checkpoints are
  BF16: page "NeuroSenko/Step-5-Preview-Int4-g128", first paragraph);
* router weight N(0, 0.02) float32; given router logits N(0, 1) float32;
* skewed routing: bias_e = -s * ln(rank_e) with s = 1.1 and rank a seeded
  permutation of 1..E (a Zipf(s) popularity on the sigmoid's logit scale).

Large weight banks for the benchmark are drawn on the GPU by torch's own
generator (see `device_normal`), chunk by chunk, since 6.6 G numpy draws
would take minutes.
"""
import numpy as np

T_X, T_WR, T_LOGITS, T_ZIPF, T_NORM = 0, 1, 2, 3, 4
T_GATE, T_UP, T_DOWN = 10, 11, 12
T_SH_GATE, T_SH_UP, T_SH_DOWN = 20, 21, 22

# Workloads: the tiny layer, decode, prefill, NVFP4 and the chained stack.
CONFIGS = {
    "tiny": dict(T=(8,), H=256, E=16, K=2, F=128, act="f16", fmt="int4",
                 router="weights", root=0),
    "decode": dict(T=(1, 8, 64), H=4096, E=352, K=8, F=1536, act="f16",
                   fmt="int4", router="logits", root=2),
    "prefill": dict(T=(2048,), H=4096, E=352, K=8, F=1536, act="bf16",
                    fmt="int4", router="weights", root=3),
    "nvfp4": dict(T=(1, 256), H=4096, E=352, K=8, F=1536, act="bf16",
                  fmt="nvfp4", router="logits", root=4),
    "stack": dict(T=(32, 4096), H=4096, E=352, K=8, F=1536, act="bf16",
                  fmt="int4", router="weights+zipf", root=5, layers=8,
                  shared=True),
}


def rng(root, layer, tensor, expert=0):
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([int(root), int(layer), int(tensor), int(expert)])))


def normal(shape, std, root, layer, tensor, expert=0):
    """float32 N(0, std^2)."""
    return (rng(root, layer, tensor, expert).standard_normal(shape, dtype=np.float32)
            * np.float32(std)).astype(np.float32)


def cast16(a, dtype):
    """Round float32 values to fp16 / bf16 (round to nearest even) with torch
    and return the torch CPU tensor."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.float16 if dtype == "f16" else torch.bfloat16)


def activations(T, H, dtype, root, layer=0):
    return cast16(normal((T, H), 1.0, root, layer, T_X), dtype)


def router_weight_T(H, E, root, layer=0):
    """Router weight stored transposed, [H, E] float32, N(0, 0.02)."""
    return np.ascontiguousarray(normal((E, H), 0.02, root, layer, T_WR).T)


def router_logits(T, E, root, layer=0):
    return normal((T, E), 1.0, root, layer, T_LOGITS)


def zipf_bias(E, root, layer=0, s=1.1):
    rank = rng(root, layer, T_ZIPF).permutation(E) + 1
    return (-s * np.log(rank.astype(np.float64))).astype(np.float32)


def norm_weight(H, root, layer=0, std=0.1):
    """Zero-centred RMSNorm gain offsets w [H] float32, N(0, std^2): the
    layer scales by (1 + w)."""
    return normal((H,), std, root, layer, T_NORM)


def expert_weight_bf16(n, k, root, layer, tensor, expert):
    """One expert matrix [n, k]: N(0, 0.02) rounded to bf16 (torch tensor)."""
    return cast16(normal((n, k), 0.02, root, layer, tensor, expert), "bf16")


def device_normal(shape, std, seed, device, dtype=None):
    """N(0, std^2) drawn on `device` by torch's generator for that device,
    seeded with `seed`; optionally cast to `dtype` (torch dtype)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std
    return x if dtype is None else x.to(dtype)


def packed_int4_random(E, n, k, seed, device, scale_mean=0.0043):
    """Random int4-g128 bank drawn directly in packed form: uniform 32-bit
    words (every nibble uniform over the 16 codes) and bf16 scales
    scale_mean * (1 + 0.1 N(0, 1)), so the weights have a standard
    deviation near 0.02. For full-size tests and benchmarks where drawing
    and quantizing 6.6 G Gaussian weights on the host would take minutes."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    q = torch.randint(-2 ** 31, 2 ** 31 - 1, (E, n, k // 8), generator=g, device=device,
                      dtype=torch.int32)
    s = (torch.randn((E, n, k // 128), generator=g, device=device) * 0.1 + 1.0) * scale_mean
    return q, s.to(torch.bfloat16)


def packed_int4_variant_random(E, n, k, seed, device, group=128, asym=False, scale_mean=0.0043):
    """Random int4-g32 (group=32) or asymmetric int4-g128 (asym=True) bank
    in packed form: uniform 32-bit words, bf16 scales scale_mean * (1 + 0.1
    N(0, 1)) per group and, for the asymmetric form, zero points uniform in
    [0, 15] (uint8 [E, n, k/128]). Returns (words, scales, zero points or
    None)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    q = torch.randint(-2 ** 31, 2 ** 31 - 1, (E, n, k // 8), generator=g, device=device,
                      dtype=torch.int32)
    s = (torch.randn((E, n, k // group), generator=g, device=device) * 0.1 + 1.0) * scale_mean
    z = (torch.randint(0, 16, (E, n, k // 128), generator=g, device=device, dtype=torch.uint8)
         if asym else None)
    return q, s.to(torch.bfloat16), z


def int8_random(E, n, k, seed, device, scale_mean=0.00027):
    """Random int8-g128 bank: uniform bytes (q uniform on [-128, 127]) and
    bf16 scales scale_mean * (1 + 0.1 N(0, 1)) per 128 inputs (a weight std
    of about 0.02). Returns (q int8 [E, n, k], scales bf16 [E, n, k/128])."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    q = torch.randint(-128, 128, (E, n, k), generator=g, device=device, dtype=torch.int8)
    s = (torch.randn((E, n, k // 128), generator=g, device=device) * 0.1 + 1.0) * scale_mean
    return q, s.to(torch.bfloat16)


def csf_random(E, R, C, seed, device, rate=0.002):
    """Random CSF tensors of an NVFP4 scale tensor [E, R, C]: row bases
    uniform in [0x60, 0x6F], uniform 4-bit codes, and per expert about
    rate * R * C exceptions at distinct random positions (row-major order)
    holding bytes uniform in [0x30, 0x7E]. Every byte they stand for is a
    finite non-negative E4M3 value. Returns (fixed uint8 [E, R/16,
    16 * (1 + C/2)], exceptions int32 [n], starts int64 [E + 1])."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    fixed = torch.randint(0, 256, (E, R // 16, 16 * (1 + C // 2)), generator=g, device=device,
                          dtype=torch.uint8)
    fixed[:, :, :16] = torch.randint(0x60, 0x70, (E, R // 16, 16), generator=g, device=device,
                                     dtype=torch.uint8)
    m = max(0, int(round(rate * R * C)))
    exc, starts = [], [0]
    for e in range(E):
        pos = torch.unique(torch.randint(0, R * C, (m,), generator=g, device=device))
        byte = torch.randint(0x30, 0x7F, (pos.numel(),), generator=g, device=device)
        exc.append((pos | (byte << 24)).to(torch.int32))
        starts.append(starts[-1] + pos.numel())
    exceptions = torch.cat(exc) if exc else torch.zeros(0, dtype=torch.int32, device=device)
    return fixed, exceptions, torch.tensor(starts, dtype=torch.int64, device=device)


def packed_nvfp4_random(E, n, k, seed, device, gs_mean=2.0e-5, scale_window=None):
    """Random NVFP4 bank in packed form: uniform bytes (two uniform E2M1
    codes each), E4M3 block-scale bytes uniform in [0x70, 0x7E] (128 .. 448)
    and float32 global scales gs_mean * (1 + 0.1 N(0, 1)).

    With scale_window = w, the scale bytes of expert e are instead uniform
    in [b_e, b_e + w - 1] with b_e uniform in [0, 0x7F - w], so that over a
    layer the block scales reach every finite non-negative E4M3 byte
    (0x00 .. 0x7E: zero, subnormals and normals); the caller then picks
    global scales that bring each expert back to a common magnitude."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    q = torch.randint(0, 256, (E, n, k // 2), generator=g, device=device, dtype=torch.uint8)
    if scale_window is None:
        s = torch.randint(0x70, 0x7F, (E, n, k // 16), generator=g, device=device,
                          dtype=torch.uint8)
    else:
        w = int(scale_window)
        base = torch.randint(0, 0x80 - w, (E, 1, 1), generator=g, device=device,
                             dtype=torch.int32)
        off = torch.randint(0, w, (E, n, k // 16), generator=g, device=device, dtype=torch.int32)
        s = (base + off).to(torch.uint8)
    gs = (torch.randn((E,), generator=g, device=device) * 0.1 + 1.0) * gs_mean
    return q, s, gs.float()
