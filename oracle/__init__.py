"""CPU oracle for the W4A16 routed-expert MoE layer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call,
link or execute anything in this package: only the test suite, the smoke
check and the benchmark's CPU-baseline leg use it.

It is a plain, slow, obviously-correct restatement of what the layer
computes, in float64 (numpy) plus one small C file for the float32 router
logit chain. It shares no code, headers, tables or helpers with the HIP
library; the two meet only through the seeded input generators.

Modules
-------
formats   IEEE-style rounding to bf16 / fp16 / fp32, the E2M1 and E4M3 value
          tables built from their bit-field definitions.
quant     int4-g128 symmetric quantizer with the 17-ratio clip search,
          max-abs comparator, nibble packing, NVFP4 two-level quantizer,
          packing and dequantization.
router    canonical float32 router logits (C), top-K selection, sigmoid
          weights with renormalisation.
permute   expert histogram, stable expert-sorted permutation, padded tiles.
layer     SwiGLU expert FFN, weighted combine, shared expert, residual.
norm      the zero-centred-gain RMSNorm that feeds each layer of the stack.
csf       the compressed scale format of the NVFP4 block scales (row base +
          4-bit code, exception lists per expert): encoder and decoder.

Every function with no independent pin says "parity unpinned" in its
docstring.
"""
