"""Seeded synthetic inputs for the sparse MoE feed-forward layer (and, in
``gdn_inputs``, for the Gated DeltaNet prefill scan).

This module only draws random bytes and lays them out; it holds none of the
layer's arithmetic (no dequantisation, no routing, no matmul).  Both the CPU
oracle (``oracle/``) and the HIP library's tests and benchmark consume the
bytes it produces, so the two sides always see identical inputs.

Layouts (shared by both sides):

* activations ``x``: bf16 bit patterns, ``uint16 [T][H]`` row-major.
* router weight: ``uint16 [E][H]`` (bf16 bits) or ``float32 [E][H]``.
* router bias: ``float32 [E]`` or ``None``.
* a quantised matrix ``W[N][K]``: ``q`` is ``uint32 [N][K/8]``; element ``k`` of
  row ``n`` is the 4-bit field at bits ``4*(k%8)`` of word ``q[n][k//8]`` (low
  nibble first); ``scale`` and ``bias`` are ``float16 [N][K/64]`` (one pair per
  group of 64 consecutive ``k``).
* per layer the routed experts ``0..E-1`` and the shared expert are stacked
  along the leading axis, the shared expert at index ``E``:
  ``gate_q [E+1][I][H/8]``, ``up_q`` likewise, ``down_q [E+1][H][I/8]``.

The quantised format (4-bit codes, groups of 64 with a scale and a bias) follows
"Optimizing on-device inference for Apple Silicon", section "Prefill ›
Dequantize weights during matmul".  The configurations below are the synthetic
stand-ins for that page's Qwen3.6-35B-A3B workload (256 routed experts, top-8,
one shared expert: section "Qwen creates three different workload shapes").
"""

from .moe_inputs import (  # noqa: F401
    CONFIGS,
    LayerWeights,
    MoeShape,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_layer,
    make_x,
    shape_of,
)
from .gdn_inputs import GDN_CONFIGS, GdnInputs, GdnShape, gdn_inputs, make_gdn  # noqa: F401,E402
