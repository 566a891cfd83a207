"""Seeded generator for the MoE layer's inputs (see the package docstring for layouts).

Every tensor is drawn from its own PCG64 stream, keyed by
``SeedSequence(seed, spawn_key=(weights_cfg, layer, tensor_id[, block]))`` so that
any tensor (one layer of forty, one 4096-row block of a long prompt) can be drawn
without drawing the others.

Distributions:

* 4-bit codes uniform on {0..15}.  Eight independent uniform nibbles packed into a
  32-bit word are exactly a uniform 32-bit word, so words are drawn directly.
* scale ~ U(0.005, 0.02) rounded to float16; bias = -8*scale (exact in float16,
  a multiplication by a power of two).
* router weight ~ N(0, 0.02^2), rounded to bf16 (float32 for the tiny case).
* activations ~ N(0, 1) rounded to bf16.
* skewed case: router bias b_e = -1.2*ln(rank_e), rank = 1 + a seeded permutation
  of 0..E-1, i.e. the log of a Zipf(1.2) pmf used as a logit offset.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

TID_ROUTER_W = 0
TID_ROUTER_B = 1
TID_X = 2
TID_EXPERT0 = 3  # expert e, matrix m (0 gate, 1 up, 2 down) -> 3 + 3*e + m
TID_SHARED_GATE = 1 << 20

X_BLOCK_ROWS = 4096


@dataclasses.dataclass(frozen=True)
class MoeShape:
    name: str
    T: int            # tokens per forward
    H: int            # hidden size
    E: int            # routed experts
    k: int            # experts per token
    I: int            # intermediate size (routed and shared expert)
    router_fp32: bool  # router weight stored as float32 (else bf16)
    zipf_bias: bool   # add the skewed per-expert router bias
    layers: int = 1   # distinct weight sets (decode sweeps them back to back)
    qparam_bf16: bool = False  # scale/bias stored as bf16 (else float16)
    shared_gate: bool = False  # a learned gate vector on the shared expert
    chunk: int = 4096  # prefill chunk size used for this workload
    weights_cfg: int = -1  # config whose weight/x streams are reused (-1: own)
    x_cfg: int = -1

    @property
    def group(self) -> int:
        return 64


CONFIGS = {
    0: MoeShape("tiny", T=8, H=256, E=16, k=2, I=128, router_fp32=True, zipf_bias=False),
    1: MoeShape("decode", T=1, H=2048, E=256, k=8, I=512, router_fp32=False,
                zipf_bias=False, layers=40),
    2: MoeShape("prefill-uniform", T=4096, H=2048, E=256, k=8, I=512,
                router_fp32=False, zipf_bias=False),
    3: MoeShape("prefill-zipf", T=4096, H=2048, E=256, k=8, I=512, router_fp32=False,
                zipf_bias=True, weights_cfg=2, x_cfg=2),
    4: MoeShape("prefill-128k", T=131072, H=2048, E=256, k=8, I=512,
                router_fp32=False, zipf_bias=False, weights_cfg=2),
    # edge shapes for the parity tests (not benchmark workloads): sizes that are not
    # multiples of the kernels' tiles, and the largest sizes the library accepts
    10: MoeShape("odd-shape", T=37, H=768, E=40, k=6, I=384, router_fp32=False, zipf_bias=False,
                 chunk=16),
    11: MoeShape("max-size", T=3, H=16384, E=4, k=4, I=4096, router_fp32=False, zipf_bias=False, chunk=3),
    # gate/up items whose last round is split along K (into 2 and into 3 pieces, the
    # latter over 10 K-steps, so the pieces are uneven)
    12: MoeShape("split-2", T=1024, H=768, E=40, k=6, I=384, router_fp32=False, zipf_bias=False, chunk=1024),
    13: MoeShape("split-3", T=1024, H=1280, E=32, k=4, I=512, router_fp32=False, zipf_bias=False, chunk=1024),
    # a bf16 router whose expert count is not a multiple of 4 (scalar logit reads in the
    # selection, a partial 64-expert logits tile), over ragged 24-token chunks
    14: MoeShape("e42-bf16", T=50, H=512, E=42, k=6, I=256, router_fp32=False, zipf_bias=False, chunk=24),
    # the pages' checkpoint format: bf16 scale/bias, and a sigmoid-gated shared expert;
    # a small shape and the benchmark shape (512 tokens)
    15: MoeShape("bf16-qparams-small", T=40, H=512, E=32, k=4, I=256, router_fp32=False, zipf_bias=False,
                 chunk=16, qparam_bf16=True, shared_gate=True),
    16: MoeShape("bf16-qparams", T=512, H=2048, E=256, k=8, I=512, router_fp32=False, zipf_bias=False,
                 chunk=512, qparam_bf16=True, shared_gate=True),
}


def shape_of(cfg: int) -> MoeShape:
    return CONFIGS[cfg]


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    if not np.isfinite(a).all():
        raise ValueError("bf16 rounding is only defined here for finite values")
    # finite inputs stay below 0xFF800000, so the sum cannot wrap in 32 bits
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class LayerWeights:
    router_w: np.ndarray            # [E][H] uint16 (bf16) or float32
    router_b: Optional[np.ndarray]  # [E] float32 or None
    gate_q: np.ndarray              # [E+1][I][H/8] uint32
    gate_s: np.ndarray              # [E+1][I][H/64] float16
    gate_b: np.ndarray
    up_q: np.ndarray
    up_s: np.ndarray
    up_b: np.ndarray
    down_q: np.ndarray              # [E+1][H][I/8] uint32
    down_s: np.ndarray              # [E+1][H][I/64] float16
    down_b: np.ndarray
    shared_gate: Optional[np.ndarray] = None  # [H] uint16 (bf16) or None

    def nbytes(self) -> int:
        return sum(getattr(self, f.name).nbytes for f in dataclasses.fields(self)
                   if getattr(self, f.name) is not None)


def _quant_matrix(rng: np.random.Generator, N: int, K: int, bf16: bool = False):
    """Codes, scale and bias of one matrix: scale ~ U(0.005, 0.02) rounded to float16 (or
    to bf16, returned as uint16 bits), bias = -8*scale (exact in either format)."""
    q = rng.integers(0, 1 << 32, size=(N, K // 8), dtype=np.uint32)
    u = rng.uniform(0.005, 0.02, size=(N, K // 64))
    if bf16:
        s = f32_to_bf16_bits(u.astype(np.float32))
        b = f32_to_bf16_bits(bf16_bits_to_f32(s) * np.float32(-8.0))
    else:
        s = u.astype(np.float16)
        b = (s.astype(np.float32) * np.float32(-8.0)).astype(np.float16)
    return q, s, b


def make_layer(cfg: int, layer: int = 0, seed: int = 0, into: Optional[LayerWeights] = None) -> LayerWeights:
    """Draw one layer's weights (router, E routed experts and the shared expert).

    ``into``: a LayerWeights of the same config whose arrays are overwritten (saves
    the page faults of fresh memory when many layers are drawn one after another).
    """
    sh = CONFIGS[cfg]
    wc = sh.weights_cfg if sh.weights_cfg >= 0 else cfg
    E, H, I = sh.E, sh.H, sh.I
    r = _rng(seed, wc, layer, TID_ROUTER_W)
    w = r.standard_normal((E, H), dtype=np.float32) * np.float32(0.02)
    router_w = w.astype(np.float32) if sh.router_fp32 else f32_to_bf16_bits(w)
    router_b = None
    if sh.zipf_bias:
        rb = _rng(seed, cfg, layer, TID_ROUTER_B)
        rank = 1 + rb.permutation(E)
        router_b = (-1.2 * np.log(rank.astype(np.float64))).astype(np.float32)
    mats = {}
    for m, (nm, N, K) in enumerate((("gate", I, H), ("up", I, H), ("down", H, I))):
        if into is not None:
            q, s, b = getattr(into, nm + "_q"), getattr(into, nm + "_s"), getattr(into, nm + "_b")
            assert q.shape == (E + 1, N, K // 8)
        else:
            qdt = np.uint16 if sh.qparam_bf16 else np.float16
            q = np.empty((E + 1, N, K // 8), np.uint32)
            s = np.empty((E + 1, N, K // 64), qdt)
            b = np.empty((E + 1, N, K // 64), qdt)
        for e in range(E + 1):
            q[e], s[e], b[e] = _quant_matrix(_rng(seed, wc, layer, TID_EXPERT0 + 3 * e + m), N, K, sh.qparam_bf16)
        mats[nm] = (q, s, b)
    sg = None
    if sh.shared_gate:
        g = _rng(seed, cfg, layer, TID_SHARED_GATE).standard_normal(H, dtype=np.float32) * np.float32(0.02)
        sg = f32_to_bf16_bits(g)
    return LayerWeights(router_w, router_b, *mats["gate"], *mats["up"], *mats["down"], shared_gate=sg)


def make_x(cfg: int, layer: int = 0, seed: int = 0, rows: Optional[slice] = None) -> np.ndarray:
    """Activations as bf16 bits ``uint16 [T][H]`` (or the requested row range).

    Rows are drawn in blocks of 4096 from independent streams, so a row range of a
    long prompt can be drawn on its own.
    """
    sh = CONFIGS[cfg]
    xc = sh.x_cfg if sh.x_cfg >= 0 else cfg
    T, H = sh.T, sh.H
    start, stop, _ = (rows or slice(0, T)).indices(T)
    out = np.empty((stop - start, H), np.uint16)
    b0, b1 = start // X_BLOCK_ROWS, (stop - 1) // X_BLOCK_ROWS if stop > start else -1
    for blk in range(b0, b1 + 1):
        n = min(X_BLOCK_ROWS, T - blk * X_BLOCK_ROWS)
        v = _rng(seed, xc, layer, TID_X, blk).standard_normal((n, H), dtype=np.float32)
        lo = max(start, blk * X_BLOCK_ROWS)
        hi = min(stop, blk * X_BLOCK_ROWS + n)
        out[lo - start:hi - start] = f32_to_bf16_bits(v[lo - blk * X_BLOCK_ROWS:hi - blk * X_BLOCK_ROWS])
    return out
