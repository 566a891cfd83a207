"""Seeded generator for the Gated DeltaNet prefill scan's inputs.

Holds none of the scan's arithmetic: it draws random numbers and lays them out.
Layouts (row-major, shared by the oracle and the HIP library):

* ``q``, ``k``: bf16 bits ``uint16 [T][n_kheads][d]``;
* ``v``: bf16 bits ``uint16 [T][n_vheads][d]``;
* ``alpha`` (decay gate), ``beta`` (write strength): ``float32 [T][n_vheads]``;
* ``state``: ``float32 [n_vheads][d][d]``, one row per value channel.

Distributions (the pages give none; these follow the usual Gated DeltaNet inputs):

* ``q``, ``k``: standard normal vectors scaled to unit length per (token, head) --
  the L2-normalised keys the delta rule is used with -- ``q`` then times ``d**-0.5``
  (the attention scale), rounded to bf16;
* ``v`` ~ N(0, 1) rounded to bf16;
* ``alpha`` ~ U(0.5, 1), ``beta`` ~ U(0.05, 0.95);
* initial state: zeros (the first chunk of a prompt) or N(0, 0.1^2) (a later chunk).

The benchmark workload is the pages' 2K-token prompt ("Prefill > Keep recurrent state
on chip"); the head counts and the head width of 128 are a reading (the pages give
none): 16 key heads shared by 32 value heads.
"""

from __future__ import annotations

import dataclasses

import numpy as np

from .moe_inputs import f32_to_bf16_bits

TID_Q, TID_K, TID_V, TID_ALPHA, TID_BETA, TID_STATE = range(6)
GDN_SEED_BASE = 1 << 24  # keeps these streams apart from the MoE layer's


@dataclasses.dataclass(frozen=True)
class GdnShape:
    name: str
    T: int
    n_kheads: int
    n_vheads: int
    d: int = 128


GDN_CONFIGS = {
    0: GdnShape("gdn-small", T=37, n_kheads=2, n_vheads=4),
    1: GdnShape("gdn-2k", T=2048, n_kheads=16, n_vheads=32),
    2: GdnShape("gdn-one-head", T=70, n_kheads=1, n_vheads=1),
    3: GdnShape("gdn-no-sharing", T=33, n_kheads=3, n_vheads=3),
}


@dataclasses.dataclass
class GdnInputs:
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    alpha: np.ndarray
    beta: np.ndarray
    state: np.ndarray


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(GDN_SEED_BASE,) + key)))


def _unit_rows(g: np.ndarray) -> np.ndarray:
    n = np.sqrt((g.astype(np.float64) ** 2).sum(-1, keepdims=True))
    return (g / n).astype(np.float32)


def make_gdn(shape: GdnShape, seed: int = 0, nonzero_state: bool = False, cfg_key: int = 0) -> GdnInputs:
    T, hk, hv, d = shape.T, shape.n_kheads, shape.n_vheads, shape.d
    q = _unit_rows(_rng(seed, cfg_key, TID_Q).standard_normal((T, hk, d), dtype=np.float32))
    q = f32_to_bf16_bits(q * np.float32(d ** -0.5))
    k = f32_to_bf16_bits(_unit_rows(_rng(seed, cfg_key, TID_K).standard_normal((T, hk, d), dtype=np.float32)))
    v = f32_to_bf16_bits(_rng(seed, cfg_key, TID_V).standard_normal((T, hv, d), dtype=np.float32))
    alpha = _rng(seed, cfg_key, TID_ALPHA).uniform(0.5, 1.0, (T, hv)).astype(np.float32)
    beta = _rng(seed, cfg_key, TID_BETA).uniform(0.05, 0.95, (T, hv)).astype(np.float32)
    if nonzero_state:
        state = (_rng(seed, cfg_key, TID_STATE).standard_normal((hv, d, d), dtype=np.float32) * np.float32(0.1))
    else:
        state = np.zeros((hv, d, d), np.float32)
    return GdnInputs(q, k, v, alpha, beta, state)


def gdn_inputs(cfg: int, seed: int = 0, nonzero_state: bool = False) -> GdnInputs:
    return make_gdn(GDN_CONFIGS[cfg], seed=seed, nonzero_state=nonzero_state, cfg_key=cfg)
