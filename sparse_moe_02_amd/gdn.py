"""Gated DeltaNet prefill scan on device tensors (argument marshalling for
``moe_gdn_scan`` of ``include/gdn.h``; every step runs in the HIP kernel)."""

from __future__ import annotations

import torch

from . import binding as B

D = 128


def _ptr(t: torch.Tensor) -> int:
    return t.data_ptr()


def gdn_scan(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor, beta: torch.Tensor,
             state: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Scan T tokens.  q, k: bf16 [T][n_kheads][128]; v: bf16 [T][n_vheads][128]; alpha, beta:
    float32 [T][n_vheads]; state: float32 [n_vheads][128][128], updated in place.
    Returns out (bf16 [T][n_vheads][128])."""
    T, hk, dk = k.shape
    hv, dv = v.shape[1], v.shape[2]
    for name, t, dt in (("q", q, torch.bfloat16), ("k", k, torch.bfloat16), ("v", v, torch.bfloat16),
                        ("alpha", alpha, torch.float32), ("beta", beta, torch.float32),
                        ("state", state, torch.float32)):
        if t.dtype != dt or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name}: contiguous {dt} device tensor required")
    if q.shape != k.shape or v.shape[0] != T or alpha.shape != (T, hv) or beta.shape != (T, hv):
        raise ValueError("shape mismatch")
    if state.shape != (hv, dv, dk):
        raise ValueError("state must be [n_vheads][d_v][d_k]")
    if out is None:
        out = torch.empty((T, hv, dv), dtype=torch.bfloat16, device=v.device)
    s = stream if stream is not None else torch.cuda.current_stream(v.device).cuda_stream
    B.moe_gdn_scan(T, hk, hv, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state), _ptr(out),
                   s)
    return out
