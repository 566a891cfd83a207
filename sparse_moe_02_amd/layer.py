"""Convenience wrapper: holds one layer's device tensors, its plan and a workspace.

PyTorch is used for device memory and streams only; every step of the layer runs in
the HIP library through the C ABI (see ``binding.py``).
"""

from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import binding as B


def _dev(a: np.ndarray, device) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    view = {np.dtype(np.uint16): np.int16, np.dtype(np.float16): np.int16,
            np.dtype(np.uint32): np.int32}.get(a.dtype)
    if view is not None:
        a = a.view(view)
    return torch.from_numpy(a).to(device)


class MoeLayer:
    """One MoE layer on one GPU.

    ``weights`` holds numpy arrays: ``router_w`` [E][H] (uint16 bf16 bits or float32),
    ``router_b`` [E] float32 or None, and ``{gate,up,down}_{q,s,b}`` stacked over E+1
    experts (the shared expert last), codes row-major [E+1][N][K/8] and scale and bias
    row-major [E+1][N][K/64].  All three are rewritten on the device into the library's
    tile layouts (``moe_pack_codes``, ``moe_pack_qparams``).
    """

    def __init__(self, weights, top_k: int, max_chunk_tokens: int = 4096, device: str = "cuda:0",
                 flags: int = 0):
        self.device = torch.device(device)
        E1, I, H8 = weights.gate_q.shape
        self.E, self.I, self.H, self.k = E1 - 1, I, H8 * 8, top_k
        self.chunk = max_chunk_tokens
        self.t = {}
        for name in ("router_w", "router_b", "gate_q", "gate_s", "gate_b", "up_q", "up_s", "up_b",
                     "down_q", "down_s", "down_b", "shared_gate"):
            a = getattr(weights, name, None)
            self.t[name] = None if a is None else _dev(a, self.device)
            if name in ("gate_s", "gate_b", "up_s", "up_b", "down_s", "down_b"):
                self.t[name] = self._tiled(self.t[name])
            elif name in ("gate_q", "up_q", "down_q"):
                self.t[name] = self._tiled_codes(self.t[name])
        fp32_router = weights.router_w.dtype == np.float32
        # scale/bias: float16 values, or bf16 bit patterns stored as uint16
        qbf16 = weights.gate_s.dtype == np.uint16
        self.cfg = B.moe_config(hidden=self.H, inter=self.I, n_experts=self.E, top_k=top_k, group_size=64,
                                router_dtype=B.MOE_FP32 if fp32_router else B.MOE_BF16,
                                qparam_dtype=B.MOE_BF16 if qbf16 else B.MOE_FP16,
                                max_chunk_tokens=max_chunk_tokens, flags=flags)
        self.w = B.moe_weights()
        self.w.router_w = self.t["router_w"].data_ptr()
        self.w.router_bias = self.t["router_b"].data_ptr() if self.t["router_b"] is not None else None
        self.w.shared_gate = self.t["shared_gate"].data_ptr() if self.t["shared_gate"] is not None else None
        for mat in ("gate", "up", "down"):
            q, s, b = self.t[mat + "_q"], self.t[mat + "_s"], self.t[mat + "_b"]
            setattr(self.w, mat, B.moe_qmat(q.data_ptr(), s.data_ptr(), b.data_ptr()))
            setattr(self.w, "s_" + mat, B.moe_qmat(q[self.E].data_ptr(), s[self.E].data_ptr(), b[self.E].data_ptr()))
        self.plan, self.ws_bytes = B.moe_plan_create(self.cfg, self.w)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        B.moe_workspace_init(self.plan, self.ws.data_ptr(), self.ws_bytes, self.stream())

    def with_flags(self, flags: int, max_chunk_tokens: int | None = None) -> "MoeLayer":
        """Another plan (own workspace) over this layer's device weights, with other flags."""
        other = MoeLayer.__new__(MoeLayer)
        other.device, other.E, other.I, other.H, other.k = self.device, self.E, self.I, self.H, self.k
        other.chunk = max_chunk_tokens or self.chunk
        other.t = self.t
        other.cfg = B.moe_config(hidden=self.H, inter=self.I, n_experts=self.E, top_k=self.k, group_size=64,
                                 router_dtype=self.cfg.router_dtype, qparam_dtype=self.cfg.qparam_dtype,
                                 max_chunk_tokens=other.chunk, flags=flags)
        other.w = self.w
        other.plan, other.ws_bytes = B.moe_plan_create(other.cfg, other.w)
        other.ws = torch.empty(other.ws_bytes, dtype=torch.uint8, device=self.device)
        B.moe_workspace_init(other.plan, other.ws.data_ptr(), other.ws_bytes, other.stream())
        return other

    def _tiled(self, rm: torch.Tensor) -> torch.Tensor:
        """fp16 bits [E+1][N][G] row-major -> the same values in 16-row tiles."""
        out = torch.empty_like(rm)
        rows, G = rm.shape[0] * rm.shape[1], rm.shape[2]
        B.moe_pack_qparams(rm.data_ptr(), out.data_ptr(), rows, 64 * G, self.stream())
        return out

    def _tiled_codes(self, rm: torch.Tensor) -> torch.Tensor:
        """uint32 codes [E+1][N][K/8] row-major -> the same words in 16 x 128 tiles."""
        out = torch.empty_like(rm)
        B.moe_pack_codes(rm.data_ptr(), out.data_ptr(), rm.shape[0] * rm.shape[1], 8 * rm.shape[2], self.stream())
        return out

    def stream(self) -> int:
        return torch.cuda.current_stream(self.device).cuda_stream

    def close(self) -> None:
        if getattr(self, "plan", None) is not None:
            B.moe_plan_destroy(self.plan)
            self.plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ------------------------------------------------------------------ forwards

    def _debug(self, T: int, decode: bool, events, outputs: bool = True, logits: bool = False):
        """The debug struct (and the tensors it points at).  outputs=False: events only."""
        nch = 1 if decode else (T + self.chunk - 1) // self.chunk
        d = {}
        if outputs:
            d["topk_ids"] = torch.empty((T, self.k), dtype=torch.int32, device=self.device)
            d["gates"] = torch.empty((T, self.k), dtype=torch.float32, device=self.device)
        if outputs and logits and not decode:
            d["logits32"] = torch.empty((T, self.E), dtype=torch.float32, device=self.device)
            d["radii32"] = torch.empty((T, self.E), dtype=torch.float32, device=self.device)
        if outputs and not decode:
            d["counts"] = torch.empty((nch, self.E + 1), dtype=torch.int32, device=self.device)
            d["offsets"] = torch.empty((nch, self.E + 2), dtype=torch.int32, device=self.device)
            d["row_token"] = torch.full((nch * self.chunk * (self.k + 1),), -1, dtype=torch.int32,
                                        device=self.device)
            d["n_refined"] = torch.zeros((nch,), dtype=torch.int32, device=self.device)
        s = B.moe_debug_out()
        for key, v in d.items():
            setattr(s, key, v.data_ptr())
        if events is not None:
            s.events = events.ptr
        return s, d

    def prefill(self, x: torch.Tensor, out: torch.Tensor | None = None, debug: bool = False, events=None,
                logits: bool = False):
        """x: bf16 [T][H] on the device.  Returns out (and the debug tensors when debug).
        events alone (debug False) records the stage events and writes no debug output."""
        assert x.dtype == torch.bfloat16 and x.is_contiguous() and x.shape[1] == self.H
        T = x.shape[0]
        if out is None:
            out = torch.empty_like(x)
        dbg, d = self._debug(T, False, events, debug, logits) if (debug or events is not None) else (None, None)
        B.moe_forward_prefill(self.plan, x.data_ptr(), T, out.data_ptr(), self.ws.data_ptr(), self.ws_bytes,
                              self.stream(), dbg)
        return (out, d) if debug else out

    def decode(self, x: torch.Tensor, out: torch.Tensor | None = None, debug: bool = False, events=None):
        """x: bf16 [H] (or [1][H]) on the device."""
        assert x.dtype == torch.bfloat16 and x.is_contiguous() and x.numel() == self.H
        if out is None:
            out = torch.empty_like(x)
        dbg, d = self._debug(1, True, events, debug) if (debug or events is not None) else (None, None)
        B.moe_forward_decode(self.plan, x.data_ptr(), out.data_ptr(), self.ws.data_ptr(), self.ws_bytes,
                             self.stream(), dbg)
        return (out, d) if debug else out

    def decode_batch(self, x: torch.Tensor, out: torch.Tensor | None = None, debug: bool = False, events=None):
        """x: bf16 [T][H] on the device, 1 <= T <= 8 (one launch for the T rows)."""
        assert x.dtype == torch.bfloat16 and x.is_contiguous() and x.dim() == 2 and x.shape[1] == self.H
        T = x.shape[0]
        if out is None:
            out = torch.empty_like(x)
        dbg, d = self._debug(T, True, events, debug) if (debug or events is not None) else (None, None)
        B.moe_forward_decode_batch(self.plan, x.data_ptr(), T, out.data_ptr(), self.ws.data_ptr(), self.ws_bytes,
                                   self.stream(), dbg)
        return (out, d) if debug else out

    def decode_error(self) -> int:
        """moe_workspace_check: 0 (MOE_OK) if every decode call so far completed its internal
        hand-offs, else MOE_ERR_WAIT; waits for the stream."""
        return B.moe_workspace_check(self.plan, self.ws.data_ptr(), self.ws_bytes, self.stream())


def bf16_tensor(bits: np.ndarray, device) -> torch.Tensor:
    """bf16 bit patterns (uint16 numpy) -> bf16 device tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


__all__ = ["MoeLayer", "bf16_tensor", "bf16_bits", "ctypes"]
