"""CPU oracle for the sparse MoE feed-forward layer (binary64, plain loops).

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg are the only callers.  The HIP library in
``sparse_moe_02_amd`` never imports this package, and this package never imports
that one; the two share only the seeded inputs from ``synth``.

The arithmetic lives in ``moe_oracle.c`` (the MoE layer) and ``gdn_oracle.c`` (the
Gated DeltaNet prefill scan); see their headers for what is computed and which
passage of "Optimizing on-device inference for Apple Silicon" each step follows.
This module only builds them with gcc, loads them and marshals numpy arrays.

Parity unpinned: nothing.  Every function here is pinned by tests under
``tests/`` that do not reuse its formulas (brute force over subsets, library
routines on special cases, closed forms, invariants).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "moe_oracle.c"), os.path.join(_HERE, "gdn_oracle.c")]
_LIB = os.path.join(_HERE, "libmoe_oracle.so")
_lock = threading.Lock()
_lib = None


def build() -> str:
    """Compile the oracle with gcc (always recompiles)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-std=c11", "-Wall", "-o", tmp, *_SRCS, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def lib() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build()
            L = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            I64 = ctypes.c_int64
            L.oracle_fp16_to_double.restype = ctypes.c_double
            L.oracle_fp16_to_double.argtypes = [ctypes.c_uint16]
            L.oracle_bf16_to_double.restype = ctypes.c_double
            L.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
            L.oracle_max_threads.restype = ctypes.c_int
            L.oracle_dequant.restype = None
            L.oracle_dequant.argtypes = [P, P, P, I64, I64, ctypes.c_int, P]
            L.oracle_route.restype = ctypes.c_int
            L.oracle_route.argtypes = [P, I64, I64, I64, I64, P, ctypes.c_int, P, P, P, P, P]
            L.oracle_group.restype = ctypes.c_int
            L.oracle_group.argtypes = [P, I64, I64, I64, P, P, P, P]
            L.oracle_experts.restype = ctypes.c_int
            L.oracle_experts.argtypes = [P, I64, I64, I64, I64, I64, P, P] + [P] * 9 + [ctypes.c_int, P, P]
            L.oracle_gdn_scan.restype = ctypes.c_int
            L.oracle_gdn_scan.argtypes = [P] * 5 + [I64] * 5 + [P, P]
            _lib = L
    return _lib


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def threads() -> int:
    return lib().oracle_max_threads()


def fp16_to_double(bits: int) -> float:
    return lib().oracle_fp16_to_double(int(bits))


def bf16_to_double(bits: int) -> float:
    return lib().oracle_bf16_to_double(int(bits))


def _qparam_bits(a):
    """Scale/bias arrays: float16 values, or bf16 bit patterns as uint16.  Returns
    (uint16 bits, is_bf16)."""
    if a.dtype == np.float16:
        return _c(a, np.float16).view(np.uint16), False
    assert a.dtype == np.uint16, "scale/bias: float16 values or bf16 bits (uint16)"
    return _c(a, np.uint16), True


def dequant(q, scale, bias) -> np.ndarray:
    """Dequantise one matrix: q uint32 [N][K/8], scale/bias [N][K/64] (float16, or bf16 bits
    as uint16) -> float64 [N][K]."""
    q = _c(q, np.uint32)
    s, sbf = _qparam_bits(scale)
    b, bbf = _qparam_bits(bias)
    assert sbf == bbf
    N, K = q.shape[0], q.shape[1] * 8
    assert s.shape == (N, K // 64) and b.shape == (N, K // 64)
    w = np.empty((N, K), np.float64)
    lib().oracle_dequant(_p(q), _p(s), _p(b), N, K, int(sbf), _p(w))
    return w


def route(x_bits, router_w, router_b, k: int):
    """Logits, chosen experts (ascending), gates and selection order for each token."""
    x = _c(x_bits, np.uint16)
    T, H = x.shape
    fp32 = router_w.dtype == np.float32
    rw = _c(router_w, np.float32 if fp32 else np.uint16)
    E = rw.shape[0]
    assert rw.shape == (E, H)
    rb = None if router_b is None else _c(router_b, np.float32)
    logits = np.empty((T, E), np.float64)
    ids = np.empty((T, k), np.int32)
    gates = np.empty((T, k), np.float64)
    ranked = np.empty((T, k), np.int32)
    rc = lib().oracle_route(_p(x), T, H, E, k, _p(rw), int(fp32), _p(rb), _p(logits), _p(ids),
                            _p(gates), _p(ranked))
    if rc != 0:
        raise ValueError(f"oracle_route failed ({rc})")
    return {"logits": logits, "ids": ids, "gates": gates, "ranked": ranked}


def group(ids, E: int):
    """Histogram (E+1 bins), offsets (E+2), grouped row order and slot map."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    counts = np.empty(E + 1, np.int32)
    offsets = np.empty(E + 2, np.int32)
    row_token = np.empty(T * (k + 1), np.int32)
    slot_row = np.empty((T, k + 1), np.int32)
    rc = lib().oracle_group(_p(ids), T, E, k, _p(counts), _p(offsets), _p(row_token), _p(slot_row))
    if rc != 0:
        raise ValueError(f"oracle_group failed ({rc})")
    return {"counts": counts, "offsets": offsets, "row_token": row_token, "slot_row": slot_row}


def experts(x_bits, layer, ids, gates) -> np.ndarray:
    """Routed experts + shared expert + gate-weighted combine -> float64 [T][H]."""
    x = _c(x_bits, np.uint16)
    T, H = x.shape
    ids = _c(ids, np.int32)
    gates = _c(gates, np.float64)
    k = ids.shape[1]
    E = layer.gate_q.shape[0] - 1
    I = layer.gate_q.shape[1]
    arrs, kinds = [], set()
    for nm in ("gate", "up", "down"):
        arrs.append(_c(getattr(layer, nm + "_q"), np.uint32))
        for part in ("_s", "_b"):
            bits, is_bf = _qparam_bits(getattr(layer, nm + part))
            arrs.append(bits)
            kinds.add(is_bf)
    assert len(kinds) == 1, "all scale/bias arrays of a layer share one dtype"
    sg = getattr(layer, "shared_gate", None)
    sg = None if sg is None else _c(sg, np.uint16)
    assert sg is None or sg.shape == (H,)
    out = np.empty((T, H), np.float64)
    rc = lib().oracle_experts(_p(x), T, H, I, E, k, _p(ids), _p(gates), *[_p(a) for a in arrs], int(kinds.pop()),
                              _p(sg), _p(out))
    if rc != 0:
        raise ValueError(f"oracle_experts failed ({rc})")
    return out


def forward(x_bits, layer, k: int):
    """The whole layer: route, group, experts.  Returns a dict with every stage."""
    r = route(x_bits, layer.router_w, layer.router_b, k)
    E = layer.gate_q.shape[0] - 1
    g = group(r["ids"], E)
    out = experts(x_bits, layer, r["ids"], r["gates"])
    r.update(g)
    r["out"] = out
    return r


def gdn_scan(q_bits, k_bits, v_bits, alpha, beta, state=None):
    """Gated DeltaNet scan over T tokens.  q_bits, k_bits: bf16 bits uint16 [T][n_kheads][d_k];
    v_bits: uint16 [T][n_vheads][d_v]; alpha, beta: float32 [T][n_vheads]; state: S_0
    [n_vheads][d_v][d_k] (any float dtype; zeros if None).  Returns (out float64
    [T][n_vheads][d_v], S_T float64)."""
    q = _c(q_bits, np.uint16)
    k = _c(k_bits, np.uint16)
    v = _c(v_bits, np.uint16)
    T, hk, dk = k.shape
    assert q.shape == k.shape
    hv, dv = v.shape[1], v.shape[2]
    assert v.shape[0] == T
    a = _c(alpha, np.float32).reshape(T, hv)
    b = _c(beta, np.float32).reshape(T, hv)
    S = np.zeros((hv, dv, dk), np.float64) if state is None else np.array(state, dtype=np.float64, copy=True)
    assert S.shape == (hv, dv, dk)
    S = np.ascontiguousarray(S)
    out = np.empty((T, hv, dv), np.float64)
    rc = lib().oracle_gdn_scan(_p(q), _p(k), _p(v), _p(a), _p(b), T, hk, hv, dk, dv, _p(S), _p(out))
    if rc != 0:
        raise ValueError(f"oracle_gdn_scan failed ({rc})")
    return out, S
