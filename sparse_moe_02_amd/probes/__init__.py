"""Measured ceilings (HBM read stream, MFMA loop on constant and on random operands, the
grouped GEMM's dequant + MFMA register pipeline, launch cost, the decode step's weight
stream with and without arithmetic) for the benchmark; see ``probes.hip``.

Built into ``libmoe_probes.so`` next to this file by ``sparse_moe_02_amd._build``; the
layer itself never loads it.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_probes.so")
_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, SZ, I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        L.probe_read_stream.argtypes = [P, SZ, P, I, P]
        L.probe_mfma.argtypes = [I, P, I, P]
        L.probe_empty.argtypes = [I, I, P]
        L.probe_mfma_data.argtypes = [P, I, P, I, P]
        L.probe_dequant_mfma.argtypes = [P, I, P, I, P]
        L.probe_expert_stream.argtypes = [ctypes.POINTER(P), P, I, I, I, P, I, P]
        L.probe_flat_stream.argtypes = [P, I, P, I, P]
        L.probe_ticket.argtypes = [P, I, I, I, P]
        L.probe_handoff.argtypes = [P, ctypes.c_uint32, I, I, I, P, I, P]
        for f in (L.probe_read_stream, L.probe_mfma, L.probe_mfma_data, L.probe_dequant_mfma, L.probe_empty, L.probe_expert_stream, L.probe_flat_stream,
                  L.probe_ticket, L.probe_handoff):
            f.restype = I
        _lib = L
    return _lib


def _ok(rc: int, name: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{name}: HIP error {rc}")


def read_stream(buf_ptr: int, nbytes: int, sink_ptr: int, grid: int, stream: int) -> None:
    _ok(lib().probe_read_stream(buf_ptr, nbytes, sink_ptr, grid, stream), "probe_read_stream")


def mfma(iters: int, sink_ptr: int, grid: int, stream: int) -> None:
    _ok(lib().probe_mfma(iters, sink_ptr, grid, stream), "probe_mfma")


def mfma_data(src_ptr: int, iters: int, sink_ptr: int, grid: int, stream: int) -> None:
    """src: grid * 8 * 64 * 16 bytes of operand data (10 MFMAs per loop iteration per wave)."""
    _ok(lib().probe_mfma_data(src_ptr, iters, sink_ptr, grid, stream), "probe_mfma_data")


def dequant_mfma(src_ptr: int, iters: int, sink_ptr: int, grid: int, stream: int) -> None:
    """src as for mfma_data (80 MFMAs and 16 dequantised words per iteration per wave)."""
    _ok(lib().probe_dequant_mfma(src_ptr, iters, sink_ptr, grid, stream), "probe_dequant_mfma")


def empty(grid: int, threads: int, stream: int) -> None:
    _ok(lib().probe_empty(grid, threads, stream), "probe_empty")


def expert_stream(mats, x_ptr: int, H: int, I: int, arith: bool, sink_ptr: int, grid: int, stream: int) -> None:
    """mats: 81 device pointers, [slot 0..8][gate, up, down][codes, scale, bias]."""
    arr = (ctypes.c_void_p * 81)(*mats)
    _ok(lib().probe_expert_stream(arr, x_ptr, H, I, int(arith), sink_ptr, grid, stream), "probe_expert_stream")


def flat_table(ptrs, nbytes):
    """The device-side segment table of probe_flat_stream (384 words: base addresses, sizes
    in 16-byte units, first workgroup of each segment) as a numpy array, and the grid."""
    import numpy as np

    n16 = [b // 16 for b in nbytes]
    wg = np.concatenate([[0], np.cumsum([-(-n // 1024) for n in n16])])
    t = np.zeros(384, np.uint64)
    t[:len(ptrs)] = ptrs
    t[128:128 + len(ptrs)] = n16
    t[256:256 + len(ptrs) + 1] = wg
    return t, int(wg[-1])


def flat_stream(table_ptr: int, n: int, sink_ptr: int, grid: int, stream: int) -> None:
    """Read n device arrays (segment table at table_ptr, see flat_table) once, 16 KB per
    workgroup."""
    _ok(lib().probe_flat_stream(table_ptr, n, sink_ptr, grid, stream), "probe_flat_stream")
