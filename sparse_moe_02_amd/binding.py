"""ctypes binding of ``include/moe.h`` -- argument marshalling only.

Every function keeps the C name and raises :class:`MoeError` on a non-OK status.
All computation happens in the HIP library (``libmoe_mi355x.so``); if it has not been
built, loading fails loudly -- there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mi355x.so")

MOE_BF16, MOE_FP16, MOE_FP32 = 0, 1, 2
MOE_OK = 0
MOE_STAGE_ROUTE, MOE_STAGE_GROUP, MOE_STAGE_GATEUP, MOE_STAGE_DOWN, MOE_STAGE_FINAL = range(5)
MOE_PREFILL_STAGES = 5
MOE_DSTAGE_LAYER = 0
MOE_DECODE_STAGES = 1
PREFILL_STAGE_NAMES = ("route", "group", "gateup", "down", "final")
DECODE_STAGE_NAMES = ("layer",)
CTRL_DECODE_ERR_OFFSET = 88  # byte offset of the decode wait-failure word in the workspace

STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_NULL", 2: "MOE_ERR_SHAPE", 3: "MOE_ERR_DTYPE", 4: "MOE_ERR_ALIGN",
                5: "MOE_ERR_WORKSPACE", 6: "MOE_ERR_TOKENS", 7: "MOE_ERR_DEVICE", 8: "MOE_ERR_HIP",
                9: "MOE_ERR_ALIAS", 10: "MOE_ERR_ALLOC", 11: "MOE_ERR_WAIT"}
(MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_ALIGN, MOE_ERR_WORKSPACE, MOE_ERR_TOKENS, MOE_ERR_DEVICE,
 MOE_ERR_HIP, MOE_ERR_ALIAS, MOE_ERR_ALLOC, MOE_ERR_WAIT) = range(1, 12)
assert all(STATUS_NAMES[globals()[n] if n != "MOE_OK" else 0] == n for n in STATUS_NAMES.values())

# moe_config.flags (include/moe.h)
MOE_F_NONE = 0


def MOE_F_FORCE_BM(rows: int) -> int:
    return (rows // 32) & 0xF


MOE_F_NO_FALLBACK = 1 << 4
MOE_F_SEPARATE_DEQUANT = 1 << 5
MOE_F_HOST_ROUTING = 1 << 6

EXPORTED = ("moe_plan_create", "moe_plan_destroy", "moe_workspace_init", "moe_workspace_check",
            "moe_forward_prefill", "moe_forward_decode", "moe_forward_decode_batch", "moe_forward_decode_static",
            "moe_pack_qparams",
            "moe_pack_codes", "moe_status_string", "moe_version", "moe_gdn_scan")


class moe_config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("group_size", ctypes.c_int32), ("router_dtype", ctypes.c_int),
                ("qparam_dtype", ctypes.c_int), ("max_chunk_tokens", ctypes.c_int32),
                ("flags", ctypes.c_uint32)]


class moe_qmat(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("bias", ctypes.c_void_p)]


class moe_weights(ctypes.Structure):
    _fields_ = [("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p), ("gate", moe_qmat),
                ("up", moe_qmat), ("down", moe_qmat), ("s_gate", moe_qmat), ("s_up", moe_qmat),
                ("s_down", moe_qmat), ("shared_gate", ctypes.c_void_p)]


class moe_debug_out(ctypes.Structure):
    _fields_ = [("topk_ids", ctypes.c_void_p), ("gates", ctypes.c_void_p), ("counts", ctypes.c_void_p),
                ("offsets", ctypes.c_void_p), ("row_token", ctypes.c_void_p), ("n_refined", ctypes.c_void_p),
                ("events", ctypes.c_void_p), ("logits32", ctypes.c_void_p), ("radii32", ctypes.c_void_p)]


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)} ({status_string(status)})")


_lock = threading.Lock()
_lib = None


def lib() -> ctypes.CDLL:
    """Load the HIP library; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                                   "(there is no CPU fallback)")
            L = ctypes.CDLL(LIB_PATH)
            P, I64, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
            L.moe_plan_create.restype = ctypes.c_int
            L.moe_plan_create.argtypes = [ctypes.POINTER(moe_config), ctypes.POINTER(moe_weights),
                                          ctypes.POINTER(P), ctypes.POINTER(SZ)]
            L.moe_plan_destroy.restype = None
            L.moe_plan_destroy.argtypes = [P]
            L.moe_workspace_init.restype = ctypes.c_int
            L.moe_workspace_init.argtypes = [P, P, SZ, P]
            L.moe_workspace_check.restype = ctypes.c_int
            L.moe_workspace_check.argtypes = [P, P, SZ, P]
            L.moe_forward_prefill.restype = ctypes.c_int
            L.moe_forward_prefill.argtypes = [P, P, I64, P, P, SZ, P, ctypes.POINTER(moe_debug_out)]
            L.moe_forward_decode.restype = ctypes.c_int
            L.moe_forward_decode.argtypes = [P, P, P, P, SZ, P, ctypes.POINTER(moe_debug_out)]
            L.moe_forward_decode_batch.restype = ctypes.c_int
            L.moe_forward_decode_batch.argtypes = [P, P, ctypes.c_int32, P, P, SZ, P, ctypes.POINTER(moe_debug_out)]
            L.moe_forward_decode_static.restype = ctypes.c_int
            L.moe_forward_decode_static.argtypes = [P, P, P, P, ctypes.POINTER(moe_debug_out)]
            L.moe_pack_qparams.restype = ctypes.c_int
            L.moe_pack_qparams.argtypes = [P, P, I64, ctypes.c_int32, P]
            L.moe_pack_codes.restype = ctypes.c_int
            L.moe_pack_codes.argtypes = [P, P, I64, ctypes.c_int32, P]
            L.moe_gdn_scan.restype = ctypes.c_int
            L.moe_gdn_scan.argtypes = [ctypes.c_int32] * 5 + [P] * 7 + [P]
            L.moe_status_string.restype = ctypes.c_char_p
            L.moe_status_string.argtypes = [ctypes.c_int]
            L.moe_version.restype = ctypes.c_char_p
            L.moe_version.argtypes = []
            _lib = L
    return _lib


def _check(fn: str, st: int):
    if st != MOE_OK:
        raise MoeError(fn, st)


def moe_status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def status_string(status: int) -> str:
    try:
        return moe_status_string(status)
    except Exception:  # library not loadable: name only
        return STATUS_NAMES.get(status, str(status))


def moe_version() -> str:
    return lib().moe_version().decode()


def moe_plan_create(cfg: moe_config, weights: moe_weights):
    """Returns (plan handle, workspace bytes)."""
    plan = ctypes.c_void_p()
    ws = ctypes.c_size_t()
    _check("moe_plan_create", lib().moe_plan_create(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(plan),
                                                    ctypes.byref(ws)))
    return plan, ws.value


def moe_plan_destroy(plan) -> None:
    lib().moe_plan_destroy(plan)


def moe_workspace_init(plan, ws_ptr: int, ws_bytes: int, stream: int) -> None:
    _check("moe_workspace_init", lib().moe_workspace_init(plan, ws_ptr, ws_bytes, stream))


def moe_workspace_check(plan, ws_ptr: int, ws_bytes: int, stream: int) -> int:
    """MOE_OK or MOE_ERR_WAIT (returned, not raised); raises on other statuses."""
    st = lib().moe_workspace_check(plan, ws_ptr, ws_bytes, stream)
    if st not in (MOE_OK, MOE_ERR_WAIT):
        raise MoeError("moe_workspace_check", st)
    return st


def moe_forward_prefill(plan, x_ptr: int, T: int, out_ptr: int, ws_ptr: int, ws_bytes: int, stream: int,
                        dbg: moe_debug_out | None = None) -> None:
    _check("moe_forward_prefill", lib().moe_forward_prefill(plan, x_ptr, T, out_ptr, ws_ptr, ws_bytes, stream,
                                                            ctypes.byref(dbg) if dbg is not None else None))


def moe_forward_decode(plan, x_ptr: int, out_ptr: int, ws_ptr: int, ws_bytes: int, stream: int,
                       dbg: moe_debug_out | None = None) -> None:
    _check("moe_forward_decode", lib().moe_forward_decode(plan, x_ptr, out_ptr, ws_ptr, ws_bytes, stream,
                                                          ctypes.byref(dbg) if dbg is not None else None))


def moe_forward_decode_batch(plan, x_ptr: int, T: int, out_ptr: int, ws_ptr: int, ws_bytes: int, stream: int,
                             dbg: moe_debug_out | None = None) -> None:
    _check("moe_forward_decode_batch", lib().moe_forward_decode_batch(plan, x_ptr, T, out_ptr, ws_ptr, ws_bytes,
                                                                      stream,
                                                                      ctypes.byref(dbg) if dbg is not None else None))


def moe_forward_decode_static(plan, x_ptr: int, out_ptr: int, stream: int, dbg: moe_debug_out | None = None) -> None:
    _check("moe_forward_decode_static", lib().moe_forward_decode_static(plan, x_ptr, out_ptr, stream,
                                                                        ctypes.byref(dbg) if dbg is not None else None))


def moe_gdn_scan(T: int, n_kheads: int, n_vheads: int, d_k: int, d_v: int, q_ptr: int, k_ptr: int, v_ptr: int,
                 alpha_ptr: int, beta_ptr: int, state_ptr: int, out_ptr: int, stream: int) -> None:
    _check("moe_gdn_scan", lib().moe_gdn_scan(T, n_kheads, n_vheads, d_k, d_v, q_ptr, k_ptr, v_ptr, alpha_ptr,
                                              beta_ptr, state_ptr, out_ptr, stream))


def moe_pack_qparams(src_ptr: int, dst_ptr: int, rows: int, k: int, stream: int) -> None:
    _check("moe_pack_qparams", lib().moe_pack_qparams(src_ptr, dst_ptr, rows, k, stream))


def moe_pack_codes(src_ptr: int, dst_ptr: int, rows: int, k: int, stream: int) -> None:
    _check("moe_pack_codes", lib().moe_pack_codes(src_ptr, dst_ptr, rows, k, stream))


# ---------------------------------------------------------------- HIP events (timing)

_hip = None


def hip() -> ctypes.CDLL:
    global _hip
    if _hip is None:
        h = ctypes.CDLL("libamdhip64.so")
        P = ctypes.c_void_p
        h.hipEventCreate.argtypes = [ctypes.POINTER(P)]
        h.hipEventRecord.argtypes = [P, P]
        h.hipEventSynchronize.argtypes = [P]
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), P, P]
        h.hipEventDestroy.argtypes = [P]
        _hip = h
    return _hip


class HipEvents:
    """An array of hipEvent_t usable as moe_debug_out.events."""

    def __init__(self, n: int):
        self.n = n
        self.arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            if hip().hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.arr[i] = ev.value

    @property
    def ptr(self) -> int:
        return ctypes.addressof(self.arr)

    def record(self, i: int, stream: int) -> None:
        if hip().hipEventRecord(self.arr[i], stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, i: int, j: int) -> float:
        ms = ctypes.c_float()
        hip().hipEventSynchronize(self.arr[j])
        if hip().hipEventElapsedTime(ctypes.byref(ms), self.arr[i], self.arr[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self) -> None:
        for i in range(self.n):
            if self.arr[i]:
                hip().hipEventDestroy(self.arr[i])
                self.arr[i] = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
