"""ctypes binding of librewy.so -- argument marshalling only.

The functions here carry the C ABI's names (include/rewy.h) and forward their
arguments unchanged; every step of the operator runs in the HIP kernels.  If
the library is not built the first call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librewy.so")

REWY_OK, REWY_EINVAL, REWY_EUNSUPPORTED, REWY_EWORKSPACE, REWY_EHIP = 0, -1, -2, -3, -4
REWY_GATE_NONE, REWY_GATE_SCALAR, REWY_GATE_VECTOR = 0, 1, 2
REWY_BF16, REWY_F32 = 0, 1
REWY_RECOMPUTE, REWY_SAVE = 0, 1
REWY_SCHEDULE_JOINT, REWY_SCHEDULE_SEPARATE = 0, 1

NOALLOC_SCRATCH_BYTES = 128 << 20  # REWY_NOALLOC_SCRATCH_BYTES

EXPORTS = ("rewy_workspace_bytes", "rewy_saved_bytes", "rewy_fwd", "rewy_bwd", "rewy_fwd_noalloc",
           "rewy_fwd_gdn2",
           "rewy_bwd_gdn2", "rewy_fwd_kda_gate", "rewy_bwd_kda_gate", "rewy_recurrent_fwd",
           "rewy_recurrent_fwd_gdn2",
           "rewy_bwd_schedule", "rewy_trace_begin", "rewy_trace_end", "rewy_trace_select",
           "rewy_status_string",
           "rewy_last_error")


class RewyDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
        ("K", ctypes.c_int32), ("V", ctypes.c_int32), ("N", ctypes.c_int32),
        ("cu_seqlens", ctypes.c_void_p), ("cu_seqlens_host", ctypes.c_void_p),
        ("dtype", ctypes.c_int32), ("beta_dtype", ctypes.c_int32), ("gate", ctypes.c_int32),
        ("policy", ctypes.c_int32), ("scale", ctypes.c_float),
    ]


class RewyTraceEntry(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_char * 96), ("total_ms", ctypes.c_double),
                ("launches", ctypes.c_int)]


class RewyError(RuntimeError):
    def __init__(self, status, where):
        lib = load()
        super().__init__(f"{where}: {lib.rewy_status_string(status).decode()} "
                         f"({lib.rewy_last_error().decode()})")
        self.status = status


_lib = None


def load():
    """Load librewy.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        lib = ctypes.CDLL(LIB_PATH)
        P, S = ctypes.c_void_p, ctypes.c_size_t
        D = ctypes.POINTER(RewyDesc)
        lib.rewy_workspace_bytes.argtypes = [D, ctypes.c_int]
        lib.rewy_workspace_bytes.restype = S
        lib.rewy_saved_bytes.argtypes = [D]
        lib.rewy_saved_bytes.restype = S
        lib.rewy_fwd.argtypes = [D, P, P, P, P, P, P, P, P, P, P, S, P]
        lib.rewy_fwd.restype = ctypes.c_int
        lib.rewy_bwd.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, S, P]
        lib.rewy_bwd.restype = ctypes.c_int
        lib.rewy_fwd_noalloc.argtypes = [D, P, P, P, P, P, P, P, P, P, P]
        lib.rewy_fwd_noalloc.restype = ctypes.c_int
        lib.rewy_fwd_gdn2.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, S, P]
        lib.rewy_fwd_gdn2.restype = ctypes.c_int
        lib.rewy_bwd_gdn2.argtypes = [D] + [P] * 18 + [S, P]
        lib.rewy_bwd_gdn2.restype = ctypes.c_int
        F = ctypes.c_float
        lib.rewy_fwd_kda_gate.argtypes = [D] + [P] * 6 + [F] + [P] * 6 + [S, P]
        lib.rewy_fwd_kda_gate.restype = ctypes.c_int
        lib.rewy_bwd_kda_gate.argtypes = [D] + [P] * 6 + [F] + [P] * 14 + [S, P]
        lib.rewy_bwd_kda_gate.restype = ctypes.c_int
        lib.rewy_recurrent_fwd.argtypes = [D, P, P, P, P, P, P, P, P, P]
        lib.rewy_recurrent_fwd.restype = ctypes.c_int
        lib.rewy_recurrent_fwd_gdn2.argtypes = [D] + [P] * 10
        lib.rewy_recurrent_fwd_gdn2.restype = ctypes.c_int
        lib.rewy_bwd_schedule.argtypes = [ctypes.c_int]
        lib.rewy_bwd_schedule.restype = ctypes.c_int
        lib.rewy_trace_begin.argtypes = []
        lib.rewy_trace_begin.restype = ctypes.c_int
        lib.rewy_trace_end.argtypes = [ctypes.POINTER(RewyTraceEntry), ctypes.c_int]
        lib.rewy_trace_end.restype = ctypes.c_int
        lib.rewy_trace_select.argtypes = [ctypes.c_char_p]
        lib.rewy_trace_select.restype = ctypes.c_int
        lib.rewy_status_string.argtypes = [ctypes.c_int]
        lib.rewy_status_string.restype = ctypes.c_char_p
        lib.rewy_last_error.argtypes = []
        lib.rewy_last_error.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def rewy_workspace_bytes(desc: RewyDesc, phase: int) -> int:
    return load().rewy_workspace_bytes(ctypes.byref(desc), phase)


def rewy_saved_bytes(desc: RewyDesc) -> int:
    return load().rewy_saved_bytes(ctypes.byref(desc))


def rewy_fwd(desc, q, k, v, g, beta, h0, o, ht, saved, workspace, ws_bytes, stream) -> int:
    return load().rewy_fwd(ctypes.byref(desc), q, k, v, g, beta, h0, o, ht, saved, workspace,
                           ws_bytes, stream)


def rewy_fwd_noalloc(desc, q, k, v, g, beta, h0, o, ht, saved, stream) -> int:
    return load().rewy_fwd_noalloc(ctypes.byref(desc), q, k, v, g, beta, h0, o, ht, saved, stream)


def rewy_bwd(desc, q, k, v, g, beta, h0, dO, dht, saved, dq, dk, dv, dg, dbeta, dh0, workspace,
             ws_bytes, stream) -> int:
    return load().rewy_bwd(ctypes.byref(desc), q, k, v, g, beta, h0, dO, dht, saved, dq, dk, dv,
                           dg, dbeta, dh0, workspace, ws_bytes, stream)


def rewy_fwd_gdn2(desc, q, k, v, g, b, w, h0, o, ht, saved, workspace, ws_bytes, stream) -> int:
    return load().rewy_fwd_gdn2(ctypes.byref(desc), q, k, v, g, b, w, h0, o, ht, saved, workspace,
                                ws_bytes, stream)


def rewy_bwd_gdn2(desc, q, k, v, g, b, w, h0, dO, dht, saved, dq, dk, dv, dg, db, dw, dh0,
                  workspace, ws_bytes, stream) -> int:
    return load().rewy_bwd_gdn2(ctypes.byref(desc), q, k, v, g, b, w, h0, dO, dht, saved, dq, dk,
                                dv, dg, db, dw, dh0, workspace, ws_bytes, stream)


def rewy_fwd_kda_gate(desc, q, k, v, x, a_log, dt_bias, lower_bound, beta, h0, o, ht, saved,
                      workspace, ws_bytes, stream) -> int:
    return load().rewy_fwd_kda_gate(ctypes.byref(desc), q, k, v, x, a_log, dt_bias, lower_bound,
                                    beta, h0, o, ht, saved, workspace, ws_bytes, stream)


def rewy_bwd_kda_gate(desc, q, k, v, x, a_log, dt_bias, lower_bound, beta, h0, dO, dht, saved, dq,
                      dk, dv, dx, da_log, ddt_bias, dbeta, dh0, workspace, ws_bytes, stream) -> int:
    return load().rewy_bwd_kda_gate(ctypes.byref(desc), q, k, v, x, a_log, dt_bias, lower_bound,
                                    beta, h0, dO, dht, saved, dq, dk, dv, dx, da_log, ddt_bias,
                                    dbeta, dh0, workspace, ws_bytes, stream)


def rewy_recurrent_fwd(desc, q, k, v, g, beta, h0, o, ht, stream) -> int:
    return load().rewy_recurrent_fwd(ctypes.byref(desc), q, k, v, g, beta, h0, o, ht, stream)


def rewy_recurrent_fwd_gdn2(desc, q, k, v, g, b, w, h0, o, ht, stream) -> int:
    return load().rewy_recurrent_fwd_gdn2(ctypes.byref(desc), q, k, v, g, b, w, h0, o, ht, stream)


def rewy_bwd_schedule(schedule: int) -> int:
    """Set the chunk backward's schedule for later calls (REWY_SCHEDULE_JOINT or
    REWY_SCHEDULE_SEPARATE); returns the previous one (a negative argument only
    queries)."""
    rc = load().rewy_bwd_schedule(schedule)
    if rc < 0 and schedule >= 0:
        raise RewyError(rc, "rewy_bwd_schedule")
    return rc


def rewy_trace_begin() -> int:
    return load().rewy_trace_begin()


def rewy_trace_select(stage=None) -> int:
    """Trace only the launches of kernel `stage` (e.g. "k_fwd_prep"); None: all."""
    rc = load().rewy_trace_select(None if stage is None else stage.encode())
    if rc < 0:
        raise RewyError(rc, "rewy_trace_select")
    return rc


def rewy_trace_end(cap: int = 32):
    """Returns [(kernel, total_ms, launches)] or raises on a negative status."""
    buf = (RewyTraceEntry * cap)()
    n = load().rewy_trace_end(buf, cap)
    if n < 0:
        raise RewyError(n, "rewy_trace_end")
    return [(buf[i].kernel.decode(), buf[i].total_ms, buf[i].launches) for i in range(min(n, cap))]


def rewy_status_string(status: int) -> str:
    return load().rewy_status_string(status).decode()


def rewy_last_error() -> str:
    return load().rewy_last_error().decode()
