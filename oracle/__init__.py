"""FP64 CPU oracle for the chunkwise gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never calls it and it
never calls the HIP library; the two share no code.

Two independent evaluations live here:

* ``forward`` / ``backward`` -- the token-by-token FP64 recurrence of the ReWY
  paper ("Background / Delta-rule operators", Table 1) and the KDA blog
  (section 4, boxed equations), with a hand-derived reverse mode.  This is the
  plain definition of the operator.  Compiled from ``rewy_oracle.c``.
* ``oracle.chunked`` -- a second FP64 evaluation in the chunked matrix form
  (ReWY paper Appendix A, Algorithm 1, Appendix sections 7-10) written with
  numpy library primitives.  It is the readable statement of what each chunk
  kernel must compute and is pinned against the token recurrence.

Shapes follow the operator: q, k [B,T,H,K]; v, dO [B,T,H,V]; g is None
(DeltaNet), [B,T,H] (scalar gate, GDN) or [B,T,H,K] (vector gate, KDA), the
natural-log decay; beta [B,T,H]; h0, dht [N,H,K,V].  With ``cu_seqlens``
(N+1 offsets) the batch dimension must be 1 and sequences are packed.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rewy_oracle.c")
_LIB = os.path.join(_HERE, "librewy_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (plain -O2, IEEE semantics, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
                               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.rewy_oracle_fwd.argtypes = [I64, P, I64, I64, I64, P, P, P, P, ctypes.c_int, P, P,
                                        ctypes.c_double, P, P, P, ctypes.c_int]
        lib.rewy_oracle_fwd.restype = ctypes.c_int
        lib.rewy_oracle_bwd.argtypes = [I64, P, I64, I64, I64, P, P, P, P, ctypes.c_int, P, P,
                                        ctypes.c_double, P, P, P, P, P, P, P, P, P, P,
                                        ctypes.c_int]
        lib.rewy_oracle_bwd.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor -> numpy, exact upcast
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    """Host threads for a call: the CPUs this process may run on, or
    OMP_NUM_THREADS when that is set lower.  The oracle hands one
    (sequence, head) unit to a thread at a time, so a call uses at most
    min(this, units) of them."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


class _Prob:
    """Flattened view of one call: tokens packed as [TT, H, *]."""

    def __init__(self, q, k, v, g, beta, erase, write, h0, cu_seqlens):
        q, k, v = _f64(q), _f64(k), _f64(v)
        if q.ndim != 4:
            raise ValueError("q must be [B,T,H,K]")
        B, T, H, K = q.shape
        V = v.shape[-1]
        if k.shape != q.shape or v.shape[:3] != q.shape[:3]:
            raise ValueError("q/k/v shape mismatch")
        if cu_seqlens is not None:
            if B != 1:
                raise ValueError("cu_seqlens requires B == 1")
            cu = np.asarray(cu_seqlens, dtype=np.int64).reshape(-1)
            if cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
                raise ValueError("bad cu_seqlens")
        else:
            cu = np.arange(B + 1, dtype=np.int64) * T
        self.B, self.T, self.H, self.K, self.V = B, T, H, K, V
        self.N = len(cu) - 1
        self.cu = np.ascontiguousarray(cu)
        TT = B * T
        self.q = q.reshape(TT, H, K)
        self.k = k.reshape(TT, H, K)
        self.v = v.reshape(TT, H, V)
        if g is None:
            self.gate_kind, self.g = 0, None
        else:
            g = _f64(g)
            if g.shape == (B, T, H):
                self.gate_kind, self.g = 1, g.reshape(TT, H)
            elif g.shape == (B, T, H, K):
                self.gate_kind, self.g = 2, g.reshape(TT, H, K)
            else:
                raise ValueError("g must be [B,T,H] or [B,T,H,K]")
        if erase is None or write is None:
            if beta is None:
                raise ValueError("need beta, or both erase and write gates")
            be = _f64(beta).reshape(TT, H)
            erase = np.broadcast_to(be[:, :, None], (TT, H, K)) if erase is None else erase
            write = np.broadcast_to(be[:, :, None], (TT, H, V)) if write is None else write
        self.b = np.ascontiguousarray(_f64(erase).reshape(TT, H, K))
        self.w = np.ascontiguousarray(_f64(write).reshape(TT, H, V))
        self.h0 = None if h0 is None else _f64(h0).reshape(self.N, H, K, V)


def forward(q, k, v, g, beta, *, scale, h0=None, cu_seqlens=None, erase=None, write=None,
            threads=None):
    """Token-by-token FP64 forward.  Returns (o [B,T,H,V], ht [N,H,K,V])."""
    p = _Prob(q, k, v, g, beta, erase, write, h0, cu_seqlens)
    o = np.zeros((p.B * p.T, p.H, p.V))
    ht = np.zeros((p.N, p.H, p.K, p.V))
    rc = _load().rewy_oracle_fwd(p.N, _ptr(p.cu), p.H, p.K, p.V, _ptr(p.q), _ptr(p.k),
                                 _ptr(p.v), _ptr(p.g), p.gate_kind, _ptr(p.b), _ptr(p.w),
                                 float(scale), _ptr(p.h0), _ptr(o), _ptr(ht),
                                 int(threads or default_threads()))
    if rc != 0:
        raise MemoryError("oracle forward failed to allocate")
    return o.reshape(p.B, p.T, p.H, p.V), ht


def kda_gate(x, a_log, dt_bias, lower_bound=0.0):
    """Channel-wise log-decay from its pre-activation (GDN2 spec section 4.4,
    the layer's gate; computed inside the kernels in section 2.1 and section 3):
        g = -exp(A_log[h]) * softplus(x + dt_bias[h, k])            (lower_bound = 0)
        g = lower_bound * sigmoid(exp(A_log[h]) * (x + dt_bias[h, k]))  (lower_bound < 0)
    The second, bounded form keeps g inside (lower_bound, 0) (GDN2 spec
    section 3, the recurrent kernel's gate, and section 4.3 for the bound).
    x [B,T,H,K], A_log [H], dt_bias [H,K]; FP64, natural log."""
    z = _f64(x) + _f64(dt_bias)[None, None]
    ea = np.exp(_f64(a_log))[None, None, :, None]
    if lower_bound == 0.0:
        return -ea * np.logaddexp(0.0, z)
    return float(lower_bound) * np.exp(-np.logaddexp(0.0, -ea * z))  # sigmoid without overflow


def kda_gate_backward(x, a_log, dt_bias, dg, lower_bound=0.0):
    """Reverse mode of ``kda_gate`` for a given dg: returns (dx, dA_log,
    ddt_bias).  Softplus form: d softplus(z)/dz = sigmoid(z), dg/dA_log = g.
    Bounded form, u = exp(A_log) z: dg/dz = lower_bound s (1 - s) exp(A_log)
    with s = sigmoid(u), and dg/dA_log = (dg/dz) z."""
    z = _f64(x) + _f64(dt_bias)[None, None]
    ea = np.exp(_f64(a_log))[None, None, :, None]
    dg = _f64(dg)
    if lower_bound == 0.0:
        dx = -ea * dg / (1.0 + np.exp(-z))
        g = -ea * np.logaddexp(0.0, z)
        return dx, (dg * g).sum(axis=(0, 1, 3)), dx.sum(axis=(0, 1))
    s = np.exp(-np.logaddexp(0.0, -ea * z))
    dx = dg * float(lower_bound) * s * (1.0 - s) * ea
    return dx, (dx * z).sum(axis=(0, 1, 3)), dx.sum(axis=(0, 1))


def backward(q, k, v, g, beta, dO, *, scale, h0=None, dht=None, cu_seqlens=None, erase=None,
             write=None, threads=None):
    """Exact reverse mode of ``forward`` for l = <dO, o> + <dht, ht>.

    Returns a dict with dq, dk [B,T,H,K], dv [B,T,H,V], dg (shape of g, or None),
    dbeta [B,T,H] (erase part + write part, undivided), derase [B,T,H,K],
    dwrite [B,T,H,V] and dh0 [N,H,K,V].
    """
    p = _Prob(q, k, v, g, beta, erase, write, h0, cu_seqlens)
    TT = p.B * p.T
    dO = _f64(dO).reshape(TT, p.H, p.V)
    dht = None if dht is None else _f64(dht).reshape(p.N, p.H, p.K, p.V)
    dq = np.zeros((TT, p.H, p.K)); dk = np.zeros_like(dq); db = np.zeros_like(dq)
    dv = np.zeros((TT, p.H, p.V)); dw = np.zeros_like(dv)
    dg = None if p.gate_kind == 0 else np.zeros(p.g.shape)
    dh0 = np.zeros((p.N, p.H, p.K, p.V))
    rc = _load().rewy_oracle_bwd(p.N, _ptr(p.cu), p.H, p.K, p.V, _ptr(p.q), _ptr(p.k),
                                 _ptr(p.v), _ptr(p.g), p.gate_kind, _ptr(p.b), _ptr(p.w),
                                 float(scale), _ptr(p.h0), _ptr(dO), _ptr(dht), _ptr(dq),
                                 _ptr(dk), _ptr(dv), _ptr(dg), _ptr(db), _ptr(dw), _ptr(dh0),
                                 int(threads or default_threads()))
    if rc != 0:
        raise MemoryError("oracle backward failed to allocate")
    B, T, H, K, V = p.B, p.T, p.H, p.K, p.V
    out = {
        "dq": dq.reshape(B, T, H, K), "dk": dk.reshape(B, T, H, K), "dv": dv.reshape(B, T, H, V),
        "derase": db.reshape(B, T, H, K), "dwrite": dw.reshape(B, T, H, V),
        "dbeta": (db.sum(-1) + dw.sum(-1)).reshape(B, T, H),
        "dg": None if dg is None else dg.reshape((B, T, H) if p.gate_kind == 1 else (B, T, H, K)),
        "dh0": dh0,
    }
    return out
