"""Torch-facing wrapper of the C ABI: allocates outputs, workspace and the
saved buffer with PyTorch (device memory and streams only) and calls
``rewy_fwd`` / ``rewy_bwd`` through the ctypes binding.  No arithmetic of the
operator happens here."""
from __future__ import annotations

import ctypes
from dataclasses import dataclass, field
from typing import Optional

import torch

from . import binding as B

_DT = {torch.bfloat16: B.REWY_BF16, torch.float32: B.REWY_F32}
_POLICY = {"recompute": B.REWY_RECOMPUTE, "save": B.REWY_SAVE}


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(rc, where):
    if rc != B.REWY_OK:
        raise B.RewyError(rc, where)


@dataclass
class Problem:
    """One operator call: the C descriptor plus the host objects it points to."""
    desc: B.RewyDesc
    device: torch.device
    dtype: torch.dtype
    beta_dtype: torch.dtype
    N: int
    cu_dev: Optional[torch.Tensor] = None
    cu_host: object = None
    keep: list = field(default_factory=list)

    @property
    def state_shape(self):
        d = self.desc
        return (self.N, d.H, d.K, d.V)


def make_problem(q, v, g, beta, *, scale=None, cu_seqlens=None, policy="recompute",
                 vector_gate=False) -> Problem:
    if q.dtype not in _DT or v.dtype != q.dtype:
        raise TypeError("q, k, v must share dtype bf16 or fp32")
    if beta.dtype not in _DT:
        raise TypeError("beta must be bf16 or fp32")
    Bsz, T, H, K = q.shape
    V = v.shape[-1]
    if vector_gate:  # the gate is formed in the kernels from its pre-activation
        gate = B.REWY_GATE_VECTOR
    elif g is None:
        gate = B.REWY_GATE_NONE
    elif g.dim() == 3:
        gate = B.REWY_GATE_SCALAR
    else:
        gate = B.REWY_GATE_VECTOR
    if g is not None and g.dtype != torch.float32:
        raise TypeError("g must be fp32")
    cu_dev = cu_host = None
    if cu_seqlens is not None:
        host = [int(x) for x in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist") else cu_seqlens)]
        cu_host = (ctypes.c_int32 * len(host))(*host)
        cu_dev = torch.tensor(host, dtype=torch.int32, device=q.device)
        N = len(host) - 1
    else:
        N = Bsz
    desc = B.RewyDesc(Bsz, T, H, K, V, N if cu_seqlens is not None else 0,
                      None if cu_dev is None else cu_dev.data_ptr(),
                      None if cu_host is None else ctypes.addressof(cu_host),
                      _DT[q.dtype], _DT[beta.dtype], gate, _POLICY[policy],
                      float(K ** -0.5 if scale is None else scale))
    return Problem(desc, q.device, q.dtype, beta.dtype, N, cu_dev, cu_host)


def _stream(device, stream):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def workspace(prob: Problem, phase: int) -> torch.Tensor:
    n = B.rewy_workspace_bytes(prob.desc, phase)
    if n == 0:
        raise B.RewyError(B.REWY_EINVAL, "rewy_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=prob.device)


def forward(q, k, v, g, beta, *, scale=None, h0=None, cu_seqlens=None, policy="recompute",
            output_final_state=True, stream=None, ws=None):
    """Run rewy_fwd.  Returns (o, ht or None, ctx) where ctx feeds ``backward``."""
    prob = make_problem(q, v, g, beta, scale=scale, cu_seqlens=cu_seqlens, policy=policy)
    o = torch.empty_like(v)
    ht = torch.empty(prob.state_shape, dtype=torch.float32, device=q.device) \
        if output_final_state else None
    saved = None
    if policy == "save":
        saved = torch.empty(B.rewy_saved_bytes(prob.desc), dtype=torch.uint8, device=q.device)
    if ws is None:
        ws = workspace(prob, 0)
    rc = B.rewy_fwd(prob.desc, _p(q), _p(k), _p(v), _p(g), _p(beta), _p(h0), _p(o), _p(ht),
                    _p(saved), _p(ws), ws.numel(), _stream(q.device, stream))
    _check(rc, "rewy_fwd")
    ctx = dict(prob=prob, q=q, k=k, v=v, g=g, beta=beta, h0=h0, saved=saved)
    return o, ht, ctx


def recurrent_forward(q, k, v, g, beta, *, scale=None, h0=None, cu_seqlens=None,
                      output_final_state=True, stream=None):
    """Run rewy_recurrent_fwd (token-serial, for decoding).  Returns (o, ht or None)."""
    prob = make_problem(q, v, g, beta, scale=scale, cu_seqlens=cu_seqlens)
    o = torch.empty_like(v)
    ht = torch.empty(prob.state_shape, dtype=torch.float32, device=q.device) \
        if output_final_state else None
    rc = B.rewy_recurrent_fwd(prob.desc, _p(q), _p(k), _p(v), _p(g), _p(beta), _p(h0), _p(o),
                              _p(ht), _stream(q.device, stream))
    _check(rc, "rewy_recurrent_fwd")
    return o, ht


def recurrent_forward_gdn2(q, k, v, g, b, w, *, scale=None, h0=None, cu_seqlens=None,
                           output_final_state=True, stream=None):
    """Run rewy_recurrent_fwd_gdn2 (token-serial, erase gate b [B,T,H,K] and
    write gate w [B,T,H,V] in the feature dtype).  Returns (o, ht or None)."""
    prob = make_problem(q, v, g, b, scale=scale, cu_seqlens=cu_seqlens)
    o = torch.empty_like(v)
    ht = torch.empty(prob.state_shape, dtype=torch.float32, device=q.device) \
        if output_final_state else None
    rc = B.rewy_recurrent_fwd_gdn2(prob.desc, _p(q), _p(k), _p(v), _p(g), _p(b), _p(w), _p(h0),
                                   _p(o), _p(ht), _stream(q.device, stream))
    _check(rc, "rewy_recurrent_fwd_gdn2")
    return o, ht


def forward_gdn2(q, k, v, g, b, w, *, scale=None, h0=None, cu_seqlens=None, policy="recompute",
                 output_final_state=True, stream=None, ws=None):
    """Run rewy_fwd_gdn2: independent erase gate b [B,T,H,K] and write gate w
    [B,T,H,V] (feature dtype).  Returns (o, ht or None, ctx) for ``backward``."""
    prob = make_problem(q, v, g, b, scale=scale, cu_seqlens=cu_seqlens, policy=policy)
    o = torch.empty_like(v)
    ht = torch.empty(prob.state_shape, dtype=torch.float32, device=q.device) \
        if output_final_state else None
    saved = None
    if policy == "save":
        saved = torch.empty(B.rewy_saved_bytes(prob.desc), dtype=torch.uint8, device=q.device)
    if ws is None:
        ws = workspace(prob, 0)
    rc = B.rewy_fwd_gdn2(prob.desc, _p(q), _p(k), _p(v), _p(g), _p(b), _p(w), _p(h0), _p(o),
                         _p(ht), _p(saved), _p(ws), ws.numel(), _stream(q.device, stream))
    _check(rc, "rewy_fwd_gdn2")
    ctx = dict(prob=prob, q=q, k=k, v=v, g=g, beta=b, w=w, h0=h0, saved=saved)
    return o, ht, ctx


def forward_kda_gate(q, k, v, x, a_log, dt_bias, beta, *, lower_bound=0.0, scale=None, h0=None,
                     cu_seqlens=None, policy="recompute", output_final_state=True, stream=None,
                     ws=None):
    """Run rewy_fwd_kda_gate: the vector gate is formed in the kernels from
    x [B,T,H,K] (feature dtype), A_log [H] and dt_bias [H,K] (fp32), as
    g = -exp(A_log) softplus(x + dt_bias) (lower_bound = 0) or
    g = lower_bound sigmoid(exp(A_log) (x + dt_bias)) (-5 <= lower_bound < 0).
    Returns (o, ht or None, ctx) for ``backward``."""
    if a_log.dtype != torch.float32 or dt_bias.dtype != torch.float32:
        raise TypeError("A_log and dt_bias must be fp32")
    if x.dtype != q.dtype:
        raise TypeError("x must have the feature dtype")
    prob = make_problem(q, v, None, beta, scale=scale, cu_seqlens=cu_seqlens, policy=policy,
                        vector_gate=True)
    o = torch.empty_like(v)
    ht = torch.empty(prob.state_shape, dtype=torch.float32, device=q.device) \
        if output_final_state else None
    saved = None
    if policy == "save":
        saved = torch.empty(B.rewy_saved_bytes(prob.desc), dtype=torch.uint8, device=q.device)
    if ws is None:
        ws = workspace(prob, 0)
    rc = B.rewy_fwd_kda_gate(prob.desc, _p(q), _p(k), _p(v), _p(x), _p(a_log), _p(dt_bias),
                             float(lower_bound), _p(beta), _p(h0), _p(o), _p(ht), _p(saved),
                             _p(ws), ws.numel(), _stream(q.device, stream))
    _check(rc, "rewy_fwd_kda_gate")
    ctx = dict(prob=prob, q=q, k=k, v=v, g=None, x=x, a_log=a_log, dt_bias=dt_bias,
               lower_bound=float(lower_bound), beta=beta, h0=h0, saved=saved)
    return o, ht, ctx


def backward(ctx, dO, dht=None, *, stream=None, ws=None, want_dh0=None):
    """Run rewy_bwd (rewy_bwd_gdn2 for a ``forward_gdn2`` context,
    rewy_bwd_kda_gate for a ``forward_kda_gate`` one).  Returns dict dq, dk, dv,
    dg, dbeta, dh0 (for the erase/write form db and dw in place of dbeta; for
    the gate formed in the kernels dx, dA_log and ddt_bias in place of dg)."""
    prob = ctx["prob"]
    if ctx.get("w") is not None:
        return _backward_gdn2(ctx, dO, dht, stream=stream, ws=ws, want_dh0=want_dh0)
    if ctx.get("x") is not None:
        return _backward_kda_gate(ctx, dO, dht, stream=stream, ws=ws, want_dh0=want_dh0)
    q, k, v, g, beta, h0 = (ctx[x] for x in ("q", "k", "v", "g", "beta", "h0"))
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dg = None if g is None else torch.empty_like(g)
    dbeta = torch.empty_like(beta)
    if want_dh0 is None:
        want_dh0 = h0 is not None
    dh0 = torch.empty(prob.state_shape, dtype=torch.float32, device=q.device) if want_dh0 else None
    if ws is None:
        ws = workspace(prob, 1)
    rc = B.rewy_bwd(prob.desc, _p(q), _p(k), _p(v), _p(g), _p(beta), _p(h0), _p(dO), _p(dht),
                    _p(ctx["saved"]), _p(dq), _p(dk), _p(dv), _p(dg), _p(dbeta), _p(dh0),
                    _p(ws), ws.numel(), _stream(q.device, stream))
    _check(rc, "rewy_bwd")
    return dict(dq=dq, dk=dk, dv=dv, dg=dg, dbeta=dbeta, dh0=dh0)


def _backward_gdn2(ctx, dO, dht=None, *, stream=None, ws=None, want_dh0=None):
    prob = ctx["prob"]
    q, k, v, g, b, w, h0 = (ctx[x] for x in ("q", "k", "v", "g", "beta", "w", "h0"))
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dg = None if g is None else torch.empty_like(g)
    db, dw = torch.empty_like(k), torch.empty_like(v)
    if want_dh0 is None:
        want_dh0 = h0 is not None
    dh0 = torch.empty(prob.state_shape, dtype=torch.float32, device=q.device) if want_dh0 else None
    if ws is None:
        ws = workspace(prob, 1)
    rc = B.rewy_bwd_gdn2(prob.desc, _p(q), _p(k), _p(v), _p(g), _p(b), _p(w), _p(h0), _p(dO),
                         _p(dht), _p(ctx["saved"]), _p(dq), _p(dk), _p(dv), _p(dg), _p(db),
                         _p(dw), _p(dh0), _p(ws), ws.numel(), _stream(q.device, stream))
    _check(rc, "rewy_bwd_gdn2")
    return dict(dq=dq, dk=dk, dv=dv, dg=dg, db=db, dw=dw, dh0=dh0)


def _backward_kda_gate(ctx, dO, dht=None, *, stream=None, ws=None, want_dh0=None):
    prob = ctx["prob"]
    q, k, v, x, a_log, dt_bias, beta, h0 = (ctx[n] for n in ("q", "k", "v", "x", "a_log", "dt_bias",
                                                          "beta", "h0"))
    dq, dk, dv, dx = (torch.empty_like(t) for t in (q, k, v, x))
    da_log, ddt_bias, dbeta = torch.empty_like(a_log), torch.empty_like(dt_bias), torch.empty_like(beta)
    if want_dh0 is None:
        want_dh0 = h0 is not None
    dh0 = torch.empty(prob.state_shape, dtype=torch.float32, device=q.device) if want_dh0 else None
    if ws is None:
        ws = workspace(prob, 2)
    rc = B.rewy_bwd_kda_gate(prob.desc, _p(q), _p(k), _p(v), _p(x), _p(a_log), _p(dt_bias),
                             ctx["lower_bound"], _p(beta), _p(h0), _p(dO), _p(dht), _p(ctx["saved"]), _p(dq), _p(dk), _p(dv),
                             _p(dx), _p(da_log), _p(ddt_bias), _p(dbeta), _p(dh0), _p(ws),
                             ws.numel(), _stream(q.device, stream))
    _check(rc, "rewy_bwd_kda_gate")
    return dict(dq=dq, dk=dk, dv=dv, dx=dx, da_log=da_log, ddt_bias=ddt_bias, dbeta=dbeta, dh0=dh0)


class ChunkDeltaRule(torch.autograd.Function):
    """Autograd wrapper: o, ht = ChunkDeltaRule.apply(q, k, v, g, beta, h0, scale, cu_seqlens, policy)."""

    @staticmethod
    def forward(fctx, q, k, v, g, beta, h0, scale, cu_seqlens, policy):
        q, k, v, beta = (x.contiguous() for x in (q, k, v, beta))
        g = None if g is None else g.contiguous()
        o, ht, ctx = forward(q, k, v, g, beta, scale=scale, h0=h0, cu_seqlens=cu_seqlens,
                             policy=policy, output_final_state=True)
        fctx.rewy = ctx
        return o, ht

    @staticmethod
    def backward(fctx, do, dht):
        g = backward(fctx.rewy, do.contiguous(), None if dht is None else dht.contiguous())
        return g["dq"], g["dk"], g["dv"], g["dg"], g["dbeta"], g["dh0"], None, None, None


def chunk_delta_rule(q, k, v, g, beta, *, scale=None, initial_state=None, cu_seqlens=None,
                     policy="recompute"):
    """Differentiable chunkwise gated delta rule on the HIP path."""
    return ChunkDeltaRule.apply(q, k, v, g, beta, initial_state, scale, cu_seqlens, policy)
