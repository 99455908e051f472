"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI,
run the FP64 oracle on the same (already rounded) inputs, compare."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

import oracle

OUT_NAMES = ("o", "ht", "dq", "dk", "dv", "dg", "dbeta", "dh0")
TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def hip_run_torch(inp, policy="recompute", want_dh0=None):
    """Forward + backward of the HIP path through the C ABI; torch tensors on the GPU."""
    from chunkwise_delta_rule_chunk_amd import ops
    dev = torch.device("cuda:0")
    x = inp.to(dev)
    o, ht, ctx = ops.forward(x.q, x.k, x.v, x.g, x.beta, scale=inp.scale, h0=x.h0,
                             cu_seqlens=inp.cu_seqlens, policy=policy)
    gr = ops.backward(ctx, x.dO, x.dht, want_dh0=want_dh0)
    torch.cuda.synchronize()
    return dict(o=o, ht=ht, **gr)


def to_np(out, select=None):
    res = {}
    for k, v in out.items():
        if v is None:
            res[k] = None
            continue
        if select is not None:
            v = select(k, v)
        res[k] = v.double().cpu().numpy()
    return res


def hip_run(inp, policy="recompute", want_dh0=None):
    """Forward + backward of the HIP path; float64 numpy outputs."""
    return to_np(hip_run_torch(inp, policy, want_dh0))


def oracle_run(inp, heads=None, seqs=None):
    """Oracle outputs for all (or the selected) heads / sequences."""
    q, k, v, g, beta, dO = inp.q, inp.k, inp.v, inp.g, inp.beta, inp.dO
    h0, dht, cu = inp.h0, inp.dht, inp.cu_seqlens
    if heads is not None:
        sel = lambda t: None if t is None else t[:, :, heads]
        q, k, v, g, beta, dO = (sel(t) for t in (q, k, v, g, beta, dO))
        h0 = None if h0 is None else h0[:, heads]
        dht = None if dht is None else dht[:, heads]
    if seqs is not None:
        q, k, v, g, beta, dO = (None if t is None else t[seqs] for t in (q, k, v, g, beta, dO))
        h0 = None if h0 is None else h0[seqs]
        dht = None if dht is None else dht[seqs]
    cuv = None if cu is None else cu.tolist()
    o, ht = oracle.forward(q, k, v, g, beta, scale=inp.scale, h0=h0, cu_seqlens=cuv)
    gr = oracle.backward(q, k, v, g, beta, dO, scale=inp.scale, h0=h0, dht=dht, cu_seqlens=cuv)
    return dict(o=o, ht=ht, **gr)


def normwise(x, ref):
    """Normwise relative error ||x - ref||_F / ||ref||_F (max-abs when the
    reference is below 1e-6 everywhere).  Non-finite values fail."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    if not np.all(np.isfinite(x)):
        return float("inf")
    if ref.size == 0:
        return 0.0
    if np.abs(ref).max() < 1e-6:  # near-zero reference: max-abs <= 1e-6 decides
        return 0.0 if np.abs(x - ref).max() <= 1e-6 else float("inf")
    return float(np.linalg.norm(x - ref) / np.linalg.norm(ref))


# outputs that hold one [K, V] state per (sequence, head): [N, H, K, V]
STATE_NAMES = ("ht", "dh0")
# parameter gradients summed over every token of every sequence: one tensor,
# no (sequence, head) units
WHOLE_NAMES = ("da_log", "ddt_bias")


def unit_slices(name, shape, cu=None):
    """The (sequence, head) units of output ``name``: yields (label, index)
    pairs, index selecting the unit's elements.  Token tensors are
    [B, T, H, ...] (one unit per batch row and head, or per packed sequence
    and head with ``cu``); state tensors are [N, H, K, V]."""
    if name in WHOLE_NAMES:
        return
    if name in STATE_NAMES:
        for n in range(shape[0]):
            for h in range(shape[1]):
                yield (n, h), (n, h)
        return
    B, T, H = shape[:3]
    if cu is None:
        for b in range(B):
            for h in range(H):
                yield (b, h), (b, slice(None), h)
    else:
        cu = [int(x) for x in cu]
        for n in range(len(cu) - 1):
            for h in range(H):
                yield (n, h), (0, slice(cu[n], cu[n + 1]), h)


def compare(hip, ref, tol, names=OUT_NAMES, label="", cu=None, units=True, worst_out=None):
    """Assert every output is within ``tol``, as one tensor and, with
    ``units``, on every (sequence, head) unit on its own (a wrong sequence or
    head cannot hide inside a large tensor's norm).  Prints the whole-tensor
    error and the worst unit of each output; returns the whole-tensor table.
    ``worst_out`` (a dict), if given, keeps the largest unit error per output
    over several calls, with the label of the call and the unit."""
    errs, worst = {}, {}
    for n in names:
        a, r = hip.get(n), ref.get(n)
        if r is None:
            assert a is None, (n, "unexpected output")
            continue
        if a is None:
            continue
        errs[n] = normwise(a, r)
        if units:
            a_np, r_np = np.asarray(a), np.asarray(r)
            w = (0.0, None)
            for lab, idx in unit_slices(n, r_np.shape, cu):
                e = normwise(a_np[idx], r_np[idx])
                if w[1] is None or not e <= w[0]:  # a non-finite error always wins
                    w = (e, lab)
            if w[1] is not None:
                worst[n] = w
    say(f"[parity] {label} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    if worst:
        say(f"[parity] {label} worst unit " +
            " ".join(f"{k}={e:.2e}@{lab}" for k, (e, lab) in worst.items()))
    if worst_out is not None:
        for k, (e, lab) in worst.items():
            if k not in worst_out or not e <= worst_out[k][0]:
                worst_out[k] = (e, f"{label}{lab}")
    bad = {k: v for k, v in errs.items() if not v <= tol}
    bad.update({f"{k}{lab}": e for k, (e, lab) in worst.items() if not e <= tol})
    assert not bad, f"{label}: outside tolerance {tol}: {bad}"
    return errs


def head_select(heads, seqs=None):
    """Select heads (and batch rows) of HIP outputs to match a sampled oracle run."""
    def f(name, a):
        if name in ("ht", "dh0"):
            a = a[:, heads]
        else:
            a = a[:, :, heads]
        return a if seqs is None else a[seqs]
    return f


def gpu_available():
    return torch.cuda.is_available() and os.path.exists(
        os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                     "chunkwise_delta_rule_chunk_amd", "librewy.so"))
