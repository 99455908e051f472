"""GPU parity of the secondary measurements at the exact configurations the
benchmark times: the gate formed in the kernels and the erase/write form on
the full KDA workload (B=1, T=8192, H=32, d=128, bf16), compared with the FP64
oracle on sampled heads (the oracle recomputes them one by one), and the
decode call (64 sequences x 1 token, H=32, d=128) on every unit."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_util import TOL, compare, gpu_available, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU and librewy.so")]

WORKLOAD = "kda_t8192_h32_d128"
HEADS = [0, 17]


def _sel(t, heads):
    return None if t is None else t[:, :, heads]


def _np_heads(out, heads):
    res = {}
    for k, v in out.items():
        if v is None:
            continue
        if k in ("ht", "dh0"):
            v = v[:, heads]
        elif k == "da_log":
            v = v[heads]
        elif k == "ddt_bias":
            v = v[heads]
        else:
            v = v[:, :, heads]
        res[k] = v.double().cpu().numpy()
    return res


def test_kda_gate_full_workload_sampled():
    """rewy_fwd_kda_gate / rewy_bwd_kda_gate on the full workload, from its
    bf16 pre-activation x, A_log and dt_bias (as the benchmark runs it)."""
    from chunkwise_delta_rule_chunk_amd import ops
    say(f"[case] {WORKLOAD} gate formed in the kernels")
    inp = workloads.workload(WORKLOAD)
    dev = torch.device("cuda:0")
    t = inp.to(dev)
    x = inp.gate_x.to(inp.q.dtype)
    o, ht, ctx = ops.forward_kda_gate(t.q, t.k, t.v, x.to(dev), inp.a_log.to(dev), inp.dt_bias.to(dev),
                                      t.beta, scale=inp.scale, h0=t.h0)
    gr = ops.backward(ctx, t.dO, t.dht, want_dh0=True)
    torch.cuda.synchronize()
    hip = _np_heads(dict(o=o, ht=ht, **gr), HEADS)
    q, k, v, beta, dO = (_sel(a, HEADS) for a in (inp.q, inp.k, inp.v, inp.beta, inp.dO))
    xs, al, db = _sel(x, HEADS), inp.a_log[HEADS], inp.dt_bias[HEADS]
    say(f"[case] {WORKLOAD} gate formed in the kernels: oracle heads {HEADS}")
    g = oracle.kda_gate(xs, al, db)
    ro, rht = oracle.forward(q, k, v, g, beta, scale=inp.scale)
    rg = oracle.backward(q, k, v, g, beta, dO, scale=inp.scale)
    dx, da, dd = oracle.kda_gate_backward(xs, al, db, rg["dg"])
    ref = dict(o=ro, ht=rht, dq=rg["dq"], dk=rg["dk"], dv=rg["dv"], dx=dx, da_log=da, ddt_bias=dd,
               dbeta=rg["dbeta"], dh0=rg["dh0"])
    compare(hip, ref, TOL[inp.q.dtype], cu=inp.cu_seqlens, names=tuple(ref), label=f"{WORKLOAD}/kda-gate")


def test_erase_write_full_workload_sampled():
    """rewy_fwd_gdn2 / rewy_bwd_gdn2 on the full workload with the benchmark's
    seeded erase and write gates."""
    from chunkwise_delta_rule_chunk_amd import ops
    say(f"[case] {WORKLOAD} erase/write form")
    inp = workloads.workload(WORKLOAD)
    gen = torch.Generator().manual_seed(13)
    b = torch.sigmoid(torch.randn(*inp.k.shape, generator=gen)).to(inp.q.dtype)
    w = torch.sigmoid(torch.randn(*inp.v.shape, generator=gen)).to(inp.q.dtype)
    dev = torch.device("cuda:0")
    t = inp.to(dev)
    o, ht, ctx = ops.forward_gdn2(t.q, t.k, t.v, t.g, b.to(dev), w.to(dev), scale=inp.scale, h0=t.h0)
    gr = ops.backward(ctx, t.dO, t.dht, want_dh0=True)
    torch.cuda.synchronize()
    hip = _np_heads(dict(o=o, ht=ht, **gr), HEADS)
    q, k, v, g, dO, bs, ws = (_sel(a, HEADS) for a in (inp.q, inp.k, inp.v, inp.g, inp.dO, b, w))
    say(f"[case] {WORKLOAD} erase/write form: oracle heads {HEADS}")
    ro, rht = oracle.forward(q, k, v, g, None, scale=inp.scale, erase=bs, write=ws)
    rg = oracle.backward(q, k, v, g, None, dO, scale=inp.scale, erase=bs, write=ws)
    ref = dict(o=ro, ht=rht, dq=rg["dq"], dk=rg["dk"], dv=rg["dv"], dg=rg["dg"], db=rg["derase"],
               dw=rg["dwrite"], dh0=rg["dh0"])
    compare(hip, ref, TOL[inp.q.dtype], cu=inp.cu_seqlens, names=tuple(ref), label=f"{WORKLOAD}/erase-write")


def test_decode_bench_config():
    """The decode call the benchmark times: 64 sequences with fp32 states, one
    new token each, H=32, K=V=128, bf16, vector gate; every unit."""
    from chunkwise_delta_rule_chunk_amd import ops
    say("[case] decode 64 x 1 token, H=32, d=128")
    inp = workloads.make_inputs(64, 1, 32, 128, 128, gate="vector", dtype="bf16", h0="normal", seed=11)
    x = inp.to(torch.device("cuda:0"))
    o, ht = ops.recurrent_forward(x.q, x.k, x.v, x.g, x.beta, scale=inp.scale, h0=x.h0)
    torch.cuda.synchronize()
    ro, rht = oracle.forward(inp.q, inp.k, inp.v, inp.g, inp.beta, scale=inp.scale, h0=inp.h0)
    compare(dict(o=o.double().cpu().numpy(), ht=ht.double().cpu().numpy()), dict(o=ro, ht=rht),
            TOL[inp.q.dtype], cu=inp.cu_seqlens, names=("o", "ht"), label="decode-bench-config")
