"""GPU parity of the erase/write form (rewy_fwd_gdn2 / rewy_bwd_gdn2: an
erase gate b per key channel and a write gate w per value channel in place of
the shared beta; ReWY paper Table 1, GDN2 row) against the FP64 oracle's
token recurrence with the same separate gates, on seeded inputs: every output
and gradient (db and dw element by element) within the stated tolerances, for
each gate kind, both dtypes, varlen and both saving policies; and with
b = w = beta the form reproduces the shared-beta operator."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_util import TOL, compare, gpu_available, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU and librewy.so")]

NAMES = ("o", "ht", "dq", "dk", "dv", "dg", "db", "dw", "dh0")

CASES = [
    # name, B, T, H, K, V, gate, dtype, h0, cu
    ("gdn2_bf16_vector_k128", 2, 200, 2, 128, 128, "vector", "bf16", "normal", None),
    ("gdn2_bf16_scalar_k64_v128", 1, 150, 2, 64, 128, "scalar", "bf16", "zero", None),
    ("gdn2_bf16_none_k64", 1, 130, 2, 64, 64, "none", "bf16", "normal", None),
    ("gdn2_fp32_vector_k64", 1, 140, 2, 64, 64, "vector", "fp32", "normal", None),
    ("gdn2_fp32_scalar_k32_v64", 2, 90, 1, 32, 64, "scalar", "fp32", "normal", None),
    ("gdn2_bf16_varlen", 1, 330, 2, 64, 64, "vector", "bf16", "normal", [0, 1, 64, 128, 193, 330]),
]


def _gates(inp, seed):
    """Erase and write gates in (0, 1), rounded to the feature dtype."""
    gen = torch.Generator().manual_seed(seed)
    B, T, H, K = inp.q.shape
    V = inp.v.shape[-1]
    b = torch.sigmoid(torch.randn(B, T, H, K, generator=gen)).to(inp.q.dtype)
    w = torch.sigmoid(torch.randn(B, T, H, V, generator=gen)).to(inp.q.dtype)
    return b, w


def _oracle(inp, b, w):
    cu = None if inp.cu_seqlens is None else list(inp.cu_seqlens)
    o, ht = oracle.forward(inp.q, inp.k, inp.v, inp.g, None, scale=inp.scale, h0=inp.h0,
                           cu_seqlens=cu, erase=b, write=w)
    gr = oracle.backward(inp.q, inp.k, inp.v, inp.g, None, inp.dO, scale=inp.scale, h0=inp.h0,
                         dht=inp.dht, cu_seqlens=cu, erase=b, write=w)
    return dict(o=o, ht=ht, dq=gr["dq"], dk=gr["dk"], dv=gr["dv"], dg=gr["dg"],
                db=gr["derase"], dw=gr["dwrite"], dh0=gr["dh0"])


def _hip(inp, b, w, policy):
    from chunkwise_delta_rule_chunk_amd import ops
    dev = torch.device("cuda:0")
    x = inp.to(dev)
    bd, wd = b.to(dev), w.to(dev)
    o, ht, ctx = ops.forward_gdn2(x.q, x.k, x.v, x.g, bd, wd, scale=inp.scale, h0=x.h0,
                                  cu_seqlens=inp.cu_seqlens, policy=policy)
    gr = ops.backward(ctx, x.dO, x.dht, want_dh0=True)
    torch.cuda.synchronize()
    out = dict(o=o, ht=ht, **gr)
    return {k: (None if v is None else v.double().cpu().numpy()) for k, v in out.items()}


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("policy", ["recompute", "save"])
def test_gdn2_matches_oracle(case, policy):
    name, B, T, H, K, V, gate, dt, h0, cu = case
    say(f"[case] {name} policy={policy}")
    seed = zlib.crc32(name.encode()) % 1000
    inp = workloads.make_inputs(B, T, H, K, V, gate=gate, dtype=dt, seed=seed, h0=h0, dht=True,
                                cu_seqlens=cu)
    b, w = _gates(inp, seed + 1)
    compare(_hip(inp, b, w, policy), _oracle(inp, b, w), TOL[inp.q.dtype], cu=inp.cu_seqlens, names=NAMES,
            label=f"{name}/{policy}")


def test_gdn2_with_shared_gates_is_the_beta_operator():
    """b = w = beta (broadcast) gives the shared-beta operator's outputs, and
    the feature sums of db and dw give its dbeta."""
    from chunkwise_delta_rule_chunk_amd import ops
    say("[case] gdn2 with b = w = beta")
    inp = workloads.make_inputs(1, 150, 2, 64, 64, gate="vector", dtype="fp32", seed=12,
                                h0="normal", dht=True)
    dev = torch.device("cuda:0")
    x = inp.to(dev)
    b = x.beta[..., None].expand(*x.k.shape).contiguous()
    w = x.beta[..., None].expand(*x.v.shape).contiguous()
    o2, ht2, c2 = ops.forward_gdn2(x.q, x.k, x.v, x.g, b, w, scale=inp.scale, h0=x.h0)
    g2 = ops.backward(c2, x.dO, x.dht)
    o1, ht1, c1 = ops.forward(x.q, x.k, x.v, x.g, x.beta, scale=inp.scale, h0=x.h0)
    g1 = ops.backward(c1, x.dO, x.dht)
    torch.cuda.synchronize()
    rel = lambda a, r: (torch.linalg.norm((a - r).double()) / torch.linalg.norm(r.double())).item()
    errs = dict(o=rel(o2, o1), ht=rel(ht2, ht1), dq=rel(g2["dq"], g1["dq"]), dk=rel(g2["dk"], g1["dk"]),
                dv=rel(g2["dv"], g1["dv"]), dg=rel(g2["dg"], g1["dg"]),
                dbeta=rel(g2["db"].sum(-1) + g2["dw"].sum(-1), g1["dbeta"]))
    say("[parity] gdn2-vs-beta " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v < 1e-5 for v in errs.values()), errs


def test_gdn2_strong_decay_takes_pairwise_path():
    """Gates 30x the KDA recipe: diagonal sub-chunks exceed the centring bound,
    so the forward's pairwise diagonal (erase gate inside the feature sum) and
    the backward's pairwise block run with the erase/write gates."""
    say("[case] gdn2 strong decay pairwise")
    inp = workloads.make_inputs(1, 256, 2, 64, 64, gate="vector", dtype="bf16", seed=4,
                                gate_scale=30.0, h0="normal", dht=True)
    G = np.cumsum(inp.g.double().numpy().reshape(1, 4, 64, 2, 64), axis=2) / np.log(2)
    sub = G.reshape(1, 4, 4, 16, 2, 64)
    assert (sub.max(3) - sub.min(3)).max() > 128  # the fallback is really exercised
    b, w = _gates(inp, 41)
    compare(_hip(inp, b, w, "recompute"), _oracle(inp, b, w), TOL[inp.q.dtype], cu=inp.cu_seqlens, names=NAMES,
            label="gdn2-strong-decay")
