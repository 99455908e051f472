"""GPU parity of the token-serial forward (rewy_recurrent_fwd, the decode
form) against the FP64 oracle's token recurrence, on the same seeded inputs:
o and the final state, normwise within the stated tolerances, across gate
kinds, dtypes, ragged varlen batches, with and without an initial state, and
in decode use (one token per call, the state carried through h0 / ht)."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_util import TOL, compare, gpu_available, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU and librewy.so")]

CASES = [
    # name, B, T, H, K, V, gate, dtype, h0, cu
    ("rec_bf16_vector_k128", 2, 37, 2, 128, 128, "vector", "bf16", "normal", None),
    ("rec_bf16_scalar_k64_v32", 3, 20, 2, 64, 32, "scalar", "bf16", "zero", None),
    ("rec_bf16_none_k32_v128", 1, 70, 3, 32, 128, "none", "bf16", "normal", None),
    ("rec_fp32_vector_k64", 2, 25, 2, 64, 64, "vector", "fp32", "normal", None),
    ("rec_fp32_scalar_k32", 1, 9, 2, 32, 32, "scalar", "fp32", "zero", None),
    ("rec_bf16_varlen", 1, 100, 2, 64, 64, "vector", "bf16", "normal", [0, 1, 1, 40, 100]),
]


def _oracle_fwd(inp):
    cu = None if inp.cu_seqlens is None else list(inp.cu_seqlens)
    o, ht = oracle.forward(inp.q, inp.k, inp.v, inp.g, inp.beta, scale=inp.scale, h0=inp.h0,
                           cu_seqlens=cu)
    return dict(o=o, ht=ht)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_recurrent_matches_oracle(case):
    from chunkwise_delta_rule_chunk_amd import ops
    name, B, T, H, K, V, gate, dt, h0, cu = case
    say(f"[case] {name}")
    inp = workloads.make_inputs(B, T, H, K, V, gate=gate, dtype=dt, h0=h0, cu_seqlens=cu,
                                seed=zlib.crc32(name.encode()) % 1000)
    x = inp.to(torch.device("cuda:0"))
    o, ht = ops.recurrent_forward(x.q, x.k, x.v, x.g, x.beta, scale=inp.scale, h0=x.h0,
                                  cu_seqlens=inp.cu_seqlens)
    torch.cuda.synchronize()
    hip = dict(o=o.double().cpu().numpy(), ht=ht.double().cpu().numpy())
    compare(hip, _oracle_fwd(inp), TOL[inp.q.dtype], cu=inp.cu_seqlens, names=("o", "ht"), label=name)


def test_recurrent_decode_steps_carry_the_state():
    """One token per call with the state carried through h0 / ht equals one
    call over the whole sequence, and both match the oracle."""
    from chunkwise_delta_rule_chunk_amd import ops
    say("[case] recurrent decode steps")
    inp = workloads.make_inputs(4, 12, 2, 128, 128, gate="vector", dtype="bf16", h0="normal",
                                seed=7)
    x = inp.to(torch.device("cuda:0"))
    o_all, ht_all = ops.recurrent_forward(x.q, x.k, x.v, x.g, x.beta, scale=inp.scale, h0=x.h0)
    h = x.h0
    outs = []
    for t in range(12):
        sl = slice(t, t + 1)
        o_t, h = ops.recurrent_forward(x.q[:, sl].contiguous(), x.k[:, sl].contiguous(),
                                       x.v[:, sl].contiguous(), x.g[:, sl].contiguous(),
                                       x.beta[:, sl].contiguous(), scale=inp.scale, h0=h)
        outs.append(o_t)
    torch.cuda.synchronize()
    # the same arithmetic in the same order: identical results
    assert torch.equal(torch.cat(outs, 1), o_all) and torch.equal(h, ht_all)
    hip = dict(o=o_all.double().cpu().numpy(), ht=ht_all.double().cpu().numpy())
    compare(hip, _oracle_fwd(inp), TOL[inp.q.dtype], cu=inp.cu_seqlens, names=("o", "ht"), label="decode-steps")


def test_recurrent_agrees_with_the_chunked_forward():
    """The token-serial and the chunked forward compute the same operator."""
    from chunkwise_delta_rule_chunk_amd import ops
    say("[case] recurrent vs chunked")
    inp = workloads.make_inputs(1, 150, 2, 64, 64, gate="vector", dtype="fp32", h0="normal",
                                seed=8)
    x = inp.to(torch.device("cuda:0"))
    o_r, ht_r = ops.recurrent_forward(x.q, x.k, x.v, x.g, x.beta, scale=inp.scale, h0=x.h0)
    o_c, ht_c, _ = ops.forward(x.q, x.k, x.v, x.g, x.beta, scale=inp.scale, h0=x.h0)
    torch.cuda.synchronize()
    err_o = (torch.linalg.norm((o_r - o_c).double()) / torch.linalg.norm(o_c.double())).item()
    err_h = (torch.linalg.norm((ht_r - ht_c).double()) / torch.linalg.norm(ht_c.double())).item()
    say(f"[parity] recurrent-vs-chunked o={err_o:.2e} ht={err_h:.2e}")
    assert err_o < TOL[inp.q.dtype] and err_h < TOL[inp.q.dtype]


EW_CASES = [
    # name, B, T, H, K, V, gate, dtype, h0, cu
    ("recew_bf16_vector_k128", 2, 37, 2, 128, 128, "vector", "bf16", "normal", None),
    ("recew_bf16_scalar_k64_v32", 3, 20, 2, 64, 32, "scalar", "bf16", "zero", None),
    ("recew_fp32_none_k32_v64", 1, 30, 2, 32, 64, "none", "fp32", "normal", None),
    ("recew_bf16_varlen", 1, 100, 2, 64, 64, "vector", "bf16", "normal", [0, 1, 1, 40, 100]),
]


def _ew_gates(inp, seed):
    gen = torch.Generator().manual_seed(seed)
    b = torch.sigmoid(torch.randn(*inp.k.shape, generator=gen)).to(inp.q.dtype)
    w = torch.sigmoid(torch.randn(*inp.v.shape, generator=gen)).to(inp.q.dtype)
    return b, w


@pytest.mark.parametrize("case", EW_CASES, ids=[c[0] for c in EW_CASES])
def test_recurrent_erase_write_matches_oracle(case):
    """rewy_recurrent_fwd_gdn2: erase gate b per key feature and write gate w
    per value column (GDN2 spec section 3) against the oracle's recurrence
    with the same separate gates."""
    from chunkwise_delta_rule_chunk_amd import ops
    name, B, T, H, K, V, gate, dt, h0, cu = case
    say(f"[case] {name}")
    seed = zlib.crc32(name.encode()) % 1000
    inp = workloads.make_inputs(B, T, H, K, V, gate=gate, dtype=dt, h0=h0, cu_seqlens=cu, seed=seed)
    b, w = _ew_gates(inp, seed + 1)
    dev = torch.device("cuda:0")
    x = inp.to(dev)
    o, ht = ops.recurrent_forward_gdn2(x.q, x.k, x.v, x.g, b.to(dev), w.to(dev), scale=inp.scale,
                                       h0=x.h0, cu_seqlens=inp.cu_seqlens)
    torch.cuda.synchronize()
    cuv = None if cu is None else list(cu)
    ro, rht = oracle.forward(inp.q, inp.k, inp.v, inp.g, None, scale=inp.scale, h0=inp.h0,
                             cu_seqlens=cuv, erase=b, write=w)
    compare(dict(o=o.double().cpu().numpy(), ht=ht.double().cpu().numpy()), dict(o=ro, ht=rht),
            TOL[inp.q.dtype], cu=inp.cu_seqlens, names=("o", "ht"), label=name)


def test_recurrent_erase_write_agrees_with_chunked_and_shared_beta():
    """The token-serial erase/write forward agrees with the chunked one
    (rewy_fwd_gdn2) on the same inputs, and with b = w = beta it reproduces
    the shared-beta token-serial forward."""
    from chunkwise_delta_rule_chunk_amd import ops
    say("[case] recurrent erase/write vs chunked and vs shared beta")
    inp = workloads.make_inputs(2, 150, 2, 64, 64, gate="vector", dtype="fp32", h0="normal", seed=21)
    b, w = _ew_gates(inp, 22)
    dev = torch.device("cuda:0")
    x = inp.to(dev)
    bd, wd = b.to(dev), w.to(dev)
    o1, ht1 = ops.recurrent_forward_gdn2(x.q, x.k, x.v, x.g, bd, wd, scale=inp.scale, h0=x.h0)
    o2, ht2, _ = ops.forward_gdn2(x.q, x.k, x.v, x.g, bd, wd, scale=inp.scale, h0=x.h0)
    bb = x.beta[..., None].expand(*x.k.shape).contiguous()
    wb = x.beta[..., None].expand(*x.v.shape).contiguous()
    o3, ht3 = ops.recurrent_forward_gdn2(x.q, x.k, x.v, x.g, bb, wb, scale=inp.scale, h0=x.h0)
    o4, ht4 = ops.recurrent_forward(x.q, x.k, x.v, x.g, x.beta, scale=inp.scale, h0=x.h0)
    torch.cuda.synchronize()
    rel = lambda a, r: (torch.linalg.norm((a - r).double()) / torch.linalg.norm(r.double())).item()
    errs = dict(o_chunk=rel(o1, o2), ht_chunk=rel(ht1, ht2), o_beta=rel(o3, o4), ht_beta=rel(ht3, ht4))
    say("[parity] recurrent-ew " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert errs["o_chunk"] < 1e-4 and errs["ht_chunk"] < 1e-4, errs
    assert errs["o_beta"] < 1e-6 and errs["ht_beta"] < 1e-6, errs
