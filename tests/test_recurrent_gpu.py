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
    compare(hip, _oracle_fwd(inp), TOL[inp.q.dtype], names=("o", "ht"), label=name)


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
    compare(hip, _oracle_fwd(inp), TOL[inp.q.dtype], names=("o", "ht"), label="decode-steps")


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
