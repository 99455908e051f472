"""The allocation-free forward, rewy_fwd_noalloc, through the C ABI against
rewy_fwd with a caller-owned workspace.  Two calls in a row, the second on a
smaller problem (so stale contents of the shared device scratch would show),
under both saving policies; the outputs must be bitwise equal (the same
kernels in the same order), and under the save-all policy so must the
backward computed from each call's saved buffer."""
import pytest
import torch

import workloads
from parity_util import gpu_available, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU and librewy.so")]


def _forward(inp, policy, noalloc):
    from chunkwise_delta_rule_chunk_amd import binding as B
    from chunkwise_delta_rule_chunk_amd import ops
    dev = torch.device("cuda:0")
    x = inp.to(dev)
    prob = ops.make_problem(x.q, x.v, x.g, x.beta, scale=inp.scale, cu_seqlens=inp.cu_seqlens,
                            policy=policy)
    o = torch.empty_like(x.v)
    ht = torch.empty(prob.state_shape, dtype=torch.float32, device=dev)
    nsaved = B.rewy_saved_bytes(prob.desc)
    saved = torch.empty(nsaved, dtype=torch.uint8, device=dev) if nsaved else None
    p, s = ops._p, ops._stream(dev, None)
    if noalloc:
        assert B.rewy_workspace_bytes(prob.desc, 0) <= B.NOALLOC_SCRATCH_BYTES
        rc = B.rewy_fwd_noalloc(prob.desc, p(x.q), p(x.k), p(x.v), p(x.g), p(x.beta), p(x.h0),
                                p(o), p(ht), p(saved), s)
    else:
        ws = ops.workspace(prob, 0)
        rc = B.rewy_fwd(prob.desc, p(x.q), p(x.k), p(x.v), p(x.g), p(x.beta), p(x.h0), p(o),
                        p(ht), p(saved), p(ws), ws.numel(), s)
    assert rc == B.REWY_OK, B.rewy_last_error()
    torch.cuda.synchronize()
    ctx = dict(prob=prob, q=x.q, k=x.k, v=x.v, g=x.g, beta=x.beta, h0=x.h0, saved=saved)
    return o, ht, ctx, x


@pytest.mark.parametrize("policy", ["recompute", "save"])
def test_noalloc_forward_matches_rewy_fwd_twice(policy):
    from chunkwise_delta_rule_chunk_amd import ops
    cases = [
        workloads.make_inputs(2, 700, 8, 128, 128, gate="vector", dtype="bf16", seed=31,
                              h0="normal", dht=True),
        # second call: smaller, packed sequences of other lengths, another gate kind
        workloads.make_inputs(1, 130, 3, 64, 64, gate="scalar", dtype="bf16", seed=32,
                              h0="normal", dht=True, cu_seqlens=[0, 1, 70, 130]),
    ]
    for i, inp in enumerate(cases):
        say(f"[case] noalloc {policy} call {i}: shape {inp.shape}")
        o1, ht1, c1, x = _forward(inp, policy, noalloc=True)
        o2, ht2, c2, _ = _forward(inp, policy, noalloc=False)
        assert torch.equal(o1, o2) and torch.equal(ht1, ht2), (policy, i)
        if policy == "save":  # the saved buffers serve the backward identically
            g1 = ops.backward(c1, x.dO, x.dht, want_dh0=True)
            g2 = ops.backward(c2, x.dO, x.dht, want_dh0=True)
            torch.cuda.synchronize()
            for n in g1:
                if g1[n] is not None:
                    assert torch.equal(g1[n], g2[n]), (policy, i, n)
        say(f"[case] noalloc {policy} call {i}: bitwise equal to rewy_fwd")
