"""The separate producer-consumer schedule of the chunk backward
(rewy_bwd_schedule(REWY_SCHEDULE_SEPARATE): P, D and the write part of dbeta
go through the workspace) against the joint one: every value is rounded at
the same point in both, so every gradient must be bitwise equal; one case is
also compared with the FP64 oracle."""
import zlib

import pytest
import torch

import workloads
from parity_util import TOL, compare, gpu_available, hip_run_torch, oracle_run, say, to_np

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU and librewy.so")]

CASES = [
    # name, B, T, H, K, V, gate, dtype, h0, dht, cu
    ("sched_bf16_vector_k128_varlen", 1, 330, 2, 128, 128, "vector", "bf16", "normal", True,
     [0, 1, 64, 128, 193, 330]),
    ("sched_bf16_scalar_k128", 2, 200, 2, 128, 128, "scalar", "bf16", "normal", True, None),
    ("sched_bf16_none_k64", 1, 130, 3, 64, 64, "none", "bf16", "zero", False, None),
    ("sched_fp32_vector_k64", 1, 150, 2, 64, 64, "vector", "fp32", "normal", True, None),
    ("sched_fp32_scalar_k32_v64", 2, 100, 2, 32, 64, "scalar", "fp32", "normal", True, None),
]


@pytest.fixture
def separate():
    from chunkwise_delta_rule_chunk_amd import binding as B
    prev = B.rewy_bwd_schedule(B.REWY_SCHEDULE_SEPARATE)
    try:
        yield
    finally:
        B.rewy_bwd_schedule(prev)


def _both(inp, policy):
    from chunkwise_delta_rule_chunk_amd import binding as B
    joint = hip_run_torch(inp, policy, want_dh0=True)
    prev = B.rewy_bwd_schedule(B.REWY_SCHEDULE_SEPARATE)
    try:
        sep = hip_run_torch(inp, policy, want_dh0=True)
    finally:
        B.rewy_bwd_schedule(prev)
    return joint, sep


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("policy", ["recompute", "save"])
def test_separate_schedule_equals_joint_bitwise(case, policy):
    name, B_, T, H, K, V, gate, dt, h0, dht, cu = case
    say(f"[case] {name} policy={policy}")
    inp = workloads.make_inputs(B_, T, H, K, V, gate=gate, dtype=dt, seed=zlib.crc32(name.encode()) % 1000,
                                h0=h0, dht=dht, cu_seqlens=cu)
    joint, sep = _both(inp, policy)
    for n in joint:
        if joint[n] is not None:
            assert torch.equal(joint[n], sep[n]), (name, policy, n)


def test_separate_schedule_matches_oracle_on_the_kda_workload():
    """The KDA workload (B=1, T=8192, H=32, d=128, bf16) under the separate
    schedule, every (sequence, head) unit against the oracle."""
    from chunkwise_delta_rule_chunk_amd import binding as B
    name = "kda_t8192_h32_d128"
    say(f"[case] {name} separate schedule")
    inp = workloads.workload(name)
    prev = B.rewy_bwd_schedule(B.REWY_SCHEDULE_SEPARATE)
    try:
        hip = to_np(hip_run_torch(inp, "recompute", want_dh0=True))
    finally:
        B.rewy_bwd_schedule(prev)
    compare(hip, oracle_run(inp), TOL[inp.q.dtype], cu=inp.cu_seqlens, label=f"{name}/separate")
