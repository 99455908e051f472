"""GPU parity of the scan dispatch order on varlen batches: the chunk table
ranks sequences by chunk count (longest first) when there are at most 1024 of
them and keeps their index order beyond that; either way every (sequence,
head) is scanned exactly once, from its own initial state.  Checked against
the FP64 oracle on a skewed batch (a few long sequences among many short ones)
and on 1100 short sequences (past the ranking limit), both policies."""
import numpy as np
import pytest

import workloads
from parity_util import TOL, compare, gpu_available, hip_run, oracle_run, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU and librewy.so")]


def _cu(lens):
    return [0] + list(np.cumsum(lens).astype(int))


def _skewed():
    rng = np.random.default_rng(31)
    lens = list(rng.integers(1, 70, size=60)) + [700, 1, 333, 64, 640]
    rng.shuffle(lens)
    return [int(x) for x in lens]


def _many():
    rng = np.random.default_rng(32)
    return [int(x) for x in rng.integers(1, 40, size=1100)]


CASES = [
    ("skewed_bf16_k64", _skewed, 2, 64, 64, "bf16", "vector"),
    ("many_fp32_k32", _many, 2, 32, 32, "fp32", "scalar"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("policy", ["recompute", "save"])
def test_varlen_scan_order_matches_oracle(case, policy):
    name, mk, H, K, V, dt, gate = case
    lens = mk()
    cu = _cu(lens)
    say(f"[case] {name} policy={policy} sequences={len(lens)} tokens={cu[-1]}")
    inp = workloads.make_inputs(1, cu[-1], H, K, V, gate=gate, dtype=dt, seed=17, h0="normal",
                                dht=True, cu_seqlens=cu)
    compare(hip_run(inp, policy=policy, want_dh0=True), oracle_run(inp), TOL[inp.q.dtype], cu=inp.cu_seqlens,
            label=f"{name}/{policy}")
