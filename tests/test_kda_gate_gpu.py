"""GPU parity of the gate formed inside the kernels (rewy_fwd_kda_gate /
rewy_bwd_kda_gate: g = -exp(A_log) softplus(x + dt_bias), GDN2 spec section
4.4, or the bounded g = lower_bound sigmoid(exp(A_log)(x + dt_bias)), section
3) against the FP64 oracle: the oracle forms g from the same pre-activation
(rounded to the feature dtype, as the kernels read it), runs its token
recurrence and reverse mode, and takes dg back to dx, dA_log and ddt_bias with
its own chain rule.  Every output and gradient within the stated tolerances,
both dtypes, varlen, both saving policies, and the pairwise path of a strongly
decaying gate; the parameter gradients are identical between repeated calls."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_util import TOL, compare, gpu_available, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU and librewy.so")]

NAMES = ("o", "ht", "dq", "dk", "dv", "dx", "da_log", "ddt_bias", "dbeta", "dh0")

CASES = [
    # name, B, T, H, K, V, dtype, h0, cu
    ("kdag_bf16_k128", 2, 200, 2, 128, 128, "bf16", "normal", None),
    ("kdag_bf16_k64_v128", 1, 150, 3, 64, 128, "bf16", "zero", None),
    ("kdag_fp32_k64", 1, 140, 2, 64, 64, "fp32", "normal", None),
    ("kdag_fp32_k32_v64", 2, 90, 1, 32, 64, "fp32", "normal", None),
    ("kdag_bf16_varlen", 1, 330, 2, 64, 64, "bf16", "normal", [0, 1, 64, 128, 193, 330]),
]

# the bounded form: name, B, T, H, K, V, dtype, h0, cu, lower_bound, A_log shift
BOUNDED = [
    ("kdagb_bf16_k128_lb1", 2, 200, 2, 128, 128, "bf16", "normal", None, -1.0, 0.0),
    ("kdagb_fp32_k64_lb3", 1, 140, 2, 64, 64, "fp32", "normal", None, -3.0, 0.0),
    # exp(A_log) ~ 30: most gates sit near the bound -5, sub-chunk ranges near
    # 16 * 5 / ln 2 = 115 log2 units (the widest the bound allows)
    ("kdagb_bf16_lb5_strong", 1, 256, 2, 64, 64, "bf16", "normal", None, -5.0, 3.4),
    ("kdagb_bf16_varlen_lb2", 1, 330, 2, 64, 64, "bf16", "normal", [0, 1, 64, 128, 193, 330], -2.0, 0.0),
]


def _inputs(name, B, T, H, K, V, dt, h0, cu, a_shift=0.0):
    seed = zlib.crc32(name.encode()) % 1000
    inp = workloads.make_inputs(B, T, H, K, V, gate="vector", dtype=dt, seed=seed, h0=h0, dht=True,
                                cu_seqlens=cu)
    x = inp.gate_x.to(inp.q.dtype)  # the kernels read x in the feature dtype
    a_log = inp.a_log + a_shift
    return inp, x, a_log, inp.dt_bias


def _oracle(inp, x, a_log, dt_bias, lb=0.0):
    cu = None if inp.cu_seqlens is None else list(inp.cu_seqlens)
    g = oracle.kda_gate(x, a_log, dt_bias, lb)
    o, ht = oracle.forward(inp.q, inp.k, inp.v, g, inp.beta, scale=inp.scale, h0=inp.h0,
                           cu_seqlens=cu)
    gr = oracle.backward(inp.q, inp.k, inp.v, g, inp.beta, inp.dO, scale=inp.scale, h0=inp.h0,
                         dht=inp.dht, cu_seqlens=cu)
    dx, da, ddt = oracle.kda_gate_backward(x, a_log, dt_bias, gr["dg"], lb)
    return dict(o=o, ht=ht, dq=gr["dq"], dk=gr["dk"], dv=gr["dv"], dx=dx, da_log=da, ddt_bias=ddt,
                dbeta=gr["dbeta"], dh0=gr["dh0"])


def _hip_torch(inp, x, a_log, dt_bias, policy, lb=0.0):
    from chunkwise_delta_rule_chunk_amd import ops
    dev = torch.device("cuda:0")
    t = inp.to(dev)
    xd, ad, dd = x.to(dev), a_log.to(dev).contiguous(), dt_bias.to(dev).contiguous()
    o, ht, ctx = ops.forward_kda_gate(t.q, t.k, t.v, xd, ad, dd, t.beta, lower_bound=lb,
                                      scale=inp.scale, h0=t.h0, cu_seqlens=inp.cu_seqlens,
                                      policy=policy)
    gr = ops.backward(ctx, t.dO, t.dht, want_dh0=True)
    torch.cuda.synchronize()
    return dict(o=o, ht=ht, **gr)


def _np(out):
    return {k: (None if v is None else v.double().cpu().numpy()) for k, v in out.items()}


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("policy", ["recompute", "save"])
def test_kda_gate_matches_oracle(case, policy):
    name = case[0]
    say(f"[case] {name} policy={policy}")
    inp, x, a_log, dt_bias = _inputs(*case)
    compare(_np(_hip_torch(inp, x, a_log, dt_bias, policy)), _oracle(inp, x, a_log, dt_bias),
            TOL[inp.q.dtype], cu=inp.cu_seqlens, names=NAMES, label=f"{name}/{policy}")


@pytest.mark.parametrize("case", BOUNDED, ids=[c[0] for c in BOUNDED])
@pytest.mark.parametrize("policy", ["recompute", "save"])
def test_kda_gate_bounded_form_matches_oracle(case, policy):
    name, lb, shift = case[0], case[9], case[10]
    say(f"[case] {name} policy={policy} lower_bound={lb}")
    inp, x, a_log, dt_bias = _inputs(*case[:9], a_shift=shift)
    compare(_np(_hip_torch(inp, x, a_log, dt_bias, policy, lb)), _oracle(inp, x, a_log, dt_bias, lb),
            TOL[inp.q.dtype], cu=inp.cu_seqlens, names=NAMES, label=f"{name}/{policy}")


def test_kda_gate_agrees_with_the_explicit_gate():
    """The gate formed in the kernels gives the results of rewy_fwd / rewy_bwd
    fed with g formed on the host in fp32 from the same x (up to the rounding
    of the two fp32 evaluations of softplus), and dx, dA_log, ddt_bias are that
    dg taken through the gate's chain rule."""
    from chunkwise_delta_rule_chunk_amd import ops
    say("[case] kda gate vs explicit g")
    inp, x, a_log, dt_bias = _inputs("kdag_vs_g", 1, 256, 2, 64, 64, "fp32", "normal", None)
    dev = torch.device("cuda:0")
    g = (-torch.exp(a_log)[:, None] * torch.nn.functional.softplus(x.float() + dt_bias)).to(dev)
    t = inp.to(dev)
    o1, ht1, c1 = ops.forward(t.q, t.k, t.v, g.contiguous(), t.beta, scale=inp.scale, h0=t.h0)
    g1 = ops.backward(c1, t.dO, t.dht)
    out = _hip_torch(inp, x, a_log, dt_bias, "recompute")
    dx, da, ddt = oracle.kda_gate_backward(x, a_log, dt_bias, g1["dg"].double().cpu().numpy())
    rel = lambda a, r: float(np.linalg.norm(np.asarray(a, np.float64) - r) / np.linalg.norm(r))
    cpu = lambda a: a.double().cpu().numpy()
    errs = dict(o=rel(cpu(out["o"]), cpu(o1)), ht=rel(cpu(out["ht"]), cpu(ht1)),
                dq=rel(cpu(out["dq"]), cpu(g1["dq"])), dk=rel(cpu(out["dk"]), cpu(g1["dk"])),
                dx=rel(cpu(out["dx"]), dx), da_log=rel(cpu(out["da_log"]), da),
                ddt_bias=rel(cpu(out["ddt_bias"]), ddt))
    say("[parity] kda-gate-vs-g " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v < 1e-5 for v in errs.values()), errs


def test_kda_gate_strong_decay_takes_pairwise_path():
    """A_log shifted by log(30): diagonal sub-chunks exceed the centring bound,
    so the forward's pairwise diagonal forms the gate per element from x."""
    say("[case] kda gate strong decay pairwise")
    inp, x, a_log, dt_bias = _inputs("kdag_strong", 1, 256, 2, 64, 64, "bf16", "normal", None,
                                     a_shift=float(np.log(30.0)))
    g = oracle.kda_gate(x, a_log, dt_bias)
    G = np.cumsum(g.reshape(1, 4, 64, 2, 64), axis=2) / np.log(2)
    sub = G.reshape(1, 4, 4, 16, 2, 64)
    assert (sub.max(3) - sub.min(3)).max() > 128  # the fallback is really exercised
    compare(_np(_hip_torch(inp, x, a_log, dt_bias, "recompute")), _oracle(inp, x, a_log, dt_bias),
            TOL[inp.q.dtype], cu=inp.cu_seqlens, names=NAMES, label="kda-gate-strong-decay")


def _hip_no_host_cu(inp, x, a_log, dt_bias, lb=0.0):
    """Forward + backward through the C ABI with cu_seqlens on the device only:
    the chunk slots are then an upper bound and some hold no tokens."""
    from chunkwise_delta_rule_chunk_amd import binding as B
    from chunkwise_delta_rule_chunk_amd import ops
    dev = torch.device("cuda:0")
    t = inp.to(dev)
    xd, ad, dd = x.to(dev), a_log.to(dev).contiguous(), dt_bias.to(dev).contiguous()
    prob = ops.make_problem(t.q, t.v, None, t.beta, scale=inp.scale, cu_seqlens=inp.cu_seqlens,
                            vector_gate=True)
    prob.desc.cu_seqlens_host = None
    p = ops._p
    s = ops._stream(dev, None)
    o, ht = torch.empty_like(t.v), torch.empty(prob.state_shape, device=dev)
    ws0, ws2 = ops.workspace(prob, 0), ops.workspace(prob, 2)
    assert ws2.numel() > B.rewy_workspace_bytes(prob.desc, 1)
    ops._check(B.rewy_fwd_kda_gate(prob.desc, p(t.q), p(t.k), p(t.v), p(xd), p(ad), p(dd), lb,
                                   p(t.beta), p(t.h0), p(o), p(ht), None, p(ws0), ws0.numel(), s),
               "fwd")
    dq, dk, dv, dx = (torch.empty_like(a) for a in (t.q, t.k, t.v, xd))
    da, ddt, dbeta = torch.empty_like(ad), torch.empty_like(dd), torch.empty_like(t.beta)
    dh0 = torch.empty(prob.state_shape, device=dev)
    ops._check(B.rewy_bwd_kda_gate(prob.desc, p(t.q), p(t.k), p(t.v), p(xd), p(ad), p(dd), lb,
                                   p(t.beta), p(t.h0), p(t.dO), p(t.dht), None, p(dq), p(dk), p(dv), p(dx),
                                   p(da), p(ddt), p(dbeta), p(dh0), p(ws2), ws2.numel(), s), "bwd")
    torch.cuda.synchronize()
    return dict(o=o, ht=ht, dq=dq, dk=dk, dv=dv, dx=dx, da_log=da, ddt_bias=ddt, dbeta=dbeta,
                dh0=dh0)


def test_kda_gate_parameter_gradients_are_deterministic():
    """Two backward calls on the same inputs give bit-identical dA_log and
    ddt_bias (the sums over chunks run in a fixed order); with cu_seqlens on
    the device only, the chunk slots that hold no tokens add nothing and the
    results still match the oracle."""
    say("[case] kda gate determinism and empty chunk slots")
    cu = [0, 7, 70, 200, 333]
    inp, x, a_log, dt_bias = _inputs("kdag_det", 1, 333, 2, 128, 128, "bf16", "normal", cu)
    a = _hip_torch(inp, x, a_log, dt_bias, "recompute")
    b = _hip_torch(inp, x, a_log, dt_bias, "recompute")
    for n in ("da_log", "ddt_bias", "dx"):
        assert torch.equal(a[n], b[n]), n
    c = _hip_no_host_cu(inp, x, a_log, dt_bias)
    ref = _oracle(inp, x, a_log, dt_bias)
    compare(_np(c), ref, TOL[inp.q.dtype], cu=inp.cu_seqlens, names=NAMES, label="kda-gate-device-cu")
    compare(_np(a), ref, TOL[inp.q.dtype], cu=inp.cu_seqlens, names=NAMES, label="kda-gate-host-cu")


def test_kda_gate_bounded_form_empty_slots_and_repeatability():
    """The bounded form with cu_seqlens on the device only (chunk slots without
    tokens) matches the oracle, and repeated calls give identical parameter
    gradients."""
    say("[case] kda gate bounded form, device-only cu_seqlens")
    cu = [0, 7, 70, 200, 333]
    inp, x, a_log, dt_bias = _inputs("kdagb_det", 1, 333, 2, 128, 128, "bf16", "normal", cu)
    a = _hip_no_host_cu(inp, x, a_log, dt_bias, -4.0)
    b = _hip_no_host_cu(inp, x, a_log, dt_bias, -4.0)
    for n in ("da_log", "ddt_bias", "dx"):
        assert torch.equal(a[n], b[n]), n
    compare(_np(a), _oracle(inp, x, a_log, dt_bias, -4.0), TOL[inp.q.dtype], cu=inp.cu_seqlens, names=NAMES,
            label="kda-gate-bounded-device-cu")


@pytest.mark.timeout(600)
def test_kda_gate_long_strong_decay_two_heads_all_rows():
    """The gate formed in the kernels on the long-context strong-decay workload
    (B=4, T=32768, H=32, d=128, bf16, A_log ~ U(0, 1)) at full size.  The oracle
    computes two heads over all four batch rows, so its dA_log and ddt_bias of
    those heads sum every token of every sequence, as the kernels' do (about
    sixteen times the terms of the KDA workload, with cancellation)."""
    name = "kda_b4_t32768_h32_strong"
    say(f"[case] {name} gate formed in the kernels: GPU")
    inp = workloads.workload(name, device="cuda")
    x = inp.gate_x.to(inp.q.dtype)
    out = _hip_torch(inp, x, inp.a_log, inp.dt_bias, "recompute")
    heads = [5, 30]

    def pick(k, v):
        if k in ("ht", "dh0"):
            return v[:, heads]
        if k in ("da_log", "ddt_bias"):
            return v[heads]
        return v[:, :, heads]

    hip = {k: (None if v is None else pick(k, v).double().cpu().numpy()) for k, v in out.items()}
    del out
    cut = lambda t: t[:, :, heads].cpu()
    sub = workloads.Inputs(name, cut(inp.q), cut(inp.k), cut(inp.v), None, cut(inp.beta), None,
                           cut(inp.dO), None, None, inp.scale, inp.gate)
    say(f"[case] {name} gate formed in the kernels: oracle heads {heads}, all rows")
    ref = _oracle(sub, cut(x), inp.a_log[heads].cpu(), inp.dt_bias[heads].cpu())
    compare(hip, ref, TOL[inp.q.dtype], names=NAMES, label=f"{name}/kda-gate")
