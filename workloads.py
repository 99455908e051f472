"""Seeded synthetic inputs for the chunkwise delta-rule operator.

This module holds input recipes only -- random draws, the L2 normalisation of
q and k (pre-processing outside the operator) and the construction of the
natural-log decay g from its pieces.  None of the operator's arithmetic lives
here.  Both the HIP path's tests/benchmark and the FP64 oracle take their
inputs from these generators.

Named workloads (shapes and distributions of the ReWY paper's evaluation:
chunk 64, d_k = d_v = 128, BF16 features with FP32 log gates and states):

  deltanet_t128_d32_fp32      DeltaNet, B=1 T=128 H=1 K=V=32, fp32
  gdn_b2_t2048_h16_d128       GDN scalar gate, B=2 T=2048 H=16, bf16, h0 ~ N(0, 0.02^2)
  kda_t8192_h32_d128          KDA vector gate, B=1 T=8192 H=32, bf16, zero h0
  kda_varlen16_h16_d128       KDA, 16 packed sequences of lengths U{64..4096}, H=16, bf16
  kda_b4_t32768_h32_strong    KDA strong decay, B=4 T=32768 H=32, bf16, beta=sigmoid(N+1)

Draw order per workload is fixed: q, k, v, beta logits, gate pieces, h0, dO, dht.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

SEED_BASE = 20260

WORKLOADS = {
    "deltanet_t128_d32_fp32": dict(B=1, T=128, H=1, K=32, V=32, gate="none", dtype="fp32",
                                   h0="zero", index=0),
    "gdn_b2_t2048_h16_d128": dict(B=2, T=2048, H=16, K=128, V=128, gate="scalar", dtype="bf16",
                                  h0="normal", index=1),
    "kda_t8192_h32_d128": dict(B=1, T=8192, H=32, K=128, V=128, gate="vector", dtype="bf16",
                               h0="zero", index=2),
    "kda_varlen16_h16_d128": dict(B=1, T=None, H=16, K=128, V=128, gate="vector", dtype="bf16",
                                  h0="normal", index=3, nseq=16, lmin=64, lmax=4096),
    "kda_b4_t32768_h32_strong": dict(B=4, T=32768, H=32, K=128, V=128, gate="vector",
                                     dtype="bf16", h0="zero", index=4, strong=True),
}


@dataclasses.dataclass
class Inputs:
    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: Optional[torch.Tensor]
    beta: torch.Tensor
    h0: Optional[torch.Tensor]
    dO: torch.Tensor
    dht: Optional[torch.Tensor]
    cu_seqlens: Optional[torch.Tensor]  # int32, host
    scale: float
    gate: str  # "none" | "scalar" | "vector"
    # vector gate: the pre-activation x [B,T,H,K] (fp32 draw), A_log [H] and
    # dt_bias [H,K] that g was formed from (g = -exp(A_log) softplus(x + dt_bias))
    gate_x: Optional[torch.Tensor] = None
    a_log: Optional[torch.Tensor] = None
    dt_bias: Optional[torch.Tensor] = None

    @property
    def shape(self):
        B, T, H, K = self.q.shape
        return B, T, H, K, self.v.shape[-1]

    @property
    def nseq(self):
        return self.q.shape[0] if self.cu_seqlens is None else len(self.cu_seqlens) - 1

    def to(self, device):
        f = lambda x: None if x is None else x.to(device)
        return dataclasses.replace(self, q=f(self.q), k=f(self.k), v=f(self.v), g=f(self.g),
                                   beta=f(self.beta), h0=f(self.h0), dO=f(self.dO),
                                   dht=f(self.dht), gate_x=f(self.gate_x), a_log=f(self.a_log),
                                   dt_bias=f(self.dt_bias))


def _dt(name):
    return {"bf16": torch.bfloat16, "fp32": torch.float32}[name]


def _l2n(x):
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-12)


def varlen_lengths(nseq=16, lmin=64, lmax=4096, seed=SEED_BASE + 3):
    """Sequence lengths drawn uniformly from [lmin, lmax], redrawn until at
    least one is not a multiple of 64 (so partial chunks occur)."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    while True:
        lens = torch.randint(lmin, lmax + 1, (nseq,), generator=gen)
        if bool((lens % 64 != 0).any()):
            return [int(x) for x in lens]


def make_inputs(B, T, H, K, V, *, gate="vector", dtype="bf16", seed=0, h0="zero",
                dht=False, strong=False, cu_seqlens=None, device="cpu", name="custom",
                beta_shift=None, gate_scale=1.0):
    """Inputs with the distributions of the named workloads.

    gate "vector": g = -exp(A_log[h]) * softplus(x + dt_bias[h, k]) with
      x ~ N(0,1), dt_bias ~ N(0, 0.5^2), A_log ~ U(-2, 0) (U(0, 1) if strong);
    gate "scalar": g = -softplus(n - 2) * exp(u), n ~ N(0,1), u ~ U(-3, 0);
    gate "none":   no g (DeltaNet).
    q, k ~ N(0,1) L2-normalised per token and head in fp32, then cast; v, dO ~ N(0,1);
    beta = sigmoid(N(0,1) [+1 if strong]); h0 zero, or ~ N(0, 0.02^2) if "normal".
    ``gate_scale`` multiplies g (tests use it for extreme decay).
    """
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(seed))
    dt = _dt(dtype)
    rn = lambda *s: torch.randn(*s, generator=gen, device=dev, dtype=torch.float32)
    ru = lambda lo, hi, *s: torch.rand(*s, generator=gen, device=dev, dtype=torch.float32) * (hi - lo) + lo
    q = _l2n(rn(B, T, H, K)).to(dt)
    k = _l2n(rn(B, T, H, K)).to(dt)
    v = rn(B, T, H, V).to(dt)
    shift = (1.0 if strong else 0.0) if beta_shift is None else beta_shift
    beta = torch.sigmoid(rn(B, T, H) + shift).to(dt)
    gx = a_log = dt_bias = None
    if gate == "vector":
        a_log = ru(0.0, 1.0, H) if strong else ru(-2.0, 0.0, H)
        x = rn(B, T, H, K)
        dt_bias = rn(H, K) * 0.5
        g = -torch.exp(a_log)[:, None] * torch.nn.functional.softplus(x + dt_bias)
        gx = x
    elif gate == "scalar":
        n = rn(B, T, H)
        u = ru(-3.0, 0.0, B, T, H)
        g = -torch.nn.functional.softplus(n - 2.0) * torch.exp(u)
    elif gate == "none":
        g = None
    else:
        raise ValueError(gate)
    if g is not None and gate_scale != 1.0:
        g = g * gate_scale
    N = B if cu_seqlens is None else len(cu_seqlens) - 1
    h0_t = None
    if h0 == "normal":
        h0_t = rn(N, H, K, V) * 0.02
    elif h0 == "explicit_zero":
        h0_t = torch.zeros(N, H, K, V, device=dev)
    dO = rn(B, T, H, V).to(dt)
    dht_t = rn(N, H, K, V) * 0.1 if dht else None
    cu = None if cu_seqlens is None else torch.tensor(cu_seqlens, dtype=torch.int32)
    return Inputs(name, q, k, v, g, beta, h0_t, dO, dht_t, cu, float(K) ** -0.5, gate,
                  gx, a_log, dt_bias)


def workload(name, device="cpu"):
    """The named workload, generated on ``device`` (values differ between the
    CPU and GPU generators; each caller uses one consistently)."""
    w = WORKLOADS[name]
    seed = SEED_BASE + w["index"]
    cu = None
    T = w["T"]
    if name == "kda_varlen16_h16_d128":
        lens = varlen_lengths(w["nseq"], w["lmin"], w["lmax"], seed)
        cu = [0]
        for x in lens:
            cu.append(cu[-1] + x)
        T = cu[-1]
    return make_inputs(w["B"], T, w["H"], w["K"], w["V"], gate=w["gate"], dtype=w["dtype"],
                       seed=seed, h0=w["h0"], strong=w.get("strong", False), cu_seqlens=cu,
                       device=device, name=name)


def paper_harness(B, T, H, K, V, *, gate="vector", dtype="bf16", seed=0, device="cpu",
                  cu_seqlens=None):
    """The ReWY paper's numerical-validation harness distributions (Appendix,
    "Numerical coverage"): normalised Gaussian q/k, Gaussian v/dO, scale
    K^-1/2, Gaussian initial/terminal states x0.1, log gates log(sigmoid(x))/16,
    beta uniform in [0.1, 0.9]."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(seed))
    dt = _dt(dtype)
    rn = lambda *s: torch.randn(*s, generator=gen, device=dev, dtype=torch.float32)
    q = _l2n(rn(B, T, H, K)).to(dt)
    k = _l2n(rn(B, T, H, K)).to(dt)
    v = rn(B, T, H, V).to(dt)
    beta = (torch.rand(B, T, H, generator=gen, device=dev) * 0.8 + 0.1).to(dt)
    if gate == "vector":
        g = torch.nn.functional.logsigmoid(rn(B, T, H, K)) / 16
    elif gate == "scalar":
        g = torch.nn.functional.logsigmoid(rn(B, T, H)) / 16
    else:
        g = None
    N = B if cu_seqlens is None else len(cu_seqlens) - 1
    h0 = rn(N, H, K, V) * 0.1
    dO = rn(B, T, H, V).to(dt)
    dht = rn(N, H, K, V) * 0.1
    cu = None if cu_seqlens is None else torch.tensor(cu_seqlens, dtype=torch.int32)
    return Inputs("paper_harness", q, k, v, g, beta, h0, dO, dht, cu, float(K) ** -0.5, gate)
