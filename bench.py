"""Benchmark of the MI355X chunkwise gated delta rule: one step = rewy_fwd +
rewy_bwd (complete backward) on the KDA workload B=1, T=8192, H=32,
K=V=128, bf16 features, fp32 gates, synthetic seeded inputs resident in HBM.

Prints ONE JSON line: whole-job fwd+bwd tokens/s, algorithmic TFLOPS and the
fraction of the bf16 MFMA peak, a roofline entry for the dominant kernel
(the method's compulsory bytes and FLOPs per launch over the kernel's
HIP-event duration, measured on the launch stream), the timing protocol of
the ReWY paper (60 graph-replayed observations per pass), measured copy and
GEMM peaks, and the FP64 oracle timed on the host cores on a bounded sample.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fwd+bwd tokens/s and MFMA TFLOPS (% bf16 peak), KDA H=32 d=128 T=8192"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (public spec)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (public spec)
# The pages' own operator figures, quoted as context (other hardware, ratios
# against their reference implementation; not targets).
PAGES_CONTEXT = {
    "wy_graph_dense_flops_per_chunk_head": "7.34M expanded -> 4.19M ReWY (-42.9%), n=64, d=128 "
                                           "(ReWY paper, Arithmetic and intermediate storage)",
    "complete_backward_speedup_nvidia": "1.15-1.81x (RTX 5070Ti, A800; ReWY paper, Results)",
    "complete_backward_speedup_ascend_950dt": "1.09-2.89x (ReWY paper, Results)",
}

# ---- kernel names -------------------------------------------------------------
# The trace hook reports each kernel by its symbol exactly as rocprofv3 does:
# demangled where the host's demangler can, else mangled (the bfloat16
# instantiations, e.g. "_ZN4rewy10k_fwd_prepIDF16bLi128ELi128ELi13EEEvNS_4ArgsE").
_PREP_ROLE = {3: "forward", 15: "forward, saving", 13: "recompute"}


def parse_kernel(name):
    """(stage, template arguments) of a kernel name, demangled or mangled."""
    m = re.search(r"rewy::(k_\w+)(?:<([^>]*)>)?", name)
    if m:
        args = [a.strip() for a in m.group(2).split(",")] if m.group(2) else []
        return m.group(1), args
    m = re.match(r"_ZN4rewy(\d+)(\w+)", name)
    if m:
        n = int(m.group(1))
        stage, rest = m.group(2)[:n], m.group(2)[n:]
        args = []
        if rest.startswith("I"):
            t = re.match(r"I(DF16b|u6__bf16|f)", rest)
            if t:
                args.append("__bf16" if t.group(1) != "f" else "float")
            args += re.findall(r"Li(\d+)E", rest)
        return stage, args
    return name, []


def kernel_label(name):
    """Short label: the stage plus what its template arguments select."""
    stage, args = parse_kernel(name)
    if stage == "k_fwd_prep" and len(args) >= 4:
        mode = int(args[3])
        role = _PREP_ROLE.get(mode & 15, f"mode {mode}")
        extra = (", erase/write" if mode & 16 else "") + (", gate in kernel" if mode & 32 else "")
        return f"k_fwd_prep ({role}{extra})"
    if stage == "k_fwd_scan" and len(args) >= 5:
        return f"k_fwd_scan (BV={args[3]}{', saving' if int(args[4]) & 1 else ''})"
    if stage in ("k_scans", "k_bwd_scan") and len(args) >= 4:
        return f"{stage} (BV={args[3]})"
    if stage == "k_bwd_chunk" and len(args) >= 4:
        gx = int(args[3])
        if gx & 16:
            return "k_bwd_chunk (producer)"
        kind = {0: "no gate", 1: "scalar gate", 2: "vector gate"}[gx & 3]
        return (f"k_bwd_chunk ({'consumers, ' if gx & 32 else ''}{kind}"
                f"{', erase/write' if gx & 4 else ''}{', gate in kernel' if gx & 8 else ''})")
    return stage


def kernel_role(name):
    """Which part of the method a launch executes: prep_forward, prep_recompute,
    fwd_scan, bwd_scan, scans (recompute scan with the reverse scan),
    bwd_chunk or other."""
    stage, args = parse_kernel(name)
    if stage == "k_fwd_prep":
        return "prep_recompute" if len(args) >= 4 and (int(args[3]) & 2) == 0 else "prep_forward"
    if stage == "k_bwd_chunk" and len(args) >= 4:
        gx = int(args[3])
        return "bwd_producer" if gx & 16 else "bwd_consumers" if gx & 32 else "bwd_chunk"
    return {"k_fwd_scan": "fwd_scan", "k_bwd_scan": "bwd_scan", "k_scans": "scans",
            "k_bwd_chunk": "bwd_chunk"}.get(stage, "other")


# ---- the method's compulsory bytes per launch ----------------------------------

def method_bytes(role, n_tokens, H, K, V, esz, besz, gate, nseq, has_h0, has_dht):
    """Compulsory HBM bytes of the method that one launch of `role` moves: the
    operator's inputs it reads and outputs it writes, each counted once per
    token-head (bf16 feature rows 256 B at d=128, fp32 gate rows 4 K B), plus
    the fp32 [K, V] states it reads or writes.  The forward prep reads q, k, v,
    g, beta (1,282 B per token-head on the KDA workload); the forward scan
    writes o; the reverse scan reads dO; the chunk backward takes the whole
    backward floor, q, k, v, g, beta, dO in and dq, dk, dv, dg, dbeta out
    (2,820 B per token-head).  Intermediates of this design are not counted."""
    tk, tv = K * esz, V * esz
    gb = {0: 0, 1: 4, 2: 4 * K}[gate]
    st = nseq * H * K * V * 4
    per = {
        "prep_forward": 2 * tk + tv + gb + besz,
        "prep_recompute": 2 * tk + tv + gb + besz,
        "fwd_scan": tv,
        "bwd_scan": tv,
        "scans": tv,
        "bwd_chunk": 2 * (2 * tk + tv + gb + besz) + tv,
        # the separate schedule splits that floor: v, beta in and dv out for
        # the producer; the rest for the consumers
        "bwd_producer": 2 * tv + besz,
        "bwd_consumers": 2 * (2 * tk + gb) + tv + 2 * besz,
    }.get(role)
    if per is None:
        return None
    states = 0
    if role == "fwd_scan":
        states = st * (1 + (1 if has_h0 else 0))              # ht written, h0 read
    elif role in ("bwd_scan", "scans"):
        states = st * (1 + (1 if has_dht else 0))             # dh0 written, dht read
    return per * n_tokens * H + states


def method_flops(role, seq_lens, H, K, V, flops):
    key = {"prep_forward": "prep_forward", "fwd_scan": "fwd_scan", "bwd_scan": "bwd_scan",
           "scans": "bwd_scan", "bwd_chunk": "bwd_chunk", "bwd_producer": "bwd_producer",
           "bwd_consumers": "bwd_consumers"}.get(role)
    return 0 if key is None else flops.kernel_flops(key, seq_lens, H, K, V)


def design_bytes(role, chunk_lens, H, K, V, esz, besz, gate, nseq, policy):
    """HBM bytes one launch moves in this design: the method's inputs and
    outputs plus the intermediates the kernel reads and writes (each once;
    chunk tiles count all 64 rows).  Compared with the counter-measured traffic
    this shows re-reads; it is not the roofline numerator."""
    n = sum(chunk_lens)
    nc = len(chunk_lens)
    gb = {0: 0, 1: 4, 2: 4 * K}[gate]
    tk, tv = K * esz, V * esz
    tileK, tileV, tile64 = nc * 64 * K * esz, nc * 64 * V * esz, nc * 64 * 64 * esz
    st = nc * K * V * esz
    glast = nc * K * 4
    # G2 tile of the chunk backward: written for a scalar gate only (the chunk
    # backward rebuilds G2 of a vector gate from g and the statistics)
    g2t = {0: 0, 1: nc * 64 * 4, 2: 0}[gate]
    gst = nc * 4 * K * 16
    prep_in = n * (2 * tk + tv + gb + besz)
    w_fscan = 2 * tileK + tileV + glast                   # W, Ft, U, glast
    w_fout = tileK + tile64                                 # Qg, Cq
    w_bscan = 3 * tileK + tile64                            # F, Wt, Qgt, Cqt
    w_bchunk = tile64 + g2t + gst                           # At, G2t, Gst
    fscan_in = 2 * tileK + tileV + glast
    per_head = {
        "prep_forward": prep_in + w_fscan + w_fout + ((w_bscan + w_bchunk) if policy == "save" else 0),
        "prep_recompute": prep_in + w_fscan + w_bscan + w_bchunk,
        "fwd_scan": fscan_in + w_fout + n * tv + ((st + tileV) if policy == "save" else 0),
        "bwd_scan": w_bscan + glast + n * tv + st + tileV,
        # reads dO, v, q, k, beta, A^T, R, Rbar, S, dS+, statistics, glast and
        # g (vector gate) or the G2 tile (scalar gate); writes dq, dk, dv, dg, dbeta
        "bwd_chunk": n * (3 * tv + 4 * tk + 2 * besz) + tile64 + 2 * tileV + 2 * st + gst + glast
                     + (n * gb if gate == 2 else g2t) + n * gb,
    }
    per_head["scans"] = fscan_in + st + tileV + per_head["bwd_scan"]
    b = per_head.get(role)
    if b is None:
        return None
    extra = {"fwd_scan": 2, "bwd_scan": 2, "scans": 4}.get(role, 0) * 4 * K * V * nseq
    return b * H + extra * H


def measured_traffic(label, workload, policy):
    """HBM bytes per launch of the kernel `label` from the committed rocprofv3
    counter summary (FETCH_SIZE and WRITE_SIZE, calibrated on a plain copy),
    or None when there is no summary for this workload or the library sources
    changed since the counters were taken."""
    from chunkwise_delta_rule_chunk_amd import build
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}_{policy}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"Library source digest: `([0-9a-f]+)`", text)
    if not m or m.group(1) != build.source_digest():
        return None
    for line in text.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) >= 4 and cells[0] == f"`{label}`":
            return float(cells[3])
    return None


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


# ---- the timed step: rewy_fwd + rewy_bwd on preallocated buffers ---------------

class Step:
    """rewy_fwd and rewy_bwd of one workload and policy through the C ABI,
    with every output, the workspace and the saved buffer allocated once
    (so a call enqueues the kernels only, and graph capture sees no
    allocation)."""

    def __init__(self, x, inp, policy, torch, ops, B):
        self.B, self.torch = B, torch
        self.x = x
        self.prob = ops.make_problem(x.q, x.v, x.g, x.beta, scale=inp.scale,
                                     cu_seqlens=inp.cu_seqlens, policy=policy)
        d = self.prob.desc
        dev = x.q.device
        self.ws0, self.ws1 = ops.workspace(self.prob, 0), ops.workspace(self.prob, 1)
        nsaved = B.rewy_saved_bytes(d)
        self.saved = torch.empty(nsaved, dtype=torch.uint8, device=dev) if nsaved else None
        self.o = torch.empty_like(x.v)
        self.ht = torch.empty(self.prob.state_shape, dtype=torch.float32, device=dev)
        self.dq, self.dk, self.dv = (torch.empty_like(t) for t in (x.q, x.k, x.v))
        self.dg = None if x.g is None else torch.empty_like(x.g)
        self.dbeta = torch.empty_like(x.beta)
        self.dh0 = None if x.h0 is None else torch.empty_like(x.h0)
        self.p = ops._p
        self.stream = lambda: ops._stream(dev, None)

    def fwd(self):
        p, x, d = self.p, self.x, self.prob.desc
        rc = self.B.rewy_fwd(d, p(x.q), p(x.k), p(x.v), p(x.g), p(x.beta), p(x.h0), p(self.o),
                             p(self.ht), p(self.saved), p(self.ws0), self.ws0.numel(), self.stream())
        if rc:
            raise self.B.RewyError(rc, "rewy_fwd")

    def bwd(self):
        p, x, d = self.p, self.x, self.prob.desc
        rc = self.B.rewy_bwd(d, p(x.q), p(x.k), p(x.v), p(x.g), p(x.beta), p(x.h0), p(x.dO),
                             p(x.dht), p(self.saved), p(self.dq), p(self.dk), p(self.dv), p(self.dg),
                             p(self.dbeta), p(self.dh0), p(self.ws1), self.ws1.numel(), self.stream())
        if rc:
            raise self.B.RewyError(rc, "rewy_bwd")

    def __call__(self):
        self.fwd()
        self.bwd()


def graph_protocol(step, torch, n_obs=60):
    """The pages' timing protocol: rewy_fwd and rewy_bwd each captured twice in
    a HIP graph, then n_obs replays of each, timed separately with events on
    the replay stream and normalised per call.  Returns medians and p10/p90 in
    ms per call."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):
            step.fwd()
            step.bwd()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    gf, gb = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(gf):
        step.fwd()
        step.fwd()
    with torch.cuda.graph(gb):
        step.bwd()
        step.bwd()
    for _ in range(5):
        gf.replay()
        gb.replay()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_obs)]
    for e in ev:
        e[0].record()
        gf.replay()
        e[1].record()
        gb.replay()
        e[2].record()
    torch.cuda.synchronize()
    f = sorted(e[0].elapsed_time(e[1]) / 2 for e in ev)
    b = sorted(e[1].elapsed_time(e[2]) / 2 for e in ev)
    pc = lambda xs, q: xs[min(len(xs) - 1, int(round(q * (len(xs) - 1))))]
    out = {"observations": n_obs, "calls_per_graph": 2,
           "fwd_ms": {"median": pc(f, 0.5), "p10": pc(f, 0.1), "p90": pc(f, 0.9)},
           "bwd_ms": {"median": pc(b, 0.5), "p10": pc(b, 0.1), "p90": pc(b, 0.9)}}
    out["step_ms_median"] = out["fwd_ms"]["median"] + out["bwd_ms"]["median"]
    del gf, gb
    return out


def measured_peaks(torch):
    """A plain device copy (1 GiB read + 1 GiB written) and a large bf16 GEMM
    (8192^3, the vendor BLAS), each the median of 10 timed runs: the practical
    ceilings beside the spec peaks."""
    dev = torch.device("cuda:0")
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    ts = []
    for i in range(13):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        if i >= 3:
            ts.append(e0.elapsed_time(e1))
    copy_gbs = 2 * src.numel() * 4 / (sorted(ts)[len(ts) // 2] * 1e-3) / 1e9
    del src, dst
    n = 8192
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    ts = []
    for i in range(13):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.matmul(a, b)
        e1.record()
        torch.cuda.synchronize()
        if i >= 3:
            ts.append(e0.elapsed_time(e1))
    gemm = 2 * n ** 3 / (sorted(ts)[len(ts) // 2] * 1e-3) / 1e12
    del a, b
    return {"copy_GBps": copy_gbs, "bf16_gemm_TFLOPs": gemm,
            "source": "device copy of 1 GiB and torch.matmul 8192^3 bf16, median of 10"}


# ---- secondary measurements ----------------------------------------------------

def _time_decode(result, args, ops, binding, torch):
    """The token-serial forward (rewy_recurrent_fwd) at a decode shape: 64
    sequences with an fp32 state each, one new token per sequence and call,
    H=32, K=V=128, bf16, vector gate.  The kernel reads and writes every state
    once per call, so it is HBM-bound on the state bytes."""
    import workloads
    Bd, H, K, V = 64, 32, 128, 128
    dev = torch.device("cuda:0")
    inp = workloads.make_inputs(Bd, 1, H, K, V, gate="vector", dtype="bf16", h0="normal", seed=11)
    x = inp.to(dev)

    def call():
        return ops.recurrent_forward(x.q, x.k, x.v, x.g, x.beta, scale=inp.scale, h0=x.h0)

    for _ in range(20):
        call()
    torch.cuda.synchronize()
    n = max(args.steps, 20)
    binding.rewy_trace_select("k_recurrent")
    binding.rewy_trace_begin()
    t0 = time.perf_counter()
    for _ in range(n):
        call()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / n
    tr = binding.rewy_trace_end()
    binding.rewy_trace_select(None)
    kern_ms = sum(t for _, t, _ in tr) / max(1, sum(c for _, _, c in tr))
    state = Bd * H * K * V * 4
    nbytes = 2 * state + Bd * H * ((2 * K + 2 * V) * 2 + K * 4 + 2)  # states in/out; q k v o, g, beta
    achieved = nbytes / (kern_ms * 1e-3) / 1e9
    result["decode"] = {
        "workload": "kda_decode_b64_h32_d128: 64 sequences, one new token each, fp32 state carried",
        "tokens_per_s": Bd / (ms * 1e-3), "ms_per_call": ms, "kernel_ms": kern_ms,
        "roofline": {"kernel": tr[0][0] if tr else "k_recurrent", "bound": "hbm",
                     "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "method_bytes_per_launch": nbytes},
    }
    print(f"[bench] decode: {ms:.3f} ms per call, kernel {kern_ms * 1e3:.1f} us, "
          f"{achieved:.0f} GB/s", file=sys.stderr, flush=True)


def _timed(fn, steps, warm, torch, binding=None):
    """ms per call of fn over `steps` calls after `warm` untimed ones; with
    binding, also the per-kernel averages from a separate traced pass."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t) * 1e3 / steps
    kern = None
    if binding is not None:
        binding.rewy_trace_begin()
        for _ in range(steps):
            fn()
        tr = binding.rewy_trace_end()
        torch.cuda.synchronize()
        kern = {kernel_label(name): {"kernel": name, "avg_ms": tot / cnt,
                                     "launches_per_step": cnt / steps}
                for name, tot, cnt in tr}
    return ms, kern


def _time_gdn2(result, x, inp, B, T, args, ops, binding, torch):
    """The erase/write form (independent erase gate b [B,T,H,K] and write gate
    w [B,T,H,V]) on the same inputs: one forward + backward step."""
    gen = torch.Generator().manual_seed(13)
    b = torch.sigmoid(torch.randn(*inp.k.shape, generator=gen)).to(inp.q.dtype).to(x.q.device)
    w = torch.sigmoid(torch.randn(*inp.v.shape, generator=gen)).to(inp.q.dtype).to(x.q.device)

    def step2():
        o, ht, ctx = ops.forward_gdn2(x.q, x.k, x.v, x.g, b, w, scale=inp.scale, h0=x.h0,
                                      cu_seqlens=inp.cu_seqlens, policy=args.policy)
        return ops.backward(ctx, x.dO, x.dht)

    ms, kern = _timed(step2, args.steps, max(3, args.warmup // 4), torch, binding)
    result["gdn2"] = {"form": "erase/write gates (b, w) in place of beta", "policy": args.policy,
                      "ms_per_step": ms, "value": B * T / (ms * 1e-3), "unit": "tokens/s",
                      "kernels_ms": kern}
    print(f"[bench] erase/write form: {ms:.3f} ms/step", file=sys.stderr, flush=True)


def _time_kda_gate(result, x, inp, B, T, args, ops, binding, torch):
    """The same step with the vector gate formed inside the kernels from its
    pre-activation (g = -exp(A_log) softplus(x + dt_bias)); x in the feature
    dtype, dx, dA_log and ddt_bias returned in place of dg."""
    if inp.gate_x is None:
        return
    dev = x.q.device
    gx = inp.gate_x.to(inp.q.dtype).to(dev)
    al, db = inp.a_log.to(dev).contiguous(), inp.dt_bias.to(dev).contiguous()

    def step3():
        o, ht, ctx = ops.forward_kda_gate(x.q, x.k, x.v, gx, al, db, x.beta, scale=inp.scale,
                                          h0=x.h0, cu_seqlens=inp.cu_seqlens, policy=args.policy)
        return ops.backward(ctx, x.dO, x.dht)

    ms, kern = _timed(step3, args.steps, max(3, args.warmup // 4), torch, binding)
    result["kda_gate_in_kernel"] = {
        "form": "g = -exp(A_log) softplus(x + dt_bias) formed in the kernels; dx, dA_log, ddt_bias out",
        "policy": args.policy, "ms_per_step": ms, "value": B * T / (ms * 1e-3), "unit": "tokens/s",
        "kernels_ms": kern}
    print(f"[bench] gate formed in the kernels: {ms:.3f} ms/step", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="kda_t8192_h32_d128")
    ap.add_argument("--policy", default="recompute", choices=["recompute", "save"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=32,
                    help="heads of the workload the oracle baseline runs")
    ap.add_argument("--min-warmup-s", type=float, default=2.0,
                    help="warm-up lasts at least this long (profiler runs pass 0)")
    ap.add_argument("--no-other-policy", action="store_true",
                    help="skip timing the other saving policy (profiler runs)")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip timing the token-serial forward at a decode shape")
    ap.add_argument("--no-kda-gate", action="store_true",
                    help="skip timing the step with the gate formed in the kernels")
    ap.add_argument("--no-gdn2", action="store_true",
                    help="skip timing the erase/write form")
    ap.add_argument("--no-schedules", action="store_true",
                    help="skip timing the separate producer-consumer schedule of the backward")
    ap.add_argument("--schedule", default="joint", choices=["joint", "separate"],
                    help="the chunk backward's schedule for the headline run (profiler runs)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the graph-replayed 60-observation protocol (profiler runs)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip measuring the copy and GEMM peaks (profiler runs)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="before the steps, copy a buffer of this many MiB once (a plain "
                         "copy kernel of known size, to calibrate HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported "
              "(heads shard across GPUs with no communication, so per-GPU throughput is the "
              "N=1 figure)", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    from chunkwise_delta_rule_chunk_amd import binding, flops, ops

    dev = torch.device("cuda:0")
    if args.schedule == "separate":
        binding.rewy_bwd_schedule(binding.REWY_SCHEDULE_SEPARATE)
    inp = workloads.workload(args.workload)  # CPU generator, then resident in HBM
    x = inp.to(dev)
    B, T, H, K, V = inp.shape
    seq_lens = ([T] * B) if inp.cu_seqlens is None else \
        [int(b - a) for a, b in zip(inp.cu_seqlens[:-1], inp.cu_seqlens[1:])]
    n_tokens = sum(seq_lens)
    step = Step(x, inp, args.policy, torch, ops, binding)
    if args.copy_mib > 0:
        src = torch.ones(args.copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    torch.cuda.synchronize()

    t_w = time.perf_counter()
    done = 0
    while done < args.warmup or time.perf_counter() - t_w < args.min_warmup_s:
        step()
        done += 1
        if done % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    print(f"[bench] warmup {done} steps", file=sys.stderr, flush=True)

    def traced(fn):
        binding.rewy_trace_begin()
        for _ in range(args.steps):
            fn()
        t = binding.rewy_trace_end()
        torch.cuda.synchronize()
        return {name: (tot / cnt, cnt / args.steps) for name, tot, cnt in t}

    # Every kernel's duration first, from an untimed pass with an event pair
    # around every launch: it names the dominant kernel (time per step).
    kern = traced(step)
    dom = max(kern, key=lambda k: kern[k][0] * kern[k][1])
    dom_stage = parse_kernel(dom)[0]

    # Timed region: K steps.  Only the dominant kernel's launches carry HIP
    # events (recorded on their launch stream), so its average duration is
    # measured over exactly the timed launches while the other kernels run
    # without event overhead.  One device event at every step boundary (on the
    # same stream) gives the distribution of single-step times as well.
    torch.cuda.synchronize()
    binding.rewy_trace_select(dom_stage)
    binding.rewy_trace_begin()
    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    bounds[0].record()
    for i in range(args.steps):
        step()
        bounds[i + 1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    tr = binding.rewy_trace_end()
    binding.rewy_trace_select(None)
    ms = elapsed * 1e3 / args.steps
    step_ms = sorted(bounds[i].elapsed_time(bounds[i + 1]) for i in range(args.steps))
    pct = lambda p: step_ms[min(len(step_ms) - 1, int(round(p * (len(step_ms) - 1))))]
    print(f"[bench] timed {args.steps} steps: {ms:.3f} ms/step", file=sys.stderr, flush=True)
    timed = {name: (tot / cnt, cnt / args.steps) for name, tot, cnt in tr}
    dom_avg, dom_per = timed[dom]

    # forward / backward split from separately traced passes
    k_fwd = traced(step.fwd)
    k_bwd = traced(step.bwd)
    fwd_ms = sum(a * p for a, p in k_fwd.values())
    bwd_ms = sum(a * p for a, p in k_bwd.values())
    f_fwd, f_bwd, f_rc = flops.workload_flops(seq_lens, H, K, V)
    tflops = (f_fwd + f_bwd) / (ms * 1e-3) / 1e12
    chunk_lens = flops.chunk_lengths(seq_lens)
    esz = 2 if inp.q.dtype == torch.bfloat16 else 4
    besz = 2 if inp.beta.dtype == torch.bfloat16 else 4
    gate = {"none": 0, "scalar": 1, "vector": 2}[inp.gate]
    nseq = len(seq_lens)
    mb = lambda role: method_bytes(role, n_tokens, H, K, V, esz, besz, gate, nseq,
                                   inp.h0 is not None, inp.dht is not None)

    def kernel_entry(name, avg, per):
        role = kernel_role(name)
        b, f = mb(role), method_flops(role, seq_lens, H, K, V, flops)
        d = design_bytes(role, chunk_lens, H, K, V, esz, besz, gate, nseq, args.policy)
        return {"kernel": name, "avg_ms": avg, "launches_per_step": per,
                "method_bytes_per_launch": b,
                "method_GBps": None if b is None else b / (avg * 1e-3) / 1e9,
                "method_TFLOPs": f / (avg * 1e-3) / 1e12,
                "design_bytes_per_launch": d,
                "design_GBps": None if d is None else d / (avg * 1e-3) / 1e9}

    dlabel = kernel_label(dom)
    drole = kernel_role(dom)
    dbytes = mb(drole)
    dflops = method_flops(drole, seq_lens, H, K, V, flops)
    ddesign = design_bytes(drole, chunk_lens, H, K, V, esz, besz, gate, nseq, args.policy)
    achieved = dbytes / (dom_avg * 1e-3) / 1e9
    traffic = measured_traffic(dlabel, args.workload, args.policy)
    # whole step: the pass floors, forward 1,538 B and backward
    # 2,820 B per token-head (+ states), over the whole step's time
    step_floor = (mb("prep_forward") + mb("fwd_scan")) + mb("bwd_chunk")
    roofline = {
        "kernel": dom, "label": dlabel, "bound": "hbm",
        "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
        "frac": achieved / PEAK_HBM_GBS,
        "traffic": traffic,
        "traffic_over_method_bytes": None if traffic is None else traffic / dbytes,
        "method_bytes_per_launch": dbytes,
        "design_bytes_per_launch": ddesign,
        "mfma": {"achieved": dflops / (dom_avg * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS,
                 "unit": "TFLOP/s", "frac": dflops / (dom_avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                 "flops_per_launch": dflops},
        "avg_ms": dom_avg, "launches_per_step": dom_per,
        "duration_source": "HIP events around this kernel's launches in the timed region",
        "step": {"method_bytes": step_floor,
                 "hbm_frac": step_floor / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                 "mfma_frac": (f_fwd + f_bwd) / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS},
    }
    result = {
        "metric": METRIC, "value": n_tokens / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": done, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if esz == 2 else "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "T": T, "H": H, "K": K, "V": V,
                   "gate": inp.gate, "policy": args.policy, "global_batch": B, "seq_len": T,
                   "parallelism": "single-gpu"},
        "tflops": tflops, "pct_bf16_peak": 100 * tflops / PEAK_BF16_TFLOPS,
        "fwd_ms": fwd_ms, "bwd_ms": bwd_ms,
        "step_ms_p10": pct(0.1), "step_ms_median": pct(0.5), "step_ms_p90": pct(0.9),
        "step_ms_source": "device events at every step boundary of the timed region",
        "bwd_tflops": f_bwd / (bwd_ms * 1e-3) / 1e12,
        "bwd_pct_bf16_peak": 100 * f_bwd / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "flops_per_step": {"forward": f_fwd, "backward": f_bwd, "recompute_executed": f_rc},
        "kernels_ms": {kernel_label(name): kernel_entry(name, a, p) for name, (a, p) in kern.items()},
        "kernels_ms_source": "untimed pass with an event pair around every launch",
        "roofline": roofline,
        "pages_context": PAGES_CONTEXT,
    }
    mem = {args.policy: {"workspace_fwd": step.ws0.numel(), "workspace_bwd": step.ws1.numel(),
                         "saved": 0 if step.saved is None else step.saved.numel()}}

    if not args.no_graph:
        gp = graph_protocol(step, torch)
        gp["policy"] = args.policy
        gp["tokens_per_s"] = n_tokens / (gp["step_ms_median"] * 1e-3)
        gp["bwd_tflops"] = f_bwd / (gp["bwd_ms"]["median"] * 1e-3) / 1e12
        result["graph_protocol"] = gp
        print(f"[bench] graph protocol: fwd {gp['fwd_ms']['median']:.3f} ms, "
              f"bwd {gp['bwd_ms']['median']:.3f} ms (median of 60)", file=sys.stderr, flush=True)

    # The other saving policy, timed the same way after the headline run: under
    # "save" the forward writes the backward's operands and the backward runs no
    # recompute ("A" in the pages' R/A pairs); under "recompute" the backward
    # re-runs the forward prep and scan ("R").
    other = None if args.no_other_policy else ("save" if args.policy == "recompute" else "recompute")
    if other is not None:
        step2 = Step(x, inp, other, torch, ops, binding)
        ms2, kern2 = _timed(step2, args.steps, max(3, args.warmup // 4), torch, binding)
        result["other_policy"] = {"policy": other, "ms_per_step": ms2,
                                  "value": n_tokens / (ms2 * 1e-3), "unit": "tokens/s",
                                  "kernels_ms": kern2}
        mem[other] = {"workspace_fwd": step2.ws0.numel(), "workspace_bwd": step2.ws1.numel(),
                      "saved": 0 if step2.saved is None else step2.saved.numel()}
        if not args.no_graph:
            gp2 = graph_protocol(step2, torch)
            result["other_policy"]["graph_protocol"] = gp2
        print(f"[bench] {other} policy: {ms2:.3f} ms/step", file=sys.stderr, flush=True)
        del step2
    result["memory_bytes"] = mem

    # The other schedule of the chunk backward (ReWY paper, "Execution and
    # numerical precision": joint or separate consumers), same policy and
    # inputs: the producer hands P, D and the write part of dbeta to the
    # consumers through the workspace.
    if not args.no_schedules and args.schedule == "joint":
        prev = binding.rewy_bwd_schedule(binding.REWY_SCHEDULE_SEPARATE)
        try:
            step3 = Step(x, inp, args.policy, torch, ops, binding)
            ms3, kern3 = _timed(step3, args.steps, max(3, args.warmup // 4), torch, binding)
            sep = {"policy": args.policy, "ms_per_step": ms3, "value": n_tokens / (ms3 * 1e-3),
                   "unit": "tokens/s", "workspace_bwd": step3.ws1.numel(), "kernels_ms": kern3}
            if not args.no_graph:
                sep["graph_protocol"] = graph_protocol(step3, torch)
            result["separate_schedule"] = sep
            del step3
        finally:
            binding.rewy_bwd_schedule(prev)
        print(f"[bench] separate schedule: {ms3:.3f} ms/step", file=sys.stderr, flush=True)
    if not args.no_decode:
        _time_decode(result, args, ops, binding, torch)
    if not args.no_gdn2:
        _time_gdn2(result, x, inp, B, T, args, ops, binding, torch)
    if not args.no_kda_gate:
        _time_kda_gate(result, x, inp, B, T, args, ops, binding, torch)
    if not args.no_peaks:
        pk = measured_peaks(torch)
        pk["dominant_kernel_frac_of_copy"] = achieved / pk["copy_GBps"]
        pk["step_mfma_frac_of_gemm"] = tflops / pk["bf16_gemm_TFLOPs"]
        result["measured_peaks"] = pk
        print(f"[bench] peaks: copy {pk['copy_GBps']:.0f} GB/s, bf16 GEMM "
              f"{pk['bf16_gemm_TFLOPs']:.0f} TFLOP/s", file=sys.stderr, flush=True)

    if not args.no_cpu_baseline:
        import oracle
        hs = list(range(min(args.cpu_heads, H)))
        sel = lambda t: None if t is None else t[:, :, hs]
        threads = oracle.default_threads()
        units = len(hs) * nseq
        cu = None if inp.cu_seqlens is None else inp.cu_seqlens.tolist()
        tc = time.perf_counter()
        oracle.forward(sel(inp.q), sel(inp.k), sel(inp.v), sel(inp.g), sel(inp.beta),
                       scale=inp.scale, h0=None if inp.h0 is None else inp.h0[:, hs],
                       cu_seqlens=cu, threads=threads)
        oracle.backward(sel(inp.q), sel(inp.k), sel(inp.v), sel(inp.g), sel(inp.beta),
                        sel(inp.dO), scale=inp.scale,
                        h0=None if inp.h0 is None else inp.h0[:, hs], cu_seqlens=cu,
                        threads=threads)
        tcpu = time.perf_counter() - tc
        frac = len(hs) / H
        try:
            aff = len(os.sched_getaffinity(0))
        except AttributeError:  # pragma: no cover
            aff = os.cpu_count()
        result["cpu_baseline"] = {
            "value": n_tokens * frac / tcpu, "unit": "tokens/s", "cores": min(threads, units),
            "kind": "oracle",
            "sample": f"FP64 token-recurrence oracle, forward+backward of heads 0..{len(hs) - 1} "
                      f"of {H} of {args.workload} ({tcpu:.1f} s); tokens/s scaled by the head "
                      f"fraction {frac:g}",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(), "affinity_cpus": aff,
            "threads": threads, "units": units,
        }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
