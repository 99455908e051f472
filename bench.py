"""Benchmark of the MI355X chunkwise gated delta rule: one step = rewy_fwd +
rewy_bwd (complete backward) on the KDA workload B=1, T=8192, H=32,
K=V=128, bf16 features, fp32 gates, synthetic seeded inputs resident in HBM.

Prints ONE JSON line: whole-job fwd+bwd tokens/s, algorithmic TFLOPS and the
fraction of the bf16 MFMA peak, a roofline entry for the dominant kernel
(per-kernel HIP-event durations from the library's trace hook, measured on the
launch stream) and the FP64 oracle timed on the host cores on a bounded sample.
"""
from __future__ import annotations

import argparse
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fwd+bwd tokens/s and MFMA TFLOPS (% bf16 peak), KDA H=32 d=128 T=8192"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def kernel_bytes(kernel: str, chunk_lens, H, K, V, esz, besz, gate, nseq, policy, prep_mode=None):
    """Algorithmic HBM bytes of one launch of `kernel` in this design: its
    compulsory reads and writes, each counted once.  Token-level rows count per
    valid token; chunk tiles count their full 64 rows per chunk-head.  The
    forward prep runs in two modes under the recompute policy (forward pass,
    and the recompute in the backward pass that also writes the reverse-scan
    and chunk-backward operands); its figure is the mean of the launches of
    one step, matching the pooled average duration (prep_mode "forward" or
    "recompute" gives one launch's figure instead)."""
    n = sum(chunk_lens)                 # valid tokens per head
    nc = len(chunk_lens)                # chunks per head
    gb = {0: 0, 1: 4, 2: 4 * K}[gate]   # gate bytes per token
    tk, tv = K * esz, V * esz           # one token row of q/k, of v
    tileK, tileV, tile64 = nc * 64 * K * esz, nc * 64 * V * esz, nc * 64 * 64 * esz
    st = nc * K * V * esz               # stored per-chunk states
    glast = nc * K * 4
    g2t = {0: 0, 1: nc * 64 * 4, 2: nc * 64 * K * 4}[gate]
    gst = nc * 4 * K * 16               # sub-chunk gate statistics, float4 per (block, feature)
    prep_in = n * (2 * tk + tv + gb + besz)
    w_fscan = n * (tk + tv) + tileK + glast              # W, U, Ft, glast
    w_fout = tileK + tile64                               # Qg, Cq
    w_bscan = n * tk + 2 * tileK + tile64                 # F, Wt, Qgt, Cqt
    w_bchunk = tile64 + g2t + gst                         # At, G2t, Gst
    if policy == "save":
        prep = prep_in + w_fscan + w_fout + w_bscan + w_bchunk
    elif prep_mode == "forward":
        prep = prep_in + w_fscan + w_fout
    elif prep_mode == "recompute":
        prep = prep_in + w_fscan + w_bscan + w_bchunk
    else:
        prep = prep_in + (w_fscan + w_fout + (w_fscan + w_bscan + w_bchunk)) / 2
    per_head = {
        "k_fwd_prep": prep,
        # forward pass: reads W, U, Ft, glast, Qg, Cq; writes o (and, saving,
        # the states and R for the backward)
        "k_fwd_scan": n * (tk + tv) + tileK + glast + tileK + tile64 + n * tv
                      + (st + tileV if policy == "save" else 0),
        "k_bwd_scan": n * (tk + tv) + 2 * tileK + tile64 + glast + st + tileV,
        # reads dO, R, v, A^T, Rbar, S, dS+, k, q, G2^T, statistics, glast, beta;
        # writes dq, dk, dv, dg, dbeta
        "k_bwd_chunk": n * 3 * tv + tile64 + tileV + 2 * st + n * 2 * tk + g2t + gst + glast
                       + n * besz + n * (2 * tk + tv + gb + besz),
    }
    # the backward's forward scan and reverse scan in one launch
    per_head["k_scans"] = n * (tk + tv) + tileK + glast + st + tileV + per_head["k_bwd_scan"]
    for name, b in per_head.items():
        if f"{len(name)}{name}I" in kernel:
            extra = 0
            if name in ("k_fwd_scan", "k_bwd_scan"):
                extra = nseq * 2 * 4 * K * V  # initial / final state (fp32) per sequence
            elif name == "k_scans":
                extra = nseq * 4 * 4 * K * V
            return b * H + extra * H
    return None


def measured_traffic(kernel: str, workload: str, policy: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE, calibrated on a plain copy), or None
    when there is no summary for this workload or the library sources changed
    since the counters were taken."""
    import re
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
        if len(cells) >= 4 and cells[0] == f"`{kernel}`":
            return float(cells[3])
    return None


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
        "roofline": {"kernel": "k_recurrent", "bound": "hbm", "achieved": achieved,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "algorithmic_bytes_per_launch": nbytes},
    }
    print(f"[bench] decode: {ms:.3f} ms per call, kernel {kern_ms * 1e3:.1f} us, "
          f"{achieved:.0f} GB/s", file=sys.stderr, flush=True)


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

    for _ in range(max(3, args.warmup // 4)):
        step2()
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for _ in range(args.steps):
        step2()
    torch.cuda.synchronize()
    ms2 = (time.perf_counter() - t2) * 1e3 / args.steps
    binding.rewy_trace_begin()  # per-kernel durations from a separate, untimed pass
    for _ in range(args.steps):
        step2()
    tr = binding.rewy_trace_end()
    torch.cuda.synchronize()
    result["gdn2"] = {"form": "erase/write gates (b, w) in place of beta", "policy": args.policy,
                      "ms_per_step": ms2, "value": B * T / (ms2 * 1e-3), "unit": "tokens/s",
                      "kernels_ms": {name: {"avg_ms": tot / cnt, "launches_per_step": cnt / args.steps}
                                     for name, tot, cnt in tr}}
    print(f"[bench] erase/write form: {ms2:.3f} ms/step", file=sys.stderr, flush=True)


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

    for _ in range(max(3, args.warmup // 4)):
        step3()
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for _ in range(args.steps):
        step3()
    torch.cuda.synchronize()
    ms3 = (time.perf_counter() - t2) * 1e3 / args.steps
    binding.rewy_trace_begin()  # per-kernel durations from a separate, untimed pass
    for _ in range(args.steps):
        step3()
    tr = binding.rewy_trace_end()
    torch.cuda.synchronize()
    result["kda_gate_in_kernel"] = {
        "form": "g = -exp(A_log) softplus(x + dt_bias) formed in the kernels; dx, dA_log, ddt_bias out",
        "policy": args.policy, "ms_per_step": ms3, "value": B * T / (ms3 * 1e-3), "unit": "tokens/s",
        "kernels_ms": {name: {"avg_ms": tot / cnt, "launches_per_step": cnt / args.steps}
                       for name, tot, cnt in tr}}
    print(f"[bench] gate formed in the kernels: {ms3:.3f} ms/step", file=sys.stderr, flush=True)


def _time_other(result, other, prob2, x, inp, B, T, args, ops, torch):
    """Time K steps under the other saving policy and record them in result."""
    w20, w21 = ops.workspace(prob2, 0), ops.workspace(prob2, 1)

    def step2():
        o, ht, ctx = ops.forward(x.q, x.k, x.v, x.g, x.beta, scale=inp.scale, h0=x.h0,
                                 cu_seqlens=inp.cu_seqlens, policy=other, ws=w20)
        return ops.backward(ctx, x.dO, x.dht, ws=w21)

    for _ in range(max(3, args.warmup // 4)):
        step2()
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for _ in range(args.steps):
        step2()
    torch.cuda.synchronize()
    ms2 = (time.perf_counter() - t2) * 1e3 / args.steps
    result["other_policy"] = {"policy": other, "ms_per_step": ms2, "value": B * T / (ms2 * 1e-3),
                              "unit": "tokens/s"}
    print(f"[bench] {other} policy: {ms2:.3f} ms/step", file=sys.stderr, flush=True)


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
    inp = workloads.workload(args.workload)  # CPU generator, then resident in HBM
    x = inp.to(dev)
    B, T, H, K, V = inp.shape
    seq_lens = ([T] * B) if inp.cu_seqlens is None else \
        [int(b - a) for a, b in zip(inp.cu_seqlens[:-1], inp.cu_seqlens[1:])]
    prob = ops.make_problem(x.q, x.v, x.g, x.beta, scale=inp.scale, cu_seqlens=inp.cu_seqlens,
                            policy=args.policy)
    ws0, ws1 = ops.workspace(prob, 0), ops.workspace(prob, 1)
    if args.copy_mib > 0:
        src = torch.ones(args.copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    torch.cuda.synchronize()

    def step():
        o, ht, ctx = ops.forward(x.q, x.k, x.v, x.g, x.beta, scale=inp.scale, h0=x.h0,
                                 cu_seqlens=inp.cu_seqlens, policy=args.policy, ws=ws0)
        return ops.backward(ctx, x.dO, x.dht, ws=ws1)

    t_w = time.perf_counter()
    done = 0
    while done < args.warmup or time.perf_counter() - t_w < args.min_warmup_s:
        step()
        done += 1
        if done % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    print(f"[bench] warmup {done} steps", file=sys.stderr, flush=True)

    # Timed region: K steps with the library's event-pair trace on, so every
    # kernel's duration comes from HIP events recorded on its launch stream
    # around exactly the launches that are timed.
    # Every kernel's duration first, from an untimed pass with an event pair
    # around every launch: it names the dominant kernel.
    def traced(fn):
        binding.rewy_trace_begin()
        for _ in range(args.steps):
            fn()
        t = binding.rewy_trace_end()
        torch.cuda.synchronize()
        return {name: (tot / cnt, cnt / args.steps) for name, tot, cnt in t}

    holder = {}

    def fwd_only():
        holder["ctx"] = ops.forward(x.q, x.k, x.v, x.g, x.beta, scale=inp.scale, h0=x.h0,
                                    cu_seqlens=inp.cu_seqlens, policy=args.policy, ws=ws0)[2]

    kern = traced(step)  # per kernel: (average ms per launch, launches per step)
    dom = max(kern, key=lambda k: kern[k][0] * kern[k][1])
    dom_stage = re.search(r"rewy(?:::|\d+)(k_\w+?)(?:I|\()", dom).group(1)

    # Timed region: K steps.  Only the dominant kernel's launches carry HIP
    # events (recorded on their launch stream), so its average duration is
    # measured over exactly the timed launches while the other kernels run
    # without event overhead.
    # One device event at every step boundary (on the stream the kernels run
    # on) gives the distribution of single-step times as well.
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
    k_fwd = traced(fwd_only)
    k_bwd = traced(lambda: ops.backward(holder["ctx"], x.dO, x.dht, ws=ws1))
    fwd_ms = sum(a * p for a, p in k_fwd.values())
    bwd_ms = sum(a * p for a, p in k_bwd.values())
    f_fwd, f_bwd, f_rc = flops.workload_flops(seq_lens, H, K, V)
    tflops = (f_fwd + f_bwd) / (ms * 1e-3) / 1e12
    chunk_lens = flops.chunk_lengths(seq_lens)
    esz = 2 if inp.q.dtype == torch.bfloat16 else 4
    besz = 2 if inp.beta.dtype == torch.bfloat16 else 4
    gate = {"none": 0, "scalar": 1, "vector": 2}[inp.gate]
    dbytes = kernel_bytes(dom, chunk_lens, H, K, V, esz, besz, gate, len(seq_lens), args.policy)
    achieved = dbytes / (dom_avg * 1e-3) / 1e9 if dbytes else None
    short = next((k for k in ("k_fwd_prep", "k_fwd_scan", "k_bwd_scan", "k_bwd_chunk", "k_scans")
                  if f"{len(k)}{k}I" in dom), dom)
    roofline = {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": None if achieved is None else achieved / PEAK_HBM_GBS,
                "traffic": measured_traffic(short, args.workload, args.policy),
                "avg_ms": dom_avg, "launches_per_step": dom_per,
                "duration_source": "HIP events around this kernel's launches in the timed region",
                "algorithmic_bytes_per_launch": dbytes}
    result = {
        "metric": METRIC, "value": B * T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
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
        "kernels_ms": {name: {"avg_ms": a, "launches_per_step": p,
                              "algorithmic_GBps": (lambda b: None if b is None else b / (a * 1e-3) / 1e9)(
                                  kernel_bytes(name, chunk_lens, H, K, V, esz, besz, gate,
                                               len(seq_lens), args.policy))}
                       for name, (a, p) in kern.items()},
        "kernels_ms_source": "untimed pass with an event pair around every launch",
        "roofline": roofline,
    }
    # The other saving policy, timed the same way after the headline run: under
    # "save" the forward writes the backward's operands and the backward runs no
    # recompute ("A" in the pages' R/A pairs); under "recompute" the backward
    # re-runs the forward prep and scan ("R").
    other = "save" if args.policy == "recompute" else "recompute"
    if args.no_other_policy:
        other = None
    prob2 = None if other is None else ops.make_problem(x.q, x.v, x.g, x.beta, scale=inp.scale,
                                                         cu_seqlens=inp.cu_seqlens, policy=other)
    if other is not None:
        _time_other(result, other, prob2, x, inp, B, T, args, ops, torch)
    if not args.no_decode:
        _time_decode(result, args, ops, binding, torch)
    if not args.no_gdn2:
        _time_gdn2(result, x, inp, B, T, args, ops, binding, torch)
    if not args.no_kda_gate:
        _time_kda_gate(result, x, inp, B, T, args, ops, binding, torch)

    if not args.no_cpu_baseline:
        import oracle
        hs = list(range(min(args.cpu_heads, H)))
        sel = lambda t: None if t is None else t[:, :, hs]
        threads = oracle.default_threads()
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
        result["cpu_baseline"] = {
            "value": B * T * frac / tcpu, "unit": "tokens/s", "cores": min(threads, len(hs) * len(seq_lens)),
            "kind": "oracle",
            "sample": f"FP64 token-recurrence oracle, forward+backward of heads 0..{len(hs) - 1} "
                      f"of {H} of {args.workload} ({tcpu:.1f} s); tokens/s scaled by the head "
                      f"fraction {frac:g}",
            "host_cpus": os.cpu_count(),
        }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
