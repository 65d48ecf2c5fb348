#!/usr/bin/env python3
"""Benchmark of the M²RNN forward recurrence on one MI355X (gfx950).

One step = one full forward pass (all T steps of the recurrence for every (batch, head)) of the
16K-token workload B=2, N=32 heads, T=16384, K=V=64 with bf16 q/k/v and fp32 state, on synthetic
seeded inputs already resident in HBM: one ``m2rnn_fwd`` call (which runs long sequences in time
segments, each segment's readout finish overlapping the next segment's scan).  After the timed
region the scan kernel runs alone over the whole sequence, each launch between two HIP events on
its stream: that gives the dominant kernel's launch duration for the roofline (``--scan-only``
runs just that loop, for counter passes and kernel traces).

Prints ONE JSON line.  ``--gpus`` above 1 is refused: the recurrence of one (batch, head) pair is
a serial chain that the library runs on a single GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "M²RNN fwd head-steps/sec + % MFMA peak at K=V=64, T=16384 (1 GPU)"
# MI355X published dense peaks (TFLOP/s).
PEAK_TFLOPS = {"f32": 157.3, "f16x3": 2500.0, "bf16x3": 2500.0, "bf16": 2500.0}
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = ["m2rnn_device.h", "m2rnn_fwd_kernel.h"]
BWD_KERNEL_SOURCES = ["m2rnn_device.h", "m2rnn_fwd_kernel.h", "m2rnn_bwd_kernel.h"]


def arithmetic(math_mode: str) -> str:
    """What the path computes in: the state and every accumulation in fp32, the per-step contraction
    in the given mode (f16x3: three fp16 MFMA passes over split operands)."""
    return f"f32 state, {math_mode} contraction"


def kernel_hash(sources=KERNEL_SOURCES) -> str:
    """Hash of a kernel's sources with comments and blank lines removed: a counter summary stays
    valid across edits of comments, and goes stale with any change of code."""
    import re
    h = hashlib.sha256()
    for name in sources:
        with open(os.path.join(ROOT, "matrix_state_nonlinear_m2rnn_amd", "csrc", name)) as fh:
            text = re.sub(r"/\*.*?\*/", "", fh.read(), flags=re.S)
        for line in text.splitlines():
            code = line.split("//", 1)[0].strip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def measured_traffic(workload: str, math_mode: str, kernel: str = "m2rnn_scan_fwd", sources=KERNEL_SOURCES):
    """HBM bytes per launch of the kernel from the committed rocprofv3 counter summary, or None
    when the summary is missing or was taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_{math_mode}_pmc.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_sources_sha256_16") != kernel_hash(sources):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo, as lscpu reports it)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(d, w, seconds: float, backward: bool = False):
    """Times the fp64 oracle (as it stands) on a bounded sample of the same workload: the first
    `threads` (batch, head) units, each over the first T_s steps, one unit per thread (forward, or
    forward + manual BPTT).  T_s is sized from a one-thread probe so that the sample takes about
    `seconds` of wall time; one unit on one thread over a few seconds gives the single-thread rate."""
    import numpy as np
    import oracle

    nthreads = oracle.default_threads()
    units = min(w.B * w.N, nthreads)
    pairs = [(u // w.N, u % w.N) for u in range(w.B * w.N)]

    def run(T, nunits, threads):
        # Units become the heads of one batch entry: q [1, T, units, K], W [units, V, V], ...
        sel = pairs[:nunits]
        # q, k shared by all heads ([B,T,1,K]) are taken per unit like the per-head ones.
        g = lambda a: np.stack([a[b, :T, n if a.shape[2] > 1 else 0] for b, n in sel], axis=1)[None]  # noqa: E731
        W = np.stack([d["W"][n] for _, n in sel])
        w_r = np.stack([d["w_r"][n] for _, n in sel])
        t0 = time.perf_counter()
        if backward:
            oracle.ref_bwd(g(d["q"]), g(d["k"]), g(d["v"]), g(d["f"]), W, w_r, None, g(d["dy"]), None,
                           nthreads=threads)
        else:
            oracle.ref_fwd(g(d["q"]), g(d["k"]), g(d["v"]), g(d["f"]), W, w_r, None, nthreads=threads)
        return time.perf_counter() - t0

    probe_T = min(w.T, 128)
    per_step = run(probe_T, 1, 1) / probe_T
    T_1 = int(max(probe_T, min(w.T, 2.0 / max(per_step, 1e-9))))
    single = T_1 / run(T_1, 1, 1)
    T_s = int(max(64, min(w.T, seconds / max(per_step, 1e-9))))
    if T_s == w.T:
        # A full-length unit per thread is shorter than the target: give each thread more units.
        reps = max(1, int(seconds / max(per_step * w.T, 1e-9)))
        units = min(w.B * w.N, nthreads * reps)
    wall = run(T_s, units, nthreads)
    what = "forward + manual BPTT" if backward else "forward"
    return {"value": units * T_s / wall, "unit": "head-steps/s", "cores": min(nthreads, units), "kind": "oracle",
            "sample": f"{units} (batch, head) units x {T_s} steps of {w.name} ({what}, fp64, units spread over "
                      "threads)",
            "wall_s": round(wall, 3), "cpu_model": cpu_model(), "host_threads": os.cpu_count(),
            "single_thread_value": single,
            "single_thread_sample": f"1 unit x {T_1} steps on one thread"}


def bench_backward(args) -> int:
    """Times m2rnn_bwd (checkpoint forward + reverse scan + sums) on the BPTT workload."""
    import numpy as np
    import torch

    import matrix_state_nonlinear_m2rnn_amd as m2
    from matrix_state_nonlinear_m2rnn_amd import inputs

    name = args.workload if args.workload != "long_b2_h32_t16384_kv64" else "bwd_b4_h16_t4096_kv64"
    w = inputs.WORKLOADS[name]
    print(f"[bench] generating {w.name} inputs", file=sys.stderr, flush=True)
    d = inputs.workload_inputs(w.name, with_dy=True)
    dev = torch.device("cuda:0")
    t = {n: torch.from_numpy(np.ascontiguousarray(a)).to(dev) for n, a in d.items() if a is not None}
    if w.qkv_dtype == "bf16":
        for n in ("q", "k", "v"):
            t[n] = t[n].to(torch.bfloat16).contiguous()
    B, T, N, K, V = w.B, w.T, w.N, w.K, w.V
    dims = m2.Dims(B, T, N, K, V, 1 if w.shared_qk else N)
    dt = m2.DTYPE_BF16 if w.qkv_dtype == "bf16" else m2.DTYPE_F32
    train = getattr(args, "train", False)
    if train:
        # One training step of the layer: the forward keeping checkpoints, then the backward from them.
        ws = torch.empty(max(m2.m2rnn_bwd_ckpt_workspace_size(dims, dt, "auto"), 1), dtype=torch.uint8, device=dev)
        fws = torch.empty(max(m2.m2rnn_fwd_workspace_size(dims, dt, "auto"), 1), dtype=torch.uint8, device=dev)
        y = torch.empty((B, T, N, V), dtype=torch.float32, device=dev)
        H_T = torch.empty((B, N, K, V), dtype=torch.float32, device=dev)
        ck = torch.empty((B, N, m2.checkpoint_count(T, V), K, V), dtype=torch.float32, device=dev)

        def step():
            m2.m2rnn_fwd_ckpt(t["q"], t["k"], t["v"], t["f"], t["W"], t["w_r"], None, y=y, H_T=H_T, ckpt=ck,
                              workspace=fws)
            return m2.m2rnn_bwd_ckpt(t["q"], t["k"], t["v"], t["f"], t["W"], t["w_r"], ck, t["dy"], None,
                                     workspace=ws)
    else:
        ws = torch.empty(max(m2.m2rnn_bwd_workspace_size(dims, dt, "auto"), 1), dtype=torch.uint8, device=dev)

        def step():
            return m2.m2rnn_bwd(t["q"], t["k"], t["v"], t["f"], t["W"], t["w_r"], None, t["dy"], None,
                                workspace=ws)

    # The reverse kernel alone (with the pass that finds each pair's scale before it): checkpoints
    # from one forward, then launches of m2rnn_scan_bwd, each between two events on its stream.
    ck_r = torch.empty((B, N, m2.checkpoint_count(T, V), K, V), dtype=torch.float32, device=dev)
    y_r = torch.empty((B, T, N, V), dtype=torch.float32, device=dev)
    m2.m2rnn_fwd_ckpt(t["q"], t["k"], t["v"], t["f"], t["W"], t["w_r"], None, y=y_r, ckpt=ck_r)
    rws = torch.empty(max(m2.m2rnn_bwd_ckpt_workspace_size(dims, dt, "auto"), 1), dtype=torch.uint8, device=dev)
    e = lambda *sh: torch.empty(sh, dtype=torch.float32, device=dev)  # noqa: E731
    Nqk = dims.Nqk
    gout = {"dq": e(B, T, Nqk, K), "dk": e(B, T, Nqk, K), "dv": e(B, T, N, V), "df": e(B, T, N), "dW": e(N, V, V),
            "dw_r": e(N, V), "dH0": None}

    def scan_bwd_loop(n):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a0, a1 in evs:
            a0.record()
            m2.m2rnn_scan_bwd(t["q"], t["k"], t["v"], t["f"], t["W"], t["w_r"], ck_r, t["dy"], None,
                              workspace=rws, out=gout)
            a1.record()
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / n

    if args.copy_calibration:
        # A fill and a plain copy of 256 MiB each: their FETCH_SIZE / WRITE_SIZE readings scale the
        # reverse kernel's.
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
    if args.scan_only:
        for _ in range(args.warmup):
            m2.m2rnn_scan_bwd(t["q"], t["k"], t["v"], t["f"], t["W"], t["w_r"], ck_r, t["dy"], None,
                              workspace=rws, out=gout)
        torch.cuda.synchronize()
        scan_ms = scan_bwd_loop(args.steps)
        ms = scan_ms
    else:
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        scan_ms = scan_bwd_loop(args.steps)
    hs = B * N * T
    # Algorithmic MFMA work of the reverse kernel per head-step: the recompute of H_{t-1} W (2 K V^2),
    # the chain's D W^T (2 K V^2) and dW's H_{t-1}^T D (2 K V^2).
    flops = 6.0 * K * V * V * hs
    achieved = flops / (scan_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS["f16x3"]
    metric = ("M²RNN training step (fwd keeping checkpoints + BPTT) head-steps/sec" if train
              else "M²RNN bwd (BPTT) head-steps/sec")
    out = {"metric": metric, "value": hs / (ms * 1e-3), "unit": "head-steps/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None,
           "dtype": "f32 state, bf16x3 checkpoint forward, f16x3 reverse scan", "data": "synthetic",
           "config": {"workload": w.name, "B": B, "T": T, "N": N, "K": K, "V": V, "qkv_dtype": w.qkv_dtype,
                      "math": {"forward": "bf16x3", "reverse": "f16x3"}, "segment": m2.BWD_CHECKPOINT,
                      "checkpoint_interval": m2.m2rnn_checkpoint_interval(dims)},
           "timed": ("m2rnn_scan_bwd alone" if args.scan_only else
                     "m2rnn_fwd_ckpt + m2rnn_bwd_ckpt" if train else "m2rnn_bwd"),
           "tokens_per_s": B * T / (ms * 1e-3),
           "scan_bwd_ms": scan_ms,
           "ns_per_recurrence_step": scan_ms * 1e6 / T,
           "roofline": {"bound": "mfma", "kernel": "m2rnn_scan_bwd_kernel (with the scale pass before it)",
                        "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
                        "traffic": measured_traffic(w.name, "f16x3", "m2rnn_scan_bwd", BWD_KERNEL_SOURCES),
                        "algorithmic_flops_per_launch": flops,
                        "frac_of_fp32_mfma_peak": achieved / PEAK_TFLOPS["f32"]}}
    tr = out["roofline"]["traffic"]
    if tr:
        out["roofline"]["hbm_GBs"] = tr / (scan_ms * 1e-3) / 1e9
    if args.cpu_baseline == "on" and not args.scan_only:
        print("[bench] cpu baseline (fp64 oracle, forward + BPTT)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(d, w, args.cpu_seconds, backward=True)
    print(json.dumps(out), flush=True)
    return 0


def bench_decode(args) -> int:
    """Times m2rnn_decode_step (one token for every (batch, head), state in HBM) on the batch-128
    decode workload.  The state is updated in place, as a serving loop would."""
    import numpy as np
    import torch

    import matrix_state_nonlinear_m2rnn_amd as m2
    from matrix_state_nonlinear_m2rnn_amd import inputs

    name = args.workload if args.workload != "long_b2_h32_t16384_kv64" else "decode_b128_h32_kv64"
    w = inputs.WORKLOADS[name]
    print(f"[bench] generating {w.name} inputs", file=sys.stderr, flush=True)
    d = inputs.workload_inputs(w.name)
    dev = torch.device("cuda:0")
    qkv_t = torch.bfloat16 if w.qkv_dtype == "bf16" else torch.float32
    B, N, K, V = w.B, w.N, w.K, w.V
    t = {n: torch.from_numpy(np.ascontiguousarray(a)).to(dev) for n, a in d.items() if a is not None}
    q, k, v = (t[n][:, 0].to(qkv_t).contiguous() for n in ("q", "k", "v"))
    f = t["f"][:, 0].contiguous()
    H = t["H0"].clone()
    y = torch.empty((B, N, V), dtype=torch.float32, device=dev)

    def step():
        m2.m2rnn_decode_step(q, k, v, f, t["W"], t["w_r"], H, H_out=H, y=y)

    # A serving loop issues decode steps from a HIP graph.  The K timed steps are captured into one
    # graph (K launches of the kernel, each updating the state in place) so that the GPU runs them
    # back to back without host launch overhead between tokens; one replay is the timed region.
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for _ in range(max(args.warmup, 1)):
            step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for _ in range(args.steps):
            step()
    torch.cuda.synchronize()
    graph.replay()  # untimed: first replay uploads the graph
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e_start.record(cur)
    graph.replay()
    e_end.record(cur)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    total_ms = e_start.elapsed_time(e_end)
    # Average kernel duration: the launches run back to back inside the replay, so the per-step
    # time is the kernel duration plus the (small) gap between consecutive kernels.
    kern_ms = total_ms / args.steps
    esz = 2 if w.qkv_dtype == "bf16" else 4
    # Algorithmic HBM bytes per launch: the state read and written once, q, k, v, f read, y
    # written, and W, w_r read once per head.
    per_unit = 2 * K * V * 4 + (2 * K + V) * esz + 4 + 4 * V
    nbytes = B * N * per_unit + N * (V * V + V) * 4
    achieved = nbytes / (kern_ms * 1e-3) / 1e9
    head_steps = B * N
    out = {"metric": f"M²RNN decode step head-steps/sec (B={B}, N={N}, K={K}, V={V}, state in HBM)",
           "value": head_steps * args.steps / (total_ms * 1e-3), "unit": "head-steps/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": total_ms / args.steps,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": arithmetic("f16x3"),
           "data": "synthetic",
           "config": {"workload": w.name, "B": B, "T": 1, "N": N, "K": K, "V": V, "qkv_dtype": w.qkv_dtype,
                      "math": "f16x3", "in_place": True, "launch": "K steps captured in one hip graph"},
           "kernel_us": kern_ms * 1e3, "wall_s": wall,
           "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": achieved / PEAK_HBM_GBS, "traffic": None, "algorithmic_bytes_per_launch": nbytes}}
    if args.cpu_baseline == "on":
        import oracle
        print("[bench] cpu baseline (fp64 oracle)", file=sys.stderr, flush=True)
        nthreads = oracle.default_threads()
        reps, t_total = 0, 0.0
        while t_total < min(args.cpu_seconds, 10.0) or reps == 0:
            t0 = time.perf_counter()
            oracle.ref_fwd(d["q"], d["k"], d["v"], d["f"], d["W"], d["w_r"], d["H0"], nthreads=nthreads)
            t_total += time.perf_counter() - t0
            reps += 1
        out["cpu_baseline"] = {"value": head_steps * reps / t_total, "unit": "head-steps/s",
                               "cores": min(nthreads, head_steps), "kind": "oracle",
                               "sample": f"{reps} whole decode steps of {w.name} (fp64, units spread over threads)",
                               "wall_s": round(t_total, 3)}
    print(json.dumps(out), flush=True)
    return 0


def bench_block(args) -> int:
    """Times the steps around the recurrence (gate, causal conv4 + SiLU on q, k, v, output gate +
    RMSNorm), forward and backward, at the shapes of the 16K-token workload; each is an HBM stream,
    reported against the HBM peak with its algorithmic bytes."""
    import numpy as np
    import torch

    import matrix_state_nonlinear_m2rnn_amd as m2
    from matrix_state_nonlinear_m2rnn_amd import inputs

    w = inputs.WORKLOADS[args.workload]
    B, T, N, K, V = w.B, w.T, w.N, w.K, w.V
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(1234)
    rn = lambda *s, sd=1.0: (torch.randn(*s, generator=g) * sd).to(dev)  # noqa: E731
    bf = torch.bfloat16
    a = rn(B, T, N, sd=2.0)
    alpha, beta = rn(N).abs() + 0.5, rn(N)
    dfv = rn(B, T, N)
    C = N * K
    x = rn(B, T, C).to(bf)
    cw, cb = rn(C, 4, sd=0.5), rn(C, sd=0.2)
    du = rn(B, T, C)
    y = rn(B, T, N, V)
    gz = rn(B, T, N, V, sd=2.0).to(bf)
    gamma = rn(N, V, sd=0.1) + 1.0
    dout = rn(B, T, N, V)
    f32, b16 = 4, 2
    ops = {
        "gate_fwd": (lambda: m2.m2rnn_gate_fwd(a, alpha, beta), B * T * N * (f32 + f32)),
        "gate_bwd": (lambda: m2.m2rnn_gate_bwd(a, alpha, beta, dfv), B * T * N * (3 * f32 + 2 * f32 + 2 * f32)),
        "conv4_silu_fwd": (lambda: m2.m2rnn_conv4_silu_fwd(x, cw, cb), B * T * C * (b16 + b16)),
        "conv4_silu_bwd": (lambda: m2.m2rnn_conv4_silu_bwd(x, cw, cb, du), B * T * C * (b16 + f32 + f32)),
        "out_norm_fwd": (lambda: m2.m2rnn_out_norm_fwd(y, gz, gamma), B * T * N * V * (f32 + b16 + f32)),
        "out_norm_bwd": (lambda: m2.m2rnn_out_norm_bwd(y, gz, gamma, dout),
                         B * T * N * V * (f32 + b16 + f32 + 2 * f32)),
    }
    res = {}
    for name, (fn, nbytes) in ops.items():
        for _ in range(max(args.warmup, 1)):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        res[name] = {"us": ms * 1e3, "GB_s": nbytes / (ms * 1e-3) / 1e9, "algorithmic_bytes": nbytes}
    dom = max(res, key=lambda k: res[k]["us"])
    total_ms = sum(r["us"] for r in res.values()) * 1e-3
    out = {"metric": "M²RNN block ops (gate, conv4+SiLU, output gate+RMSNorm; fwd+bwd) token-steps/sec",
           "value": B * T / (total_ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": total_ms, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": w.name, "B": B, "T": T, "N": N, "K": K, "V": V, "conv_channels": C,
                      "activations": "bf16 in, fp32 gradients"},
           "ops": res,
           "roofline": {"bound": "hbm", "kernel": dom, "achieved": res[dom]["GB_s"], "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": res[dom]["GB_s"] / PEAK_HBM_GBS, "traffic": None}}
    print(json.dumps(out), flush=True)
    return 0


def bench_fused_block(args) -> int:
    """Times the block forward from the gate pre-activation to the normalised output: the fused
    entry point (m2rnn_fwd_block: gate pass, scan, one epilogue pass per token) next to the three
    separate calls it replaces (m2rnn_gate_fwd, m2rnn_fwd, m2rnn_out_norm_fwd)."""
    import numpy as np
    import torch

    import matrix_state_nonlinear_m2rnn_amd as m2
    from matrix_state_nonlinear_m2rnn_amd import inputs

    w = inputs.WORKLOADS[args.workload]
    math_mode = "bf16x3" if args.math == "auto" else args.math
    d = inputs.workload_inputs(w.name)
    dev = torch.device("cuda:0")
    qkv_t = torch.bfloat16 if w.qkv_dtype == "bf16" else torch.float32
    t = {n: torch.from_numpy(np.ascontiguousarray(a)).to(dev) for n, a in d.items() if a is not None}
    for n in ("q", "k", "v"):
        t[n] = t[n].to(qkv_t).contiguous()
    B, T, N, K, V = w.B, w.T, w.N, w.K, w.V
    g = torch.Generator(device="cpu").manual_seed(4321)
    a = (torch.randn(B, T, N, generator=g) * 2.0).to(dev)
    alpha, beta = (torch.rand(N, generator=g) * 2.0 + 0.5).to(dev), torch.randn(N, generator=g).to(dev)
    gz = (torch.randn(B, T, N, V, generator=g) * 2.0).to(torch.bfloat16).to(dev)
    gamma = (torch.randn(N, V, generator=g) * 0.1 + 1.0).to(dev)
    out = torch.empty((B, T, N, V), dtype=torch.float32, device=dev)
    H_T = torch.empty((B, N, K, V), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, _fwd_block_ws(m2, w, math_mode, args.row_blocks)), dtype=torch.uint8, device=dev)

    def fused():
        m2.m2rnn_fwd_block(t["q"], t["k"], t["v"], a, alpha, beta, t["W"], t["w_r"], gz, gamma, None,
                           math=math_mode, row_blocks=args.row_blocks, out=out, H_T=H_T, workspace=ws)

    def unfused():
        f = m2.m2rnn_gate_fwd(a, alpha, beta)
        y, _ = m2.m2rnn_fwd(t["q"], t["k"], t["v"], f, t["W"], t["w_r"], None, math=math_mode,
                            row_blocks=args.row_blocks, H_T=H_T)
        m2.m2rnn_out_norm_fwd(y, gz, gamma, out=out)

    res = {}
    for name, fn in (("fused", fused), ("unfused", unfused)):
        for _ in range(max(args.warmup, 1)):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / args.steps
    ms = res["fused"]
    line = {"metric": "M²RNN block forward (gate, recurrence, output gate + RMSNorm) head-steps/sec",
            "value": B * T * N / (ms * 1e-3), "unit": "head-steps/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": arithmetic(math_mode), "data": "synthetic",
            "config": {"workload": w.name, "B": B, "T": T, "N": N, "K": K, "V": V, "qkv_dtype": w.qkv_dtype,
                       "gz_dtype": "bf16", "math": math_mode, "entry": "m2rnn_fwd_block"},
            "unfused_ms": res["unfused"], "saved_ms": res["unfused"] - ms}
    print(json.dumps(line), flush=True)
    return 0


def bench_layer(args) -> int:
    """Times one training step of the whole M²RNN layer around the recurrence: causal conv4 + SiLU
    on q, k, v, the gate, the recurrence keeping checkpoints, the output gate + RMSNorm, then the
    backward of each (RMSNorm, recurrence from the checkpoints, gate, the three convs), on the BPTT
    workload's shapes with fp32 activations and random-init parameters."""
    import numpy as np
    import torch

    import matrix_state_nonlinear_m2rnn_amd as m2
    from matrix_state_nonlinear_m2rnn_amd import inputs

    name = args.workload if args.workload != "long_b2_h32_t16384_kv64" else "bwd_b4_h16_t4096_kv64"
    w = inputs.WORKLOADS[name]
    B, T, N, K, V = w.B, w.T, w.N, w.K, w.V
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(2468)
    rn = lambda *s, sd=1.0: (torch.randn(*s, generator=g) * sd).to(dev)  # noqa: E731
    x = {c: rn(B, T, N * (V if c == "v" else K), sd=0.7) for c in "qkv"}
    cw = {c: rn(x[c].shape[-1], 4, sd=0.5) for c in "qkv"}
    cb = {c: rn(x[c].shape[-1], sd=0.1) for c in "qkv"}
    a, alpha, beta = rn(B, T, N, sd=2.0), rn(N).abs() + 0.5, rn(N)
    W = torch.stack([torch.linalg.qr(torch.randn(V, V, generator=g))[0] for _ in range(N)]).mul(0.9).to(dev)
    w_r, gz, gamma = rn(N, V, sd=0.3), rn(B, T, N, V, sd=2.0), rn(N, V, sd=0.1) + 1.0
    dout = rn(B, T, N, V)

    def step():
        u = {c: m2.m2rnn_conv4_silu_fwd(x[c], cw[c], cb[c]).view(B, T, N, -1) for c in "qkv"}
        f = m2.m2rnn_gate_fwd(a, alpha, beta)
        y, _, ck = m2.m2rnn_fwd_ckpt(u["q"], u["k"], u["v"], f, W, w_r)
        m2.m2rnn_out_norm_fwd(y, gz, gamma)
        gn = m2.m2rnn_out_norm_bwd(y, gz, gamma, dout)
        gs = m2.m2rnn_bwd_ckpt(u["q"], u["k"], u["v"], f, W, w_r, ck, gn["dy"], want_dH0=False)
        m2.m2rnn_gate_bwd(a, alpha, beta, gs["df"])
        for c, du in (("q", gs["dq"]), ("k", gs["dk"]), ("v", gs["dv"])):
            m2.m2rnn_conv4_silu_bwd(x[c], cw[c], cb[c], du.view(B, T, -1))

    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    line = {"metric": "M²RNN layer training step (conv4+SiLU on q,k,v, gate, recurrence, output gate + RMSNorm; "
                      "fwd + bwd) tokens/sec",
            "value": B * T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f32 state, bf16x3 forward, f16x3 reverse scan", "data": "synthetic",
            "config": {"workload": w.name, "B": B, "T": T, "N": N, "K": K, "V": V, "activations": "fp32",
                       "math": {"forward": "bf16x3", "reverse": "f16x3"}, "params": "random init"}}
    print(json.dumps(line), flush=True)
    return 0


def _fwd_block_ws(m2, w, math_mode, row_blocks) -> int:
    import ctypes
    n = ctypes.c_size_t(0)
    dims = m2.Dims(w.B, w.T, w.N, w.K, w.V, 1 if w.shared_qk else w.N)
    dt = m2.DTYPE_BF16 if w.qkv_dtype == "bf16" else m2.DTYPE_F32
    st = m2.lib().m2rnn_fwd_block_workspace_size(ctypes.byref(dims), dt, m2.MATH[math_mode], int(row_blocks),
                                                 ctypes.byref(n))
    if st != m2.M2RNN_OK:
        raise RuntimeError(f"m2rnn_fwd_block_workspace_size: {m2.status_string(st)}")
    return int(n.value)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="long_b2_h32_t16384_kv64")
    ap.add_argument("--math", default="auto", choices=["auto", "f32", "f16x3", "bf16x3", "bf16"])
    ap.add_argument("--row-blocks", type=int, default=0)
    ap.add_argument("--cpu-baseline", default="on", choices=["on", "off"])
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--backward", action="store_true",
                    help="time m2rnn_bwd on the BPTT workload instead of the forward (its own JSON line)")
    ap.add_argument("--train", action="store_true",
                    help="time one training step of the layer (m2rnn_fwd_ckpt + m2rnn_bwd_ckpt) on the BPTT workload")
    ap.add_argument("--block", action="store_true",
                    help="time the gate, conv4 + SiLU and output gate + RMSNorm (fwd and bwd) at the workload's shapes")
    ap.add_argument("--fused-block", action="store_true",
                    help="time m2rnn_fwd_block (gate, scan, fused output gate + RMSNorm) against the separate calls")
    ap.add_argument("--layer", action="store_true",
                    help="time one training step of the whole layer (convs, gate, recurrence, norm; fwd + bwd)")
    ap.add_argument("--decode", action="store_true",
                    help="time m2rnn_decode_step on the batch-128 decode workload (its own JSON line)")
    ap.add_argument("--scan-only", action="store_true",
                    help="time the forward scan kernel alone over the whole sequence (with --backward: the reverse "
                         "scan alone), for counters and traces")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain device copy of known size (for HBM counter scaling)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}): the recurrence of a "
              "(batch, head) pair is a serial chain and the library has no multi-GPU path.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import matrix_state_nonlinear_m2rnn_amd as m2
    from matrix_state_nonlinear_m2rnn_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.backward or args.train:
        return bench_backward(args)
    if args.decode:
        return bench_decode(args)
    if args.block:
        return bench_block(args)
    if args.fused_block:
        return bench_fused_block(args)
    if args.layer:
        return bench_layer(args)
    w = inputs.WORKLOADS[args.workload]
    math_mode = "bf16x3" if args.math == "auto" else args.math
    print(f"[bench] generating {w.name} inputs", file=sys.stderr, flush=True)
    d = inputs.workload_inputs(w.name)
    dev = torch.device("cuda:0")
    qkv_t = torch.bfloat16 if w.qkv_dtype == "bf16" else torch.float32
    t = {n: torch.from_numpy(np.ascontiguousarray(a)).to(dev) for n, a in d.items() if a is not None}
    for n in ("q", "k", "v"):
        t[n] = t[n].to(qkv_t).contiguous()
    B, T, N, K, V = w.B, w.T, w.N, w.K, w.V
    y = torch.empty((B, T, N, V), dtype=torch.float32, device=dev)
    H_T = torch.empty((B, N, K, V), dtype=torch.float32, device=dev)
    dims = m2.Dims(B, T, N, K, V, 1 if w.shared_qk else N)
    dt = m2.DTYPE_BF16 if w.qkv_dtype == "bf16" else m2.DTYPE_F32
    nbytes = m2.m2rnn_fwd_workspace_size(dims, dt, math_mode, args.row_blocks)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    common = dict(math=math_mode, row_blocks=args.row_blocks, y=y, H_T=H_T, workspace=ws)
    fwd_in = (t["q"], t["k"], t["v"], t["f"], t["W"], t["w_r"], None)

    def scan_loop(n):
        """n launches of the scan alone over the whole sequence, each between two events on the
        stream it runs on: the dominant kernel's launch duration for the roofline."""
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for e0, e1 in evs:
            e0.record()
            m2.m2rnn_scan_fwd(*fwd_in, **common)
            e1.record()
        torch.cuda.synchronize()
        ms = [a.elapsed_time(b) for a, b in evs]
        return sum(ms) / len(ms)

    if args.scan_only:
        # The scan kernel alone (the counter passes and the roofline's kernel trace run this).
        for _ in range(args.warmup):
            m2.m2rnn_scan_fwd(*fwd_in, **common)
        torch.cuda.synchronize()
        total_ms = None
        scan_avg = scan_loop(args.steps)
        wall = None
    else:
        # One step is m2rnn_fwd, the forward a caller runs (for long sequences: time segments whose
        # finish passes overlap the next segment's scan).
        print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
        for _ in range(args.warmup):
            m2.m2rnn_fwd(*fwd_in, **common)
        torch.cuda.synchronize()
        e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
        w0 = time.perf_counter()
        e_start.record()
        for _ in range(args.steps):
            m2.m2rnn_fwd(*fwd_in, **common)
        e_end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        total_ms = e_start.elapsed_time(e_end)
        # After the timed region: the scan kernel alone over the whole sequence, for the roofline.
        scan_avg = scan_loop(args.steps)
    if total_ms is None:
        total_ms = scan_avg * args.steps
    head_steps = B * N * T
    value = head_steps * args.steps / (total_ms * 1e-3)
    flops = 2.0 * K * V * V * head_steps
    achieved = flops / (scan_avg * 1e-3) / 1e12
    peak = PEAK_TFLOPS[math_mode]
    traffic = measured_traffic(w.name, math_mode)
    esz = 2 if w.qkv_dtype == "bf16" else 4
    # Algorithmic HBM bytes per head-step: q, k, v, f read and y written once.
    alg_bytes = head_steps * ((2 * K + V) * esz + 4 + 4 * V)

    if args.copy_calibration:
        # A plain copy of known size: its FETCH_SIZE / WRITE_SIZE readings scale the scan's.
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    out = {
        "metric": METRIC if w.name == "long_b2_h32_t16384_kv64" else f"M²RNN fwd head-steps/sec ({w.name}, 1 GPU)",
        "value": value,
        "unit": "head-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": total_ms / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": arithmetic(math_mode),
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "T": T, "N": N, "K": K, "V": V, "qkv_dtype": w.qkv_dtype,
                   "math": math_mode, "row_blocks": args.row_blocks or "auto"},
        "tokens_per_s": B * T * args.steps / (total_ms * 1e-3),
        "ns_per_recurrence_step": scan_avg * 1e6 / T,
        "scan_ms": scan_avg,
        "timed": "m2rnn_scan_fwd alone (whole sequence)" if args.scan_only else "m2rnn_fwd",
        "wall_s": wall,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": traffic,
                     "algorithmic_flops_per_launch": flops,
                     "frac_of_fp32_mfma_peak": achieved / PEAK_TFLOPS["f32"],
                     "algorithmic_hbm_bytes_per_launch": alg_bytes,
                     "algorithmic_hbm_GBs": alg_bytes / (scan_avg * 1e-3) / 1e9,
                     "hbm_GBs": traffic / (scan_avg * 1e-3) / 1e9 if traffic else None},
    }
    if args.cpu_baseline == "on":
        print("[bench] cpu baseline (fp64 oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(d, w, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
