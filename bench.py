#!/usr/bin/env python3
"""Benchmark of the gated delta rule hot path on one MI355X.

A step is one chunkwise forward pass (gate scan, gated Gram, UT transform, chunk operators,
state propagation and output: gdn_chunk_prepare + gdn_chunk_propagate, exactly the launches
gdn_chunk_fwd makes) over the training-shape workload B4 H16 T2048 d_k=d_v=128, bf16
q/k/v/o, fp32 gates and state, chunk 64: the headline line. Inputs are resident in HBM before
timing and rotate over 4 independent sets (~540 MB) so that no step is served from the 256 MB
Infinity Cache. The same run times every other workload the same way and reports each under
"workloads": the tiny fp32 forward, the long-context forward (B1 H16 T32768, h0 != 0), the
packed variable-length forward (8 sequences, H32) and the decode step (256 sequences x H32,
d128, fp32 state, bf16 o, 64 chained steps), each with per-call percentiles, algorithmic
TFLOP/s and HBM rate against the chip's peaks, and the CPU oracle on a bounded sample.

Prints one JSON line (rank 0, one GPU).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GDN chunk-fwd tokens/s + %MFMA peak (B4 H16 T2048 d128); decode %HBM BW"
PEAK_BF16_FLOPS = 2516.6e12   # 256 CU x 2.4 GHz x 4096 dense bf16/fp16 FLOP/clk/CU (MI355X, ~2.5 PF)
PEAK_F32_FLOPS = 157.3e12     # dense fp32 matrix core
PEAK_HBM_BPS = 8.0e12         # MI355X HBM3E
CHUNK = 64


def fwd_counts(dk, dv, C=CHUNK, elem=2):
    """Algorithmic counts per token-head of the chunkwise forward: FLOP of the method's
    eight chunk matmuls at full tile size, and the bytes it must move (q, k, v, o, g, beta).
    The bytes split by kernel: stage 2 moves q, k, v, o; stage 1 moves g, beta."""
    flops = 6 * dk * dv + 2 * C * (3 * dk + 2 * dv)
    stage2_bytes = (2 * dk + dv) * elem + dv * elem
    stage1_bytes = 8
    # FLOP actually issued per token-head by each stage of this implementation
    stage1_flops = 2 * C * dk * 2                      # K K^T, Q K^T (plus the small 64x64 solve)
    stage2_flops = 6 * dk * dv + 4 * C * dv            # K S^T, Q S^T, Delta^T K, Mmat R, P Delta
    return dict(flops=flops, bytes=stage1_bytes + stage2_bytes, stage1_bytes=stage1_bytes,
                stage2_bytes=stage2_bytes, stage1_flops=stage1_flops, stage2_flops=stage2_flops)


def bwd_counts(dk, dv, C=CHUNK):
    """Algorithmic FLOP per token-head of the two backward kernels of this implementation
    (the second fp16 MFMA of operands carried as hi + lo pairs is not counted): the reverse walk (K dS'^T, P^T dO, Mmat^T dDelta, the two rank-C state-gradient
    updates) and the per-chunk gradients (K S^T, Q S^T, K dS'^T, Mmat R, P^T dO, Mmat^T dDelta,
    dO Delta^T, dDelta R^T, E dO S, E dR S, Ed Delta dS', dT T^T, T^T X, K K^T, dPg K,
    dPg^T Q, dG K, dG^T K)."""
    state = 2 * (3 * dk * dv + 2 * C * dv)
    grad = 2 * (6 * dk * dv + 5 * C * dv + 2 * C * C + 5 * C * dk)
    return dict(state_flops=state, grad_flops=grad)


def bwd_bytes(dk, dv, elem=2):
    """Algorithmic HBM bytes per token-head of one backward call: q, k, v, dO read and dq, dk, dv
    written (elem bytes each), g and beta read and dg, dbeta written (fp32)."""
    return (2 * dk + 2 * dv) * elem + (2 * dk + dv) * elem + 16


def kda_bytes(dk, dv, elem=2):
    """Algorithmic HBM bytes per token-head of one channel-wise-decay forward call: q, k, v read
    and o written (elem bytes each), the per-channel g (fp32, d_k) and beta read."""
    return (2 * dk + 2 * dv) * elem + 4 * dk + 4


def decode_bytes(dk, dv, elem=2, o_elem=4):
    """Bytes one decode step moves per (sequence, head): the fp32 state read and written,
    plus q, k, v (elem bytes), o (o_elem bytes) and the two gates."""
    return 2 * dk * dv * 4 + (2 * dk + dv) * elem + dv * o_elem + 8


def measured_traffic(kernel, instance=None):
    """HBM bytes per launch (read + write) that rocprofv3 counters measured for `kernel` on
    the benchmark workload (profiles/traffic.json), or None when the kernel's sources have
    changed since the counters were taken (or, with `instance`, when the record is of another
    template instance than the one whose name contains it)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    recs = json.load(open(path))
    rec = recs.get(kernel)
    if instance is not None and (not rec or instance not in rec["kernel"]):
        # another instance of the family measured on the same workload (key kernel<...>@workload)
        fam, _, wl = kernel.partition("@")
        rec = next((r for r in recs.values() if r["kernel"].startswith(fam + "<") and r.get("workload") == wl
                    and instance in r["kernel"]), None)
    if not rec:
        return None
    csrc = os.path.join(ROOT, "gated_delta_rule_42_amd", "csrc")
    h = hashlib.sha256(b"".join(open(os.path.join(csrc, f), "rb").read() for f in rec["sources"])).hexdigest()
    return rec["read_bytes"] + rec["write_bytes"] if h == rec["source_sha256"] else None


def call_traffic(launches):
    """Measured HBM bytes of one call that makes the given launches ((traffic.json key, instance
    name fragment or None) each once), or None unless every launch has a current record."""
    total = 0.0
    for key, inst in launches:
        t = measured_traffic(key, inst)
        if t is None:
            return None
        total += t
    return total


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=64)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall-clock budget of the CPU oracle baseline (0 disables it)")
    ap.add_argument("--only", choices=["all", "fwd", "decode", "bwd", "kda"], default="all")
    ap.add_argument("--bwd-steps", type=int, default=10)
    ap.add_argument("--fwd-workloads", default="all",
                    help="comma-separated forward workloads to time (train_1p3b, the headline; "
                         "tiny_fp32, long_ctx, varlen_packed), or 'all'; profiling runs name one")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="also run plain device copies of this many MiB (counter calibration)")
    return ap.parse_args()


def median(xs):
    xs = sorted(xs)
    return xs[len(xs) // 2] if xs else float("nan")


# One timed step in EVENT_EVERY carries the HIP events that give the per-kernel durations:
# each event marker on the stream adds a few microseconds of dispatch gap before the next
# kernel, so events on every step would inflate the wall-clock throughput they sit in.
EVENT_EVERY = 5


def event_steps(n, per, torch):
    """Events for the instrumented steps among n timed steps: {step: [per events]}."""
    return {i: [torch.cuda.Event(enable_timing=True) for _ in range(per)] for i in range(n) if i % EVENT_EVERY == 0}


def pcts(xs):
    """p10, median and p90 of a list of samples (nearest rank)."""
    xs = sorted(xs)
    if not xs:
        return {"p10": None, "median": None, "p90": None}
    q = lambda f: xs[min(len(xs) - 1, int(round(f * (len(xs) - 1))))]  # noqa: E731
    return {"p10": q(0.1), "median": q(0.5), "p90": q(0.9)}


def fwd_path(N, H, dk, dv, dtype):
    """The path gdn_chunk_fwd takes for a shape, by the library's own rule: the one-kernel
    forward for bf16 inputs with d_k = d_v = 128 and fewer than 64 (sequence, head) pairs, the
    two stages (gdn_chunk_prepare, gdn_chunk_propagate) otherwise; GDN_FUSED=0/1 forces it."""
    if dtype != "bf16" or dk != 128 or dv != 128:
        return "staged"
    env = os.environ.get("GDN_FUSED")
    if env is not None:
        return "fused" if int(env) != 0 else "staged"
    return "fused" if N * H < 64 else "staged"


def bench_forward(wid, steps, warmup, nsets, torch, gb, SY):
    """gdn_chunk_fwd on forward workload `wid` (o in the input dtype), nsets rotating input sets:
    `steps` back-to-back calls timed by the wall clock, then as many calls (at least 10) each
    bracketed by HIP events on the launch stream. When the call runs the two stages, they are
    also timed as gdn_chunk_prepare + gdn_chunk_propagate (checked equal to the call first)."""
    w = SY.WORKLOADS[wid]
    dev = torch.device("cuda:0")
    sets = []
    for s in range(nsets):
        x = SY.make_forward_inputs(wid, seed=w.id + 100 * s)
        t = {n: (None if x[n] is None else x[n].to(dev)) for n in ("q", "k", "v", "g", "beta", "h0", "cu_seqlens")}
        B, T, H, dk = t["q"].shape
        dv = t["v"].shape[-1]
        N = B if t["cu_seqlens"] is None else t["cu_seqlens"].numel() - 1
        t["o"] = torch.empty((B, T, H, dv), dtype=t["q"].dtype, device=dev)
        t["hT"] = torch.empty((N, H, dv, dk), dtype=torch.float32, device=dev)
        sets.append(t)
    cu0 = sets[0]["cu_seqlens"]
    need = gb.gdn_chunk_fwd_workspace_bytes(B, T, H, dk, dv, N, cu0 is not None, dtype=sets[0]["q"].dtype)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    path = fwd_path(N, H, dk, dv, w.dtype)

    def call(t):
        gb.gdn_chunk_fwd(*(t[n] for n in ("q", "k", "v", "g", "beta", "h0", "cu_seqlens")), o=t["o"], hT=t["hT"],
                         workspace=ws)

    def stages(t, ev):
        ev[0].record()
        gb.gdn_chunk_prepare(t["q"], t["k"], t["g"], t["beta"], ws, t["cu_seqlens"], dv=dv)
        ev[1].record()
        gb.gdn_chunk_propagate(t["q"], t["k"], t["v"], ws, t["h0"], t["cu_seqlens"], o=t["o"], hT=t["hT"])
        ev[2].record()

    for i in range(warmup):
        call(sets[i % nsets])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        call(sets[i % nsets])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    n_ev = max(10, steps)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_ev)]
    for i, e in enumerate(evs):
        e[0].record()
        call(sets[i % nsets])
        e[1].record()
    torch.cuda.synchronize()
    out = dict(wid=wid, name=w.name, B=B, T=T, H=H, dk=dk, dv=dv, N=N, dtype=w.dtype, path=path,
               h0=sets[0]["h0"] is not None, tokens=B * T, ms=wall / steps * 1e3, steps=steps,
               call_ms=[e[0].elapsed_time(e[1]) for e in evs], prep_ms=None, prop_ms=None)
    if path == "staged":
        # the two stage calls are exactly gdn_chunk_fwd on this path
        t = sets[0]
        call(t)
        o_ref, h_ref = t["o"].clone(), t["hT"].clone()
        stages(t, [torch.cuda.Event() for _ in range(3)])
        torch.cuda.synchronize()
        assert torch.equal(o_ref, t["o"]) and torch.equal(h_ref, t["hT"])
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_ev)]
        for i, e in enumerate(evs):
            stages(sets[i % nsets], e)
        torch.cuda.synchronize()
        out["prep_ms"] = [e[0].elapsed_time(e[1]) for e in evs]
        out["prop_ms"] = [e[1].elapsed_time(e[2]) for e in evs]
    return out


def forward_report(f):
    """Throughput, algorithmic rates against the chip's peaks and the per-call distribution of
    one forward workload."""
    elem = 4 if f["dtype"] == "f32" else 2
    c = fwd_counts(f["dk"], f["dv"], elem=elem)
    th = f["tokens"] * f["H"]
    state_bytes = f["N"] * f["H"] * f["dk"] * f["dv"] * 4 * (2 if f["h0"] else 1)   # h0 read, hT written
    flops, byts = c["flops"] * th, c["bytes"] * th + state_bytes
    peak = PEAK_F32_FLOPS if f["dtype"] == "f32" else PEAK_BF16_FLOPS
    sec = f["ms"] / 1e3
    # the whole call against its nearer roof: algorithmic bytes at peak HBM vs FLOP at peak MFMA
    hbm_bound = byts / PEAK_HBM_BPS >= flops / peak
    return {"workload": f"{f['name']}: B{f['B']} T{f['T']} H{f['H']} d_k={f['dk']} d_v={f['dv']} N={f['N']} "
                        f"{f['dtype']} q/k/v/o, fp32 gates and state" + (", h0 != 0" if f["h0"] else ""),
            "tokens": f["tokens"], "ms_per_call": f["ms"], "calls_timed": f["steps"],
            "ms_per_call_events": pcts(f["call_ms"]),
            "tokens_per_s": f["tokens"] / sec, "tflops": flops / sec / 1e12,
            "mfma_frac": flops / sec / peak, "mfma_peak_tflops": peak / 1e12,
            "hbm_GBps_algorithmic": byts / sec / 1e9, "hbm_frac": byts / sec / PEAK_HBM_BPS,
            "algorithmic_flops_per_call": flops, "algorithmic_bytes_per_call": byts,
            "path": ("two stages (gdn_chunk_prepare, gdn_chunk_propagate)" if f["path"] == "staged"
                     else "one kernel (chunk_fused_kernel)"),
            "stages_ms_median": ({"chunk_prepare": pcts(f["prep_ms"])["median"],
                                  "chunk_propagate": pcts(f["prop_ms"])["median"]} if f["prep_ms"] else None),
            "call_roofline": {"bound": "hbm" if hbm_bound else "mfma",
                              "achieved": byts / sec / 1e9 if hbm_bound else flops / sec / 1e12,
                              "peak": PEAK_HBM_BPS / 1e9 if hbm_bound else peak / 1e12,
                              "unit": "GB/s" if hbm_bound else "TFLOP/s",
                              "frac": byts / sec / PEAK_HBM_BPS if hbm_bound else flops / sec / peak}}


def bench_backward(args, torch, gb, SY):
    """gdn_chunk_bwd on the training-shape workload (bf16 q/k/v/dO and gradients, no initial
    or final state), two rotating input sets."""
    w = SY.WORKLOADS[1]
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
    dev = torch.device("cuda:0")
    sets = []
    for s in range(2):
        x = SY.make_forward_inputs(1, seed=1 + 100 * s)
        t = {n: x[n].to(dev) for n in ("q", "k", "v", "g", "beta")}
        t["do"] = SY.make_cotangents(x, 7 + s, dhT=False)["do"].to(dev)
        sets.append(t)
    need = gb.gdn_chunk_bwd_workspace_bytes(B, T, H, dk, dv, B, False)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)

    def step(t):
        return gb.gdn_chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["do"], need_dh0=False,
                                workspace=ws)

    for i in range(2):
        step(sets[i % 2])
    evs = event_steps(args.bwd_steps, 2, torch)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.bwd_steps):
        if i in evs:
            evs[i][0].record()
        step(sets[i % 2])
        if i in evs:
            evs[i][1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return dict(B=B, T=T, H=H, dk=dk, dv=dv, wall_s=t1 - t0,
                step_ms=[e[0].elapsed_time(e[1]) for e in evs.values()])


def bench_kda(args, torch, gb, SY):
    """gdn_kda_chunk_fwd on the training-shape workload with one decay per key channel (bf16
    q/k/v/o, fp32 gates and state), two rotating input sets; then 16 chained
    gdn_kda_decode_step calls on the decode workload with per-channel gates."""
    w = SY.WORKLOADS[1]
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
    dev = torch.device("cuda:0")
    sets = []
    for s in range(2):
        x = SY.channel_gates(SY.make_forward_inputs(1, seed=1 + 100 * s), 55 + s)
        t = {n: x[n].to(dev) for n in ("q", "k", "v", "g", "beta")}
        t["o"] = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
        t["hT"] = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
        sets.append(t)
    need = gb.gdn_kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, B, False)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)

    def step(t):
        gb.gdn_kda_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], o=t["o"], hT=t["hT"], workspace=ws)

    for i in range(2):
        step(sets[i % 2])
    n = max(args.bwd_steps, 5)
    evs = event_steps(n, 2, torch)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        if i in evs:
            evs[i][0].record()
        step(sets[i % 2])
        if i in evs:
            evs[i][1].record()
    torch.cuda.synchronize()
    fwd_ms = (time.perf_counter() - t0) / n * 1e3

    wd = SY.WORKLOADS[4]
    steps = 16
    d = SY.channel_gates(SY.make_decode_inputs(4, steps=steps), 57)
    toks = [{n_: d[n_][s].to(dev) for n_ in ("q", "k", "v", "g", "beta")} for s in range(steps)]
    state = d["state"].to(dev)
    o = torch.empty((wd.decode_seqs, wd.H, wd.dv), dtype=torch.float32, device=dev)
    gb.gdn_kda_decode_step(*(toks[0][n_] for n_ in ("q", "k", "v", "g", "beta")), state.clone(), o)
    devs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    for s in range(steps):
        devs[s][0].record()
        gb.gdn_kda_decode_step(*(toks[s][n_] for n_ in ("q", "k", "v", "g", "beta")), state, o)
        devs[s][1].record()
    torch.cuda.synchronize()
    dec_ms = [e[0].elapsed_time(e[1]) for e in devs]

    # decoupled erase / write gates on the same workload
    for i, t in enumerate(sets):
        x = SY.decoupled_gates(dict(meta=dict(dv=dv), g=t["g"].cpu(), beta=t["beta"].cpu()), 58 + i)
        t["erase"], t["write"] = x["erase"].to(dev), x["write"].to(dev)

    def dstep(t):
        gb.gdn_decoupled_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["erase"], t["write"], o=t["o"], hT=t["hT"],
                                   workspace=ws)

    dstep(sets[0])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        dstep(sets[i % 2])
    torch.cuda.synchronize()
    dc_ms = (time.perf_counter() - t0) / n * 1e3
    return dict(B=B, T=T, H=H, dk=dk, dv=dv, fwd_ms=fwd_ms, fwd_step_ms=[e[0].elapsed_time(e[1]) for e in evs.values()],
                dec_ms=dec_ms, N=wd.decode_seqs, Hd=wd.H, dc_ms=dc_ms)


def bench_decode(args, torch, gb, SY):
    """gdn_decode_step on the decode workload (fp32 state, bf16 q/k/v and o), args.decode_steps
    chained steps, each bracketed by HIP events."""
    w = SY.WORKLOADS[4]
    d = SY.make_decode_inputs(4, steps=args.decode_steps)
    dev = torch.device("cuda:0")
    N, H, dk, dv = w.decode_seqs, w.H, w.dk, w.dv
    toks = [{n: d[n][s].to(dev) for n in ("q", "k", "v", "g", "beta")} for s in range(args.decode_steps)]
    state = d["state"].to(dev)
    o = torch.empty((N, H, dv), dtype=torch.bfloat16, device=dev)
    warm = state.clone()
    for s in range(min(3, args.decode_steps)):
        gb.gdn_decode_step(*(toks[s][n] for n in ("q", "k", "v", "g", "beta")), warm, o)
    del warm
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.decode_steps):
        gb.gdn_decode_step(*(toks[s][n] for n in ("q", "k", "v", "g", "beta")), state, o)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    state = d["state"].to(dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.decode_steps)]
    for s, e in enumerate(evs):
        e[0].record()
        gb.gdn_decode_step(*(toks[s][n] for n in ("q", "k", "v", "g", "beta")), state, o)
        e[1].record()
    torch.cuda.synchronize()
    return dict(N=N, H=H, dk=dk, dv=dv, ms=wall / args.decode_steps * 1e3,
                step_ms=[e[0].elapsed_time(e[1]) for e in evs])


def cpu_forward(wid, seconds):
    """The CPU fp64 oracle (C twin: the token recurrence, OpenMP over (sequence, head) pairs)
    on the whole of forward workload `wid`, repeated until `seconds` of wall clock have passed
    (at least once)."""
    from gated_delta_rule_42_amd import synthetic as SY
    from oracle import ctwin

    w = SY.WORKLOADS[wid]
    x = SY.make_forward_inputs(wid)
    p = ctwin.prepare_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], x["cu_seqlens"])
    reps, used = 0, 1
    t0 = time.perf_counter()
    while True:
        _, _, used = ctwin.forward_prepared(p)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or el / reps * (reps + 1) > 3 * seconds:
            break
    tokens = reps * p["B"] * p["T"]
    return {"value": tokens / el, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": f"the full {w.name} workload x{reps} (fp64 token recurrence, {el:.1f} s wall, "
                      f"{os.cpu_count()} host CPUs visible)"}


def cpu_decode(seconds):
    """The CPU fp64 oracle decode step (C twin, OpenMP over (sequence, head) pairs) on the whole
    decode workload, chained steps until `seconds` have passed."""
    import numpy as np

    from gated_delta_rule_42_amd import synthetic as SY
    from oracle import ctwin

    w = SY.WORKLOADS[4]
    d = SY.make_decode_inputs(4, steps=8)
    lib = ctwin.load()
    f64 = lambda t: np.ascontiguousarray(t.double().numpy())  # noqa: E731
    S = f64(d["state"])
    N, H, dv, dk = S.shape
    toks = [[f64(d[n][s]) for n in ("q", "k", "v", "g", "beta")] for s in range(8)]
    o = np.zeros((N, H, dv))
    P = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    steps, used = 0, 1
    t0 = time.perf_counter()
    while True:
        q, k, v, g, b = toks[steps % 8]
        used = lib.gdn_oracle_decode(P(S), P(q), P(k), P(v), P(g), P(b), P(o), N * H, dk, dv)
        steps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": steps * N / el, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": f"{steps} chained steps of the whole {w.name} workload (fp64 step, {el:.1f} s wall)"}


def cpu_baseline_slices(kind, seconds):
    """The fp64 numpy oracle of a path beyond the headline (kind "bwd": the gradient oracle,
    "kda": the channel-wise-decay forward) on one (sequence, head) slice of the training-shape
    workload at a time, over successive slices until `seconds` have passed, with one BLAS
    thread. A slice is T tokens of one head, i.e. T / H tokens of the full workload."""
    from threadpoolctl import threadpool_limits

    from gated_delta_rule_42_amd import synthetic as SY
    from oracle import backward as BW
    from oracle import kda as KD

    x = SY.make_forward_inputs(1)
    B, T, H = x["q"].shape[0], x["q"].shape[1], x["q"].shape[2]
    if kind == "bwd":
        extra = SY.make_cotangents(x, 7, dhT=False)["do"]
    else:
        x = SY.channel_gates(x, 55)
        extra = None
    n, t0 = 0, time.perf_counter()
    with threadpool_limits(1):
        while True:
            b, h = n % B, (n // B) % H
            sl = lambda t: t[b:b + 1, :, h:h + 1].contiguous()  # noqa: E731
            if kind == "bwd":
                BW.backward(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["g"]), sl(x["beta"]), sl(extra))
            else:
                KD.forward(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["g"]), sl(x["beta"]))
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    return {"value": n * T / H / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} (sequence, head) slices of T {T} of the B{B} H{H} T{T} d128 workload "
                      f"({'gradient oracle' if kind == 'bwd' else 'channel-wise-decay oracle'}, "
                      f"numpy fp64, one BLAS thread, {el:.1f} s wall), scaled to tokens of all {H} heads"}


def calib_copy(torch, mb):
    n = mb * 1024 * 1024 // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the operator "
              "shards over (sequence, head) pairs with no exchange; see the sharding notes)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from gated_delta_rule_42_amd import binding as gb
    from gated_delta_rule_42_amd import synthetic as SY

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    gb.lib()
    out = {"metric": METRIC, "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded; q,k unit-norm, v ~ N(0,1), g = -softplus(N(0,1)), "
                   "beta = sigmoid(N(0,1)))",
           "config": {"workload": "chunkwise forward B4 H16 T2048 d_k=d_v=128 chunk 64, bf16 "
                                  "q/k/v/o, fp32 gates and state, h0 = 0",
                      "B": 4, "T": 2048, "H": 16, "d_k": 128, "d_v": 128, "chunk": 64,
                      "global_batch": 4, "seq_len": 2048, "parallelism": "single GPU"}}
    if args.calib_copy_mb:
        calib_copy(torch, args.calib_copy_mb)
    if args.only in ("all", "fwd"):
        wl = {}
        names = {w.name: i for i, w in SY.WORKLOADS.items() if i != 4}
        want = set(names.values()) if args.fwd_workloads == "all" else {names[n] for n in args.fwd_workloads.split(",")}
        if 1 in want:
            # the headline: the training shape over 4 rotating input sets (beyond the Infinity Cache)
            f1 = bench_forward(1, args.steps, args.warmup, 4, torch, gb, SY)
            r1 = forward_report(f1)
            wl["train_1p3b"] = r1
            out["value"] = r1["tokens_per_s"]
            out["ms_per_step"] = r1["ms_per_call"]
            out["mfma_frac"] = r1["mfma_frac"]
            out["tflops"] = r1["tflops"]
            out["hbm_frac_algorithmic"] = r1["hbm_frac"]
            out["ms_per_step_events"] = r1["ms_per_call_events"]
            out["forward_call_roofline"] = r1["call_roofline"]
            out["forward_path"] = r1["path"]
            c = fwd_counts(f1["dk"], f1["dv"])
            th = f1["tokens"] * f1["H"]
            # the method's algorithmic bytes per call (q, k, v, o, g, beta per token-head; hT),
            # charged to the dominant kernel's launch
            alg = r1["algorithmic_bytes_per_call"]
            if f1["path"] == "fused":
                # one kernel family per call: the call's events time it
                mean_call = sum(f1["call_ms"]) / len(f1["call_ms"])
                ach = alg / (mean_call / 1e3)
                out["roofline"] = {"kernel": "chunk_fused_kernel", "bound": "hbm",
                                   "achieved": ach / 1e9, "peak": PEAK_HBM_BPS / 1e9, "unit": "GB/s",
                                   "frac": ach / PEAK_HBM_BPS, "traffic": measured_traffic("chunk_fused_kernel"),
                                   "algorithmic_bytes_per_launch": alg}
            else:
                out["stages_ms"] = {"chunk_prepare_median": pcts(f1["prep_ms"])["median"],
                                    "chunk_propagate_median": pcts(f1["prop_ms"])["median"],
                                    "chunk_prepare_mean": sum(f1["prep_ms"]) / len(f1["prep_ms"]),
                                    "chunk_propagate_mean": sum(f1["prop_ms"]) / len(f1["prop_ms"])}
                mean_prep, mean_prop = out["stages_ms"]["chunk_prepare_mean"], out["stages_ms"]["chunk_propagate_mean"]
                if mean_prop >= mean_prep:
                    ach = alg / (mean_prop / 1e3)
                    # the training shape's 32-column tiles run on chain and output waves unless
                    # GDN_SPLIT_OUT=0 selects the four-wave kernel
                    kname = ("chunk_propagate_bf16_kernel" if os.environ.get("GDN_SPLIT_OUT", "1") == "0"
                             else "chunk_propagate_split_kernel")
                    out["roofline"] = {"kernel": kname, "bound": "hbm",
                                       "achieved": ach / 1e9, "peak": PEAK_HBM_BPS / 1e9, "unit": "GB/s",
                                       "frac": ach / PEAK_HBM_BPS,
                                       "traffic": measured_traffic(kname),
                                       "algorithmic_bytes_per_launch": alg}
                else:
                    ach = c["stage1_flops"] * th / (mean_prep / 1e3)
                    out["roofline"] = {"kernel": "chunk_prepare_kernel", "bound": "mfma",
                                       "achieved": ach / 1e12, "peak": PEAK_BF16_FLOPS / 1e12,
                                       "unit": "TFLOP/s", "frac": ach / PEAK_BF16_FLOPS,
                                       "traffic": measured_traffic("chunk_prepare_kernel"),
                                       "algorithmic_flops_per_launch": c["stage1_flops"] * th}
        # the other forward workloads, one input set each (each exceeds the Infinity Cache but
        # the tiny one, which is latency-bound anyway)
        for wid, steps in ((0, args.steps), (2, max(5, args.steps // 3)), (3, max(5, args.steps // 3))):
            if wid in want:
                f = bench_forward(wid, steps, min(args.warmup, 3), 1, torch, gb, SY)
                wl[SY.WORKLOADS[wid].name] = forward_report(f)
        if "long_ctx" in wl and "train_1p3b" in wl:
            t1 = wl["train_1p3b"]["ms_per_call"] / (wl["train_1p3b"]["tokens"] * 16)
            lw = wl["long_ctx"]
            t2 = lw["ms_per_call"] / (lw["tokens"] * 16)
            out["long_vs_train_time_per_token_head"] = t2 / t1
        out["workloads"] = wl
    if args.only in ("all", "decode"):
        d = bench_decode(args, torch, gb, SY)
        per = decode_bytes(d["dk"], d["dv"], o_elem=2) * d["N"] * d["H"]
        sec = d["ms"] / 1e3
        rd = {"workload": "decode: 256 sequences x H32 d128, fp32 state, bf16 q/k/v/o, "
                          f"{args.decode_steps} chained steps",
              "ms_per_step": d["ms"], "ms_per_step_events": pcts(d["step_ms"]),
              "tokens_per_s": d["N"] / sec, "hbm_GBps": per / sec / 1e9, "hbm_frac": per / sec / PEAK_HBM_BPS,
              "bytes_per_step": per, "traffic": measured_traffic("decode_kernel"),
              "call_roofline": {"bound": "hbm", "achieved": per / sec / 1e9, "peak": PEAK_HBM_BPS / 1e9,
                                "unit": "GB/s", "frac": per / sec / PEAK_HBM_BPS}}
        out.setdefault("workloads", {})["decode"] = rd
        out["decode"] = rd
        if args.only == "decode":
            out["value"] = rd["tokens_per_s"]
            out["ms_per_step"] = d["ms"]
            out["roofline"] = dict(rd["call_roofline"], kernel="decode_kernel", traffic=rd["traffic"],
                                   algorithmic_bytes_per_launch=per)
    if args.only in ("all", "bwd"):
        b = bench_backward(args, torch, gb, SY)
        th = b["B"] * b["T"] * b["H"]
        ms = b["wall_s"] / args.bwd_steps * 1e3
        c = bwd_counts(b["dk"], b["dv"])
        fl = (c["state_flops"] + c["grad_flops"]) * th
        bb = bwd_bytes(b["dk"], b["dv"]) * th
        out["bwd"] = {"workload": "chunkwise backward B4 H16 T2048 d_k=d_v=128 chunk 64, bf16 "
                                  "q/k/v/dO and gradients, fp16 matrix-core operands with fp32 "
                                  "accumulation, states and gate gradients, no h0 / dhT",
                      "ms_per_step": ms, "ms_per_step_median": median(b["step_ms"]),
                      "tokens_per_s": b["B"] * b["T"] / (ms / 1e3),
                      "tflops": fl / (ms / 1e3) / 1e12,
                      "mfma_frac": fl / (ms / 1e3) / PEAK_BF16_FLOPS,
                      "grad_kernel_flops_per_launch": c["grad_flops"] * th,
                      "state_kernel_flops_per_launch": c["state_flops"] * th,
                      "mfma_peak_tflops": PEAK_BF16_FLOPS / 1e12,
                      # whole call (four launches in one entry point): HBM is the nearer bound
                      # (algorithmic bytes at peak take longer than algorithmic FLOP at peak)
                      "roofline": {"kernel": "gdn_chunk_bwd (whole call)", "bound": "hbm",
                                   "achieved": bb / (ms / 1e3) / 1e9, "peak": PEAK_HBM_BPS / 1e9,
                                   "unit": "GB/s", "frac": bb / (ms / 1e3) / PEAK_HBM_BPS,
                                   "traffic": call_traffic([("chunk_prepare_kernel@bwd", "128, true>"),
                                                            ("chunk_propagate_bf16_kernel@bwd", "false>"),
                                                            ("chunk_bwd_state16_kernel@bwd", None),
                                                            ("chunk_bwd_grad16_kernel@bwd", None)]),
                                   "algorithmic_bytes_per_call": bb}}
        if args.cpu_seconds > 0:
            out["bwd"]["cpu_baseline"] = cpu_baseline_slices("bwd", args.cpu_seconds / 2)
        if args.only == "bwd":
            out["value"] = b["B"] * b["T"] / (ms / 1e3)
            out["ms_per_step"] = ms
    if args.only in ("all", "kda"):
        k = bench_kda(args, torch, gb, SY)
        th = k["B"] * k["T"] * k["H"]
        c = fwd_counts(k["dk"], k["dv"])
        dmean = sum(k["dec_ms"]) / len(k["dec_ms"])
        per = (decode_bytes(k["dk"], k["dv"]) + 4 * (k["dk"] - 1)) * k["N"] * k["Hd"]
        out["kda"] = {"workload": "channel-wise decay: chunkwise forward B4 H16 T2048 d128 bf16 q/k/v/o "
                                  "(stage 1 fp32, its Gram blocks below the diagonal on fp16 operands; stage 2 on fp16 "
                                  "matrix-core operands with fp32 "
                                  "accumulation and state), and decode 256 seq x H32 d128 (16 chained steps)",
                      "fwd_ms_per_step": k["fwd_ms"], "fwd_ms_median": median(k["fwd_step_ms"]),
                      "fwd_tokens_per_s": k["B"] * k["T"] / (k["fwd_ms"] / 1e3),
                      "fwd_tflops_algorithmic": c["flops"] * th / (k["fwd_ms"] / 1e3) / 1e12,
                      "decode_ms_per_step_mean": dmean,
                      "decode_hbm_GBps": per / (dmean / 1e3) / 1e9,
                      "decode_hbm_frac": per / (dmean / 1e3) / PEAK_HBM_BPS,
                      "decoupled_gates_fwd_ms_per_step": k["dc_ms"],
                      "decoupled_gates_fwd_tokens_per_s": k["B"] * k["T"] / (k["dc_ms"] / 1e3)}
        kb = kda_bytes(k["dk"], k["dv"]) * th
        # the channel-wise-decay forward, whole call (two launches in one entry point): HBM is the
        # nearer bound
        out["kda"]["roofline"] = {"kernel": "gdn_kda_chunk_fwd (whole call)", "bound": "hbm",
                                  "achieved": kb / (k["fwd_ms"] / 1e3) / 1e9, "peak": PEAK_HBM_BPS / 1e9,
                                  "unit": "GB/s", "frac": kb / (k["fwd_ms"] / 1e3) / PEAK_HBM_BPS,
                                  # the instances without decoupled gates (template flag false)
                                  "traffic": call_traffic([("kda_prepare_kernel@kda", "128, false>"),
                                                           ("kda_propagate_dma_kernel@kda", "false>")]),
                                  "algorithmic_bytes_per_call": kb}
        if args.cpu_seconds > 0:
            out["kda"]["cpu_baseline"] = cpu_baseline_slices("kda", args.cpu_seconds / 2)
        if args.only == "kda":
            out["value"] = k["B"] * k["T"] / (k["fwd_ms"] / 1e3)
            out["ms_per_step"] = k["fwd_ms"]
    if args.cpu_seconds > 0 and args.only in ("all", "fwd"):
        # the headline's oracle gets the budget, the other workloads a fifth of it each
        if "train_1p3b" in out["workloads"]:
            out["cpu_baseline"] = cpu_forward(1, args.cpu_seconds)
            out["workloads"]["train_1p3b"]["cpu_baseline"] = out["cpu_baseline"]
        for wid in (0, 2, 3):
            if SY.WORKLOADS[wid].name in out["workloads"]:
                out["workloads"][SY.WORKLOADS[wid].name]["cpu_baseline"] = cpu_forward(wid, args.cpu_seconds / 5)
    if args.cpu_seconds > 0 and args.only in ("all", "decode"):
        out["workloads"]["decode"]["cpu_baseline"] = cpu_decode(args.cpu_seconds / 5)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
