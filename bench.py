"""Benchmark of the KDA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Headline: chunked prefill of one 4096-token sequence (H=32, dk=dv=128, conv
kernel 4, 64-token chunks, bf16 inputs, fp32 state).  One step is the whole
prefill path over one batch already resident in HBM, from raw inputs to the
gated output, the final fp32 state and the outgoing conv cache: kda_prefill
(kda_prefill_prepare: short conv + SiLU + L2 + sigmoid(beta) fused into the
chunk preparation; kda_prefill_scan: state pass + sigmoid output gate).
`--path unfused` times kda_prologue + kda_chunk_forward instead.  Two input
sets alternate between steps so the 256 MB Infinity Cache cannot hold one
step's inputs for the next.  value = prefill tokens/s.

The metric's second half, decode, is measured in the same run on the batched
decode workload (256 resident fp32 states x 1 token, 64 consecutive
kda_decode_step calls with distinct inputs) and reported under "decode".
The chunked backward (kda_chunk_backward) on the prefill workload's shapes is
reported under "backward", the packed varlen and long-context prefill
workloads under "prefill_workloads", and the KDA mixer (input projection,
prefill, output projection at a synthetic hidden size) under "mixer", and
the MLA decode token under "mla_decode" (informative; the headline stays the
4096-token sequence).

The headline's W warm-up steps (600 by default, about 0.1 s) and a time-based
warm-up of 0.1 s before every other leg let the GPU's clocks settle before
anything is timed (a few calls are not enough: the first timed batch then
runs several percent slow).  Every kernel is timed with HIP events on the
stream it is launched on.  The
roofline object counts the path's algorithmic bytes only (49,216 B per token:
q, k, v, log alpha, gate and beta in, y out, plus the fp32 state and conv
cache in and out), never the chunk records the two stages pass between them:
"frac" is those bytes over the longest kernel's own time, "path.frac" over
the whole step; "traffic" is what the counters measured for both kernels.
The oracle (CPU, fp64) is timed on the same prefill workload as
"cpu_baseline".  Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s (%MFMA peak) + decode tokens/s (%HBM BW), H=32 d=128"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s

H, D, K, CHUNK = 32, 128, 4, 64
# Algorithmic bytes per token of the prefill path (all 32 heads, bf16): q, k,
# v, log alpha and gate in (8,192 B each), beta in (64 B), y out (8,192 B).
PATH_B_PER_TOK = 5 * 8192 + 64 + 8192                                          # 49,216
STATE_B = H * D * D * 4                                                        # one sequence's fp32 state
CONV_CACHE_B = 3 * (K - 1) * H * D * 4
FLOP_PER_TOK = 4_496_032                                                       # useful chunked-form flops (H=32)
DECODE_B_PER_ROW = 2 * STATE_B + 2 * CONV_CACHE_B + 3 * 8192 + 8192 + 64 + 8192 + 16384   # 4,546,624
# kda_chunk_backward: the dense fp32 products it executes per (64-token chunk,
# head), in multiply-adds (C = 64, d = 128): WY quantities 4 C^2 d; forward
# state pass 2 C d^2; backward state pass C^2 d + 3 C d^2; per-chunk gradients
# 4 C d^2 + 11 C^2 d + 2 C^3 (O 1.57, dPm 0.52, dQd 1.57, dW 1.05, dKg 1.05,
# dTB 1.05, dKd 1.05, dV 0.52, T^T dT 0.26, dA 0.26, Kd Ki^T 0.52, dKi 1.05
# million): 18,350,080 in all.
BWD_FLOP_PER_CHUNK_HEAD = 2 * 18_350_080
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 vector, TFLOP/s


# bench timing slot -> the kernel it launches at head dim 128, conv 4, SiLU
# (the batched varlen scan runs the two-tiles-per-block instance), and the
# sources that kernel is built from: a counter record is used only while the
# hash of those sources matches the one stored with it
TRAFFIC_KERNEL = {"prologue": "prologue128_kernel<4, 1>", "chunk_prepare": "prepare_kernel<false, 4, 0>",
                  "chunk_scan": "scan_kernel<true, 1>", "prefill_prepare": "prepare_kernel<true, 4, 1>",
                  "prefill_scan": "scan_kernel<true, 1>", "decode": "decode_kernel<128, 1, 0>",
                  "in_projection": "gemm_kernel<1, 256>", "in_projection_beta": "gemm_narrow_kernel",
                  "out_projection": "gemm_kernel<0, 224 or 256>",
                  "mla_attend": "mla_attend_kernel<3, 2, true, true>", "mla_combine": "mla_combine_kernel"}
KERNEL_SOURCES = {"prologue": ["prologue.hip"], "chunk_prepare": ["chunk.hip"], "chunk_scan": ["chunk.hip"],
                  "prefill_prepare": ["chunk.hip"], "prefill_scan": ["chunk.hip"], "decode": ["decode.hip"],
                  "in_projection": ["proj.hip"], "in_projection_beta": ["proj.hip"], "out_projection": ["proj.hip"],
                  "mla_attend": ["mla.hip"],
                  "mla_combine": ["mla.hip"]}


def _src_sha(slot):
    import hashlib

    h = hashlib.sha256()
    for fn in KERNEL_SOURCES[slot] + ["kda_device.h", "kda_internal.h"]:
        with open(os.path.join(ROOT, "kimi_delta_attention_07_amd", "csrc", fn), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _counter_record(fname, slot, workload="T4096"):
    """The record of the kernel behind a bench timing slot in a counter file
    under profiles/ (written from rocprofv3 runs of this bench), or None when
    the file is missing or the kernel's sources changed since."""
    path = os.path.join(ROOT, "profiles", fname)
    if slot not in KERNEL_SOURCES or not os.path.exists(path):
        return None
    rec = json.load(open(path)).get("records", {}).get(f"{slot} @ {workload}")
    if not rec or rec.get("src_sha") != _src_sha(slot):
        return None
    return rec


def measured_traffic(slot, workload="T4096"):
    """HBM bytes per launch measured by rocprofv3 (FETCH_SIZE, WRITE_SIZE, both
    calibrated against a 1 GiB copy) and kept in profiles/traffic.json, or None
    when that file is missing or the kernel's sources changed since."""
    rec = _counter_record("traffic.json", slot, workload)
    return rec["bytes_per_launch"] if rec else None


def measured_mfma(slot, workload="T4096"):
    """Matrix-core counters per launch (rocprofv3 --pmc), from
    profiles/mfma.json: bf16 MFMA flops executed and MFMA-busy cycles."""
    return _counter_record("mfma.json", slot, workload)


def path_roofline(path_bytes, per_kernel_ms, ms_step, slots, workload="T4096", tokens=4096):
    """The roofline object of one prefill workload: the path's algorithmic
    bytes over the longest kernel's time (frac) and over the whole step
    (path.frac), the measured traffic of the step's kernels beside them, and
    the matrix-core fractions (useful flops from the flop model; executed
    flops and busy cycles from the counters when they are current)."""
    dom = max(per_kernel_ms, key=per_kernel_ms.get)
    t_dom = per_kernel_ms[dom] * 1e-3
    ach = path_bytes / t_dom / 1e9
    tr = {k: measured_traffic(k, workload) for k in slots}
    traffic = sum(tr.values()) if all(v is not None for v in tr.values()) else None
    useful = FLOP_PER_TOK * tokens
    mf = {k: measured_mfma(k, workload) for k in slots}
    out = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
           "traffic": traffic, "kernel": TRAFFIC_KERNEL.get(dom, dom), "bytes_per_launch": path_bytes,
           "traffic_over_algorithmic": traffic / path_bytes if traffic else None,
           "traffic_per_kernel": tr,
           "path": {"achieved": path_bytes / (ms_step * 1e-3) / 1e9,
                    "frac": path_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "floor_us": path_bytes / (HBM_PEAK_GBS * 1e9) * 1e6},
           "mfma": {"useful_flop_per_step": useful,
                    "useful_frac": useful / (ms_step * 1e-3) / (BF16_PEAK_TFLOPS * 1e12)}}
    if all(v is not None for v in mf.values()):
        ex = sum(v["bf16_flop"] for v in mf.values())
        out["mfma"]["executed_bf16_flop_per_step"] = ex
        out["mfma"]["executed_frac"] = ex / (ms_step * 1e-3) / (BF16_PEAK_TFLOPS * 1e12)
        out["mfma"]["busy_frac_per_kernel"] = {k: v["busy_frac"] for k, v in mf.items()}
    return out


def spin_up(torch, fn, ms=100.0):
    """Untimed warm-up: call fn until ms of wall time have passed (the GPU's
    clocks settle well after a few calls; every leg starts after CPU-side
    input generation has left the GPU idle)."""
    t0 = time.perf_counter()
    n = 0
    while (time.perf_counter() - t0) * 1e3 < ms or n < 2:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=600,
                    help="untimed prefill steps before the timed ones (600: about 0.1 s, enough for the clocks)")
    ap.add_argument("--decode-reps", type=int, default=3, help="timed passes of 64 decode steps")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode measurement")
    ap.add_argument("--no-backward", action="store_true", help="skip the chunked backward measurement")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the varlen and long-context prefill measurements")
    ap.add_argument("--no-mixer", action="store_true", help="skip the KDA mixer (projections) measurement")
    ap.add_argument("--no-mla", action="store_true", help="skip the MLA decode measurement")
    ap.add_argument("--mixer-hidden", type=int, default=7168, help="hidden size of the mixer measurement")
    ap.add_argument("--backward-steps", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--path", choices=("fused", "unfused"), default="fused")
    return ap.parse_args()


def prefill_sets(torch, ki, dev, n_sets=2):
    sets = []
    for i in range(n_sets):
        inp = ki.prefill_inputs(1 + 100 * i, [4096], H=H, d=D, K=K)
        g = {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in inp.items()}
        g["pro"] = dict(q=torch.empty_like(g["q_raw"]), k=torch.empty_like(g["k_raw"]), v=torch.empty_like(g["v_raw"]),
                        beta=torch.empty(4096, H, dtype=torch.float32, device=dev),
                        gate=torch.empty_like(g["gate_logit"]))
        g["cache_out"] = torch.empty_like(g["conv_cache"])
        g["y"] = torch.empty_like(g["v_raw"])
        g["final_state"] = torch.empty_like(g["initial_state"])
        g["cu_host"] = inp["cu_seqlens"]
        sets.append(g)
    return sets


def run_fused_step(kda, g, ws, ev=None):
    """kda_prefill_prepare -> kda_prefill_scan; ev: 3 events recorded around them."""
    if ev:
        ev[0].record()
    kda.prefill_prepare(g["q_raw"], g["k_raw"], g["v_raw"], g["conv_w"], g["log_alpha"], g["beta_logit"],
                        g["cu_seqlens"], ws, g["conv_cache"], g["cache_out"], cu_seqlens_host=g["cu_host"])
    if ev:
        ev[1].record()
    kda.prefill_scan(g["gate_logit"], g["cu_seqlens"], ws, g["y"], g["initial_state"], g["final_state"], H=H,
                     cu_seqlens_host=g["cu_host"])
    if ev:
        ev[2].record()


def run_prefill_step(kda, g, ws, ev=None):
    """prologue -> chunk_prepare -> chunk_scan; ev: 4 events recorded between them."""
    if ev:
        ev[0].record()
    kda.prologue(g["q_raw"], g["k_raw"], g["v_raw"], g["conv_w"], g["cu_seqlens"], g["beta_logit"], g["gate_logit"],
                 g["conv_cache"], g["cache_out"], cu_seqlens_host=g["cu_host"], outs=g["pro"])
    if ev:
        ev[1].record()
    p = g["pro"]
    kda.chunk_prepare(p["q"], p["k"], p["v"], g["log_alpha"], p["beta"], g["cu_seqlens"], ws,
                      cu_seqlens_host=g["cu_host"])
    if ev:
        ev[2].record()
    kda.chunk_scan(p["gate"], g["cu_seqlens"], ws, g["y"], g["initial_state"], g["final_state"], H=H,
                   cu_seqlens_host=g["cu_host"])
    if ev:
        ev[3].record()


def bench_prefill(torch, kda, ki, args, dev):
    sets = prefill_sets(torch, ki, dev)
    ws = kda.chunk_workspace(H, D, sets[0]["cu_host"], dev)
    fused = args.path == "fused"
    step = run_fused_step if fused else run_prefill_step
    slots = ["prefill_prepare", "prefill_scan"] if fused else ["prologue", "chunk_prepare", "chunk_scan"]
    for i in range(args.warmup):
        step(kda, sets[i % 2], ws)
    torch.cuda.synchronize()
    # headline: K back-to-back steps bracketed by two events only (an event
    # recorded between kernels costs several microseconds of its own)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        step(kda, sets[i % 2], ws)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(stop)
    # per-kernel times (and the roofline's kernel duration): the same K steps
    # again, with events between the kernels
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(slots) + 1)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(kda, sets[i % 2], ws, evs[i])
    torch.cuda.synchronize()
    per = {k: 0.0 for k in slots}
    for e in evs:
        for j, k in enumerate(slots):
            per[k] += e[j].elapsed_time(e[j + 1])
    per = {k: v / args.steps for k, v in per.items()}
    # per-step times: the same K steps once more, one event at each step
    # boundary only; their median is reported beside the K-step mean
    bev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    bev[0].record()
    for i in range(args.steps):
        step(kda, sets[i % 2], ws)
        bev[i + 1].record()
    torch.cuda.synchronize()
    steps_ms = sorted(bev[i].elapsed_time(bev[i + 1]) for i in range(args.steps))
    n = len(steps_ms)
    median = steps_ms[n // 2] if n % 2 else 0.5 * (steps_ms[n // 2 - 1] + steps_ms[n // 2])
    return dict(ms_per_step=total_ms / args.steps, wall_s=wall, per_kernel_ms=per, step_ms_median=median,
                step_ms_min=steps_ms[0], step_ms_max=steps_ms[-1])


def bench_prefill_workloads(torch, kda, ki, args, dev):
    """The two other prefill workloads, timed the same way on one input set
    each (they are far larger than the 256 MB last-level cache): packed varlen
    (32 sequences of U[256, 8192] tokens, seed 3) and long context (one
    65,536-token sequence with slow decay, seed 4).  Reported beside the
    headline, with the path's HBM floor (49,216 B per token plus the fp32
    states and conv caches in and out)."""
    out = {}
    cases = [("varlen", dict(seed=3, lengths=None, draw_lengths=(256, 8192, 32)),
              "packed varlen prefill, 32 sequences of U[256, 8192] tokens"),
             ("long_context", dict(seed=4, lengths=[65536], la_range=(-8.0, -2.0), tail_steps=128),
              "long-context prefill, 1 sequence x 65,536 tokens, log alpha = -exp(U(-8, -2))")]
    for name, kw, desc in cases:
        inp = ki.prefill_inputs(kw.pop("seed"), kw.pop("lengths"), H=H, d=D, K=K, **kw)
        T, N = inp["T"], inp["N"]
        g = {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in inp.items()}
        g["cache_out"] = torch.empty_like(g["conv_cache"])
        g["y"] = torch.empty_like(g["v_raw"])
        g["final_state"] = torch.empty_like(g["initial_state"])
        g["cu_host"] = inp["cu_seqlens"]
        ws = kda.chunk_workspace(H, D, g["cu_host"], dev)
        spin_up(torch, lambda: run_fused_step(kda, g, ws))
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        a.record()
        for _ in range(reps):
            run_fused_step(kda, g, ws)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
        for e in evs:
            run_fused_step(kda, g, ws, e)
        torch.cuda.synchronize()
        per = {"prefill_prepare": sum(e[0].elapsed_time(e[1]) for e in evs) / reps,
               "prefill_scan": sum(e[1].elapsed_time(e[2]) for e in evs) / reps}
        floor_b = T * PATH_B_PER_TOK + N * (2 * STATE_B + 2 * CONV_CACHE_B)
        n_chunks = sum((int(x) + CHUNK - 1) // CHUNK for x in inp["lengths"])
        out[name] = {"workload": desc + f" ({T} tokens), H=32 dk=dv=128, conv 4, chunk 64, bf16 inputs",
                     "tokens": T, "sequences": N, "chunks": n_chunks, "ms_per_call": ms,
                     "value": T / (ms * 1e-3), "unit": "tokens/s", "per_kernel_ms": per,
                     "roofline": path_roofline(floor_b, per, ms, list(per), name, T)}
        if inp["tail"]:
            out[name]["decode_tail"] = decode_tail(torch, kda, g, inp["tail"], dev)
        del g, ws
        torch.cuda.empty_cache()
    return out


def decode_tail(torch, kda, g, tail, dev):
    """The long-context workload's decode tail: kda_decode_step for one
    sequence, token after token, continuing from the prefill's final state
    and conv cache (the state is updated in place; a warm-up pass of the same
    tokens runs first).  One workgroup per head, so the step is set by
    latency, not bandwidth; bytes per token are the 32 fp32 states read and
    written."""
    steps = [{k: v.to(dev) for k, v in st.items()} for st in tail]
    state, cache = g["final_state"], g["cache_out"]
    y = torch.empty(1, H, D, dtype=torch.float32, device=dev)

    def run():
        for st in steps:
            kda.decode_step(st["q_raw"], st["k_raw"], st["v_raw"], g["conv_w"], cache, state, st["log_alpha"],
                            st["beta_logit"], st["gate_logit"], out=y)

    spin_up(torch, run)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    run()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / len(steps)
    # the same 128 launches replayed from a HIP graph (captured on torch's
    # capture stream after a warm-up there): launch overhead mostly gone
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    spin_up(torch, graph.replay)
    a.record()
    graph.replay()
    b.record()
    torch.cuda.synchronize()
    us_graph = a.elapsed_time(b) * 1e3 / len(steps)
    return {"steps": len(steps), "us_per_token": us, "value": 1e6 / us, "unit": "tokens/s",
            "us_per_token_graph": us_graph, "state_bytes_per_token": DECODE_B_PER_ROW,
            "achieved_gbs": DECODE_B_PER_ROW / (us * 1e-6) / 1e9}


def bench_decode(torch, kda, ki, args, dev):
    dec = ki.config_decode(2)
    state, cache, cw = dec["state"].to(dev), dec["conv_cache"].to(dev), dec["conv_w"].to(dev)
    steps = [{k: v.to(dev) for k, v in s.items()} for s in dec["steps"]]
    out = torch.empty(256, H, D, dtype=torch.float32, device=dev)

    def one(s):
        kda.decode_step(s["q_raw"], s["k_raw"], s["v_raw"], cw, cache, state, s["log_alpha"], s["beta_logit"],
                        s["gate_logit"], out=out)

    it = iter(range(1 << 30))
    spin_up(torch, lambda: one(steps[next(it) % len(steps)]))
    times = []
    for _ in range(args.decode_reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for s in steps:
            one(s)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) / len(steps))
    ms = sorted(times)[len(times) // 2]
    gbs = 256 * DECODE_B_PER_ROW / (ms * 1e-3) / 1e9
    return {"workload": "batched decode: 256 resident fp32 states x 1 token, H=32 d=128 conv 4, 64 steps",
            "value": 256 / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": measured_traffic("decode", "B256"),
                         "bytes_per_launch": 256 * DECODE_B_PER_ROW}}


def copy_bandwidth(torch, dev):
    a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(5):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / 5
    return 2 * a.numel() * 4 / (ms * 1e-3) / 1e9


def cpu_baseline(ki, seconds):
    import oracle

    orc = oracle.get()
    inp = ki.config_prefill(1)
    threads = orc.num_threads()
    reps, t0 = 0, time.perf_counter()
    while True:
        orc.prefill(inp)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 50:
            break
    cores = min(orc.num_threads(), H)   # one (sequence, head) pair per thread at most
    # the same workload on one thread, once (about 16 times one run above)
    orc.set_num_threads(1)
    t1 = time.perf_counter()
    orc.prefill(inp)
    el1 = time.perf_counter() - t1
    orc.set_num_threads(threads)
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": reps * 4096 / el, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"the full T=4096 H=32 prefill workload, fp64 oracle, {reps} run(s) in {el:.1f} s "
                      f"on {cores} OpenMP threads (heads in parallel)",
            "cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0)), "omp_threads": threads,
            "single_thread": {"value": 4096 / el1, "unit": "tokens/s", "cores": 1,
                              "sample": f"one run of the same workload on one thread, {el1:.1f} s"}}


def bench_backward(torch, kda, ki, args, dev):
    """kda_chunk_backward on the prefill workload's shapes (T=4096, H=32):
    the forward inputs come from the library's own prologue, dy and the
    final-state gradient are seeded random."""
    inp = ki.prefill_inputs(3, [4096], H=H, d=D, K=K)
    g = {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in inp.items()}
    cu_h = inp["cu_seqlens"]
    pro = kda.prologue(g["q_raw"], g["k_raw"], g["v_raw"], g["conv_w"], g["cu_seqlens"], g["beta_logit"],
                       g["gate_logit"], g["conv_cache"], torch.empty_like(g["conv_cache"]), cu_seqlens_host=cu_h)
    gen = torch.Generator().manual_seed(5)
    dy = torch.randn(4096, H, D, generator=gen).to(torch.bfloat16).to(dev)
    dsf = (torch.randn(1, H, D, D, generator=gen) * 0.1).to(dev)
    ws = torch.empty(kda.chunk_backward_workspace_bytes(H, D, cu_h), dtype=torch.uint8, device=dev)

    def one():
        return kda.chunk_backward(pro["q"], pro["k"], pro["v"], g["log_alpha"], pro["beta"], pro["gate"],
                                  g["cu_seqlens"], dy, g["initial_state"], dsf, workspace=ws, cu_seqlens_host=cu_h)

    grads = one()
    spin_up(torch, one)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.backward_steps):
        one()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.backward_steps
    # the prologue's backward on the same shapes, from the chunk backward's gradients
    pws = torch.empty(kda._lib.load().kda_prologue_backward_workspace_bytes(
        ctypes.byref(kda._lib.geom(H, D, K)), 4096), dtype=torch.uint8, device=dev)

    def one_pro():
        return kda.prologue_backward(g["q_raw"], g["k_raw"], g["v_raw"], g["conv_w"], g["cu_seqlens"],
                                     g["beta_logit"], g["gate_logit"], g["conv_cache"], grads["dq"], grads["dk"],
                                     grads["dv"], grads["dbeta"], grads["dgate"], cu_seqlens_host=cu_h, workspace=pws)

    spin_up(torch, one_pro)
    a.record()
    for _ in range(args.backward_steps):
        one_pro()
    b.record()
    torch.cuda.synchronize()
    ms_pro = a.elapsed_time(b) / args.backward_steps
    # compulsory bytes: raw q, k, v, gate and beta logits (bf16) and the five
    # upstream gradients (fp32) in; four fp32 gradients [T, H, d] and dbeta
    # logits out (conv taps and caches are negligible)
    pro_bytes = 4096 * H * D * (4 * 2 + 4 * 4 + 4 * 4) + 4096 * H * (2 + 4 + 4)
    flop = (4096 // CHUNK) * H * BWD_FLOP_PER_CHUNK_HEAD
    tf = flop / (ms * 1e-3) / 1e12
    return {"workload": "chunked backward, 1 sequence x 4096 tokens, H=32 dk=dv=128, chunk 64, bf16 inputs and dy, "
                        "fp32 gradients (dq, dk, dv, dlog alpha, dbeta, dgate, d initial state)",
            "value": 4096 / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms, "steps": args.backward_steps,
            "roofline": {"bound": "alu", "achieved": tf, "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": tf / FP32_PEAK_TFLOPS, "traffic": None,
                         "kernel": "kda_chunk_backward (prep, fwd_states, bwd_states, grads)",
                         "flop_per_launch": flop},
            "prologue_backward": {"workload": "kda_prologue_backward on the same shapes, from the chunk "
                                              "backward's gradients to raw q, k, v, conv taps, conv cache, "
                                              "beta and gate logits",
                                  "ms_per_call": ms_pro, "value": 4096 / (ms_pro * 1e-3), "unit": "tokens/s",
                                  "hbm_gbs": pro_bytes / (ms_pro * 1e-3) / 1e9,
                                  "hbm_frac": pro_bytes / (ms_pro * 1e-3) / 1e9 / HBM_PEAK_GBS}}


def bench_mixer(torch, kda, ki, args, dev):
    """The KDA mixer on one 4096-token sequence: input projection (hidden ->
    q, k, v, gate, decay, beta), the fused prefill, output projection.  The
    pages give no hidden size; --mixer-hidden sets a synthetic one.  The two
    projections are MFMA-bound GEMMs: each is timed alone and priced on its
    dense bf16 flops, 2 T hidden N."""
    T, hidden = 4096, args.mixer_hidden
    inp = ki.mixer_inputs(11, [T], hidden, H, D, K)
    g = {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in inp.items()}
    cu_h = inp["cu_seqlens"]
    n_in, n_out = 5 * H * D + H, hidden
    outs = kda.in_projection(g["x"], g["w_in"], H, D, g["a_log"], g["dt_bias"])
    y = torch.empty(T, H * D, dtype=torch.bfloat16, device=dev).normal_()
    o = kda.out_projection(y, g["w_out"])
    ws = torch.empty(kda.mixer_workspace_bytes(H, D, 1, T), dtype=torch.uint8, device=dev)
    fs = torch.empty(1, H, D, D, dtype=torch.float32, device=dev)
    cco = torch.empty_like(g["conv_cache"])

    def mixer():
        kda.mixer_prefill(g["x"], g["w_in"], g["w_out"], g["conv_w"], g["cu_seqlens"], g["a_log"], g["dt_bias"],
                          g["initial_state"], g["conv_cache"], cco, H=H, d=D, final_state=fs, out=o,
                          workspace=ws, cu_seqlens_host=cu_h)

    def timed(fn, reps):
        spin_up(torch, fn)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    reps = max(args.steps // 2, 5)
    ms_in = timed(lambda: kda.in_projection(g["x"], g["w_in"], H, D, g["a_log"], g["dt_bias"], outs=outs), reps)
    ms_out = timed(lambda: kda.out_projection(y, g["w_out"], out=o), reps)
    ms_mix = timed(mixer, reps)
    f_in, f_out = 2.0 * T * hidden * n_in, 2.0 * T * H * D * n_out
    tf_in, tf_out = f_in / (ms_in * 1e-3) / 1e12, f_out / (ms_out * 1e-3) / 1e12
    tf_mix = (f_in + f_out) / (ms_mix * 1e-3) / 1e12
    tr_in = [measured_traffic("in_projection", "mixer"), measured_traffic("in_projection_beta", "mixer")]
    in_traffic = sum(tr_in) if all(t is not None for t in tr_in) else None
    return {"workload": f"KDA mixer, 1 sequence x {T} tokens, hidden {hidden} (synthetic), H=32 dk=dv=128, conv 4: "
                        "input projection, fused prefill, output projection; bf16 weights and activations",
            "value": T / (ms_mix * 1e-3), "unit": "tokens/s", "ms_per_step": ms_mix, "steps": reps,
            "in_projection": {"ms_per_call": ms_in, "shape": f"[{T} x {hidden}] x [{n_in} x {hidden}]^T",
                              "tflops": tf_in, "mfma_frac": tf_in / BF16_PEAK_TFLOPS},
            "out_projection": {"ms_per_call": ms_out, "shape": f"[{T} x {H * D}] x [{n_out} x {H * D}]^T",
                               "tflops": tf_out, "mfma_frac": tf_out / BF16_PEAK_TFLOPS},
            "roofline": {"bound": "mfma", "achieved": tf_in, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": tf_in / BF16_PEAK_TFLOPS, "traffic": in_traffic,
                         "kernel": "gemm_kernel<1, 256> + gemm_narrow_kernel (input projection: the 5 H d columns, "
                                   "then the H beta columns)", "flop_per_launch": f_in,
                         "mfma_counters": {"gemm_kernel<1, 256>": measured_mfma("in_projection", "mixer"),
                                           "gemm_narrow_kernel": measured_mfma("in_projection_beta", "mixer")}},
            "projection_flops_frac_of_step": (f_in + f_out) / (ms_mix * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "step_tflops": tf_mix}


def bench_mla(torch, kda, ki, args, dev):
    """The MLA decode token on 16 sequences x 64 heads, 192 q/k channels
    (128 nope + 64 rope), 128 value channels, a 4096-slot bf16 K/V cache
    filled to U[1024, 4095] tokens (the pages give the tiny config's widths
    only; these are synthetic).  Repeated calls rewrite the same slot, so
    every call does the same work.  Priced on HBM bytes: the cached k and v
    of every sequence's tokens, q, the new k and v (read, then written into
    the cache), the gate logits in and the output out."""
    B, Hq, Hkv, dqk, dv, L = 16, 64, 64, 192, 128, 4096
    inp = ki.mla_inputs(45, B, Hq, Hkv, dqk, dv, L, len_range=(1024, 4095))
    g = {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in inp.items()}
    ws = torch.empty(kda.mla_decode_workspace_bytes(Hq, Hkv, dqk, dv, B, L), dtype=torch.uint8, device=dev)
    out = torch.empty(B, Hq, dv, dtype=torch.bfloat16, device=dev)

    def one():
        kda.mla_decode_step(g["q"], g["k_new"], g["v_new"], g["k_cache"], g["v_cache"], g["cache_len"],
                            g["gate_logit"], out=out, workspace=ws)

    spin_up(torch, one)
    reps = max(args.steps, 20)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    evs[0].record()
    for i in range(reps):
        one()
        evs[i + 1].record()
    torch.cuda.synchronize()
    per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(reps))
    ms = per[reps // 2]
    tokens = int(inp["cache_len"].sum())
    nbytes = (tokens * Hkv * (dqk + dv) * 2 + B * Hq * dqk * 2 + 2 * B * Hkv * (dqk + dv) * 2
              + 2 * B * Hq * dv * 2)
    gbs = nbytes / (ms * 1e-3) / 1e9
    tr = [measured_traffic("mla_attend", "mla"), measured_traffic("mla_combine", "mla")]
    mla_traffic = sum(tr) if all(t is not None for t in tr) else None
    return {"workload": f"MLA decode token, {B} sequences x {Hq} heads ({Hkv} kv heads), q/k {dqk} (128 nope + 64 "
                        f"rope, NoPE), v {dv}, bf16 K/V cache of {L} slots holding U[1024, 4095] tokens "
                        f"({tokens} in all), gated",
            "value": B / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms, "steps": reps,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": mla_traffic,
                         "kernel": "mla_attend_kernel<3, 2, true, true> + mla_combine_kernel (one call)",
                         "bytes_per_launch": nbytes,
                         "traffic_over_algorithmic": mla_traffic / nbytes if mla_traffic else None}}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported by this single-GPU build "
              "(heads and sequences are independent, so N GPUs would each run this kernel on their share).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import kda_inputs as ki
    import kimi_delta_attention_07_amd as kda

    kda.load()
    dev = torch.device("cuda:0")
    pre = bench_prefill(torch, kda, ki, args, dev)
    ms = pre["ms_per_step"]
    tok_s = 4096 / (ms * 1e-3)
    per = pre["per_kernel_ms"]
    path_bytes = 4096 * PATH_B_PER_TOK + 2 * STATE_B + 2 * CONV_CACHE_B   # 206,077,952
    res = {
        "metric": METRIC, "value": tok_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "chunked prefill, 1 sequence x 4096 tokens, H=32 dk=dv=128, conv 4, chunk 64, "
                               "bf16 inputs, fp32 initial/final state", "global_batch": 1, "seq_len": 4096,
                   "parallelism": "single GPU", "path": "kda_prefill (fused)" if args.path == "fused"
                   else "kda_prologue + kda_chunk_forward"},
        "step_ms_median": pre["step_ms_median"],
        "roofline": path_roofline(path_bytes, per, ms, list(per)),
        "prefill": {"per_kernel_ms": per, "step_ms_median": pre["step_ms_median"],
                    "step_ms_min": pre["step_ms_min"], "step_ms_max": pre["step_ms_max"]},
    }
    if not args.no_workloads:
        res["prefill_workloads"] = bench_prefill_workloads(torch, kda, ki, args, dev)
    if not args.no_decode:
        res["decode"] = bench_decode(torch, kda, ki, args, dev)
    if not args.no_backward:
        res["backward"] = bench_backward(torch, kda, ki, args, dev)
    if not args.no_mixer:
        res["mixer"] = bench_mixer(torch, kda, ki, args, dev)
    if not args.no_mla:
        res["mla_decode"] = bench_mla(torch, kda, ki, args, dev)
    res["copy_gbs"] = copy_bandwidth(torch, dev)
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(ki, args.cpu_seconds)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
