#!/usr/bin/env python3
"""Benchmark of the MoE decode tail on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one pass of the whole tail at b=64 tokens, P=3584:

  1. EP finalize of tp=8 simulated ranks' GEMM2 rows (top-16 routes, 2 local
     per rank) into each rank's BF16 latent partial [8, 64, 3584];
  2. the shared expert 7168 -> 6144 (gate/up, SiLU) -> 7168 into the
     reduce-scatter partial rs [64, 7168];
  3. the rank-order combine of the 8 partials, RMSNorm, and the 3584 -> 7168
     up projection plus rs -> out [64, 7168] (moetail_combine_norm_upproj).

The step is one moetail_decode_tail call (three launches: the finalize, the
gate/up projection forming h with y beside it, the down and up projections
forming rs and out); --tail fused runs it as moetail_finalize then
moetail_tail (the same three launches), --tail calls as moetail_finalize and
the tail's two entry points (eight launches): the same bits every way.

The timed steps replay one HIP graph of G steps on one stream, G the
largest divisor of the step count up to 40 (a replay boundary costs about
8 us of launch, paid once per graph), the two input sets (weights and rows)
alternating so that the 315 MB of weights per step stream from HBM, not
from the 256 MB Infinity Cache.  (--tail calls --streams 2 puts the finalize
on a side stream beside the shared expert: measured slower, the cross-stream
fork and join inside the graph cost more than the overlap gains.)  Inputs
are resident in HBM before the timed region starts.

The line's roofline object is the step's dominant kernel, its gate/up launch
(the gate/up projection forming h, the latent norm's y beside it), timed
alone with HIP events through moetail_gate_up; every entry point's time and
fraction (the gate/up projection's split-K stage alone among them), the
per-config kernels, the targets, a same-size device copy and the CPU
oracle's rate (on all of this process's host threads and on one) ride along.
Rank 0 prints one JSON line (progress goes to stderr).
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

B, P, TP, K = 64, 3584, 8, 16
H, I = 7168, 6144
HBM_PEAK_GBPS = 8000.0
METRIC = "MoE-tail tokens/s and achieved HBM GB/s (% peak) at b=64, P=3584"
MAX_GRAPH_STEPS = 40  # most steps per captured graph


def graph_steps(steps: int) -> int:
    """Steps per captured graph: the largest divisor of the step count up to
    MAX_GRAPH_STEPS, so that every timed step sits in a graph of that size
    (a decode loop holds many layers' tails in one graph; a replay boundary
    costs about 8 us of launch, paid once per graph)."""
    return max(g for g in range(1, min(steps, MAX_GRAPH_STEPS) + 1) if steps % g == 0)


# HBM bytes of one launch of the dominant kernel -- the step's gate/up launch
# at b=64 (moetail_gate_up with y) -- from two rocprofv3 --pmc passes over
# `bench.py --counters` (FETCH_SIZE, then WRITE_SIZE, per dispatch, that
# call's dispatches averaged), scaled by what each reads for the calibration
# kernel (256 MiB in, 256 MiB out: FETCH_SIZE x 2.0, WRITE_SIZE x 1.0).
# They hold for the kernel sources with this digest only (None: not taken
# for these sources).
TRAFFIC = dict(source_digest="1d2d1e8c1dd4ef36", fetch_bytes=93308 * 2 * 1024,
               write_bytes=7420 * 1024)


def kernel_source_digest():
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "expert_finalize_rmsnorm_amd", "csrc")
    # the sources of the fused tail's kernels and of its launch plans
    for name in ("common.h", "kernels.h", "norm_device.h", "project.hip", "api.hip"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes():
    """Bytes each call must move at least (inputs read once, outputs written
    once), per entry point of the step."""
    fin = TP * (B * K // TP) * P * 2 + TP * B * K * 4 + B * K * 4 + P * 2 + TP * B * P * 2
    shared = 3 * H * I * 2 + B * H * 2 + B * H * 2
    upproj = TP * B * P * 2 + P * 2 + H * P * 2 + B * H * 2 + B * H * 2
    # the gate/up projection's split-K stage: its two weight matrices and x
    # (its FP32 partials are an artifact of the split, not counted)
    gate_up = 2 * I * H * 2 + B * H * 2
    # the step's gate/up launch (moetail_gate_up with y): the stage's bytes,
    # h out, and the latent norm's partials and gamma in, y out
    gate_up_h = gate_up + B * I * 2 + TP * B * P * 2 + P * 2 + B * P * 2
    return dict(finalize=fin, shared_expert=shared, combine_norm_upproj=upproj,
                tail=shared + upproj - B * H * 2 * 2, gate_up_stage=gate_up,
                gate_up_h=gate_up_h)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernels", action="store_true", help="skip the per-config kernel table")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="end with two launches of a plain elementwise kernel over 256 MiB "
                         "(reads 256 MiB, writes 256 MiB): the scale for HBM byte counters")
    ap.add_argument("--tail", choices=("decode", "fused", "calls"), default="decode",
                    help="decode: the whole step as one moetail_decode_tail call; "
                         "fused: moetail_finalize, then the shared expert and "
                         "combine+norm+upproj as one moetail_tail call; calls: "
                         "moetail_finalize and the tail's two entry points")
    ap.add_argument("--weights", choices=("tiled", "rows"), default="tiled",
                    help="tiled: the projections read weights packed once by "
                         "moetail_pack_weights; rows: row-major weights")
    ap.add_argument("--streams", type=int, choices=(1, 2), default=1,
                    help="2: the finalize on a side stream beside the shared expert; "
                         "1: the three calls in order on one stream")
    ap.add_argument("--counters", action="store_true",
                    help="for rocprofv3 counter passes: a few eager calls of each workload (the "
                         "decode step at b=64; finalize+combine b=64; expert TP b=128; combine+"
                         "norm+up projection b=32; shared expert b=32 and 128), then two "
                         "launches of the 256 MiB calibration kernel; no timing, no JSON line")
    ap.add_argument("--cpu-baseline-child", action="store_true", help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.cpu_baseline_child:
        cpu_baseline_child()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the tp rank partials are a resident buffer on one device).", file=sys.stderr)
        sys.exit(2)
    # The CPU baseline runs in a child process, started before the GPU is
    # touched and idle until the GPU timing is done: its OpenMP threads end
    # with it, and nothing of it outlives this process.
    child = None
    if not args.no_cpu_baseline and not args.counters:
        child = subprocess.Popen([sys.executable, os.path.abspath(__file__),
                                  "--cpu-baseline-child"], stdin=subprocess.PIPE,
                                 stdout=subprocess.PIPE, text=True)

    import torch

    import expert_finalize_rmsnorm_amd as mt
    import workloads
    from tests.gpu_util import dev

    torch.cuda.set_device(0)
    nsets = 2
    log("drawing inputs")
    sets = []
    for s in range(nsets):
        ep = workloads.ep_finalize(s, b=B, K=K, P=P, tp=TP)
        up = workloads.upproj(s, b=B, tp=TP, L=P, N=H)
        sh = workloads.shared(s, b=B, H=H, I=I)
        # the weights as the projections read them: row-major, or packed
        # once (at load time, outside every timed region) into the tiled
        # layout
        wl = (lambda a: mt.pack_weights(dev(a))) if args.weights == "tiled" else dev
        d = dict(rows=dev(ep["rows"]), idx=dev(ep["idx"]), w=dev(ep["w32"]),
                 gamma=dev(ep["gamma"]), x=dev(sh["x"]), wg=wl(sh["w_gate"]),
                 wu=wl(sh["w_up"]), wd=wl(sh["w_down"]), lgamma=dev(up["gamma"]),
                 w_up=wl(up["w_up"]),
                 lat=torch.empty((TP, B, P), dtype=torch.int16, device="cuda"),
                 rs=torch.empty((B, H), dtype=torch.int16, device="cuda"),
                 out=torch.empty((B, H), dtype=torch.int16, device="cuda"),
                 ws_sh=mt.new_workspace(mt.OP_SHARED_EXPERT, B, H, I),
                 ws_up=mt.new_workspace(mt.OP_COMBINE_NORM_UPPROJ, B, P, H, TP),
                 ws_tail=mt.new_workspace(mt.OP_TAIL, B, P, H, I))
        sets.append(d)
    torch.cuda.synchronize()

    def finalize(d):
        mt.moetail_finalize(d["rows"], d["idx"], d["w"], d["gamma"], 1.0, 1e-6, True,
                            partials=d["lat"])

    lay = mt.W_TILED if args.weights == "tiled" else mt.W_ROWS

    def shared(d):
        mt.moetail_shared_expert(d["x"], d["wg"], d["wu"], d["wd"], d["rs"], workspace=d["ws_sh"],
                                 w_layout=lay)

    def upproj(d):
        mt.moetail_combine_norm_upproj(d["lat"], d["lgamma"], 1e-6, d["w_up"], d["out"],
                                       rs=d["rs"], workspace=d["ws_up"], w_layout=lay)

    def tail(d):
        mt.moetail_tail(d["lat"], d["lgamma"], 1e-6, d["w_up"], d["x"], d["wg"], d["wu"], d["wd"],
                        d["out"], rs=d["rs"], workspace=d["ws_tail"], w_layout=lay)

    side = torch.cuda.Stream()

    def decode(d):
        mt.moetail_decode_tail(d["rows"], d["idx"], d["w"], d["gamma"], 1.0, 1e-6, True, d["lat"],
                               d["lgamma"], 1e-6, d["w_up"], d["x"], d["wg"], d["wu"], d["wd"],
                               d["out"], rs=d["rs"], workspace=d["ws_tail"], w_layout=lay)

    def step(d):
        """finalize runs on a side stream beside the shared expert; the up
        projection waits for both (a fork/join inside the captured graph)."""
        if args.tail == "decode":
            decode(d)
            return
        if args.tail == "fused":
            finalize(d)
            tail(d)
            return
        if args.streams == 1:
            finalize(d)
            shared(d)
            upproj(d)
            return
        main = torch.cuda.current_stream()
        fork, join = torch.cuda.Event(), torch.cuda.Event()
        fork.record(main)
        with torch.cuda.stream(side):
            side.wait_event(fork)
            finalize(d)
            join.record(side)
        shared(d)
        main.wait_event(join)
        upproj(d)

    if args.counters:
        counter_workloads(sets, step, log, mt.W_TILED if args.weights == "tiled" else mt.W_ROWS)
        return

    log("capturing the step graph")
    for d in sets:
        step(d)  # eager once before capture
    torch.cuda.synchronize()
    # One graph of G steps, the input sets alternating; the timed region
    # replays it steps / G times (G divides the step count).
    G = graph_steps(args.steps)
    cap = torch.cuda.Stream()
    many = torch.cuda.CUDAGraph()
    with torch.cuda.graph(many, stream=cap):
        for i in range(G):
            step(sets[i % nsets])
    torch.cuda.synchronize()

    def run_steps(n):
        for _ in range((n + G - 1) // G):
            many.replay()

    log(f"warmup {args.warmup}, timed {args.steps} steps")
    run_steps(args.warmup)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    run_steps(args.steps)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    tokens_per_s = B / (ms_per_step * 1e-3)
    algo0 = algorithmic_bytes()
    step_bytes = algo0["finalize"] + algo0["shared_expert"] + algo0["combine_norm_upproj"]
    log(f"step {ms_per_step * 1e3:.1f} us wall, {gpu_ms * 1e3:.1f} us GPU events")

    # Per entry point: a HIP graph of back-to-back calls (rotating the input
    # sets), HIP events around each of 20 replays, the median; the host's
    # launch rate is out of the measurement.
    def time_calls(fn, reps=20):
        return graph_time(lambda i: fn(sets[i % nsets]), reps)

    # The dominant kernel alone: the gate/up projection's split-K stage (one
    # launch of the streamed projection kernel), through its own entry point.
    gu_part = torch.empty(mt.workspace_bytes(mt.OP_PROJECTION, B, 2 * I, H, mt.PROJ_GATEUP) // 4,
                          dtype=torch.float32, device="cuda")

    def gate_up_stage(d):
        mt.moetail_projection_partials(mt.PROJ_GATEUP, d["wg"], d["wu"], d["x"], gu_part,
                                       w_layout=lay)

    # The step's dominant kernel: its gate/up launch (h formed in the launch,
    # y beside it), as its own call.
    gu_ws = mt.new_workspace(mt.OP_GATE_UP, B, H, I)
    gu_h = torch.empty((B, I), dtype=torch.int16, device="cuda")
    gu_y = torch.empty((B, P), dtype=torch.int16, device="cuda")

    def gate_up_h(d):
        mt.moetail_gate_up(d["x"], d["wg"], d["wu"], gu_h, d["lat"], d["lgamma"], 1e-6, gu_y,
                           workspace=gu_ws, w_layout=lay)

    per_call = {n: time_calls(f) for n, f in
                (("finalize", finalize), ("shared_expert", shared),
                 ("combine_norm_upproj", upproj), ("tail", tail),
                 ("gate_up_stage", gate_up_stage), ("gate_up_h", gate_up_h))}
    algo = algorithmic_bytes()
    entry = {n: dict(us=round(per_call[n], 2), bytes=algo[n],
                     GBps=round(algo[n] / per_call[n] / 1e3, 1),
                     frac=round(algo[n] / per_call[n] / 1e3 / HBM_PEAK_GBPS, 4))
             for n in per_call}
    dom = "gate_up_h"
    traffic = traffic_bytes = None
    if TRAFFIC["source_digest"] and kernel_source_digest() == TRAFFIC["source_digest"]:
        traffic_bytes = TRAFFIC["fetch_bytes"] + TRAFFIC["write_bytes"]
        traffic = round(traffic_bytes / per_call[dom] / 1e3, 1)
    roofline = dict(bound="hbm",
                    kernel="px_gateup_fused_kernel<4, 6, 8>: the decode step's gate/up launch at "
                           "b=64 (2 x 6144 x 7168 BF16 weights and x in, h formed in the launch; "
                           "the latent norm's 8 x 64 x 3584 partials in, y out, beside it), one "
                           "launch (moetail_gate_up)",
                    achieved=entry[dom]["GBps"], peak=HBM_PEAK_GBPS, unit="GB/s",
                    frac=entry[dom]["frac"], traffic=traffic, traffic_bytes=traffic_bytes,
                    algorithmic_bytes=algo[dom], us_per_launch=entry[dom]["us"])

    kernels = None
    if not args.no_kernels:
        log("per-config kernel timings")
        kernels = config_kernels(sets[0], log, lay)

    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(2):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log("copy calibration: 2 x neg over 268435456 B in, 268435456 B out")
        del src, dst

    log("copy ceiling")
    ceiling = copy_ceiling(step_bytes)

    cpu = None
    if child is not None:
        log("CPU oracle baseline (child process)")
        out, _ = child.communicate("go\n", timeout=900)
        if child.returncode != 0:
            raise RuntimeError(f"the CPU baseline process failed ({child.returncode})")
        cpu = json.loads(out.strip().splitlines()[-1])

    line = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; shapes and distributions of the pages' workloads)",
        "graph_steps": G,
        "config": {"workload": "MoE decode tail step: EP finalize tp=8 K=16 P=3584 -> shared "
                               "expert 7168x6144 SiLU -> latent combine + RMSNorm + up "
                               "projection 3584->7168 (+rs)",
                   "b": B, "P": P, "tp": TP, "K": K, "H": H, "I": I,
                   "global_batch": B, "tail": args.tail, "streams": args.streams,
                   "weights": args.weights,
                   "parallelism": "one GPU, tp rank partials resident"},
        "gpu_ms_per_step_events": round(gpu_ms, 5),
        "step_algorithmic_bytes": step_bytes,
        "step_GBps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "entry_points": entry,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "copy_ceiling": ceiling,
        "targets": targets_of(kernels),
        "kernels": kernels,
    }
    print(json.dumps(line), flush=True)


def graph_time(fn, reps, replays=20):
    """Microseconds per call of fn(i), i = 0..reps-1: a HIP graph holds the
    reps calls; after one untimed replay, HIP events time `replays` replays
    one by one, and the median replay is taken."""
    import statistics
    import torch
    for i in range(min(reps, 4)):
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        for i in range(reps):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(replays):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) * 1e3 / reps)
    return statistics.median(times)


def config_kernels(base, log, lay):
    """Per-config timings on cold inputs: enough distinct input sets rotate
    that their total exceeds twice the 256 MB Infinity Cache."""
    import numpy as np
    import torch

    import expert_finalize_rmsnorm_amd as mt
    import workloads
    from tests.gpu_util import dev

    gen = torch.Generator("cuda").manual_seed(1234)

    def randn_bf16(shape, std):
        return (torch.randn(shape, device="cuda", generator=gen) * std).to(torch.bfloat16).view(
            torch.int16)

    def timed(fn, nsets, reps=None):
        return graph_time(lambda i: fn(i % nsets), reps or max(2 * nsets, 12))

    res = []

    def add(name, us, nbytes, **extra):
        gbps = nbytes / us / 1e3
        res.append(dict(name=name, us=round(us, 2), bytes=nbytes, GBps=round(gbps, 1),
                        frac=round(gbps / HBM_PEAK_GBPS, 4), **extra))
        log(f"  {name}: {us:.2f} us, {gbps:.0f} GB/s")

    # EP finalize + rank combine at decode scale (the metric's b=64, P=3584)
    rows = [randn_bf16((TP, B * K // TP, P), 2.0) for _ in range(48)]
    part = torch.empty((TP, B, P), dtype=torch.int16, device="cuda")
    out = torch.empty((B, P), dtype=torch.int16, device="cuda")
    fin_in = TP * (B * K // TP) * P * 2 + TP * B * K * 4 + B * K * 4 + P * 2
    for wbn in (True, False):
        us = timed(lambda i: mt.moetail_finalize(rows[i], base["idx"], base["w"], base["gamma"],
                                                 1.0, 1e-6, wbn, partials=part, out=out), 48)
        add(f"finalize+combine b=64 P=3584 tp=8 wbn={int(wbn)}", us,
            fin_in + TP * B * P * 2 + B * P * 2, tokens_per_s=round(B / (us * 1e-6), 1))
    us = timed(lambda i: mt.moetail_finalize(rows[i], base["idx"], base["w"], base["gamma"],
                                             1.0, 1e-6, True, out=out), 48)
    add("finalize+combine b=64, out only (partials not written)", us, fin_in + B * P * 2,
        tokens_per_s=round(B / (us * 1e-6), 1))
    us = timed(lambda i: mt.moetail_finalize(rows[i], base["idx"], base["w"], base["gamma"],
                                             1.0, 1e-6, True, partials=part), 48)
    add("finalize b=64, partials only", us, fin_in + TP * B * P * 2,
        tokens_per_s=round(B / (us * 1e-6), 1))
    # without a per-route norm (the Kimi finalize): partials, and out only
    us = timed(lambda i: mt.moetail_finalize(rows[i], base["idx"], base["w"], None, 0.0, 1e-6,
                                             mt.NO_NORM, partials=part), 48)
    add("finalize, no norm (Kimi) b=64, partials only", us, fin_in - P * 2 + TP * B * P * 2,
        tokens_per_s=round(B / (us * 1e-6), 1))
    us = timed(lambda i: mt.moetail_finalize(rows[i], base["idx"], base["w"], None, 0.0, 1e-6,
                                             mt.NO_NORM, out=out), 48)
    add("finalize+combine, no norm (Kimi) b=64, out only", us, fin_in - P * 2 + B * P * 2,
        tokens_per_s=round(B / (us * 1e-6), 1))
    del rows

    # expert-TP finalize: b=128, K=16, P=7168, tp=8 (235 MB of K-partials)
    g0 = torch.Generator("cpu").manual_seed(0)
    w32, _ = workloads.route_weights(g0, 128, 16)
    tgamma = workloads.normal_bf16(g0, (7168,), 1.0, 0.05)
    idx = torch.from_numpy(np.random.default_rng(0).permutation(2048).astype(np.int32).reshape(
        128, 16)).cuda()
    kp = [randn_bf16((8, 2048, 7168), 0.5) for _ in range(3)]
    tout = torch.empty((128, 7168), dtype=torch.int16, device="cuda")
    w, gamma = dev(w32), dev(tgamma)
    tws = mt.new_workspace(mt.OP_TP_FINALIZE, 128, 16, 7168, 8)
    us = timed(lambda i: mt.moetail_tp_finalize(kp[i], idx, w, gamma, 0.0, 1e-6, False, tout,
                                                workspace=tws), 3, reps=12)
    add("tp_finalize b=128 K=16 P=7168 tp=8", us,
        8 * 2048 * 7168 * 2 + 128 * 16 * 8 + 7168 * 2 + 128 * 7168 * 2,
        tokens_per_s=round(128 / (us * 1e-6), 1))
    del kp

    # latent combine + norm + up projection, b in {1, 8, 32, 64}
    def wl(t):
        return mt.pack_weights(t) if lay == mt.W_TILED else t

    wups = [wl(randn_bf16((H, P), 0.02)) for _ in range(12)]
    for b in (1, 8, 32, 64):
        lat = randn_bf16((TP, b, P), 1.0)
        o = torch.empty((b, H), dtype=torch.int16, device="cuda")
        ws = mt.new_workspace(mt.OP_COMBINE_NORM_UPPROJ, b, P, H, TP)
        us = timed(lambda i: mt.moetail_combine_norm_upproj(lat, base["lgamma"], 1e-6, wups[i], o,
                                                            workspace=ws, w_layout=lay), 12)
        add(f"combine_norm_upproj b={b}", us, H * P * 2 + TP * b * P * 2 + P * 2 + b * H * 2,
            weight_roofline_us=round(H * P * 2 / HBM_PEAK_GBPS / 1e3, 2))
    del wups

    # shared expert, b in {16, 32, 64, 128}
    ws_sets = [(wl(randn_bf16((I, H), 0.02)), wl(randn_bf16((I, H), 0.02)),
                wl(randn_bf16((H, I), 0.02))) for _ in range(2)]
    for b in (16, 32, 64, 128):
        x = randn_bf16((b, H), 1.0)
        rs = torch.empty((b, H), dtype=torch.int16, device="cuda")
        ws = mt.new_workspace(mt.OP_SHARED_EXPERT, b, H, I)
        us = timed(lambda i: mt.moetail_shared_expert(x, *ws_sets[i], rs, workspace=ws,
                                                      w_layout=lay), 2, reps=12)
        add(f"shared_expert b={b}", us, 3 * H * I * 2 + 2 * b * H * 2,
            weight_roofline_us=round(3 * H * I * 2 / HBM_PEAK_GBPS / 1e3, 2))
    return res


def counter_workloads(sets, step, log, lay, reps=2):
    """Eager calls of every workload, reps each, for counter passes (each
    dispatch is its own row in rocprofv3's output): the decode step (five
    kernels), then each workload of the per-config table once more."""
    import numpy as np
    import torch

    import expert_finalize_rmsnorm_amd as mt
    import workloads
    from tests.gpu_util import dev

    base = sets[0]
    for i in range(reps):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()
    log(f"counters: {reps} decode steps")
    gu_part = torch.empty(mt.workspace_bytes(mt.OP_PROJECTION, B, 2 * I, H, mt.PROJ_GATEUP) // 4,
                          dtype=torch.float32, device="cuda")
    for _ in range(reps):
        mt.moetail_projection_partials(mt.PROJ_GATEUP, base["wg"], base["wu"], base["x"], gu_part,
                                       w_layout=lay)
    gws = mt.new_workspace(mt.OP_GATE_UP, B, H, I)
    gh = torch.empty((B, I), dtype=torch.int16, device="cuda")
    gy = torch.empty((B, P), dtype=torch.int16, device="cuda")
    for _ in range(reps):
        mt.moetail_gate_up(base["x"], base["wg"], base["wu"], gh, base["lat"], base["lgamma"],
                           1e-6, gy, workspace=gws, w_layout=lay)
    part = torch.empty((TP, B, P), dtype=torch.int16, device="cuda")
    out = torch.empty((B, P), dtype=torch.int16, device="cuda")
    for _ in range(reps):
        mt.moetail_finalize(base["rows"], base["idx"], base["w"], base["gamma"], 1.0, 1e-6, True,
                            partials=part, out=out)
    g0 = torch.Generator("cpu").manual_seed(0)
    w32, _ = workloads.route_weights(g0, 128, 16)
    tgamma = workloads.normal_bf16(g0, (7168,), 1.0, 0.05)
    idx = torch.from_numpy(np.random.default_rng(0).permutation(2048).astype(np.int32).reshape(
        128, 16)).cuda()
    gen = torch.Generator("cuda").manual_seed(1234)
    kp = (torch.randn((8, 2048, 7168), device="cuda", generator=gen) * 0.5).to(
        torch.bfloat16).view(torch.int16)
    tout = torch.empty((128, 7168), dtype=torch.int16, device="cuda")
    tws = mt.new_workspace(mt.OP_TP_FINALIZE, 128, 16, 7168, 8)
    for _ in range(reps):
        mt.moetail_tp_finalize(kp, idx, dev(w32), dev(tgamma), 0.0, 1e-6, False, tout,
                               workspace=tws)
    del kp
    for b in (8, 32):  # (b = 8: the block-local kernel, one launch after the norm)
        lat = torch.randn((TP, b, P), device="cuda", generator=gen).to(torch.bfloat16).view(
            torch.int16)
        o = torch.empty((b, H), dtype=torch.int16, device="cuda")
        ws = mt.new_workspace(mt.OP_COMBINE_NORM_UPPROJ, b, P, H, TP)
        for _ in range(reps):
            mt.moetail_combine_norm_upproj(lat, base["lgamma"], 1e-6, base["w_up"], o,
                                           workspace=ws, w_layout=lay)
    for b in (32, 128):
        x = torch.randn((b, H), device="cuda", generator=gen).to(torch.bfloat16).view(torch.int16)
        rs = torch.empty((b, H), dtype=torch.int16, device="cuda")
        ws = mt.new_workspace(mt.OP_SHARED_EXPERT, b, H, I)
        for _ in range(reps):
            mt.moetail_shared_expert(x, base["wg"], base["wu"], base["wd"], rs, workspace=ws,
                                     w_layout=lay)
    torch.cuda.synchronize()
    src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(2):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log("counters: gate/up stage b=64, gate/up + y b=64, finalize+combine b=64, expert TP b=128, "
        "combine+norm+upproj b=8 and b=32, shared expert b=32 and b=128, calibration 2 x neg "
        "over 256 MiB in, 256 MiB out")


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def host_threads():
    """The threads this process may use: the host's CPUs, capped by the
    OpenMP thread setting where one is given (on a shared GPU host that is
    this GPU's share of the cores)."""
    n = os.cpu_count() or 1
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return n


def cpu_baseline_child():
    """The CPU baseline's process: waits for a line "go" on stdin (the
    parent's GPU timing done; end of input: exit at once), draws input set 0
    as the parent does, times the oracle and prints the result as one JSON
    line."""
    if sys.stdin.readline().strip() != "go":
        return
    import workloads
    host = (workloads.ep_finalize(0, b=B, K=K, P=P, tp=TP),
            workloads.upproj(0, b=B, tp=TP, L=P, N=H), workloads.shared(0, b=B, H=H, I=I))
    print(json.dumps(cpu_baseline(host, log)), flush=True)


def cpu_baseline(host_inputs, log, seconds=(8.0, 10.0)):
    """The oracle (as it stands) on the step's full b=64 batch on host cores:
    whole steps repeated until the time given has passed, once on one thread
    and once on host_threads() threads (the results do not depend on the
    thread count)."""
    import oracle
    ep, up, sh = host_inputs

    def run(threads, min_seconds):
        steps = 0
        t0 = time.perf_counter()
        while True:
            lat, _ = oracle.finalize(ep["rows"], ep["idx"], ep["w32"], ep["gamma"], 1.0, 1e-6,
                                     True, combine=False, nthreads=threads)
            _, rs = oracle.shared_expert(sh["x"], sh["w_gate"], sh["w_up"], sh["w_down"],
                                         nthreads=threads)
            oracle.combine_norm_upproj(lat, up["gamma"], 1e-6, up["w_up"], rs, nthreads=threads)
            steps += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds:
                return steps, dt

    n = host_threads()
    s1, t1 = run(1, seconds[0])
    log(f"oracle: {s1} steps in {t1:.2f} s on 1 thread")
    sn, tn = run(n, seconds[1])
    log(f"oracle: {sn} steps in {tn:.2f} s on {n} threads")
    return {"value": round(sn * B / tn, 2), "unit": "tokens/s", "cores": n, "kind": "oracle",
            "sample": f"{sn} full b={B} steps (finalize, shared expert, combine+norm+upproj) of "
                      f"input set 0, {tn:.2f} s wall on {n} threads",
            "single_thread": {"value": round(s1 * B / t1, 2), "unit": "tokens/s", "cores": 1,
                              "sample": f"{s1} full b={B} steps, {t1:.2f} s wall on 1 thread"},
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model()}


def copy_ceiling(nbytes, reps=10):
    """A device-to-device copy of nbytes (read nbytes, write nbytes), HIP
    events around replays of a graph of reps copies (the median): the bandwidth a
    plain copy reaches on this GPU, as the practical ceiling beside the
    8 TB/s peak."""
    import torch
    n = nbytes // 2
    src = [torch.empty(n, dtype=torch.int16, device="cuda").fill_(1) for _ in range(2)]
    dst = torch.empty(n, dtype=torch.int16, device="cuda")
    us = graph_time(lambda i: dst.copy_(src[i % 2]), reps)
    del src, dst
    return {"bytes_copied": n * 2, "us": round(us, 2),
            "GBps_read_plus_write": round(2 * n * 2 / us / 1e3, 1)}


def targets_of(kernels):
    """Each workload's figure against its target (finalize and combine: at
    least 70% of the 8 TB/s peak; the up projection and the shared expert at
    b=32: at least 60% of the weight-streaming roofline)."""
    if not kernels:
        return None
    by = {k["name"]: k for k in kernels}
    res = []

    def frac_target(name, key):
        k = by.get(key)
        if k:
            res.append(dict(name=name, measured_frac=k["frac"], target_frac=0.70,
                            us=k["us"], met=k["frac"] >= 0.70))

    def time_target(name, key, roof_us):
        k = by.get(key)
        if k:
            res.append(dict(name=name, us=k["us"], target_us=round(roof_us / 0.6, 2),
                            measured_frac=round(roof_us / k["us"], 4), target_frac=0.60,
                            met=k["us"] <= roof_us / 0.6))

    frac_target("EP finalize + combine (b=64, partials and out)",
                "finalize+combine b=64 P=3584 tp=8 wbn=1")
    frac_target("EP finalize, partials only (b=64)", "finalize b=64, partials only")
    frac_target("expert-TP finalize (b=128, P=7168)", "tp_finalize b=128 K=16 P=7168 tp=8")
    time_target("combine + norm + up projection b=32", "combine_norm_upproj b=32",
                H * P * 2 / HBM_PEAK_GBPS / 1e3)
    time_target("shared expert b=32", "shared_expert b=32", 3 * H * I * 2 / HBM_PEAK_GBPS / 1e3)
    return res


if __name__ == "__main__":
    main()
