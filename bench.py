#!/usr/bin/env python3
"""Throughput of the seven-estimator scan path on one MI355X.

Workload: num_envs = 4096, seq_len = 128, fp32 (the pages' headline shape).
One step = every estimator once without truncations (prefix sum in fp32) and
the five truncating estimators once more with truncations: 12 library calls,
each one pass over its [4096, 128] inputs.

Inputs sit in HBM before timing starts.  The batch is replicated R times
(>= 1 GiB in all, four times the 256 MB Infinity Cache) and step k uses
replica k mod R, so every call reads its inputs from HBM rather than from a
cache ("cold"); --warm reuses one replica.  Each replica's 12 calls are
captured once into a HIP graph (torch.cuda.CUDAGraph), so the timed loop is
K graph replays and host launch overhead stays off the critical path.

Prints one JSON line.  value = 12 * num_envs * seq_len / step time (Gelem/s).
roofline: the call with the longest average duration, its algorithmic bytes
(one read of every input stream, one write of every output) over its
average duration, measured with HIP events around a graph of R back-to-back
launches of that call on the launch stream.
cpu_baseline: the fp64 oracle on the host cores, full steps on the same batch.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Gelem/s + HBM GB/s (% peak), 7 estimators, 4096 envs×T=128..131072"
HBM_PEAK_GBPS = 8000.0
WORKLOAD = "all7_4096x128"
BACKWARD = ("gae", "vtrace", "retrace", "lambda_returns", "discounted_returns")
CALLS = [("gae", False), ("vtrace", False), ("retrace", False), ("lambda_returns", False),
         ("discounted_returns", False), ("eligibility_traces", False), ("prefix_sum_f32", False),
         ("gae", True), ("vtrace", True), ("retrace", True), ("lambda_returns", True),
         ("discounted_returns", True)]
# bytes per element: one read of each dense input, one write of each output
DENSE_BYTES = {"gae": 13, "vtrace": 21, "retrace": 21, "lambda_returns": 13,
               "discounted_returns": 9, "eligibility_traces": 9, "prefix_sum_f32": 9}


def key(est, trunc):
    return est + ("+trunc" if trunc else "")


def alg_bytes(est, trunc, n, t):
    """One read of each input stream and one write of each output:
    DENSE_BYTES per element, plus 5 B per element with truncations (the
    uint8 mask and the fp32 trunc_values), plus 4 B of bootstrap per env."""
    b = DENSE_BYTES[est] * n * t
    if trunc:
        b += 5 * n * t
    if est in BACKWARD:
        b += 4 * n
    return b


def make_call(lrs, est, trunc, D, O, g, lam):
    kg = dict(truncateds=D["truncateds"] if trunc else None,
              trunc_values=D["trunc_values"] if trunc else None,
              bootstrap_value=D["bootstrap_value"])
    k = key(est, trunc)
    if est == "gae":
        return lambda: lrs.compute_gae(D["rewards"], D["values"], D["terminateds"], g, lam,
                                       out=O[k], **kg)
    if est == "vtrace":
        return lambda: lrs.compute_vtrace(D["log_rhos"], D["rewards"], D["values"],
                                          D["terminateds"], g, lam, rho_bar=1.0, c_bar=1.0,
                                          out=(O[k], O[k + "/pg"]), **kg)
    if est == "retrace":
        return lambda: lrs.compute_retrace(D["log_rhos"], D["rewards"], D["q_values"], D["values"],
                                           D["terminateds"], g, lam, c_bar=1.0, out=O[k], **kg)
    if est == "lambda_returns":
        return lambda: lrs.compute_lambda_returns(D["rewards"], D["values"], D["terminateds"], g,
                                                  lam, out=O[k], **kg)
    if est == "discounted_returns":
        return lambda: lrs.compute_discounted_returns(D["rewards"], D["terminateds"], g, out=O[k],
                                                      **kg)
    if est == "eligibility_traces":
        return lambda: lrs.compute_eligibility_traces(D["x"], D["dones"], g, lam, out=O[k])
    if est == "prefix_sum_f32":
        return lambda: lrs.compute_episodic_prefix_sum(D["x"], D["dones"], out=O[k])
    raise KeyError(est)


def cpu_baseline(ro, seconds):
    import oracle
    a = ro.arrays
    g, lam = ro.gamma, ro.lambda_
    kt = dict(truncateds=a["truncateds"], trunc_values=a["trunc_values"],
              bootstrap_value=a["bootstrap_value"])
    kn = dict(bootstrap_value=a["bootstrap_value"])

    def step():
        for kk in (kn, kt):
            oracle.gae(a["rewards"], a["values"], a["terminateds"], g, lam, **kk)
            oracle.vtrace(a["log_rhos"], a["rewards"], a["values"], a["terminateds"], g, lam, **kk)
            oracle.retrace(a["log_rhos"], a["rewards"], a["q_values"], a["values"],
                           a["terminateds"], g, lam, **kk)
            oracle.lambda_returns(a["rewards"], a["values"], a["terminateds"], g, lam, **kk)
            oracle.discounted_returns(a["rewards"], a["terminateds"], g, **kk)
        oracle.eligibility_traces(a["x"], a["dones"], g, lam)
        oracle.prefix_sum(a["x"], a["dones"])

    step()  # warm-up (also builds/loads the library)
    n, t0 = 0, time.perf_counter()
    while True:
        step()
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    elems = n * len(CALLS) * ro.num_envs * ro.seq_len
    return {"value": round(elems / el / 1e9, 4), "unit": "Gelem/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"{n} full steps (12 calls each) of the {ro.num_envs}x{ro.seq_len} batch, "
                      f"{el:.1f} s, fp64 sequential recursion, OpenMP over envs"}


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "hbm_traffic_all7_4096x128.md")
CALIBRATION_BYTES = 64 << 20  # one --calibrate-copy dispatch reads and writes this much


def source_hash():
    """sha256 of the kernel sources: counters taken on other sources are stale."""
    import hashlib
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "linear_recurrence_scan_env_amd", "csrc")
    for f in sorted(os.listdir(pkg)) + ["../../include/lrs.h"]:
        with open(os.path.join(pkg, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def call_of_kernel(name):
    """Map a demangled kernel name to a bench call key."""
    ops = {"GaeOp": "gae", "VtraceOp": "vtrace", "RetraceOp": "retrace",
           "LambdaOp": "lambda_returns", "DiscOp": "discounted_returns",
           "EligOp": "eligibility_traces", "PrefixF32Op": "prefix_sum_f32",
           "PrefixI32Op": "prefix_sum_i32"}
    for op, est in ops.items():
        if f"lrs::{op}<" in name:
            return key(est, ", true>" in name.split(op, 1)[1][:12])
    return None


def summarize_stats(csv_path, command):
    import csv
    rows = list(csv.DictReader(open(csv_path)))
    out = ["# rocprofv3 kernel statistics: seven estimators at 4096 x 128", "",
           "Command:", "", "```", command, "```", "",
           "| kernel | call | dispatches | avg us | min us | max us |", "|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{r['Name'].split('(')[0]}` | {call_of_kernel(r['Name']) or '-'} | "
                   f"{r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} | "
                   f"{float(r['MinNs']) / 1e3:.3f} | {float(r['MaxNs']) / 1e3:.3f} |")
    print("\n".join(out))


def summarize_counters(fetch_csv, write_csv, command_fetch, command_write):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) scaled by what the same
    counters read for the calibration copy of CALIBRATION_BYTES."""
    import csv
    import collections

    def load(path):
        per = collections.defaultdict(list)
        calib = []
        for r in csv.DictReader(open(path)):
            v = float(r["Counter_Value"]) * 1024.0
            k = call_of_kernel(r["Kernel_Name"])
            if k:
                per[k].append(v)
            elif "copyBuffer" in r["Kernel_Name"] and int(r["Grid_Size"]) == CALIBRATION_BYTES // 512:
                calib.append(v)
        return per, calib

    fetch, fcal = load(fetch_csv)
    write, wcal = load(write_csv)
    ff = CALIBRATION_BYTES / (sum(fcal) / len(fcal))
    wf = CALIBRATION_BYTES / (sum(wcal) / len(wcal))
    n, t = 4096, 128
    out = ["# HBM traffic per launch: seven estimators at 4096 x 128 (cold inputs)", "",
           "Commands (one counter per pass):", "", "```", command_fetch, command_write, "```", "",
           f"Calibration: a device copy of {CALIBRATION_BYTES >> 20} MiB reads FETCH_SIZE "
           f"{sum(fcal) / len(fcal) / 1024:.1f} KiB and WRITE_SIZE {sum(wcal) / len(wcal) / 1024:.1f} KiB "
           f"per dispatch, so the scale factors are fetch x{ff:.4f}, write x{wf:.4f}.", "",
           "| call | FETCH KiB (raw) | WRITE KiB (raw) | traffic bytes (scaled) | algorithmic bytes | traffic / algorithmic |",
           "|---|---|---|---|---|---|"]
    data = {}
    for k in fetch:
        fr = sum(fetch[k]) / len(fetch[k])
        wr = sum(write[k]) / len(write[k])
        traffic = int(round(fr * ff + wr * wf))
        est, tr = k.split("+")[0], k.endswith("+trunc")
        ab = alg_bytes(est, tr, n, t)
        data[k] = traffic
        out.append(f"| {k} | {fr / 1024:.1f} | {wr / 1024:.1f} | {traffic} | {ab} | {traffic / ab:.3f} |")
    out += ["", "Machine-readable (read by bench.py; valid only for these kernel sources):", "",
            f"source_sha256: {source_hash()}",
            "traffic_bytes: " + json.dumps(data, sort_keys=True)]
    print("\n".join(out))


def committed_traffic(call):
    """Scaled HBM bytes per launch of `call` from the committed counter
    summary, or None when it is missing or was taken on other sources."""
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    sha = traffic = None
    for line in text.splitlines():
        if line.startswith("source_sha256:"):
            sha = line.split(":", 1)[1].strip()
        if line.startswith("traffic_bytes:"):
            traffic = json.loads(line.split(":", 1)[1])
    if sha != source_hash() or not traffic:
        return None
    return traffic.get(call)


def run_eager(args, lrs, reps, R, N, T, g, lam, stream, dev):
    """Counter-collection mode: the same calls, launched one by one."""
    import torch
    calls = [[make_call(lrs, e, tr, D, O, g, lam) for e, tr in CALLS] for D, O in reps]
    with torch.cuda.stream(stream):
        for k in range(args.warmup + args.steps):
            for f in calls[k % R]:
                f()
        torch.cuda.synchronize()
    print(json.dumps({"mode": "eager", "steps": args.steps, "warmup": args.warmup,
                      "workload": WORKLOAD, "replicas": R}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--replicas", type=int, default=0, help="0: enough for >= 1 GiB")
    ap.add_argument("--warm", action="store_true", help="one replica: cache-resident inputs")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--roofline-reps", type=int, default=20)
    ap.add_argument("--eager", action="store_true",
                    help="launch calls one by one instead of replaying HIP graphs "
                         "(for counter collection)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run 5 device copies of a 64 MiB tensor: a kernel of known "
                         "HBM traffic for scaling FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--summarize-stats", nargs=2, metavar=("CSV", "COMMAND"),
                    help="print a markdown summary of a rocprofv3 kernel_stats.csv")
    ap.add_argument("--summarize-counters", nargs=4,
                    metavar=("FETCH_CSV", "WRITE_CSV", "FETCH_COMMAND", "WRITE_COMMAND"),
                    help="print the HBM-traffic summary of two rocprofv3 --pmc runs")
    args = ap.parse_args()

    if args.summarize_stats:
        return summarize_stats(*args.summarize_stats)
    if args.summarize_counters:
        return summarize_counters(*args.summarize_counters)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(sharding over environments needs no communication; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import linear_recurrence_scan_env_amd as lrs
    from linear_recurrence_scan_env_amd import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lrs.load()

    p = workloads.WORKLOADS[WORKLOAD]
    N, T = p["num_envs"], p["seq_len"]
    ro = workloads.rollout(N, T, seed=0, term_p=p["term_p"], trunc_p=p["trunc_p"],
                           gamma=p["gamma"], lambda_=p["lambda_"], done_p=p["term_p"],
                           streams=["rewards", "values", "q_values", "log_rhos", "terminateds",
                                    "truncateds", "trunc_values", "bootstrap_value", "x", "dones"])
    g, lam = ro.gamma, ro.lambda_

    host = {k: torch.from_numpy(v) for k, v in ro.arrays.items()}
    per_rep = sum(v.numel() * v.element_size() for v in host.values()) + 13 * N * T * 4
    R = 1 if args.warm else (args.replicas or max(8, -(-(1 << 30) // per_rep)))
    reps = []
    for _ in range(R):
        D = {k: v.to(dev) for k, v in host.items()}
        O = {}
        for est, tr in CALLS:
            O[key(est, tr)] = torch.empty(N, T, device=dev)
            if est == "vtrace":
                O[key(est, tr) + "/pg"] = torch.empty(N, T, device=dev)
        reps.append((D, O))

    stream = torch.cuda.Stream(dev)
    if args.calibrate_copy:
        src = torch.ones(16 << 20, device=dev)
        dst = torch.empty_like(src)
        with torch.cuda.stream(stream):
            for _ in range(5):
                dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.eager:
        return run_eager(args, lrs, reps, R, N, T, g, lam, stream, dev)
    with torch.cuda.stream(stream):
        # Eager warm-up on the capture stream (allocates its workspace outside capture).
        for D, O in reps[:2]:
            for est, tr in CALLS:
                make_call(lrs, est, tr, D, O, g, lam)()
        stream.synchronize()

        def capture(fns):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=stream):
                for f in fns:
                    f()
            return gr

        step_graphs = [capture([make_call(lrs, e, tr, D, O, g, lam) for e, tr in CALLS])
                       for D, O in reps]
        call_graphs = {key(e, tr): capture([make_call(lrs, e, tr, D, O, g, lam) for D, O in reps])
                       for e, tr in CALLS}
        torch.cuda.synchronize()

        # ---- timed steps
        for k in range(args.warmup):
            step_graphs[k % R].replay()
        torch.cuda.synchronize()
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        t_start.record(stream)
        for k in range(args.steps):
            step_graphs[k % R].replay()
        t_end.record(stream)
        torch.cuda.synchronize()
        ms_per_step = t_start.elapsed_time(t_end) / args.steps

        # ---- per-call average launch duration (graph of R launches, events around it)
        per_call = {}
        for e, tr in CALLS:
            k_ = key(e, tr)
            call_graphs[k_].replay()
            ev0 = torch.cuda.Event(enable_timing=True)
            ev1 = torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            for _ in range(args.roofline_reps):
                call_graphs[k_].replay()
            ev1.record(stream)
            torch.cuda.synchronize()
            us = ev0.elapsed_time(ev1) * 1e3 / (args.roofline_reps * R)
            b = alg_bytes(e, tr, N, T)
            per_call[k_] = {"us": round(us, 3), "alg_bytes": b, "GBps": round(b / us / 1e3, 1)}

    elems_per_step = len(CALLS) * N * T
    value = elems_per_step / (ms_per_step * 1e-3) / 1e9
    dom = max(per_call, key=lambda k_: per_call[k_]["us"])
    achieved = per_call[dom]["GBps"]
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "Gelem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "num_envs": N, "seq_len": T, "calls_per_step": len(CALLS),
                   "cache": "warm" if args.warm else "cold", "replicas": R,
                   "launch": "hip graph per step"},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": committed_traffic(dom),
                     "alg_bytes": per_call[dom]["alg_bytes"]},
        "per_call": per_call,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(ro, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
