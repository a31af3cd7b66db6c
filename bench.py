#!/usr/bin/env python3
"""Throughput of the scan path on one MI355X.

Default workload (the pages' headline shape): num_envs = 4096, seq_len = 128,
fp32.  One step = every estimator once without truncations (prefix sum in
fp32) and the five truncating estimators once more with truncations: 12
library calls, each one pass over its [4096, 128] inputs.  --workload picks
one of the other benchmark workloads (their steps are listed in WORKLOADS).

Inputs sit in HBM before timing starts.  Each workload's batch is replicated
R times (>= 1 GiB in all, four times the 256 MB Infinity Cache) and step k
uses replica k mod R, so every call reads its inputs from HBM rather than
from a cache ("cold"); --warm reuses one replica.  The calls are captured
into HIP graphs (torch.cuda.CUDAGraph) of G consecutive steps each (G = 1 for
steps of 24 or more calls, more for short steps), so the timed loop is K / G
graph replays and host launch overhead stays off the critical path.

Prints one JSON line.  value = elements processed per step / step time
(Gelem/s).  roofline: the call with the longest average duration, its
algorithmic bytes (one read of every input stream, one write of every
output) over its average duration, measured with HIP events around a graph
of >= 64 back-to-back launches of that call (cycling over its replicas) on
the launch stream; copy_same_bytes times a plain device copy of the same
bytes the same way, for context.  cpu_baseline:
the fp64 oracle on the host cores, whole steps on the same batch.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Gelem/s + HBM GB/s (% peak), 7 estimators, 4096 envs×T=128..131072"
HBM_PEAK_GBPS = 8000.0
BACKWARD = ("gae", "vtrace", "retrace", "lambda_returns", "discounted_returns")
ALL7 = [("gae", False), ("vtrace", False), ("retrace", False), ("lambda_returns", False),
        ("discounted_returns", False), ("eligibility_traces", False), ("prefix_sum_f32", False),
        ("gae", True), ("vtrace", True), ("retrace", True), ("lambda_returns", True),
        ("discounted_returns", True)]
# workload -> the calls of one step: (estimator, with truncations, num_envs, seq_len)
WORKLOADS = {
    "all7_4096x128": [(e, tr, 4096, 128) for e, tr in ALL7],
    "gae_64x512": [("gae", False, 64, 512)],
    "long_64x131072": [(e, True, 64, 131072) for e in ("gae", "vtrace", "retrace")],
    # all seven estimators on the long rows (the 12 calls of all7_4096x128)
    "all7_64x131072": [(e, tr, 64, 131072) for e, tr in ALL7],
    "sweep_4096xT": [(e, False, 4096, t) for t in (32, 128, 512, 2048, 8192)
                     for e in ("discounted_returns", "lambda_returns", "eligibility_traces")],
    "prefix_16384x1024": [("prefix_sum_i32", False, 16384, 1024),
                          ("prefix_sum_f32", False, 16384, 1024)],
    "affine_4096x8192": [("affine_fwd", False, 4096, 8192), ("affine_rev", False, 4096, 8192)],
    # the same calls with bfloat16 storage of every floating-point stream
    "all7_4096x128_bf16": [(e, tr, 4096, 128) for e, tr in ALL7],
    "long_64x131072_bf16": [(e, True, 64, 131072) for e in ("gae", "vtrace", "retrace")],
    "sweep_4096xT_bf16": [(e, False, 4096, t) for t in (32, 128, 512, 2048, 8192)
                          for e in ("discounted_returns", "lambda_returns", "eligibility_traces")],
    # the same calls on time-major [seq_len, num_envs] arrays
    "all7_4096x128_tm": [(e, tr, 4096, 128) for e, tr in ALL7],
    "sweep_4096xT_tm": [(e, False, 4096, t) for t in (32, 128, 512, 2048, 8192)
                        for e in ("discounted_returns", "lambda_returns", "eligibility_traces")],
}
# workloads on time-major arrays
TIME_MAJOR = {"all7_4096x128_tm", "sweep_4096xT_tm"}
# storage type of the floating-point streams (fp32 unless listed); arithmetic is fp32 throughout
STORAGE = {"all7_4096x128_bf16": "bf16", "long_64x131072_bf16": "bf16", "sweep_4096xT_bf16": "bf16"}
BASE_WORKLOAD = {"all7_64x131072": "long_64x131072",
                 "all7_4096x128_bf16": "all7_4096x128", "long_64x131072_bf16": "long_64x131072",
                 "sweep_4096xT_bf16": "sweep_4096xT", "all7_4096x128_tm": "all7_4096x128",
                 "sweep_4096xT_tm": "sweep_4096xT"}
DEFAULT_WORKLOAD = "all7_4096x128"
# input streams each estimator reads
NEEDS = {
    "gae": ("rewards", "values", "terminateds", "bootstrap_value"),
    "vtrace": ("log_rhos", "rewards", "values", "terminateds", "bootstrap_value"),
    "retrace": ("log_rhos", "rewards", "q_values", "values", "terminateds", "bootstrap_value"),
    "lambda_returns": ("rewards", "values", "terminateds", "bootstrap_value"),
    "discounted_returns": ("rewards", "terminateds", "bootstrap_value"),
    "eligibility_traces": ("x", "dones"),
    "prefix_sum_f32": ("x", "dones"),
    "prefix_sum_i32": ("x_int", "dones"),
    "affine_fwd": ("alpha", "beta", "reset", "carry_in"),
    "affine_rev": ("alpha", "beta", "reset", "carry_in"),
}
# dense per-element streams of each call: (data streams read or written, uint8 masks read).
# With 4-byte data: GAE and TD(lambda) 13 B/elem, V-trace and Retrace 21, the others 9,
# the affine scan 13.
STREAMS = {"gae": (3, 1), "vtrace": (5, 1), "retrace": (5, 1), "lambda_returns": (3, 1),
           "discounted_returns": (2, 1), "eligibility_traces": (2, 1), "prefix_sum_f32": (2, 1),
           "prefix_sum_i32": (2, 1), "affine_fwd": (3, 1), "affine_rev": (3, 1)}


def steps_per_graph(calls_per_step):
    """Steps captured per graph: enough for at least 24 calls."""
    return max(1, -(-24 // calls_per_step))


def replay_plan(R, G, K):
    """Graphs of G steps over R replicas for K timed steps: graph i holds the
    steps on replicas i*G, ..., i*G + G - 1 (mod R), R / gcd(R, G) graphs in
    all, replayed in order; a last graph holds the K mod G remaining steps.
    Returns (first replica of each graph, number of full replays, first
    replica of the remainder graph or None).  Step k of the timed loop then
    uses replica k mod R."""
    n_graphs = R // math.gcd(R, G)
    full, rest = divmod(K, G)
    return [(i * G) % R for i in range(n_graphs)], full, ((full * G) % R if rest else None)


def key(est, trunc, n=None, t=None):
    k = est + ("+trunc" if trunc else "")
    return k if n is None else f"{k}@{n}x{t}"


def make_batches(name):
    """Seeded host inputs of a workload, one batch per (num_envs, seq_len)."""
    from linear_recurrence_scan_env_amd import workloads
    calls = WORKLOADS[name]
    p = workloads.WORKLOADS[BASE_WORKLOAD.get(name, name)]
    batches = {}
    for n, t in sorted({(n, t) for _, _, n, t in calls}):
        if name.startswith("affine"):
            arrs = workloads.affine_inputs(n, t, seed=0, reset_p=p["reset_p"],
                                           beta_range=p["beta_range"])
            batches[(n, t)] = workloads.Rollout(n, t, 1.0, 1.0, arrs)
            continue
        streams = {s_ for e, tr, n_, t_ in calls if (n_, t_) == (n, t) for s_ in NEEDS[e]}
        if any(tr for e, tr, n_, t_ in calls if (n_, t_) == (n, t)):
            streams.add("truncateds")
        batches[(n, t)] = workloads.rollout(
            n, t, seed=0, term_p=p["term_p"], trunc_p=p["trunc_p"], gamma=p["gamma"],
            lambda_=p["lambda_"], done_p=p["term_p"], streams=sorted(streams))
    return batches


def trunc_counts(batches):
    """Truncations per batch (the trunc_values the method reads)."""
    out = {}
    for s_, b in batches.items():
        tr = b.arrays.get("truncateds")
        out[s_] = int(np.count_nonzero(tr)) if tr is not None else 0
    return out


def alg_bytes(est, trunc, n, t, width=4, n_trunc=None):
    """One read of each input stream and one write of each output, with
    `width`-byte data: STREAMS per element, plus one datum of bootstrap (or
    carry) per env.  With truncations: one mask byte per element, and one
    datum of trunc_values per truncation (n_trunc of them), the only ones
    the method uses and the only ones the row-major kernels read; without a
    count, one per element."""
    data, masks = STREAMS[est]
    b = (data * width + masks) * n * t
    if trunc:
        b += n * t + width * (n * t if n_trunc is None else n_trunc)
    if est in BACKWARD or est.startswith("affine"):
        b += width * n
    return b


def make_call(lrs, est, trunc, D, O, g, lam, tm=False):
    kg = dict(truncateds=D["truncateds"] if trunc else None,
              trunc_values=D["trunc_values"] if trunc else None,
              bootstrap_value=D.get("bootstrap_value"), time_major=tm)
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
        return lambda: lrs.compute_eligibility_traces(D["x"], D["dones"], g, lam, out=O[k],
                                                      time_major=tm)
    if est == "prefix_sum_f32":
        return lambda: lrs.compute_episodic_prefix_sum(D["x"], D["dones"], out=O[k], time_major=tm)
    if est == "prefix_sum_i32":
        return lambda: lrs.compute_episodic_prefix_sum(D["x_int"], D["dones"], out=O[k],
                                                       time_major=tm)
    if est in ("affine_fwd", "affine_rev"):
        return lambda: lrs.compute_affine_scan(D["alpha"], D["beta"], reset=D.get("reset"),
                                               carry_in=D.get("carry_in"),
                                               reverse=est == "affine_rev", out=O[k],
                                               time_major=tm)
    raise KeyError(est)


def oracle_call(oracle, est, trunc, ro):
    a = ro.arrays
    g, lam = ro.gamma, ro.lambda_
    kk = dict(bootstrap_value=a.get("bootstrap_value"))
    if trunc:
        kk.update(truncateds=a["truncateds"], trunc_values=a["trunc_values"])
    if est == "gae":
        return lambda: oracle.gae(a["rewards"], a["values"], a["terminateds"], g, lam, **kk)
    if est == "vtrace":
        return lambda: oracle.vtrace(a["log_rhos"], a["rewards"], a["values"], a["terminateds"],
                                     g, lam, **kk)
    if est == "retrace":
        return lambda: oracle.retrace(a["log_rhos"], a["rewards"], a["q_values"], a["values"],
                                      a["terminateds"], g, lam, **kk)
    if est == "lambda_returns":
        return lambda: oracle.lambda_returns(a["rewards"], a["values"], a["terminateds"], g, lam,
                                             **kk)
    if est == "discounted_returns":
        return lambda: oracle.discounted_returns(a["rewards"], a["terminateds"], g, **kk)
    if est == "eligibility_traces":
        return lambda: oracle.eligibility_traces(a["x"], a["dones"], g, lam)
    if est == "prefix_sum_f32":
        return lambda: oracle.prefix_sum(a["x"], a["dones"])
    if est == "prefix_sum_i32":
        return lambda: oracle.prefix_sum(a["x_int"], a["dones"])
    if est in ("affine_fwd", "affine_rev"):
        return lambda: oracle.affine_scan(a["alpha"], a["beta"], reset=a.get("reset"),
                                          carry_in=a.get("carry_in"), reverse=est == "affine_rev")
    raise KeyError(est)


def cpu_baseline(name, batches, seconds):
    """The oracle, untuned, timed on whole steps of the same batch until
    `seconds` have passed (at least one step after a warm-up step)."""
    import oracle
    calls = [oracle_call(oracle, e, tr, batches[(n, t)]) for e, tr, n, t in WORKLOADS[name]]

    def step():
        for f in calls:
            f()

    step()  # warm-up (also builds/loads the library)
    k, t0 = 0, time.perf_counter()
    while True:
        step()
        k += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    elems = k * sum(n * t for _, _, n, t in WORKLOADS[name])
    return {"value": round(elems / el / 1e9, 4), "unit": "Gelem/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"{k} whole steps ({len(calls)} calls each) of the {name} batch, {el:.1f} s, "
                      f"fp64 sequential recursion, OpenMP over envs"}


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "hbm_traffic_all7_4096x128.md")
CALIBRATION_BYTES = 64 << 20  # one --calibrate-copy dispatch reads and writes this much


def source_hash():
    """sha256 of the kernel sources (csrc/): counters taken on other sources are stale."""
    import hashlib
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "linear_recurrence_scan_env_amd", "csrc")
    for f in sorted(os.listdir(pkg)):
        if f.endswith((".hip", ".hpp")):
            with open(os.path.join(pkg, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def call_of_kernel(name):
    """Map a demangled kernel name (scan_kernel<Op<E, ...>, E, W, Acc>) to a bench call key."""
    import re
    ops = {"GaeOp": "gae", "VtraceOp": "vtrace", "RetraceOp": "retrace",
           "LambdaOp": "lambda_returns", "DiscOp": "discounted_returns",
           "EligOp": "eligibility_traces", "PrefixF32Op": "prefix_sum_f32",
           "PrefixI32Op": "prefix_sum_i32"}
    m = re.search(r"lrs::(\w+Op)<([^<>]*)>", name)
    if not m:
        return None
    op, args = m.group(1), [a.strip() for a in m.group(2).split(",")]
    if op in ops:
        trunc = op in ("GaeOp", "VtraceOp", "RetraceOp", "LambdaOp", "DiscOp") and args[1] == "true"
        return key(ops[op], trunc)
    if op == "AffineOp":
        return "affine_rev" if args[1] == "true" else "affine_fwd"
    return None


def summarize_stats(csv_path, command, title="seven estimators at 4096 x 128"):
    import csv
    rows = list(csv.DictReader(open(csv_path)))
    out = [f"# rocprofv3 kernel statistics: {title}", "",
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
    n_trunc = trunc_counts(make_batches(DEFAULT_WORKLOAD))[(n, t)]
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
        ab = alg_bytes(est, tr, n, t, 4, n_trunc)
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


def copy_reference(alg_bytes, stream, reps):
    """A plain device copy moving the dominant call's algorithmic bytes (half
    read, half written), timed like the calls: cold buffers (>= 1 GiB of
    them, cycled), a HIP graph of >= 64 back-to-back launches, events around
    it.  The per-launch time no kernel of this size can beat by much, for
    context beside the roofline fraction."""
    import torch
    half = max(4, alg_bytes // 2) // 4  # fp32 elements per side
    pairs = max(8, -(-(1 << 30) // (8 * half)))
    bufs = [(torch.empty(half, device=stream.device), torch.empty(half, device=stream.device))
            for _ in range(pairs)]
    launches = max(64, pairs)
    with torch.cuda.stream(stream):
        for src, dst in bufs[:2]:
            dst.copy_(src)
        stream.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=stream):
            for i in range(launches):
                src, dst = bufs[i % pairs]
                dst.copy_(src)
        gr.replay()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(reps):
            gr.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / (reps * launches)
    del bufs
    return {"us": round(us, 3), "GBps": round(8 * half / us / 1e3, 1)}


def run_eager(args, steps_fns, stream):
    """Counter-collection mode: the same calls, launched one by one."""
    import torch
    R = len(steps_fns)
    with torch.cuda.stream(stream):
        for k in range(args.warmup + args.steps):
            for f in steps_fns[k % R]:
                f()
        torch.cuda.synchronize()
    print(json.dumps({"mode": "eager", "steps": args.steps, "warmup": args.warmup,
                      "workload": args.workload, "step_graphs": R}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(WORKLOADS))
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
    ap.add_argument("--summarize-stats", nargs="+", metavar="CSV COMMAND [TITLE]",
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

    name = args.workload
    calls = WORKLOADS[name]
    p = workloads.WORKLOADS[BASE_WORKLOAD.get(name, name)]
    storage = STORAGE.get(name, "f32")
    width = 2 if storage in ("bf16", "f16") else 4
    store_dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[storage]
    shapes = sorted({(n, t) for _, _, n, t in calls})
    batches = make_batches(name)
    n_trunc = trunc_counts(batches)
    ro0 = batches[shapes[0]]
    g, lam = ro0.gamma, ro0.lambda_

    hosts = {s_: {k: torch.from_numpy(v) for k, v in b.arrays.items() if v is not None}
             for s_, b in batches.items()}
    if storage != "f32":
        for h in hosts.values():
            for k, v in h.items():
                if v.dtype == torch.float32:
                    h[k] = v.to(store_dt)
    tm = name in TIME_MAJOR
    if tm:  # per-step arrays as [seq_len, num_envs]
        for h in hosts.values():
            for k, v in h.items():
                if v.dim() == 2:
                    h[k] = v.t().contiguous()

    # Replicas per shape: enough copies of that shape's inputs and outputs
    # for >= 1 GiB, so that each call reads cold data however small it is.
    def shape_bytes(s_):
        b = sum(v.numel() * v.element_size() for v in hosts[s_].values())
        return b + sum((2 if e == "vtrace" else 1) * n * t * width for e, _, n, t in calls
                       if (n, t) == s_)

    if args.warm:
        nrep = {s_: 1 for s_ in shapes}
    elif args.replicas:
        nrep = {s_: args.replicas for s_ in shapes}
    else:
        nrep = {s_: max(2, -(-(1 << 30) // shape_bytes(s_))) for s_ in shapes}
    R = max(nrep.values())
    store = {}  # (shape, replica) -> (inputs, outputs)
    for s_ in shapes:
        for i in range(nrep[s_]):
            D = {k: v.to(dev) for k, v in hosts[s_].items()}
            O = {}
            for e, tr, n, t in calls:
                if (n, t) != s_:
                    continue
                dt = torch.int32 if e == "prefix_sum_i32" else store_dt
                oshape = (t, n) if tm else (n, t)
                O[key(e, tr)] = torch.empty(oshape, device=dev, dtype=dt)
                if e == "vtrace":
                    O[key(e, tr) + "/pg"] = torch.empty(oshape, device=dev, dtype=dt)
            store[(s_, i)] = (D, O)

    def fn(e, tr, n, t, i):
        D, O = store[((n, t), i % nrep[(n, t)])]
        return make_call(lrs, e, tr, D, O, g, lam, tm)

    def step_fns(i):
        return [fn(e, tr, n, t, i) for e, tr, n, t in calls]

    stream = torch.cuda.Stream(dev)
    if args.calibrate_copy:
        src = torch.ones(CALIBRATION_BYTES // 4, device=dev)
        dst = torch.empty_like(src)
        with torch.cuda.stream(stream):
            for _ in range(5):
                dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.eager:
        return run_eager(args, [step_fns(i) for i in range(R)], stream)

    with torch.cuda.stream(stream):
        # Eager warm-up on the capture stream (allocates its workspace outside capture).
        for i in range(min(R, 2)):
            for f in step_fns(i):
                f()
        stream.synchronize()

        def capture(fns):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=stream):
                for f in fns:
                    f()
            return gr

        # Several consecutive steps per graph when a step has few calls (at least 24
        # calls per graph), so that host-side replay cost never paces the GPU.  Graph
        # i holds the steps on replicas i*G, i*G+1, ... (mod R): replaying the graphs
        # in order walks the replicas in order, so no call reuses recent inputs.
        G = steps_per_graph(len(calls))
        starts, full, tail_start = replay_plan(R, G, args.steps)
        n_graphs = len(starts)

        def steps_graph(first, count):
            fns = []
            for k in range(first, first + count):
                fns += step_fns(k % R)
            return capture(fns)

        step_graphs = [steps_graph(first, G) for first in starts]
        tail_graph = steps_graph(tail_start, args.steps % G) if tail_start is not None else None
        call_keys = [key(e, tr, n, t) for e, tr, n, t in calls]
        # per call: a graph of >= 64 launches cycling over that call's replicas
        launches = {k_: max(64, nrep[(n, t)]) for k_, (e, tr, n, t) in zip(call_keys, calls)}
        call_graphs = {k_: capture([fn(e, tr, n, t, i) for i in range(launches[k_])])
                       for k_, (e, tr, n, t) in zip(call_keys, calls)}
        torch.cuda.synchronize()

        # ---- timed steps: exactly args.steps steps (full graphs, then the rest)
        for k in range(-(-args.warmup // G)):
            step_graphs[k % n_graphs].replay()
        torch.cuda.synchronize()
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        t_start.record(stream)
        for k in range(full):
            step_graphs[k % n_graphs].replay()
        if tail_graph is not None:
            tail_graph.replay()
        t_end.record(stream)
        torch.cuda.synchronize()
        ms_per_step = t_start.elapsed_time(t_end) / args.steps

        # ---- per-call average launch duration (graph of R launches, events around it)
        per_call = {}
        for (e, tr, n, t), k_ in zip(calls, call_keys):
            call_graphs[k_].replay()
            ev0 = torch.cuda.Event(enable_timing=True)
            ev1 = torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            for _ in range(args.roofline_reps):
                call_graphs[k_].replay()
            ev1.record(stream)
            torch.cuda.synchronize()
            us = ev0.elapsed_time(ev1) * 1e3 / (args.roofline_reps * launches[k_])
            b = alg_bytes(e, tr, n, t, width, n_trunc[(n, t)])
            per_call[k_ if len(shapes) > 1 else key(e, tr)] = {
                "us": round(us, 3), "alg_bytes": b, "GBps": round(b / us / 1e3, 1),
                "Gelem/s": round(n * t / us / 1e3, 2)}

    elems_per_step = sum(n * t for _, _, n, t in calls)
    value = elems_per_step / (ms_per_step * 1e-3) / 1e9
    dom = max(per_call, key=lambda k_: per_call[k_]["us"])
    achieved = per_call[dom]["GBps"]
    copy_ref = copy_reference(per_call[dom]["alg_bytes"], stream, args.roofline_reps)
    cfg = {"workload": name, "calls_per_step": len(calls),
           "cache": "warm" if args.warm else "cold",
           "replicas": {f"{n}x{t}": nrep[(n, t)] for n, t in shapes},
           "launch": f"hip graphs of {G} step(s)", "storage": storage,
           "layout": "time-major [seq_len, num_envs]" if tm else "row-major [num_envs, seq_len]"}
    if len(shapes) == 1:
        cfg.update(num_envs=shapes[0][0], seq_len=shapes[0][1])
    else:
        cfg.update(shapes=[f"{n}x{t}" for n, t in shapes])
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
        "dtype": "i32" if all(e == "prefix_sum_i32" for e, *_ in calls) else "f32",
        "data": "synthetic",
        "config": cfg,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": committed_traffic(dom) if name == DEFAULT_WORKLOAD else None,
                     "alg_bytes": per_call[dom]["alg_bytes"],
                     "copy_same_bytes": copy_ref},
        "per_call": per_call,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(name, batches, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
