#!/usr/bin/env python3
"""Throughput of the scan path on one MI355X.

Default workload (the pages' headline shape): num_envs = 4096, seq_len = 128,
fp32.  One step = every estimator once without truncations (prefix sum in
fp32) and the five truncating estimators once more with truncations: 12
library calls, each one pass over its [4096, 128] inputs.  --workload picks
one of the other benchmark workloads (their steps are listed in WORKLOADS).

Inputs sit in HBM before timing starts.  Each shape's batch is replicated R
times and step k uses replica k mod R, so every call reads its inputs from HBM
rather than from a cache ("cold"): R is chosen so that every single call
cycles over at least 1 GiB of its own inputs and outputs, four times the
256 MB Infinity Cache; --warm reuses one replica.  The calls are captured into
HIP graphs (torch.cuda.CUDAGraph) of G consecutive steps each (G = 1 for steps
of 24 or more calls, more for short steps), so the timed loop is K / G graph
replays and host launch overhead stays off the critical path; it starts at the
graph after the last one warm-up replayed.

Prints one JSON line.  value = elements processed per step / step time
(Gelem/s).  per_call: each call's average launch duration from HIP events
around graphs of >= 64 back-to-back launches of that call (cycling over its
replicas) on the launch stream, the inter-launch gap included.  roofline: the
call with the longest average duration, its algorithmic bytes (one read of
every input stream, one write of every output) over that duration; beside it
the same fraction from the committed rocprofv3 kernel trace of this command
(kernel time alone, no gap) while the kernel sources match; floor: an empty
kernel and a streaming kernel that moves the call's bytes on the call's own
grid, timed the same way; copy_same_bytes: a plain device copy of the bytes.
With the default workload, long_path reports the chunked-path calls (GAE,
V-trace and Retrace with truncations at 64 x 131072) the same way.
cpu_baseline: the fp64 oracle on the host cores, whole steps on the same batch.
"""
from __future__ import annotations

import argparse
import ctypes
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
MIN_CYCLE_BYTES = 1 << 30  # every timed call cycles over at least this much of its own data
BACKWARD = ("gae", "vtrace", "retrace", "lambda_returns", "discounted_returns")
ALL7 = [("gae", False), ("vtrace", False), ("retrace", False), ("lambda_returns", False),
        ("discounted_returns", False), ("eligibility_traces", False), ("prefix_sum_f32", False),
        ("gae", True), ("vtrace", True), ("retrace", True), ("lambda_returns", True),
        ("discounted_returns", True)]
LONG3 = [(e, True, 64, 131072) for e in ("gae", "vtrace", "retrace")]
SWEEP = [(e, False, 4096, t) for t in (32, 128, 512, 2048, 8192)
         for e in ("discounted_returns", "lambda_returns", "eligibility_traces")]
# workload -> the calls of one step: (estimator, with truncations, num_envs, seq_len)
WORKLOADS = {
    "all7_4096x128": [(e, tr, 4096, 128) for e, tr in ALL7],
    "gae_64x512": [("gae", False, 64, 512)],
    "long_64x131072": LONG3,
    # all seven estimators on the long rows (the 12 calls of all7_4096x128)
    "all7_64x131072": [(e, tr, 64, 131072) for e, tr in ALL7],
    "sweep_4096xT": SWEEP,
    "prefix_16384x1024": [("prefix_sum_i32", False, 16384, 1024),
                          ("prefix_sum_f32", False, 16384, 1024)],
    "affine_4096x8192": [("affine_fwd", False, 4096, 8192), ("affine_rev", False, 4096, 8192)],
    # the same calls with bfloat16 storage of every floating-point stream
    "all7_4096x128_bf16": [(e, tr, 4096, 128) for e, tr in ALL7],
    "long_64x131072_bf16": LONG3,
    "sweep_4096xT_bf16": SWEEP,
    # the same calls on time-major [seq_len, num_envs] arrays
    "all7_4096x128_tm": [(e, tr, 4096, 128) for e, tr in ALL7],
    "sweep_4096xT_tm": SWEEP,
    # the same calls on views of wider buffers: every per-step array a slice
    # [:, :T] of an [N, T + pad] buffer (its own row stride), read in place
    "all7_4096x128_strided": [(e, tr, 4096, 128) for e, tr in ALL7],
    "long_64x131072_strided": LONG3,
}
# workloads on time-major arrays
TIME_MAJOR = {"all7_4096x128_tm", "sweep_4096xT_tm"}
# storage type of the floating-point streams (fp32 unless listed); arithmetic is fp32 throughout
STORAGE = {"all7_4096x128_bf16": "bf16", "long_64x131072_bf16": "bf16", "sweep_4096xT_bf16": "bf16"}
# row padding (elements) of the strided workloads: rows stay 16-byte aligned
STRIDE_PAD = {"all7_4096x128_strided": 4, "long_64x131072_strided": 64}
BASE_WORKLOAD = {"all7_64x131072": "long_64x131072",
                 "all7_4096x128_bf16": "all7_4096x128", "long_64x131072_bf16": "long_64x131072",
                 "sweep_4096xT_bf16": "sweep_4096xT", "all7_4096x128_tm": "all7_4096x128",
                 "sweep_4096xT_tm": "sweep_4096xT", "all7_4096x128_strided": "all7_4096x128",
                 "long_64x131072_strided": "long_64x131072"}
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
# dense per-element streams of each call: (data streams read, data streams
# written, uint8 masks read).  With 4-byte data: GAE and TD(lambda) 13 B/elem,
# V-trace and Retrace 21, the others 9, the affine scan 13.
STREAMS = {"gae": (2, 1, 1), "vtrace": (3, 2, 1), "retrace": (4, 1, 1),
           "lambda_returns": (2, 1, 1), "discounted_returns": (1, 1, 1),
           "eligibility_traces": (1, 1, 1), "prefix_sum_f32": (1, 1, 1),
           "prefix_sum_i32": (1, 1, 1), "affine_fwd": (2, 1, 1), "affine_rev": (2, 1, 1)}
# estimator id of lrs_debug_schedule and flags
EST_ID = {"gae": 0, "vtrace": 1, "retrace": 2, "lambda_returns": 3, "discounted_returns": 4,
          "eligibility_traces": 5, "prefix_sum_i32": 6, "prefix_sum_f32": 7, "affine_fwd": 8,
          "affine_rev": 8}


def steps_per_graph(calls_per_step):
    """Steps captured per graph: enough for at least 24 calls."""
    return max(1, -(-24 // calls_per_step))


def replay_plan(R, G, K, first_graph=0):
    """Graphs of G steps over R replicas for K timed steps: graph i holds the
    steps on replicas i*G, ..., i*G + G - 1 (mod R), R / gcd(R, G) graphs in
    all, replayed in order from graph `first_graph`; a last graph holds the
    K mod G remaining steps.  Returns (first replica of each graph, number of
    full replays, first replica of the remainder graph or None).  Step k of
    the timed loop then uses replica (first_graph * G + k) mod R."""
    n_graphs = R // math.gcd(R, G)
    full, rest = divmod(K, G)
    starts = [(i * G) % R for i in range(n_graphs)]
    tail = ((first_graph + full) * G) % R if rest else None
    return starts, full, tail


def replicas_for(call_bytes, min_bytes=MIN_CYCLE_BYTES, multiple=1):
    """Replicas of a shape's batch so that each call cycles over at least
    min_bytes of its own data: the largest need among its calls, >= 2, rounded
    up to a multiple of the steps per graph."""
    r = max([2] + [-(-min_bytes // b) for b in call_bytes])
    return -(-r // multiple) * multiple


def key(est, trunc, n=None, t=None):
    k = est + ("+trunc" if trunc else "")
    return k if n is None else f"{k}@{n}x{t}"


def make_batches(name, calls=None):
    """Seeded host inputs of a workload, one batch per (num_envs, seq_len)."""
    from linear_recurrence_scan_env_amd import workloads
    calls = WORKLOADS[name] if calls is None else calls
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


def alg_bytes_rw(est, trunc, n, t, width=4, n_trunc=None):
    """(bytes read, bytes written) of one call: one read of each input stream
    and one write of each output, with `width`-byte data, plus one datum of
    bootstrap (or carry) per env.  With truncations: one mask byte per
    element, and one datum of trunc_values per truncation (n_trunc of them),
    the only ones the method uses and the only ones the row-major kernels
    read; without a count, one per element."""
    rd, wr, masks = STREAMS[est]
    r = (rd * width + masks) * n * t
    if trunc:
        r += n * t + width * (n * t if n_trunc is None else n_trunc)
    if est in BACKWARD or est.startswith("affine"):
        r += width * n
    return r, wr * width * n * t


def alg_bytes(est, trunc, n, t, width=4, n_trunc=None):
    return sum(alg_bytes_rw(est, trunc, n, t, width, n_trunc))


def beta_max(est, g, lam, c_bar=1.0):
    """The largest beta a call's maps hold, as the library derives it."""
    if est in ("gae", "lambda_returns", "eligibility_traces"):
        return g * lam
    if est == "discounted_returns":
        return g
    if est in ("vtrace", "retrace"):
        return g * lam * c_bar
    if est.startswith("prefix"):
        return 1.0
    return float("inf")


class SchedInfo(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int64), ("num_tiles", ctypes.c_int64),
                ("tile_elems", ctypes.c_int64), ("tile_steps", ctypes.c_int64),
                ("groups", ctypes.c_int64), ("envs_per_group", ctypes.c_int64),
                ("time_major", ctypes.c_int32), ("carries", ctypes.c_int32),
                ("backward", ctypes.c_int32), ("tiles_per_row", ctypes.c_int32),
                ("elems_per_lane", ctypes.c_int32), ("waves_per_block", ctypes.c_int32),
                ("composition_fp64", ctypes.c_int32), ("reserved", ctypes.c_int32)]


def launch_grid(lib, est, trunc, n, t, g, lam, tm=False, half=False):
    """(blocks, threads per block) of a call, from the library's own plan."""
    flags = (1 if trunc else 0) | (2 if est == "affine_rev" else 0) | (4 if tm else 0) | \
        (8 if half else 0)
    info = SchedInfo()
    fn = lib.lrs_debug_schedule
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
                   ctypes.POINTER(SchedInfo), ctypes.c_void_p, ctypes.c_int64]
    st = fn(EST_ID[est], flags, n, t, beta_max(est, g, lam), ctypes.byref(info), None, 0)
    if st != 0:
        raise RuntimeError(lib.lrs_last_error().decode())
    return int(info.num_blocks), int(info.waves_per_block) * 64


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


# ------------------------------------------------------------ profiles

PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_PROFILE = os.path.join(PROFILES, "hbm_traffic_all7_4096x128.md")
CALIBRATION_BYTES = 64 << 20  # one --calibrate-copy dispatch reads and writes this much
# grid of the calibration dispatch (lrs_debug_floor's streaming kernel, eight
# 16-byte vectors per lane): unique among the dispatches of a counter run
CALIBRATION_GRID = (CALIBRATION_BYTES // 16 // 8 // 256, 256)


def source_hash():
    """sha256 of the kernel sources (csrc/): figures taken on other sources are stale."""
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
    if "floor_empty" in name:
        return "floor:empty"
    if "floor_stream" in name:
        return "floor:stream"
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


def profile_path(workload):
    return os.path.join(PROFILES, f"kernel_stats_{workload}.md")


def summarize_trace(trace_csv, command, workload, title):
    """Markdown summary of a rocprofv3 kernel trace of `bench.py --workload
    workload`: per-kernel statistics, then each call's average duration
    (dispatches matched to calls by kernel and grid), and a machine-readable
    block that bench.py reads while the kernel sources are unchanged."""
    import csv
    import collections
    import linear_recurrence_scan_env_amd as lrs
    lib = lrs.load()
    calls = list(WORKLOADS[workload]) + (LONG3 if workload == DEFAULT_WORKLOAD else [])
    p = make_batches(workload).popitem()[1]
    tm, half = workload in TIME_MAJOR, workload in STORAGE
    grids = {}
    for e, tr, n, t in calls:
        b, th = launch_grid(lib, e, tr, n, t, p.gamma, p.lambda_, tm, half)
        grids.setdefault((key(e, tr), b * th), key(e, tr, n, t))
    per_kernel = collections.defaultdict(list)
    per_call = collections.defaultdict(list)
    for r in csv.DictReader(open(trace_csv)):
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        name = r["Kernel_Name"]
        per_kernel[name].append(us)
        c = call_of_kernel(name)
        grid = int(r.get("Grid_Size_X") or r.get("Grid_Size") or 0)
        if c and c.startswith("floor:"):
            per_call[c].append(us)
        elif c and (c, grid) in grids:
            per_call[grids[(c, grid)]].append(us)
    out = [f"# rocprofv3 kernel statistics: {title}", "",
           "Command:", "", "```", command, "```", "",
           "| kernel | call | dispatches | avg us | min us | max us |", "|---|---|---|---|---|---|"]
    for name, v in sorted(per_kernel.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"| `{name.split('(')[0]}` | {call_of_kernel(name) or '-'} | {len(v)} | "
                   f"{sum(v) / len(v):.3f} | {min(v):.3f} | {max(v):.3f} |")
    out += ["", "Average duration per call (dispatches matched by kernel and grid size):", "",
            "| call | dispatches | avg us |", "|---|---|---|"]
    avg = {}
    for c in sorted(per_call):
        v = per_call[c]
        avg[c] = round(sum(v) / len(v), 3)
        out.append(f"| {c} | {len(v)} | {avg[c]:.3f} |")
    out += ["", "Machine-readable (read by bench.py; valid only for these kernel sources):", "",
            f"source_sha256: {source_hash()}", "kernel_avg_us: " + json.dumps(avg, sort_keys=True)]
    print("\n".join(out))


def committed_profile(workload):
    """Per-call average kernel durations (us) from the committed rocprofv3
    summary of this workload, or None when missing or taken on other sources."""
    try:
        text = open(profile_path(workload)).read()
    except OSError:
        return None
    sha = avg = None
    for line in text.splitlines():
        if line.startswith("source_sha256:"):
            sha = line.split(":", 1)[1].strip()
        if line.startswith("kernel_avg_us:"):
            avg = json.loads(line.split(":", 1)[1])
    return avg if sha == source_hash() and avg else None


def summarize_counters(fetch_csv, write_csv, command_fetch, command_write):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) scaled by what the same
    counters read for the calibration dispatch: the streaming kernel reading
    and writing CALIBRATION_BYTES (matched by kernel name and grid size)."""
    import csv
    import collections

    def load(path):
        per = collections.defaultdict(list)
        calib = []
        for r in csv.DictReader(open(path)):
            v = float(r["Counter_Value"]) * 1024.0
            k = call_of_kernel(r["Kernel_Name"])
            if k and not k.startswith("floor:"):
                per[k].append(v)
            elif k == "floor:stream" and int(r["Grid_Size"]) == CALIBRATION_GRID[0] * CALIBRATION_GRID[1]:
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
           f"Calibration: the streaming kernel reading and writing {CALIBRATION_BYTES >> 20} MiB "
           f"(grid {CALIBRATION_GRID[0]} x {CALIBRATION_GRID[1]}) reads FETCH_SIZE "
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


# ------------------------------------------------------------ timing

def time_graph(gr, stream, reps, launches):
    """Average time per launch of a graph of `launches` launches, from HIP
    events around `reps` replays on `stream` (after one untimed replay)."""
    import torch
    gr.replay()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(reps):
        gr.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) * 1e3 / (reps * launches)


def capture(fns, stream):
    import torch
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=stream):
        for f in fns:
            f()
    return gr


def copy_reference(alg_bytes, stream, reps):
    """A plain device copy moving the dominant call's algorithmic bytes (half
    read, half written), timed like the calls: cold buffers (>= 1 GiB of
    them, cycled), a HIP graph of >= 64 back-to-back launches, events around
    it.  The per-launch time no kernel of this size can beat by much, for
    context beside the roofline fraction."""
    import torch
    half = max(4, alg_bytes // 2) // 4  # fp32 elements per side
    pairs = max(8, -(-MIN_CYCLE_BYTES // (8 * half)))
    bufs = [(torch.empty(half, device=stream.device), torch.empty(half, device=stream.device))
            for _ in range(pairs)]
    launches = max(64, pairs)
    with torch.cuda.stream(stream):
        for src, dst in bufs[:2]:
            dst.copy_(src)
        stream.synchronize()
        gr = capture([(lambda s=src, d=dst: d.copy_(s)) for src, dst in
                      (bufs[i % pairs] for i in range(launches))], stream)
        us = time_graph(gr, stream, reps, launches)
    del bufs
    return {"us": round(us, 3), "GBps": round(8 * half / us / 1e3, 1)}


def floor_reference(lib, grid, rw_bytes, stream, reps):
    """The dominant call's grid with no work (an empty kernel) and with only
    its bytes (lrs_debug_floor's streaming kernel reading and writing the
    call's byte counts, cold buffers cycled over >= 1 GiB), each in a graph of
    >= 64 back-to-back launches timed like the calls.  call - empty is the
    call's own time beyond a launch of its grid; stream - empty is what the
    bytes alone cost on that grid."""
    import torch
    blocks, threads = grid
    rd = -(-rw_bytes[0] // 16) * 16
    wr = -(-rw_bytes[1] // 16) * 16
    fn = lib.lrs_debug_floor
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
                   ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    pairs = max(8, -(-MIN_CYCLE_BYTES // (rd + wr)))
    bufs = [(torch.empty(rd, dtype=torch.uint8, device=stream.device),
             torch.empty(wr, dtype=torch.uint8, device=stream.device)) for _ in range(pairs)]
    launches = max(64, pairs)
    sid = stream.cuda_stream

    def empty():
        if fn(0, blocks, threads, None, 0, None, 0, sid) != 0:
            raise RuntimeError(lib.lrs_last_error().decode())

    def streamer(s, d):
        def f():
            if fn(1, blocks, threads, s.data_ptr(), rd, d.data_ptr(), wr, sid) != 0:
                raise RuntimeError(lib.lrs_last_error().decode())
        return f

    with torch.cuda.stream(stream):
        empty()
        streamer(*bufs[0])()
        stream.synchronize()
        ge = capture([empty] * 64, stream)
        gs = capture([streamer(*bufs[i % pairs]) for i in range(launches)], stream)
        e_us = time_graph(ge, stream, reps, 64)
        s_us = time_graph(gs, stream, reps, launches)
    del bufs
    return {"grid": [blocks, threads], "empty_us": round(e_us, 3), "stream_us": round(s_us, 3),
            "stream_bytes": rd + wr, "stream_GBps": round((rd + wr) / s_us / 1e3, 1)}


class Store:
    """Device replicas of a workload's batches and its calls' outputs."""

    def __init__(self, lrs, name, calls, batches, dev, storage, tm, pad, nrep_fn):
        import torch
        self.calls, self.tm = calls, tm
        width = 2 if storage in ("bf16", "f16") else 4
        store_dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[storage]
        shapes = sorted({(n, t) for _, _, n, t in calls})
        hosts = {s_: {k: torch.from_numpy(v) for k, v in b.arrays.items() if v is not None}
                 for s_, b in batches.items() if s_ in shapes}
        for h in hosts.values():
            for k, v in list(h.items()):
                if v.dtype == torch.float32 and storage != "f32":
                    v = v.to(store_dt)
                if tm and v.dim() == 2:  # per-step arrays as [seq_len, num_envs]
                    v = v.t().contiguous()
                h[k] = v
        self.nrep = {}
        self.data = {}  # (shape, replica) -> (inputs, outputs)

        def place(v0):
            """A copy of device tensor v0; per-step arrays as views of
            [rows, cols + pad] buffers when pad > 0."""
            if pad and v0.dim() == 2:
                rows, cols = v0.shape
                buf = torch.empty((rows, cols + pad), dtype=v0.dtype, device=dev)
                view = buf[:, :cols]
                view.copy_(v0)
                return view
            return v0.clone()

        for s_ in shapes:
            ntr = int(np.count_nonzero(batches[s_].arrays.get("truncateds"))) \
                if batches[s_].arrays.get("truncateds") is not None else 0
            cb = [alg_bytes(e, tr, n, t, width, ntr) for e, tr, n, t in calls if (n, t) == s_]
            R = nrep_fn(cb)
            self.nrep[s_] = R
            first = {k: v.to(dev) for k, v in hosts[s_].items()}
            for i in range(R):
                D = {k: place(v) for k, v in first.items()}
                O = {}
                for e, tr, n, t in calls:
                    if (n, t) != s_:
                        continue
                    dt = torch.int32 if e == "prefix_sum_i32" else store_dt
                    oshape = (t, n) if tm else (n, t)
                    k = key(e, tr)
                    O[k] = place(torch.empty(oshape, device=dev, dtype=dt))
                    if e == "vtrace":
                        O[k + "/pg"] = place(torch.empty(oshape, device=dev, dtype=dt))
                D["_O"] = O
                self.data[(s_, i)] = D
            del first
        self.lrs = lrs
        self.g, self.lam = batches[shapes[0]].gamma, batches[shapes[0]].lambda_

    def fn(self, e, tr, n, t, i):
        D = self.data[((n, t), i % self.nrep[(n, t)])]
        return make_call(self.lrs, e, tr, D, D["_O"], self.g, self.lam, self.tm)

    def step_fns(self, i):
        return [self.fn(e, tr, n, t, i) for e, tr, n, t in self.calls]


def time_per_call(st, stream, reps, width, n_trunc, shapes_in_key):
    """Each call's average launch duration: a graph of max(64, R) launches
    cycling over the call's R replicas (>= 1 GiB of its own data)."""
    per_call = {}
    for e, tr, n, t in st.calls:
        R = st.nrep[(n, t)]
        launches = max(64, R)
        gr = capture([st.fn(e, tr, n, t, i) for i in range(launches)], stream)
        us = time_graph(gr, stream, reps, launches)
        del gr
        b = alg_bytes(e, tr, n, t, width, n_trunc[(n, t)])
        per_call[key(e, tr, n, t) if shapes_in_key else key(e, tr)] = {
            "us": round(us, 3), "alg_bytes": b, "GBps": round(b / us / 1e3, 1),
            "frac": round(b / us / 1e3 / HBM_PEAK_GBPS, 4), "Gelem/s": round(n * t / us / 1e3, 2),
            "cycle_bytes": b * R}
    return per_call


def run_eager(args, st, stream):
    """Counter-collection mode: the same calls, launched one by one."""
    import torch
    R = max(st.nrep.values())
    with torch.cuda.stream(stream):
        for k in range(args.warmup + args.steps):
            for f in st.step_fns(k % R):
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
    ap.add_argument("--replicas", type=int, default=0,
                    help="0: enough for >= 1 GiB of every call's own data")
    ap.add_argument("--warm", action="store_true", help="one replica: cache-resident inputs")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-long-path", action="store_true",
                    help="default workload: skip the 64 x 131072 chunked-path calls")
    ap.add_argument("--roofline-reps", type=int, default=20)
    ap.add_argument("--eager", action="store_true",
                    help="launch calls one by one instead of replaying HIP graphs "
                         "(for counter collection)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run the streaming kernel 5 times over 64 MiB in and 64 MiB out: a "
                         "kernel of known HBM traffic for scaling FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--summarize-trace", nargs=4,
                    metavar=("TRACE_CSV", "COMMAND", "WORKLOAD", "TITLE"),
                    help="print the markdown summary of a rocprofv3 kernel_trace.csv of a run "
                         "of WORKLOAD")
    ap.add_argument("--summarize-counters", nargs=4,
                    metavar=("FETCH_CSV", "WRITE_CSV", "FETCH_COMMAND", "WRITE_COMMAND"),
                    help="print the HBM-traffic summary of two rocprofv3 --pmc runs")
    args = ap.parse_args()

    if args.summarize_trace:
        return summarize_trace(*args.summarize_trace)
    if args.summarize_counters:
        return summarize_counters(*args.summarize_counters)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(sharding over environments needs no communication; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import linear_recurrence_scan_env_amd as lrs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = lrs.load()

    name = args.workload
    calls = WORKLOADS[name]
    storage = STORAGE.get(name, "f32")
    width = 2 if storage in ("bf16", "f16") else 4
    tm = name in TIME_MAJOR
    pad = STRIDE_PAD.get(name, 0)
    shapes = sorted({(n, t) for _, _, n, t in calls})
    batches = make_batches(name)
    n_trunc = trunc_counts(batches)
    G = steps_per_graph(len(calls))

    def nrep_fn(call_bytes):
        if args.warm:
            return 1
        if args.replicas:
            return args.replicas
        return replicas_for(call_bytes, MIN_CYCLE_BYTES, G)

    st = Store(lrs, name, calls, batches, dev, storage, tm, pad, nrep_fn)
    R = max(st.nrep.values())
    stream = torch.cuda.Stream(dev)
    if args.calibrate_copy:
        src = torch.ones(CALIBRATION_BYTES // 4, device=dev)
        dst = torch.empty_like(src)
        fl = lib.lrs_debug_floor
        fl.restype = ctypes.c_int
        fl.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
                       ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        for _ in range(5):
            if fl(1, CALIBRATION_GRID[0], CALIBRATION_GRID[1], src.data_ptr(), CALIBRATION_BYTES,
                  dst.data_ptr(), CALIBRATION_BYTES, stream.cuda_stream) != 0:
                raise RuntimeError(lib.lrs_last_error().decode())
        torch.cuda.synchronize()
        del src, dst
    if args.eager:
        return run_eager(args, st, stream)

    with torch.cuda.stream(stream):
        # Eager warm-up on the capture stream (allocates its workspace outside capture).
        for i in range(min(R, 2)):
            for f in st.step_fns(i):
                f()
        stream.synchronize()

        # Several consecutive steps per graph when a step has few calls (at least 24
        # calls per graph), so that host-side replay cost never paces the GPU.  Graph
        # i holds the steps on replicas i*G, i*G+1, ... (mod R): replaying the graphs
        # in order walks the replicas in order, so no call reuses recent inputs.
        warm_graphs = -(-args.warmup // G)
        starts, full, tail_start = replay_plan(R, G, args.steps)
        n_graphs = len(starts)
        first_graph = warm_graphs % n_graphs
        _, full, tail_start = replay_plan(R, G, args.steps, first_graph)

        def steps_graph(first, count):
            fns = []
            for k in range(first, first + count):
                fns += st.step_fns(k % R)
            return capture(fns, stream)

        step_graphs = [steps_graph(first, G) for first in starts]
        tail_graph = steps_graph(tail_start, args.steps % G) if tail_start is not None else None
        torch.cuda.synchronize()

        # ---- timed steps: exactly args.steps steps (full graphs, then the rest),
        # starting at the graph after the last one the warm-up replayed
        for k in range(warm_graphs):
            step_graphs[k % n_graphs].replay()
        torch.cuda.synchronize()
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        t_start.record(stream)
        for k in range(full):
            step_graphs[(first_graph + k) % n_graphs].replay()
        if tail_graph is not None:
            tail_graph.replay()
        t_end.record(stream)
        torch.cuda.synchronize()
        ms_per_step = t_start.elapsed_time(t_end) / args.steps
        del step_graphs, tail_graph

        # ---- per-call average launch duration
        per_call = time_per_call(st, stream, args.roofline_reps, width, n_trunc, len(shapes) > 1)

    elems_per_step = sum(n * t for _, _, n, t in calls)
    value = elems_per_step / (ms_per_step * 1e-3) / 1e9
    dom = max(per_call, key=lambda k_: per_call[k_]["us"])
    dom_call = next(c for c in calls if key(c[0], c[1], c[2], c[3]) == dom or
                    key(c[0], c[1]) == dom)
    e_d, tr_d, n_d, t_d = dom_call
    achieved = per_call[dom]["GBps"]
    rw = alg_bytes_rw(e_d, tr_d, n_d, t_d, width, n_trunc[(n_d, t_d)])
    grid = launch_grid(lib, e_d, tr_d, n_d, t_d, st.g, st.lam, tm, width == 2)
    floor = floor_reference(lib, grid, rw, stream, args.roofline_reps)
    floor["call_minus_empty_us"] = round(per_call[dom]["us"] - floor["empty_us"], 3)
    floor["stream_minus_empty_us"] = round(floor["stream_us"] - floor["empty_us"], 3)
    copy_ref = copy_reference(per_call[dom]["alg_bytes"], stream, args.roofline_reps)
    prof = committed_profile(name)
    dom_full = key(e_d, tr_d, n_d, t_d)
    rocprof = None
    if prof and dom_full in prof:
        us = prof[dom_full]
        rocprof = {"us": us, "frac": round(per_call[dom]["alg_bytes"] / us / 1e3 / HBM_PEAK_GBPS, 4),
                   "profile": os.path.relpath(profile_path(name), ROOT),
                   "source": "rocprofv3 kernel trace of this command: kernel time alone"}
    cfg = {"workload": name, "calls_per_step": len(calls),
           "cache": "warm" if args.warm else "cold",
           "replicas": {f"{n}x{t}": st.nrep[(n, t)] for n, t in shapes},
           "launch": f"hip graphs of {G} step(s)", "storage": storage,
           "layout": ("time-major [seq_len, num_envs]" if tm else "row-major [num_envs, seq_len]") +
                     (f", views of [rows, cols + {pad}] buffers" if pad else "")}
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
                     "traffic": committed_traffic(key(e_d, tr_d)) if name == DEFAULT_WORKLOAD
                     else None,
                     "alg_bytes": per_call[dom]["alg_bytes"],
                     "duration_source": "HIP events around graphs of back-to-back launches of "
                                        "the call on its stream (inter-launch gap included)",
                     "rocprof": rocprof, "floor": floor, "copy_same_bytes": copy_ref},
        "per_call": per_call,
    }
    if name == DEFAULT_WORKLOAD and not args.no_long_path:
        out["long_path"] = long_path(lrs, lib, dev, stream, args)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(name, batches, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def long_path(lrs, lib, dev, stream, args):
    """The chunked path's calls (GAE, V-trace and Retrace with truncations at
    64 x 131072: multi-block carries along 131072-step rows), each timed like
    the per-call figures above, with the rocprof kernel time of the committed
    default-workload profile beside it."""
    import torch
    batches = make_batches("long_64x131072")
    st = Store(lrs, "long_64x131072", LONG3, batches, dev, "f32", False, 0,
               lambda cb: replicas_for(cb, MIN_CYCLE_BYTES, 1))
    with torch.cuda.stream(stream):
        for f in st.step_fns(0):
            f()
        stream.synchronize()
        per = time_per_call(st, stream, max(4, args.roofline_reps // 4), 4,
                            trunc_counts(batches), True)
    prof = committed_profile(DEFAULT_WORKLOAD) or {}
    for k, v in per.items():
        if k in prof:
            v["rocprof_us"] = prof[k]
            v["rocprof_frac"] = round(v["alg_bytes"] / prof[k] / 1e3 / HBM_PEAK_GBPS, 4)
    del st
    return per


if __name__ == "__main__":
    main()
