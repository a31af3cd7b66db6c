"""Python binding of liblrs.so: the seven estimators and the generic
segmented affine scan on torch tensors (float32, bfloat16 or float16 data;
the dtype of the first data tensor picks the _f32 / _bf16 / _f16 entry).
Per-step tensors are [num_envs, seq_len]; with time_major=True they are
[seq_len, num_envs] and the _tm_ entry points run (outputs in the same
layout); per-env tensors are [num_envs] either way.

Argument marshalling only: every step of every estimator runs in the gfx950
kernels behind the C ABI (include/lrs.h).  torch supplies device memory and
the current stream.  There is no CPU path: calling any compute_* function
without the built library, or on tensors that are not on a GPU, raises.

Strided views.  A per-step tensor whose last dimension has unit stride and
whose rows do not overlap (for example buffer[:, :T] of a wider rollout
buffer, or a column slice of a time-major buffer) is passed in place with its
own row stride: no copy is made.  Any other layout (a transposed view, a
stride along the last dimension other than 1) is first copied with
.contiguous(), which costs one extra read and write of that tensor in HBM
outside the kernel.  out= tensors must already have unit inner stride.

Names and keyword arguments follow the rl-triton README (Kernels table and
Usage section): compute_gae(rewards, values, terminateds, gamma, lambda_).
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

import torch

from . import build as _build

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_F = ctypes.c_float
_SZ = ctypes.c_size_t

# every call ends with (strides, workspace, workspace_bytes, stream)
_TAIL = [_P, _P, _SZ, _P]
_BASE_SIGS = {
    "lrs_gae_f32": [_I64, _I64, _P, _P, _P, _P, _P, _P, _F, _F, _P] + _TAIL,
    "lrs_vtrace_f32": [_I64, _I64, _P, _P, _P, _P, _P, _P, _P, _F, _F, _F, _F, _F, _P, _P] + _TAIL,
    "lrs_retrace_f32": [_I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _F, _F, _F, _P] + _TAIL,
    "lrs_lambda_returns_f32": [_I64, _I64, _P, _P, _P, _P, _P, _P, _F, _F, _P] + _TAIL,
    "lrs_discounted_returns_f32": [_I64, _I64, _P, _P, _P, _P, _P, _F, _P] + _TAIL,
    "lrs_eligibility_traces_f32": [_I64, _I64, _P, _P, _F, _F, _P] + _TAIL,
    "lrs_episodic_prefix_sum_i32": [_I64, _I64, _P, _P, _P] + _TAIL,
    "lrs_episodic_prefix_sum_f32": [_I64, _I64, _P, _P, _P] + _TAIL,
    "lrs_affine_scan_f32": [_I64, _I64, _P, _P, _P, _P, ctypes.c_int, _P] + _TAIL,
}
# the 16-bit variants take the same arguments (pointers to 16-bit data), and
# so do the time-major (_tm_) variants of every call
_SIGS = dict(_BASE_SIGS)
for _name, _args in _BASE_SIGS.items():
    if _name.endswith("_f32"):
        for _sfx in ("bf16", "f16"):
            _SIGS[_name[:-3] + _sfx] = _args
for _name, _args in list(_SIGS.items()):
    _stem, _sfx = _name.rsplit("_", 1)
    _SIGS[f"{_stem}_tm_{_sfx}"] = _args

# storage dtype of the floating-point streams -> entry-point suffix
_SUFFIX = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16"}


def _suffix(x, name):
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    try:
        return _SUFFIX[x.dtype]
    except KeyError:
        raise TypeError(f"{name} must be float32, bfloat16 or float16, got {x.dtype}") from None

ESTIMATOR_ID = {"gae": 0, "vtrace": 1, "retrace": 2, "lambda_returns": 3,
                "discounted_returns": 4, "eligibility_traces": 5, "prefix_sum_i32": 6,
                "prefix_sum_f32": 7, "affine_scan": 8}

_lib = None
_lock = threading.Lock()


class LrsError(RuntimeError):
    pass


def lib_path() -> str:
    return _build.LIB


def load():
    """Load liblrs.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = _build.LIB
        if not os.path.exists(path):
            raise LrsError(f"{path} is not built: run `python -m linear_recurrence_scan_env_amd.build`"
                           " (there is no CPU fallback)")
        lib = ctypes.CDLL(path)
        for name, args in _SIGS.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        lib.lrs_version.restype = ctypes.c_int
        lib.lrs_status_string.restype = ctypes.c_char_p
        lib.lrs_status_string.argtypes = [ctypes.c_int]
        lib.lrs_last_error.restype = ctypes.c_char_p
        lib.lrs_workspace_bytes.restype = _SZ
        lib.lrs_workspace_bytes.argtypes = [ctypes.c_int, _I64, _I64]
        lib.lrs_debug_set_schedule.restype = ctypes.c_int
        lib.lrs_debug_set_schedule.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
        lib.lrs_debug_set_time_major_waves.argtypes = [ctypes.c_int]
        _check_single_hip_runtime()
        _lib = lib
    return _lib


def _check_single_hip_runtime():
    """Two different libamdhip64 images in one process would make torch's
    stream handles meaningless to the library: refuse to run then."""
    try:
        with open("/proc/self/maps") as f:
            paths = {line.split()[-1] for line in f if "libamdhip64" in line}
    except OSError:
        return
    real = {os.path.realpath(p) for p in paths}
    if len(real) > 1:
        raise LrsError(f"more than one HIP runtime is loaded: {sorted(real)}")


def _check(status: int, name: str):
    if status != 0:
        lib = load()
        msg = lib.lrs_last_error().decode()
        kind = lib.lrs_status_string(status).decode()
        if status in (1, 2):
            raise ValueError(f"{name}: {kind}: {msg}")
        raise LrsError(f"{name}: {kind}: {msg}")


def set_schedule(force_lookback: bool = False, elems_per_lane: int = 0, waves_per_block: int = 0):
    """Diagnostics: force the carry-propagation path and/or a fixed tile."""
    _check(load().lrs_debug_set_schedule(int(force_lookback), int(elems_per_lane),
                                         int(waves_per_block)), "set_schedule")


def set_time_major_waves(waves_per_block: int = 0):
    """Diagnostics: waves per block of the time-major calls (2, 4, 8 or 16: tiles of
    16 to 128 steps of 64 environments; 0 = automatic, which also uses blocks of 32
    environments for rows of up to 128 steps when there are few environments)."""
    _check(load().lrs_debug_set_time_major_waves(int(waves_per_block)), "set_time_major_waves")


# ------------------------------------------------------------ marshalling

_workspaces = {}
# Workspaces replaced by larger ones stay allocated: a HIP graph captured
# earlier keeps the pointer it saw, and its replays still use that memory.
_retired = []


def workspace(device: torch.device, stream: torch.cuda.Stream, est: str, n: int, t: int):
    """Zero-filled workspace cached per (device, stream), grown on demand.
    Under graph capture, run each call eagerly on the capture stream first,
    so that capturing allocates nothing.

    Calls that share a workspace must run one after another: its header
    counts the blocks of one launch at a time.  Eager calls on one stream are
    ordered by the stream.  A graph captured on a stream keeps that stream's
    workspace, and replays run on the caller's current stream, so graphs
    captured on the same stream (torch.cuda.graph uses one shared side stream
    unless given another) must be replayed one after another, and not beside
    eager calls issued on their capture stream.  Replaying such graphs
    concurrently on different streams races: carry waits then give up and the
    affected outputs are NaN, with the header's error word set (see
    workspace_state).  To replay graphs concurrently, capture each on its own
    stream."""
    need = int(load().lrs_workspace_bytes(ESTIMATOR_ID[est], n, t))
    key = (device.index, stream.cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < need:
        if ws is not None:
            _retired.append(ws)
        ws = torch.zeros(max(need, 4096), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def workspace_state():
    """Diagnostics: synchronize, then read the header of every cached workspace.
    Returns a list of dicts: epoch (launches that used the carry protocol),
    error (nonzero: a carry wait gave up, bit 2 = timeout), top and
    counters_nonzero (both 0 between launches: every launch resets them), and
    epochs_in_step (every count word carries the header's epoch)."""
    import numpy as np
    torch.cuda.synchronize()
    out = []
    for ws in _workspaces.values():
        h = ws[:4224].cpu().numpy().view(np.uint32)
        counts = h[32::32][:32]  # count words, one per 128-byte line after the first:
        epochs = h[33::32][:32]  # low half the count, high half the epoch
        out.append({"epoch": int(h[0]), "error": int(h[1]), "top": int(h[2]),
                    "counters_nonzero": int(np.count_nonzero(counts)),
                    "epochs_in_step": bool((epochs == h[0]).all())})
    return out


def _checked(x, name, dtype, shape, device):
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if x.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (there is no CPU path)")
    if device is not None and x.device != device:
        raise ValueError(f"{name} is on {x.device}, expected {device}")
    if x.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {x.dtype}")
    if shape is not None and tuple(x.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(x.shape)}")
    return x


def _dev_tensor(x, name, dtype, shape, device):
    """A per-env tensor (contiguous, copied if it is not)."""
    return _checked(x, name, dtype, shape, device).contiguous()


def _row_stride(x):
    """Row stride of a 2-D tensor the kernels can read in place (unit stride
    along the last dimension, rows that do not overlap), else None."""
    rows, cols = x.shape
    if cols > 1 and x.stride(1) != 1:
        return None
    if rows == 1:
        return cols
    return x.stride(0) if x.stride(0) >= cols else None


class _Step:
    """A per-step [rows, cols] tensor as passed to a call: the tensor (a view
    of the caller's memory, or a contiguous copy when its layout cannot be
    read in place) and its row stride."""
    __slots__ = ("t", "ld")

    def __init__(self, t, ld):
        self.t, self.ld = t, ld


def _step(x, name, dtype, shape, device):
    x = _checked(x, name, dtype, shape, device)
    ld = _row_stride(x)
    if ld is None:
        x = x.contiguous()
        ld = x.shape[1]
    return _Step(x, ld)


def _strides(*arrays):
    """The strides argument of a call: None when every array is contiguous,
    else a host int64 array in signature order (0 for absent arrays)."""
    vals = [0 if a is None else a.ld for a in arrays]
    cols = next(a.t.shape[1] for a in arrays if a is not None)
    if all(v in (0, cols) for v in vals):
        return None
    return (ctypes.c_int64 * len(vals))(*vals)


def _mask(x, name, shape, device):
    """bool/uint8 masks pass through (strided views in place); other dtypes
    become (x != 0) first."""
    if x is None:
        return None
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if x.dtype == torch.bool:
        x = x.view(torch.uint8)
    elif x.dtype != torch.uint8:
        x = (x != 0).view(torch.uint8)
    return _step(x, name, torch.uint8, shape, device)


def _ptr(x):
    if x is None:
        return None
    return x.t.data_ptr() if isinstance(x, _Step) else x.data_ptr()


def _rows(x, name, time_major=False):
    """(num_envs, seq_len, shape of the per-step arrays)."""
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        layout = "[seq_len, num_envs]" if time_major else "[num_envs, seq_len]"
        raise ValueError(f"{name} must be a 2-D {layout} tensor")
    if time_major:
        return x.shape[1], x.shape[0], (x.shape[0], x.shape[1])
    return x.shape[0], x.shape[1], (x.shape[0], x.shape[1])


def _entry(stem, sfx, time_major):
    return getattr(load(), f"{stem}_tm_{sfx}" if time_major else f"{stem}_{sfx}")


def _prep_boundary(shape, n, device, dtype, terminateds, truncateds, trunc_values,
                   bootstrap_value):
    term = _mask(terminateds, "terminateds", shape, device)
    if term is None:
        raise ValueError("terminateds is required")
    trunc = _mask(truncateds, "truncateds", shape, device)
    tv = None
    if trunc is not None:
        if trunc_values is None:
            raise ValueError("truncateds given without trunc_values")
        tv = _step(trunc_values, "trunc_values", dtype, shape, device)
    boot = None
    if bootstrap_value is not None:
        boot = _dev_tensor(bootstrap_value, "bootstrap_value", dtype, (n,), device)
    return term, trunc, tv, boot


def _out(out, like, name):
    """The output: a new contiguous tensor, or the caller's out= tensor in
    place (unit stride along its last dimension, rows not overlapping)."""
    if out is None:
        return _Step(torch.empty(like.t.shape, dtype=like.t.dtype, device=like.t.device),
                     like.t.shape[1])
    o = _checked(out, name, like.t.dtype, like.t.shape, like.t.device)
    ld = _row_stride(o)
    if ld is None:
        raise ValueError(f"{name} must have unit stride along its last dimension and "
                         "non-overlapping rows")
    return _Step(o, ld)


def _launch_ctx(device, est, n, t):
    stream = torch.cuda.current_stream(device)
    ws = workspace(device, stream, est, n, t)
    return ws, ws.numel(), stream.cuda_stream


def compute_gae(rewards, values, terminateds, gamma=0.99, lambda_=0.95, *, truncateds=None,
                trunc_values=None, bootstrap_value=None, out=None,
                time_major=False):
    """Generalized advantage estimates, [num_envs, seq_len], in the dtype of
    rewards (float32, bfloat16 or float16; every float input must match)."""
    n, t, shape = _rows(rewards, "rewards", time_major)
    dev, sfx, dt = rewards.device, _suffix(rewards, "rewards"), rewards.dtype
    r = _step(rewards, "rewards", dt, shape, None)
    v = _step(values, "values", dt, shape, dev)
    term, trunc, tv, boot = _prep_boundary(shape, n, dev, dt, terminateds, truncateds,
                                           trunc_values, bootstrap_value)
    adv = _out(out, r, "out")
    ws, wsb, st = _launch_ctx(dev, "gae", n, t)
    fn = _entry("lrs_gae", sfx, time_major)
    _check(fn(n, t, _ptr(r), _ptr(v), _ptr(term), _ptr(trunc), _ptr(tv),
              _ptr(boot), gamma, lambda_, _ptr(adv), _strides(r, v, term, trunc, tv, adv),
              _ptr(ws), wsb, st),
           "compute_gae")
    return adv.t


def compute_vtrace(log_rhos, rewards, values, terminateds, gamma=0.99, lambda_=1.0, *,
                   rho_bar=1.0, c_bar=1.0, pg_rho_bar=None, truncateds=None, trunc_values=None,
                   bootstrap_value=None, out=None, time_major=False):
    """V-trace targets and policy-gradient advantages: returns (vs, pg_advantages)."""
    n, t, shape = _rows(rewards, "rewards", time_major)
    dev, sfx, dt = rewards.device, _suffix(rewards, "rewards"), rewards.dtype
    r = _step(rewards, "rewards", dt, shape, None)
    lr = _step(log_rhos, "log_rhos", dt, shape, dev)
    v = _step(values, "values", dt, shape, dev)
    term, trunc, tv, boot = _prep_boundary(shape, n, dev, dt, terminateds, truncateds,
                                           trunc_values, bootstrap_value)
    vs = _out(None if out is None else out[0], r, "out[0]")
    pg = _out(None if out is None else out[1], r, "out[1]")
    if pg_rho_bar is None:
        pg_rho_bar = rho_bar
    ws, wsb, st = _launch_ctx(dev, "vtrace", n, t)
    fn = _entry("lrs_vtrace", sfx, time_major)
    _check(fn(n, t, _ptr(lr), _ptr(r), _ptr(v), _ptr(term), _ptr(trunc),
              _ptr(tv), _ptr(boot), gamma, lambda_, _inf(rho_bar), _inf(c_bar),
              _inf(pg_rho_bar), _ptr(vs), _ptr(pg), _strides(lr, r, v, term, trunc, tv, vs, pg),
              _ptr(ws), wsb, st),
           "compute_vtrace")
    return vs.t, pg.t


def compute_retrace(log_rhos, rewards, q_values, values, terminateds, gamma=0.99, lambda_=0.95, *,
                    c_bar=1.0, truncateds=None, trunc_values=None, bootstrap_value=None, out=None,
                    time_major=False):
    """Retrace(lambda) targets for Q(s_t, a_t); values = E_pi Q(s_t, .)."""
    n, t, shape = _rows(rewards, "rewards", time_major)
    dev, sfx, dt = rewards.device, _suffix(rewards, "rewards"), rewards.dtype
    r = _step(rewards, "rewards", dt, shape, None)
    lr = _step(log_rhos, "log_rhos", dt, shape, dev)
    q = _step(q_values, "q_values", dt, shape, dev)
    v = _step(values, "values", dt, shape, dev)
    term, trunc, tv, boot = _prep_boundary(shape, n, dev, dt, terminateds, truncateds,
                                           trunc_values, bootstrap_value)
    g = _out(out, r, "out")
    ws, wsb, st = _launch_ctx(dev, "retrace", n, t)
    fn = _entry("lrs_retrace", sfx, time_major)
    _check(fn(n, t, _ptr(lr), _ptr(r), _ptr(q), _ptr(v), _ptr(term),
              _ptr(trunc), _ptr(tv), _ptr(boot), gamma, lambda_, _inf(c_bar),
              _ptr(g), _strides(lr, r, q, v, term, trunc, tv, g), _ptr(ws), wsb, st),
           "compute_retrace")
    return g.t


def compute_lambda_returns(rewards, values, terminateds, gamma=0.99, lambda_=0.95, *,
                           truncateds=None, trunc_values=None, bootstrap_value=None, out=None,
                           time_major=False):
    """TD(lambda) returns."""
    n, t, shape = _rows(rewards, "rewards", time_major)
    dev, sfx, dt = rewards.device, _suffix(rewards, "rewards"), rewards.dtype
    r = _step(rewards, "rewards", dt, shape, None)
    v = _step(values, "values", dt, shape, dev)
    term, trunc, tv, boot = _prep_boundary(shape, n, dev, dt, terminateds, truncateds,
                                           trunc_values, bootstrap_value)
    g = _out(out, r, "out")
    ws, wsb, st = _launch_ctx(dev, "lambda_returns", n, t)
    fn = _entry("lrs_lambda_returns", sfx, time_major)
    _check(fn(n, t, _ptr(r), _ptr(v), _ptr(term), _ptr(trunc),
              _ptr(tv), _ptr(boot), gamma, lambda_, _ptr(g),
              _strides(r, v, term, trunc, tv, g), _ptr(ws), wsb, st),
           "compute_lambda_returns")
    return g.t


def compute_discounted_returns(rewards, terminateds, gamma=0.99, *, truncateds=None,
                               trunc_values=None, bootstrap_value=None, out=None,
                               time_major=False):
    """Discounted reward-to-go."""
    n, t, shape = _rows(rewards, "rewards", time_major)
    dev, sfx, dt = rewards.device, _suffix(rewards, "rewards"), rewards.dtype
    r = _step(rewards, "rewards", dt, shape, None)
    term, trunc, tv, boot = _prep_boundary(shape, n, dev, dt, terminateds, truncateds,
                                           trunc_values, bootstrap_value)
    g = _out(out, r, "out")
    ws, wsb, st = _launch_ctx(dev, "discounted_returns", n, t)
    fn = _entry("lrs_discounted_returns", sfx, time_major)
    _check(fn(n, t, _ptr(r), _ptr(term), _ptr(trunc), _ptr(tv),
              _ptr(boot), gamma, _ptr(g), _strides(r, term, trunc, tv, g), _ptr(ws), wsb, st),
           "compute_discounted_returns")
    return g.t


def compute_eligibility_traces(x, dones, gamma=0.99, lambda_=0.95, *, out=None,
                               time_major=False):
    """Accumulating eligibility traces, forward in time (dtype of x)."""
    n, t, shape = _rows(x, "x", time_major)
    dev, sfx = x.device, _suffix(x, "x")
    xs = _step(x, "x", x.dtype, shape, None)
    d = _mask(dones, "dones", shape, dev)
    if d is None:
        raise ValueError("dones is required")
    e = _out(out, xs, "out")
    ws, wsb, st = _launch_ctx(dev, "eligibility_traces", n, t)
    fn = _entry("lrs_eligibility_traces", sfx, time_major)
    _check(fn(n, t, _ptr(xs), _ptr(d), gamma, lambda_, _ptr(e), _strides(xs, d, e),
              _ptr(ws), wsb, st), "compute_eligibility_traces")
    return e.t


def compute_episodic_prefix_sum(x, dones, *, out=None, time_major=False):
    """Inclusive prefix sum with done resets; int32 (exact), float32, bfloat16
    or float16 input, output of the same dtype."""
    n, t, shape = _rows(x, "x", time_major)
    dev = x.device
    if isinstance(x, torch.Tensor) and x.dtype == torch.int32:
        xs = _step(x, "x", torch.int32, shape, None)
        fn, est = _entry("lrs_episodic_prefix_sum", "i32", time_major), "prefix_sum_i32"
    else:
        sfx = _suffix(x, "x")
        xs = _step(x, "x", x.dtype, shape, None)
        fn, est = _entry("lrs_episodic_prefix_sum", sfx, time_major), "prefix_sum_f32"
    d = _mask(dones, "dones", shape, dev)
    if d is None:
        raise ValueError("dones is required")
    s = _out(out, xs, "out")
    ws, wsb, st = _launch_ctx(dev, est, n, t)
    _check(fn(n, t, _ptr(xs), _ptr(d), _ptr(s), _strides(xs, d, s), _ptr(ws), wsb, st),
           "compute_episodic_prefix_sum")
    return s.t


def compute_affine_scan(alpha, beta, *, reset=None, carry_in=None, reverse=False, out=None,
                        time_major=False):
    """Segmented first-order linear recurrence over given coefficients, per row:
    y_t = alpha_t + beta_t * y_{t-1} (forward) or y_t = alpha_t + beta_t * y_{t+1}
    (reverse=True).  carry_in [num_envs] is the y before each row's first step
    in scan order (0 if None); where reset is set, y_t = alpha_t."""
    n, t, shape = _rows(alpha, "alpha", time_major)
    dev, sfx, dt = alpha.device, _suffix(alpha, "alpha"), alpha.dtype
    a = _step(alpha, "alpha", dt, shape, None)
    b = _step(beta, "beta", dt, shape, dev)
    rs = _mask(reset, "reset", shape, dev)
    c = None if carry_in is None else _dev_tensor(carry_in, "carry_in", dt, (n,), dev)
    y = _out(out, a, "out")
    ws, wsb, st = _launch_ctx(dev, "affine_scan", n, t)
    _check(_entry("lrs_affine_scan", sfx, time_major)(n, t, _ptr(a), _ptr(b), _ptr(rs), _ptr(c),
                                                      1 if reverse else 0, _ptr(y),
                                                      _strides(a, b, rs, y), _ptr(ws), wsb, st),
           "compute_affine_scan")
    return y.t


def _inf(x):
    x = float(x)
    return math.inf if math.isinf(x) and x > 0 else x
