"""fp64 CPU oracle for the seven RL credit-assignment estimators and the
generic segmented affine scan they reduce to.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import this package.  The product
library never loads it and has no CPU fallback.

The arithmetic lives in ``lrs_oracle.c`` (plain sequential recursions in
double precision, one function per estimator, each citing the passage it
follows).  This module only builds that file with gcc, loads it with ctypes
and marshals numpy arrays.  It shares no code with the HIP path.

Inputs are the exact fp32 / uint8 / int32 arrays the GPU reads; scalars are
doubles.  Parity tests pass fp32-rounded scalars (``float(np.float32(g))``)
so both sides use the same gamma and lambda.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lrs_oracle.c")
_LIB = os.path.join(_HERE, "liblrs_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile lrs_oracle.c into liblrs_oracle.so next to it (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-shared", "-fPIC",
               "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def compile_variant(src_text: str, out_path: str) -> str:
    """Compile a modified copy of the oracle source (used by the mutation test)."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O1", "-std=c99", "-fopenmp", "-shared", "-fPIC", src, "-o",
                    out_path, "-lm"], check=True, capture_output=True)
    return out_path


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


@contextlib.contextmanager
def use_library(path: str):
    """Temporarily route every oracle call through another compiled variant."""
    global _lib
    saved = _lib
    _lib = _open(path)
    try:
        yield
    finally:
        _lib = saved


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build(force=True)
    _lib = _open(_LIB)
    return _lib


def _open(path):
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int64
    D = ctypes.c_double
    sig = {
        "lrs_oracle_gae": [I, I, P, P, P, P, P, P, D, D, P],
        "lrs_oracle_lambda_returns": [I, I, P, P, P, P, P, P, D, D, P],
        "lrs_oracle_discounted_returns": [I, I, P, P, P, P, P, D, P],
        "lrs_oracle_vtrace": [I, I, P, P, P, P, P, P, P, D, D, D, D, D, P, P],
        "lrs_oracle_retrace": [I, I, P, P, P, P, P, P, P, P, D, D, D, P],
        "lrs_oracle_eligibility_traces": [I, I, P, P, D, D, P],
        "lrs_oracle_prefix_sum_f32": [I, I, P, P, P],
        "lrs_oracle_prefix_sum_i32": [I, I, P, P, P],
        "lrs_oracle_affine_scan": [I, I, P, P, P, P, ctypes.c_int, P],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = None
    lib.lrs_oracle_threads.restype = ctypes.c_int
    return lib


def threads() -> int:
    """OpenMP threads the oracle's parallel loop over environments uses."""
    return int(_load().lrs_oracle_threads())


def _f32(a, shape=None):
    a = np.ascontiguousarray(a, dtype=np.float32)
    if shape is not None and a.shape != shape:
        raise ValueError(f"expected shape {shape}, got {a.shape}")
    return a


def _mask(a, shape):
    if a is None:
        return None
    a = np.ascontiguousarray(np.asarray(a) != 0, dtype=np.uint8)
    if a.shape != shape:
        raise ValueError(f"expected shape {shape}, got {a.shape}")
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data


def _boundary(shape, terminateds, truncateds, trunc_values, bootstrap_value):
    n, _ = shape
    term = _mask(terminateds, shape)
    trunc = _mask(truncateds, shape)
    tv = None
    if trunc is not None:
        if trunc_values is None:
            raise ValueError("truncateds given without trunc_values")
        tv = _f32(trunc_values, shape)
    boot = None if bootstrap_value is None else _f32(bootstrap_value, (n,))
    return term, trunc, tv, boot


def gae(rewards, values, terminateds, gamma, lambda_, *, truncateds=None,
        trunc_values=None, bootstrap_value=None):
    r = _f32(rewards)
    v = _f32(values, r.shape)
    term, trunc, tv, boot = _boundary(r.shape, terminateds, truncateds, trunc_values, bootstrap_value)
    out = np.empty(r.shape, np.float64)
    _load().lrs_oracle_gae(r.shape[0], r.shape[1], _ptr(r), _ptr(v), _ptr(term), _ptr(trunc),
                           _ptr(tv), _ptr(boot), float(gamma), float(lambda_), _ptr(out))
    return out


def lambda_returns(rewards, values, terminateds, gamma, lambda_, *, truncateds=None,
                   trunc_values=None, bootstrap_value=None):
    r = _f32(rewards)
    v = _f32(values, r.shape)
    term, trunc, tv, boot = _boundary(r.shape, terminateds, truncateds, trunc_values, bootstrap_value)
    out = np.empty(r.shape, np.float64)
    _load().lrs_oracle_lambda_returns(r.shape[0], r.shape[1], _ptr(r), _ptr(v), _ptr(term),
                                      _ptr(trunc), _ptr(tv), _ptr(boot), float(gamma),
                                      float(lambda_), _ptr(out))
    return out


def discounted_returns(rewards, terminateds, gamma, *, truncateds=None, trunc_values=None,
                       bootstrap_value=None):
    r = _f32(rewards)
    term, trunc, tv, boot = _boundary(r.shape, terminateds, truncateds, trunc_values, bootstrap_value)
    out = np.empty(r.shape, np.float64)
    _load().lrs_oracle_discounted_returns(r.shape[0], r.shape[1], _ptr(r), _ptr(term),
                                          _ptr(trunc), _ptr(tv), _ptr(boot), float(gamma),
                                          _ptr(out))
    return out


def vtrace(log_rhos, rewards, values, terminateds, gamma, lambda_=1.0, *, rho_bar=1.0,
           c_bar=1.0, pg_rho_bar=None, truncateds=None, trunc_values=None,
           bootstrap_value=None):
    """Returns (vs, pg_advantages), both float64."""
    lr = _f32(log_rhos)
    r = _f32(rewards, lr.shape)
    v = _f32(values, lr.shape)
    term, trunc, tv, boot = _boundary(lr.shape, terminateds, truncateds, trunc_values, bootstrap_value)
    if pg_rho_bar is None:
        pg_rho_bar = rho_bar
    vs = np.empty(lr.shape, np.float64)
    pg = np.empty(lr.shape, np.float64)
    _load().lrs_oracle_vtrace(lr.shape[0], lr.shape[1], _ptr(lr), _ptr(r), _ptr(v), _ptr(term),
                              _ptr(trunc), _ptr(tv), _ptr(boot), float(gamma), float(lambda_),
                              float(rho_bar), float(c_bar), float(pg_rho_bar), _ptr(vs), _ptr(pg))
    return vs, pg


def retrace(log_rhos, rewards, q_values, values, terminateds, gamma, lambda_, *, c_bar=1.0,
            truncateds=None, trunc_values=None, bootstrap_value=None):
    lr = _f32(log_rhos)
    r = _f32(rewards, lr.shape)
    q = _f32(q_values, lr.shape)
    v = _f32(values, lr.shape)
    term, trunc, tv, boot = _boundary(lr.shape, terminateds, truncateds, trunc_values, bootstrap_value)
    out = np.empty(lr.shape, np.float64)
    _load().lrs_oracle_retrace(lr.shape[0], lr.shape[1], _ptr(lr), _ptr(r), _ptr(q), _ptr(v),
                               _ptr(term), _ptr(trunc), _ptr(tv), _ptr(boot), float(gamma),
                               float(lambda_), float(c_bar), _ptr(out))
    return out


def eligibility_traces(x, dones, gamma, lambda_):
    xs = _f32(x)
    d = _mask(dones, xs.shape)
    out = np.empty(xs.shape, np.float64)
    _load().lrs_oracle_eligibility_traces(xs.shape[0], xs.shape[1], _ptr(xs), _ptr(d),
                                          float(gamma), float(lambda_), _ptr(out))
    return out


def prefix_sum(x, dones):
    """Integer input -> int32 output (exact, modulo 2^32); float -> float64."""
    a = np.asarray(x)
    if np.issubdtype(a.dtype, np.integer):
        xs = np.ascontiguousarray(a, dtype=np.int32)
        d = _mask(dones, xs.shape)
        out = np.empty(xs.shape, np.int32)
        _load().lrs_oracle_prefix_sum_i32(xs.shape[0], xs.shape[1], _ptr(xs), _ptr(d), _ptr(out))
        return out
    xs = _f32(a)
    d = _mask(dones, xs.shape)
    out = np.empty(xs.shape, np.float64)
    _load().lrs_oracle_prefix_sum_f32(xs.shape[0], xs.shape[1], _ptr(xs), _ptr(d), _ptr(out))
    return out


def affine_scan(alpha, beta, *, reset=None, carry_in=None, reverse=False):
    """y_t = alpha_t + beta_t * y_prev along each row (prev = t-1, or t+1 when
    reverse); y_prev of the first step in scan order is carry_in[n] (0 if
    None); a nonzero reset[t] drops the beta_t * y_prev term.  float64 out."""
    a = _f32(alpha)
    b = _f32(beta, a.shape)
    rs = _mask(reset, a.shape)
    c = None if carry_in is None else _f32(carry_in, (a.shape[0],))
    out = np.empty(a.shape, np.float64)
    _load().lrs_oracle_affine_scan(a.shape[0], a.shape[1], _ptr(a), _ptr(b), _ptr(rs), _ptr(c),
                                   1 if reverse else 0, _ptr(out))
    return out
