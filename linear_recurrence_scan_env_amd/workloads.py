"""Seeded synthetic rollout generators.

This module holds no arithmetic of the estimators: it only draws random
arrays with the shapes and distributions of the benchmark workloads, so the
same bytes can be fed to the HIP library and to any CPU reference.

Every named stream comes from its own generator,
``numpy.random.default_rng([seed, STREAM_KEY[name]])``, so a stream's values
do not depend on which other streams a workload draws.

Layout: every per-step array is ``[num_envs, seq_len]`` row-major
(contiguous along time); floats are float32, masks uint8 (0/1), integer
inputs int32; ``bootstrap_value`` is ``[num_envs]`` float32.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

STREAM_KEY = {
    "rewards": 1, "values": 2, "q_values": 3, "log_rhos": 4,
    "terminateds": 5, "truncateds": 6, "trunc_values": 7,
    "bootstrap_value": 8, "x": 9, "x_int": 10, "dones": 11,
    "alpha": 12, "beta": 13, "reset": 14, "carry_in": 15,
}


def _rng(seed: int, name: str) -> np.random.Generator:
    return np.random.default_rng([int(seed), STREAM_KEY[name]])


def normal(seed, name, shape, sigma=1.0):
    a = _rng(seed, name).standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    return a


def bernoulli(seed, name, shape, p):
    return (_rng(seed, name).random(shape, dtype=np.float64) < p).astype(np.uint8)


def uniform(seed, name, shape, lo, hi):
    """Floats uniform on [lo, hi), float32."""
    return _rng(seed, name).uniform(lo, hi, size=shape).astype(np.float32)


def uniform_int(seed, name, shape, lo, hi):
    """Integers uniform on [lo, hi] inclusive, int32."""
    return _rng(seed, name).integers(lo, hi, size=shape, endpoint=True, dtype=np.int32)


@dataclass
class Rollout:
    """One synthetic batch; absent streams are None."""
    num_envs: int
    seq_len: int
    gamma: float
    lambda_: float
    arrays: dict = field(default_factory=dict)

    def __getitem__(self, k):
        return self.arrays.get(k)


def rollout(num_envs, seq_len, *, seed=0, term_p=0.01, trunc_p=0.0, logrho_sigma=0.5,
            gamma=0.99, lambda_=0.95, bootstrap=True, streams=None, int_range=(-1000, 1000),
            done_p=None):
    """Draw a batch.  ``streams`` limits which arrays are drawn (default: all).

    Distributions: rewards, values, q_values, trunc_values, bootstrap_value,
    x ~ N(0,1); log_rhos ~ N(0, logrho_sigma^2); terminateds ~ Bern(term_p);
    truncateds ~ Bern(trunc_p) (absent when trunc_p == 0); dones ~
    Bern(done_p, default term_p); x_int ~ U{int_range}.
    """
    shape = (int(num_envs), int(seq_len))
    want = set(streams) if streams is not None else set(STREAM_KEY)
    a = {}
    for name in ("rewards", "values", "q_values", "x"):
        if name in want:
            a[name] = normal(seed, name, shape)
    if "log_rhos" in want:
        a["log_rhos"] = normal(seed, "log_rhos", shape, logrho_sigma)
    if "terminateds" in want:
        a["terminateds"] = bernoulli(seed, "terminateds", shape, term_p)
    if trunc_p > 0 and "truncateds" in want:
        a["truncateds"] = bernoulli(seed, "truncateds", shape, trunc_p)
        a["trunc_values"] = normal(seed, "trunc_values", shape)
    if bootstrap and "bootstrap_value" in want:
        a["bootstrap_value"] = normal(seed, "bootstrap_value", (shape[0],))
    if "dones" in want:
        a["dones"] = bernoulli(seed, "dones", shape, term_p if done_p is None else done_p)
    if "x_int" in want:
        a["x_int"] = uniform_int(seed, "x_int", shape, *int_range)
    return Rollout(shape[0], shape[1], float(np.float32(gamma)), float(np.float32(lambda_)), a)


def affine_inputs(num_envs, seq_len, *, seed=0, reset_p=0.02, beta_range=(0.9, 1.0),
                  carry=True):
    """Coefficients for the generic affine scan: alpha ~ N(0,1), beta ~
    U[beta_range), reset ~ Bern(reset_p) (None when reset_p == 0), carry_in ~
    N(0,1) per env (None unless carry)."""
    shape = (int(num_envs), int(seq_len))
    return {
        "alpha": normal(seed, "alpha", shape),
        "beta": uniform(seed, "beta", shape, *beta_range),
        "reset": bernoulli(seed, "reset", shape, reset_p) if reset_p > 0 else None,
        "carry_in": normal(seed, "carry_in", (shape[0],)) if carry else None,
    }


# The benchmark workloads, as (name, sizes, drawing parameters).
WORKLOADS = {
    # GAE, 64 x 512, terminations Bern(0.01), no truncations.
    "gae_64x512": dict(num_envs=64, seq_len=512, term_p=0.01, trunc_p=0.0,
                       gamma=0.99, lambda_=0.95),
    # All seven estimators, 4096 x 128, terminations Bern(1/64); the
    # truncating pass adds truncations Bern(1/128).
    "all7_4096x128": dict(num_envs=4096, seq_len=128, term_p=1 / 64, trunc_p=1 / 128,
                          gamma=0.99, lambda_=0.95),
    # GAE / V-trace / Retrace, 64 x 131072, Bern(1e-4) terminations and truncations.
    "long_64x131072": dict(num_envs=64, seq_len=131072, term_p=1e-4, trunc_p=1e-4,
                           gamma=0.99, lambda_=0.95),
    # Sequence sweep for discounted / TD(lambda) / traces, done Bern(0.02).
    "sweep_4096xT": dict(num_envs=4096, seq_len=(32, 128, 512, 2048, 8192), term_p=0.02,
                         trunc_p=0.0, gamma=0.99, lambda_=0.9),
    # Episodic prefix sum, 16384 x 1024, done Bern(0.02), int32 in [-1000, 1000].
    "prefix_16384x1024": dict(num_envs=16384, seq_len=1024, term_p=0.02, trunc_p=0.0,
                              gamma=1.0, lambda_=1.0),
    # Generic affine scan over stored coefficients, both directions, 4096 x
    # 8192: beta ~ U[0.9, 1), resets Bern(0.02), a carry per env.
    "affine_4096x8192": dict(num_envs=4096, seq_len=8192, reset_p=0.02, beta_range=(0.9, 1.0)),
}


def device_stream(seed, name, shape, device, *, kind, p=None, sigma=1.0, lo=-1000, hi=1000,
                  chunk=1 << 28):
    """Draws one stream straight into device memory, for arrays too large to
    draw on the host (billions of elements).  torch's device generator (Philox)
    is seeded with ``(seed << 8) | STREAM_KEY[name]`` and fills the flat array
    in chunks of ``chunk`` elements, in order, so the values depend only on
    (seed, name, shape).  The values are not the numpy draws of the same seed.

    kind: "normal" -> float32 N(0, sigma^2); "bernoulli" -> uint8 with
    P(1) = p; "int" -> int32 uniform on [lo, hi] inclusive.
    """
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed((int(seed) << 8) | STREAM_KEY[name])
    dtype = {"normal": torch.float32, "bernoulli": torch.uint8, "int": torch.int32}[kind]
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    for s in range(0, flat.numel(), chunk):
        n = min(chunk, flat.numel() - s)
        if kind == "normal":
            flat[s:s + n].normal_(0.0, sigma, generator=gen)
        elif kind == "bernoulli":
            flat[s:s + n] = torch.rand(n, generator=gen, device=device) < p
        else:
            flat[s:s + n].random_(lo, hi + 1, generator=gen)
    return out
