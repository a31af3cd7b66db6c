"""Pins of the fp64 oracle against things other than itself (CPU only).

* brute force: O(T^2) sum definitions (tests/bruteforce.py) on tiny inputs;
* exact hand-worked values with dyadic inputs;
* closed forms and library routines (scipy.signal.lfilter IIR filter,
  numpy cumsum, geometric series);
* cross-estimator identities that hold by the definitions (TD(lambda) =
  GAE + V, on-policy V-trace = TD(lambda), on-policy Retrace = TD(lambda) on Q);
* the no-leakage invariant across episode boundaries (exact equality);
* the algebra of the combine operator: composition of affine maps is
  associative, and a tree-ordered scan reproduces the sequential recursion.
"""
import itertools

import numpy as np
import pytest
from scipy.signal import lfilter

import bruteforce as bf
import oracle

F32 = lambda x: float(np.float32(x))  # noqa: E731


def case(seed, N, T, p_term, p_trunc, boot=True, logrho_sigma=0.7):
    rng = np.random.default_rng(seed)
    d = dict(
        r=rng.standard_normal((N, T)).astype(np.float32),
        V=rng.standard_normal((N, T)).astype(np.float32),
        Q=rng.standard_normal((N, T)).astype(np.float32),
        lr=(logrho_sigma * rng.standard_normal((N, T))).astype(np.float32),
        term=(rng.random((N, T)) < p_term).astype(np.uint8),
        trunc=(rng.random((N, T)) < p_trunc).astype(np.uint8) if p_trunc > 0 else None,
        tv=rng.standard_normal((N, T)).astype(np.float32) if p_trunc > 0 else None,
        boot=rng.standard_normal(N).astype(np.float32) if boot else None,
        x=rng.standard_normal((N, T)).astype(np.float32),
    )
    return d


def kw(c):
    return dict(truncateds=c["trunc"], trunc_values=c["tv"], bootstrap_value=c["boot"])


def close(a, b, tol=1e-10):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape
    err = np.abs(a - b) / (1.0 + np.abs(b))
    assert err.max(initial=0.0) <= tol, f"max rel err {err.max()}"


# ---------------------------------------------------------------- brute force

GAMMAS = [0.0, 0.5, F32(0.99), 1.0]
LAMBDAS = [0.0, F32(0.95), 1.0]
SHAPES = [(1, 1), (2, 7), (3, 23), (2, 40)]
MASKS = [(0.0, 0.0), (0.15, 0.0), (0.1, 0.1), (0.5, 0.3)]


def brute_cases():
    seed = 0
    for (N, T), (pt, pk) in itertools.product(SHAPES, MASKS):
        for boot in (True, False):
            seed += 1
            yield seed, N, T, pt, pk, boot


@pytest.mark.parametrize("seed,N,T,pt,pk,boot", list(brute_cases()))
def test_bruteforce_backward(seed, N, T, pt, pk, boot):
    c = case(seed, N, T, pt, pk, boot)
    rng = np.random.default_rng(seed + 1000)
    g = GAMMAS[rng.integers(len(GAMMAS))]
    lam = LAMBDAS[rng.integers(len(LAMBDAS))]
    tk = dict(trunc=c["trunc"], tv=c["tv"], boot=c["boot"])
    close(oracle.gae(c["r"], c["V"], c["term"], g, lam, **kw(c)),
          bf.gae(c["r"], c["V"], c["term"], g, lam, **tk))
    close(oracle.discounted_returns(c["r"], c["term"], g, **kw(c)),
          bf.discounted(c["r"], c["term"], g, **tk))
    close(oracle.lambda_returns(c["r"], c["V"], c["term"], g, lam, **kw(c)),
          bf.lambda_returns(c["r"], c["V"], c["term"], g, lam, **tk))
    rho_bar, c_bar, pg_bar = [(1.0, 1.0, 1.0), (2.0, 0.5, 1.5), (np.inf, np.inf, np.inf)][seed % 3]
    vs, pg = oracle.vtrace(c["lr"], c["r"], c["V"], c["term"], g, lam, rho_bar=rho_bar,
                           c_bar=c_bar, pg_rho_bar=pg_bar, **kw(c))
    vs_b, pg_b = bf.vtrace(c["lr"], c["r"], c["V"], c["term"], g, lam, rho_bar, c_bar, pg_bar, **tk)
    close(vs, vs_b)
    close(pg, pg_b)
    close(oracle.retrace(c["lr"], c["r"], c["Q"], c["V"], c["term"], g, lam, c_bar=c_bar, **kw(c)),
          bf.retrace(c["lr"], c["r"], c["Q"], c["V"], c["term"], g, lam, c_bar, **tk))


@pytest.mark.parametrize("seed,N,T,pt", [(s, N, T, p) for s, ((N, T), p) in
                                         enumerate(itertools.product(SHAPES, [0.0, 0.1, 0.5]))])
def test_bruteforce_forward(seed, N, T, pt):
    c = case(seed, N, T, pt, 0.0)
    d = c["term"]
    for g, lam in [(0.0, 1.0), (0.5, 0.5), (F32(0.99), F32(0.9)), (1.0, 1.0)]:
        close(oracle.eligibility_traces(c["x"], d, g, lam), bf.eligibility(c["x"], d, g, lam))
    close(oracle.prefix_sum(c["x"], d), bf.prefix(c["x"], d))
    xi = np.random.default_rng(seed).integers(-1000, 1001, size=(N, T)).astype(np.int32)
    assert np.array_equal(oracle.prefix_sum(xi, d), bf.prefix(xi, d).astype(np.int32))


# ---------------------------------------------------------- hand-worked values

def test_hand_worked_gae():
    # gamma = lambda = 1/2, r = [1, 2, 3], V = 0, bootstrap 4, no cuts:
    # delta = [1, 2, 3 + 0.5*4] = [1, 2, 5]
    # A_2 = 5; A_1 = 2 + 0.25*5 = 3.25; A_0 = 1 + 0.25*3.25 = 1.8125
    r = np.array([[1, 2, 3]], np.float32)
    V = np.zeros((1, 3), np.float32)
    term = np.zeros((1, 3), np.uint8)
    out = oracle.gae(r, V, term, 0.5, 0.5, bootstrap_value=np.array([4], np.float32))
    assert out.tolist() == [[1.8125, 3.25, 5.0]]


def test_hand_worked_terminated_vs_truncated():
    # gamma = 1/2, lambda = 1, r = 1, V = [2, 2, 2, 2], cut after step 1.
    # Terminated at 1: successor value 0 -> delta_1 = 1 + 0 - 2 = -1,
    #   A_1 = -1, A_0 = (1 + 1 - 2) + 0.5*(-1) = -0.5 ; steps 2,3 (boot 8):
    #   delta_3 = 1 + 4 - 2 = 3, A_3 = 3, delta_2 = 1 + 1 - 2 = 0, A_2 = 1.5.
    # Truncated at 1 with trunc value 6: delta_1 = 1 + 3 - 2 = 2,
    #   A_1 = 2, A_0 = 0 + 0.5*2 = 1 ; steps 2,3 unchanged.
    r = np.ones((1, 4), np.float32)
    V = np.full((1, 4), 2, np.float32)
    cut = np.array([[0, 1, 0, 0]], np.uint8)
    none = np.zeros((1, 4), np.uint8)
    boot = np.array([8], np.float32)
    a_term = oracle.gae(r, V, cut, 0.5, 1.0, bootstrap_value=boot)
    assert a_term.tolist() == [[-0.5, -1.0, 1.5, 3.0]]
    a_trunc = oracle.gae(r, V, none, 0.5, 1.0, truncateds=cut,
                         trunc_values=np.full((1, 4), 6, np.float32), bootstrap_value=boot)
    assert a_trunc.tolist() == [[1.0, 2.0, 1.5, 3.0]]
    # Both set at once: termination wins (successor value 0).
    a_both = oracle.gae(r, V, cut, 0.5, 1.0, truncateds=cut,
                        trunc_values=np.full((1, 4), 6, np.float32), bootstrap_value=boot)
    assert a_both.tolist() == a_term.tolist()


def test_hand_worked_forward():
    # e_t = x_t + gamma*lambda*(1 - d_{t-1}) e_{t-1}, gamma*lambda = 1/4,
    # x = [4, 8, 16, 32], done at t=1 -> reset at t=2:
    # e = [4, 8 + 1, 16, 32 + 4] = [4, 9, 16, 36]
    x = np.array([[4, 8, 16, 32]], np.float32)
    d = np.array([[0, 1, 0, 0]], np.uint8)
    assert oracle.eligibility_traces(x, d, 0.5, 0.5).tolist() == [[4, 9, 16, 36]]
    assert oracle.prefix_sum(x, d).tolist() == [[4, 12, 16, 48]]
    assert oracle.prefix_sum(x.astype(np.int32), d).tolist() == [[4, 12, 16, 48]]


def test_hand_worked_retrace_and_vtrace():
    # Two steps, gamma = 1/2, lambda = 1, no cuts, bootstrap B = 2.
    # log-ratios 0 -> w = 1; r = [1, 1]; Q = [0, 4]; V = [0, 2].
    # Retrace: G_1 = r_1 + g*B = 2; G_0 = 1 + g*(V_1 + c_1*(G_1 - Q_1))
    #          = 1 + 0.5*(2 + (2 - 4)) = 1.
    z = np.zeros((1, 2), np.float32)
    r = np.ones((1, 2), np.float32)
    Q = np.array([[0, 4]], np.float32)
    V = np.array([[0, 2]], np.float32)
    boot = np.array([2], np.float32)
    term = np.zeros((1, 2), np.uint8)
    assert oracle.retrace(z, r, Q, V, term, 0.5, 1.0, bootstrap_value=boot).tolist() == [[1.0, 2.0]]
    # V-trace, rho = c = 1: A_1 = 1 + 1 - 2 = 0, vs_1 = 2; A_0 = (1 + 1 - 0) + 0.5*0 = 2, vs_0 = 2
    # pg_1 = 1 + 0.5*2 - 2 = 0; pg_0 = 1 + 0.5*vs_1 - 0 = 2
    vs, pg = oracle.vtrace(z, r, V, term, 0.5, 1.0, bootstrap_value=boot)
    assert vs.tolist() == [[2.0, 2.0]] and pg.tolist() == [[2.0, 0.0]]
    # Halve the target policy at step 0 (log-ratio -log 2 is not exact in
    # fp32, so use exact w via rho_bar clipping): rho_bar = c_bar = 0.5 with w = 1
    # gives rho_0 = rho_1 = 0.5, c = 0.5:
    # A_1 = 0.5*(1 + 1 - 2) = 0; A_0 = 0.5*2 + 0.5*0.5*0 = 1; vs = [1, 2]
    # pg (pg clip 0.5): pg_1 = 0.5*(0) = 0; pg_0 = 0.5*(1 + 0.5*2 - 0) = 1
    vs, pg = oracle.vtrace(z, r, V, term, 0.5, 1.0, rho_bar=0.5, c_bar=0.5,
                           bootstrap_value=boot)
    assert vs.tolist() == [[1.0, 2.0]] and pg.tolist() == [[1.0, 0.0]]


# ------------------------------------------------- closed forms and libraries

def segments(term_row, trunc_row=None):
    """(start, end) index pairs of the backward segments of one row."""
    T = len(term_row)
    ends = [t for t in range(T) if term_row[t] or (trunc_row is not None and trunc_row[t])
            or t == T - 1]
    out, s = [], 0
    for e in ends:
        out.append((s, e))
        s = e + 1
    return out


def vend_row(c, n, e):
    if c["term"][n, e]:
        return 0.0
    if c["trunc"] is not None and c["trunc"][n, e]:
        return float(c["tv"][n, e])
    return 0.0 if c["boot"] is None else float(c["boot"][n])


def mc_return_lfilter(c, gamma):
    """Per-segment discounted return with terminal bootstrap via an IIR filter."""
    r = c["r"].astype(np.float64)
    out = np.zeros_like(r)
    for n in range(r.shape[0]):
        for s, e in segments(c["term"][n], None if c["trunc"] is None else c["trunc"][n]):
            y = r[n, s:e + 1].copy()
            y[-1] += gamma * vend_row(c, n, e)
            out[n, s:e + 1] = lfilter([1.0], [1.0, -gamma], y[::-1])[::-1]
    return out


def vnext_array(c):
    V = c["V"].astype(np.float64)
    N, T = V.shape
    vn = np.zeros_like(V)
    vn[:, :-1] = V[:, 1:]
    for n in range(N):
        for t in range(T):
            end = c["term"][n, t] or (c["trunc"] is not None and c["trunc"][n, t]) or t == T - 1
            if end:
                vn[n, t] = vend_row(c, n, t)
    return vn


def end_array(c):
    e = c["term"].astype(bool).copy()
    if c["trunc"] is not None:
        e |= c["trunc"].astype(bool)
    e[:, -1] = True
    return e


@pytest.mark.parametrize("seed,pt,pk", [(1, 0.0, 0.0), (2, 0.05, 0.0), (3, 0.05, 0.05)])
def test_gae_lambda_limits(seed, pt, pk):
    c = case(seed, 4, 300, pt, pk)
    g = F32(0.99)
    # lambda = 1: A = Monte-Carlo return (bootstrapped at the episode end) - V
    a1 = oracle.gae(c["r"], c["V"], c["term"], g, 1.0, **kw(c))
    close(a1, mc_return_lfilter(c, g) - c["V"].astype(np.float64), 1e-11)
    # lambda = 0: A = one-step TD error
    a0 = oracle.gae(c["r"], c["V"], c["term"], g, 0.0, **kw(c))
    delta = c["r"].astype(np.float64) + g * vnext_array(c) - c["V"].astype(np.float64)
    close(a0, delta, 1e-14)


def test_discounted_geometric_series():
    N, T, g, rc = 3, 500, F32(0.97), 0.75
    r = np.full((N, T), rc, np.float32)
    term = np.zeros((N, T), np.uint8)
    t = np.arange(T)
    want = rc * (1.0 - g ** (T - t)) / (1.0 - g)
    close(oracle.discounted_returns(r, term, g), np.broadcast_to(want, (N, T)), 1e-12)


@pytest.mark.parametrize("seed,pt,pk", [(4, 0.0, 0.0), (5, 0.02, 0.02), (6, 0.3, 0.1)])
def test_discounted_lfilter_and_gamma_one(seed, pt, pk):
    c = case(seed, 3, 400, pt, pk)
    g = F32(0.99)
    close(oracle.discounted_returns(c["r"], c["term"], g, **kw(c)), mc_return_lfilter(c, g), 1e-11)
    # gamma = 1: reverse cumulative sum over each segment plus the end value
    got = oracle.discounted_returns(c["r"], c["term"], 1.0, **kw(c))
    r = c["r"].astype(np.float64)
    want = np.zeros_like(r)
    for n in range(r.shape[0]):
        for s, e in segments(c["term"][n], None if c["trunc"] is None else c["trunc"][n]):
            want[n, s:e + 1] = np.cumsum(r[n, s:e + 1][::-1])[::-1] + vend_row(c, n, e)
    close(got, want, 1e-11)
    # gamma = 0: G = r
    close(oracle.discounted_returns(c["r"], c["term"], 0.0, **kw(c)), r, 0.0)


@pytest.mark.parametrize("seed,pt,pk", [(7, 0.0, 0.0), (8, 0.05, 0.05)])
def test_lambda_returns_identities(seed, pt, pk):
    c = case(seed, 3, 300, pt, pk)
    g, lam = F32(0.99), F32(0.95)
    G = oracle.lambda_returns(c["r"], c["V"], c["term"], g, lam, **kw(c))
    A = oracle.gae(c["r"], c["V"], c["term"], g, lam, **kw(c))
    close(G, A + c["V"].astype(np.float64), 1e-11)
    close(oracle.lambda_returns(c["r"], c["V"], c["term"], g, 1.0, **kw(c)),
          mc_return_lfilter(c, g), 1e-11)
    close(oracle.lambda_returns(c["r"], c["V"], c["term"], g, 0.0, **kw(c)),
          c["r"].astype(np.float64) + g * vnext_array(c), 1e-14)


@pytest.mark.parametrize("seed,pt,pk", [(9, 0.0, 0.0), (10, 0.05, 0.05)])
def test_vtrace_identities(seed, pt, pk):
    c = case(seed, 3, 300, pt, pk)
    g, lam = F32(0.99), F32(0.95)
    zero = np.zeros_like(c["lr"])
    # on-policy (log-ratio 0) with rho_bar = c_bar = 1: vs = TD(lambda) returns
    vs, pg = oracle.vtrace(zero, c["r"], c["V"], c["term"], g, lam, rho_bar=1.0, c_bar=1.0, **kw(c))
    close(vs, oracle.lambda_returns(c["r"], c["V"], c["term"], g, lam, **kw(c)), 1e-11)
    vs1, _ = oracle.vtrace(zero, c["r"], c["V"], c["term"], g, 1.0, **kw(c))
    close(vs1, mc_return_lfilter(c, g), 1e-11)
    # pg_t = min(pg_rho_bar, w_t) * (r_t + gamma * target_{t+1} - V_t), recomputed from vs
    rho_bar, c_bar, pg_bar = 1.3, 0.8, 0.6
    vs, pg = oracle.vtrace(c["lr"], c["r"], c["V"], c["term"], g, lam, rho_bar=rho_bar,
                           c_bar=c_bar, pg_rho_bar=pg_bar, **kw(c))
    nxt = vnext_array(c)
    nxt[:, :-1] = np.where(end_array(c)[:, :-1], nxt[:, :-1], vs[:, 1:])
    w = np.exp(c["lr"].astype(np.float64))
    want_pg = np.minimum(pg_bar, w) * (c["r"] + g * nxt - c["V"].astype(np.float64))
    close(pg, want_pg, 1e-12)
    # c_bar = 0 kills the trace: vs = V + rho * delta
    vs0, _ = oracle.vtrace(c["lr"], c["r"], c["V"], c["term"], g, lam, rho_bar=rho_bar, c_bar=0.0,
                           **kw(c))
    delta = c["r"] + g * vnext_array(c) - c["V"].astype(np.float64)
    close(vs0, c["V"] + np.minimum(rho_bar, w) * delta, 1e-13)


@pytest.mark.parametrize("seed,pt,pk", [(11, 0.0, 0.0), (12, 0.05, 0.05)])
def test_retrace_identities(seed, pt, pk):
    c = case(seed, 3, 300, pt, pk)
    g, lam = F32(0.99), F32(0.95)
    zero = np.zeros_like(c["lr"])
    # on-policy with expected values equal to Q: TD(lambda) returns computed on Q
    cq = dict(c)
    cq["V"] = c["Q"]
    got = oracle.retrace(zero, c["r"], c["Q"], c["Q"], c["term"], g, lam, c_bar=1.0, **kw(c))
    close(got, oracle.lambda_returns(c["r"], c["Q"], c["term"], g, lam, **kw(c)), 1e-11)
    # lambda = 0: expected-SARSA target r + gamma * Vnext
    got0 = oracle.retrace(c["lr"], c["r"], c["Q"], c["V"], c["term"], g, 0.0, **kw(c))
    close(got0, c["r"].astype(np.float64) + g * vnext_array(c), 1e-14)


@pytest.mark.parametrize("seed,pd", [(13, 0.0), (14, 0.05)])
def test_forward_identities(seed, pd):
    c = case(seed, 3, 500, pd, 0.0)
    d = c["term"]
    x = c["x"].astype(np.float64)
    # gamma*lambda = 1: traces equal the prefix sum; gamma*lambda = 0: traces equal x
    close(oracle.eligibility_traces(c["x"], d, 1.0, 1.0), oracle.prefix_sum(c["x"], d), 0.0)
    close(oracle.eligibility_traces(c["x"], d, 0.0, 0.9), x, 0.0)
    # per-segment IIR filter / cumsum
    gl = F32(0.99) * F32(0.9)
    want_e = np.zeros_like(x)
    want_s = np.zeros_like(x)
    for n in range(x.shape[0]):
        starts = [0] + [t + 1 for t in range(x.shape[1] - 1) if d[n, t]]
        for s, e in zip(starts, starts[1:] + [x.shape[1]]):
            want_e[n, s:e] = lfilter([1.0], [1.0, -gl], x[n, s:e])
            want_s[n, s:e] = np.cumsum(x[n, s:e])
    close(oracle.eligibility_traces(c["x"], d, F32(0.99), F32(0.9)), want_e, 1e-11)
    close(oracle.prefix_sum(c["x"], d), want_s, 1e-12)


def test_prefix_int_exact_and_wrap():
    rng = np.random.default_rng(15)
    x = rng.integers(-1000, 1001, size=(5, 777)).astype(np.int32)
    d = (rng.random((5, 777)) < 0.02).astype(np.uint8)
    want = np.zeros_like(x)
    for n in range(5):
        starts = [0] + [t + 1 for t in range(776) if d[n, t]]
        for s, e in zip(starts, starts[1:] + [777]):
            want[n, s:e] = np.cumsum(x[n, s:e].astype(np.int64)).astype(np.int32)
    assert np.array_equal(oracle.prefix_sum(x, d), want)
    # Sums past int32 range wrap modulo 2^32, as numpy's int32 cumsum does.
    big = np.full((1, 8), 2**30 + 7, np.int32)
    got = oracle.prefix_sum(big, np.zeros((1, 8), np.uint8))
    assert np.array_equal(got, np.cumsum(big, axis=1, dtype=np.int32))


# -------------------------------------------------------------- invariants

@pytest.mark.parametrize("seed", [16, 17, 18])
def test_no_leakage_backward(seed):
    """Changing anything strictly after a cut leaves outputs up to the cut unchanged."""
    c = case(seed, 2, 120, 0.0, 0.0)
    cut_at = 50 + seed
    term = np.zeros((2, 120), np.uint8)
    trunc = np.zeros((2, 120), np.uint8)
    term[0, cut_at] = 1
    trunc[1, cut_at] = 1
    tv = c["r"].copy()
    g, lam = F32(0.99), F32(0.95)

    def run(cc):
        k = dict(truncateds=trunc, trunc_values=tv, bootstrap_value=cc["boot"])
        return [
            oracle.gae(cc["r"], cc["V"], term, g, lam, **k),
            oracle.lambda_returns(cc["r"], cc["V"], term, g, lam, **k),
            oracle.discounted_returns(cc["r"], term, g, **k),
            *oracle.vtrace(cc["lr"], cc["r"], cc["V"], term, g, lam, **k),
            oracle.retrace(cc["lr"], cc["r"], cc["Q"], cc["V"], term, g, lam, **k),
        ]

    base = run(c)
    p = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in c.items()}
    rng = np.random.default_rng(seed)
    for name in ("r", "V", "Q", "lr"):
        p[name][:, cut_at + 1:] = rng.standard_normal((2, 120 - cut_at - 1)) * 5
    p["boot"] = p["boot"] + 100
    for a, b in zip(base, run(p)):
        assert np.array_equal(a[:, :cut_at + 1], b[:, :cut_at + 1])
        assert not np.array_equal(a[:, cut_at + 1:], b[:, cut_at + 1:])


@pytest.mark.parametrize("seed", [19, 20])
def test_no_leakage_forward(seed):
    """Changing anything at or before a done step leaves later outputs unchanged."""
    c = case(seed, 2, 90, 0.0, 0.0)
    d = np.zeros((2, 90), np.uint8)
    d[:, 40] = 1
    xi = np.random.default_rng(seed).integers(-9, 10, size=(2, 90)).astype(np.int32)
    base = [oracle.eligibility_traces(c["x"], d, 0.99, 0.9), oracle.prefix_sum(c["x"], d),
            oracle.prefix_sum(xi, d)]
    x2, xi2 = c["x"].copy(), xi.copy()
    x2[:, :41] += 3.0
    xi2[:, :41] += 3
    new = [oracle.eligibility_traces(x2, d, 0.99, 0.9), oracle.prefix_sum(x2, d),
           oracle.prefix_sum(xi2, d)]
    for a, b in zip(base, new):
        assert np.array_equal(a[:, 41:], b[:, 41:])


def test_trunc_values_read_only_at_truncations():
    c = case(21, 3, 200, 0.03, 0.03)
    g, lam = F32(0.99), F32(0.95)
    tv2 = c["tv"].copy()
    tv2[c["trunc"] == 0] = 1e6
    k2 = dict(truncateds=c["trunc"], trunc_values=tv2, bootstrap_value=c["boot"])
    assert np.array_equal(oracle.gae(c["r"], c["V"], c["term"], g, lam, **kw(c)),
                          oracle.gae(c["r"], c["V"], c["term"], g, lam, **k2))
    assert np.array_equal(oracle.retrace(c["lr"], c["r"], c["Q"], c["V"], c["term"], g, lam, **kw(c)),
                          oracle.retrace(c["lr"], c["r"], c["Q"], c["V"], c["term"], g, lam, **k2))


def test_bootstrap_ignored_when_last_step_is_cut():
    c = case(22, 2, 30, 0.0, 0.0)
    term = np.zeros((2, 30), np.uint8)
    term[:, -1] = 1
    a = oracle.gae(c["r"], c["V"], term, 0.9, 0.9, bootstrap_value=np.array([1, 2], np.float32))
    b = oracle.gae(c["r"], c["V"], term, 0.9, 0.9, bootstrap_value=np.array([50, -7], np.float32))
    assert np.array_equal(a, b)


# ---------------------------------------------------- the combine operator

def combine(near, far):
    """(a_B, b_B) (+) (a_A, b_A) = (a_B + b_B a_A, b_A b_B): compose x -> a + b x maps."""
    return (near[0] + near[1] * far[0], near[1] * far[1])


def test_combine_associative_exact():
    rng = np.random.default_rng(23)
    for _ in range(500):
        x, y, z = [(int(rng.integers(-99, 100)), int(rng.integers(-3, 4))) for _ in range(3)]
        assert combine(combine(x, y), z) == combine(x, combine(y, z))
    for _ in range(200):
        x, y, z = [tuple(rng.standard_normal(2)) for _ in range(3)]
        l, r = combine(combine(x, y), z), combine(x, combine(y, z))
        assert np.allclose(l, r, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("seed", [24, 25])
def test_tree_scan_reproduces_recursion(seed):
    """A Hillis-Steele (log-depth) scan with the operator equals the recursion."""
    c = case(seed, 2, 97, 0.05, 0.05)
    g, lam = 0.9, 0.8
    A = oracle.gae(c["r"], c["V"], c["term"], g, lam, **kw(c))
    end = end_array(c)
    alpha = c["r"] + g * vnext_array(c) - c["V"].astype(np.float64)
    beta = np.where(end, 0.0, g * lam)
    for n in range(2):
        # backward scan: element t composes with t+d, ..., reading from higher index
        s = [(alpha[n, t], beta[n, t]) for t in range(97)]
        d = 1
        while d < 97:
            s = [combine(s[t], s[t + d]) if t + d < 97 else s[t] for t in range(97)]
            d *= 2
        close([v[0] for v in s], A[n], 1e-12)


# ------------------------------------------------ generic segmented affine scan
def affine_case(seed, N, T, p_reset):
    rng = np.random.default_rng(seed)
    return dict(alpha=rng.standard_normal((N, T)).astype(np.float32),
                beta=rng.uniform(-1.2, 1.2, (N, T)).astype(np.float32),
                reset=(rng.random((N, T)) < p_reset).astype(np.uint8),
                carry=rng.standard_normal(N).astype(np.float32))


@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("seed,N,T,pr", [(40, 3, 17, 0.15), (41, 2, 1, 0.5), (42, 4, 9, 0.0),
                                         (43, 2, 23, 0.4)])
def test_affine_bruteforce(seed, N, T, pr, reverse):
    c = affine_case(seed, N, T, pr)
    for reset in (c["reset"], None):
        for carry in (c["carry"], None):
            got = oracle.affine_scan(c["alpha"], c["beta"], reset=reset, carry_in=carry,
                                     reverse=reverse)
            want = bf.affine(c["alpha"], c["beta"], reset, carry, reverse)
            close(got, want, 1e-12)


def test_affine_hand_worked():
    # one row, T = 4, beta = 0.5 everywhere, reset at t = 2, carry 8:
    # forward  y0 = 1 + 0.5*8 = 5, y1 = 2 + 2.5 = 4.5, y2 = 3 (reset), y3 = 4 + 1.5 = 5.5
    # reverse  y3 = 4 + 4 = 8, y2 = 3 (reset), y1 = 2 + 1.5 = 3.5, y0 = 1 + 1.75 = 2.75
    a = np.array([[1, 2, 3, 4]], np.float32)
    b = np.full((1, 4), 0.5, np.float32)
    r = np.array([[0, 0, 1, 0]], np.uint8)
    cin = np.array([8.0], np.float32)
    assert oracle.affine_scan(a, b, reset=r, carry_in=cin).tolist() == [[5.0, 4.5, 3.0, 5.5]]
    assert oracle.affine_scan(a, b, reset=r, carry_in=cin, reverse=True).tolist() == \
        [[2.75, 3.5, 3.0, 8.0]]


@pytest.mark.parametrize("seed", [44, 45])
def test_affine_mirror_exact(seed):
    """Reversing every row turns a reverse scan into a forward one, bit for bit."""
    c = affine_case(seed, 5, 31, 0.1)
    back = oracle.affine_scan(c["alpha"], c["beta"], reset=c["reset"], carry_in=c["carry"],
                              reverse=True)
    fwd = oracle.affine_scan(c["alpha"][:, ::-1], c["beta"][:, ::-1], reset=c["reset"][:, ::-1],
                             carry_in=c["carry"])
    assert np.array_equal(back, fwd[:, ::-1])


def test_affine_geometric_closed_form():
    """Constant alpha = a, beta = b, no resets, carry c (reverse):
    y_t = a (1 - b^L) / (1 - b) + b^L c with L = T - t."""
    T, a, b, cin = 40, 0.75, 0.875, -2.5
    y = oracle.affine_scan(np.full((1, T), a, np.float32), np.full((1, T), b, np.float32),
                           carry_in=np.array([cin], np.float32), reverse=True)[0]
    L = T - np.arange(T)
    close(y, a * (1 - b ** L) / (1 - b) + b ** L * cin, 1e-13)


@pytest.mark.parametrize("seed", [46, 47])
def test_affine_lfilter(seed):
    """Forward, constant beta, no resets: a first-order IIR filter whose
    initial state is beta * carry."""
    rng = np.random.default_rng(seed)
    N, T, b = 3, 50, 0.93
    a = rng.standard_normal((N, T)).astype(np.float32)
    cin = rng.standard_normal(N).astype(np.float32)
    y = oracle.affine_scan(a, np.full((N, T), b, np.float32), carry_in=cin)
    bb = float(np.float32(b))
    for n in range(N):
        want, _ = lfilter([1.0], [1.0, -bb], a[n].astype(np.float64),
                                       zi=[bb * float(cin[n])])
        close(y[n], want, 1e-12)


@pytest.mark.parametrize("reverse", [False, True])
def test_affine_integer_segmented_cumsum(reverse):
    """beta = 1 with resets is a segmented cumulative sum (numpy.cumsum per
    segment), exact on integers."""
    rng = np.random.default_rng(48)
    N, T = 3, 60
    a = rng.integers(-9, 10, (N, T)).astype(np.float32)
    r = (rng.random((N, T)) < 0.1).astype(np.uint8)
    y = oracle.affine_scan(a, np.ones((N, T), np.float32), reset=r, reverse=reverse)
    for n in range(N):
        row, rr = (a[n, ::-1], r[n, ::-1]) if reverse else (a[n], r[n])
        want = np.empty(T)
        starts = [0] + [t for t in range(1, T) if rr[t]]
        for s, e in zip(starts, starts[1:] + [T]):
            want[s:e] = np.cumsum(row[s:e])
        assert np.array_equal(y[n], want[::-1] if reverse else want)


def test_affine_reduces_to_gae():
    """GAE is the reverse affine scan with alpha = delta and beta = gamma*lambda
    cut at episode ends (Methodology 1).  Dyadic inputs keep both sides exact."""
    rng = np.random.default_rng(49)
    N, T, g, lam = 3, 40, 0.5, 0.75
    r = rng.integers(-8, 9, (N, T)).astype(np.float32)
    v = rng.integers(-8, 9, (N, T)).astype(np.float32)
    term = (rng.random((N, T)) < 0.1).astype(np.uint8)
    boot = rng.integers(-8, 9, N).astype(np.float32)
    vn = np.concatenate([v[:, 1:], boot[:, None]], axis=1).astype(np.float64)
    vn[term != 0] = 0.0
    delta = r + g * vn - v
    beta = np.where(term != 0, 0.0, g * lam)
    beta[:, -1] = 0.0
    got = oracle.affine_scan(delta.astype(np.float32), beta.astype(np.float32), reverse=True)
    assert np.array_equal(got, oracle.gae(r, v, term, g, lam, bootstrap_value=boot))
