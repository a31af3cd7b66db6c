"""O(T^2) brute-force definitions of the seven estimators (tests only).

Each function evaluates the closed SUM form of its estimator directly, in
plain Python floats (fp64), with no recursion, so that it can pin the
oracle's sequential recursions.  It is deliberately written from the sum
definitions, not from the recursions:

  GAE (Schulman et al. 2016, eq. 16):
      A_t = sum_{k=t..e} (gamma*lambda)^(k-t) * delta_k
  discounted return:
      G_t = sum_{k=t..e} gamma^(k-t) r_k + gamma^(e-t+1) * Vend
  TD(lambda) (Sutton & Barto sec. 12.1, truncated at the episode end):
      G_t = (1-lambda) sum_{n=1..L} lambda^(n-1) G_t^(n) + lambda^L G_t^(L+1)
  V-trace (Espeholt et al. 2018, eq. 1):
      vs_s = V_s + sum_{t=s..e} gamma^(t-s) (prod_{i=s..t-1} c_i) rho_t delta_t
  Retrace (Munos et al. 2016):
      Q_s + sum_{t=s..e} gamma^(t-s) (prod_{i=s+1..t} c_i) (r_t + gamma Vnext_t - Q_t)
  eligibility trace / prefix sum:
      e_t = sum_{k=s..t} (gamma*lambda)^(t-k) x_k    (s = segment start)

where e is the first step >= t that ends the segment (terminated, truncated
or the last column), L = e - t, Vnext_k = V_{k+1} inside the segment and
Vend at e (0 if terminated, trunc_values if truncated, the bootstrap value
at the window end).
"""
import math

import numpy as np


def _f(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def _m(a):
    return None if a is None else (np.asarray(a) != 0)


class Ctx:
    def __init__(self, T, term, trunc=None, tv=None, boot=None):
        self.T = T
        self.term = _m(term)
        self.trunc = _m(trunc)
        self.tv = _f(tv)
        self.boot = _f(boot)

    def is_end(self, n, k):
        return bool(self.term[n, k]) or (self.trunc is not None and bool(self.trunc[n, k])) \
            or k == self.T - 1

    def seg_end(self, n, t):
        e = t
        while not self.is_end(n, e):
            e += 1
        return e

    def vend(self, n, e):
        if self.term[n, e]:
            return 0.0
        if self.trunc is not None and self.trunc[n, e]:
            return float(self.tv[n, e])
        return 0.0 if self.boot is None else float(self.boot[n])

    def vnext(self, V, n, k, e):
        return float(V[n, k + 1]) if k < e else self.vend(n, e)


def gae(r, V, term, gamma, lam, trunc=None, tv=None, boot=None):
    r, V = _f(r), _f(V)
    N, T = r.shape
    c = Ctx(T, term, trunc, tv, boot)
    out = np.zeros((N, T))
    for n in range(N):
        for t in range(T):
            e = c.seg_end(n, t)
            s = 0.0
            for k in range(t, e + 1):
                delta = r[n, k] + gamma * c.vnext(V, n, k, e) - V[n, k]
                s += (gamma * lam) ** (k - t) * delta
            out[n, t] = s
    return out


def discounted(r, term, gamma, trunc=None, tv=None, boot=None):
    r = _f(r)
    N, T = r.shape
    c = Ctx(T, term, trunc, tv, boot)
    out = np.zeros((N, T))
    for n in range(N):
        for t in range(T):
            e = c.seg_end(n, t)
            s = sum(gamma ** (k - t) * r[n, k] for k in range(t, e + 1))
            out[n, t] = s + gamma ** (e - t + 1) * c.vend(n, e)
    return out


def lambda_returns(r, V, term, gamma, lam, trunc=None, tv=None, boot=None):
    r, V = _f(r), _f(V)
    N, T = r.shape
    c = Ctx(T, term, trunc, tv, boot)
    out = np.zeros((N, T))
    for n in range(N):
        for t in range(T):
            e = c.seg_end(n, t)
            L = e - t

            def nstep(m):  # m-step return, m <= L uses V inside the segment
                g = sum(gamma ** k * r[n, t + k] for k in range(m))
                boot_v = V[n, t + m] if m <= L else c.vend(n, e)
                return g + gamma ** m * boot_v

            g = (1.0 - lam) * sum(lam ** (m - 1) * nstep(m) for m in range(1, L + 1))
            out[n, t] = g + lam ** L * nstep(L + 1)
    return out


def vtrace(lr, r, V, term, gamma, lam, rho_bar, c_bar, pg_rho_bar=None, trunc=None, tv=None,
           boot=None):
    lr, r, V = _f(lr), _f(r), _f(V)
    if pg_rho_bar is None:
        pg_rho_bar = rho_bar
    N, T = r.shape
    c = Ctx(T, term, trunc, tv, boot)
    w = np.exp(lr)
    rho = np.minimum(rho_bar, w)
    cc = lam * np.minimum(c_bar, w)
    vs = np.zeros((N, T))
    for n in range(N):
        for s in range(T):
            e = c.seg_end(n, s)
            acc = 0.0
            for t in range(s, e + 1):
                prod = math.prod(cc[n, i] for i in range(s, t))
                delta = rho[n, t] * (r[n, t] + gamma * c.vnext(V, n, t, e) - V[n, t])
                acc += gamma ** (t - s) * prod * delta
            vs[n, s] = V[n, s] + acc
    pg = np.zeros((N, T))
    for n in range(N):
        for s in range(T):
            nxt = c.vend(n, s) if c.is_end(n, s) else vs[n, s + 1]
            pg[n, s] = min(pg_rho_bar, w[n, s]) * (r[n, s] + gamma * nxt - V[n, s])
    return vs, pg


def retrace(lr, r, Q, V, term, gamma, lam, c_bar, trunc=None, tv=None, boot=None):
    lr, r, Q, V = _f(lr), _f(r), _f(Q), _f(V)
    N, T = r.shape
    c = Ctx(T, term, trunc, tv, boot)
    cc = lam * np.minimum(c_bar, np.exp(lr))
    out = np.zeros((N, T))
    for n in range(N):
        for s in range(T):
            e = c.seg_end(n, s)
            acc = 0.0
            for t in range(s, e + 1):
                prod = math.prod(cc[n, i] for i in range(s + 1, t + 1))
                acc += gamma ** (t - s) * prod * (r[n, t] + gamma * c.vnext(V, n, t, e) - Q[n, t])
            out[n, s] = Q[n, s] + acc
    return out


def _seg_start(done, n, t):
    s = t
    while s > 0 and not done[n, s - 1]:
        s -= 1
    return s


def eligibility(x, done, gamma, lam):
    x = _f(x)
    d = _m(done)
    N, T = x.shape
    out = np.zeros((N, T))
    for n in range(N):
        for t in range(T):
            s = _seg_start(d, n, t)
            out[n, t] = sum((gamma * lam) ** (t - k) * x[n, k] for k in range(s, t + 1))
    return out


def prefix(x, done):
    d = _m(done)
    xa = np.asarray(x)
    N, T = xa.shape
    if np.issubdtype(xa.dtype, np.integer):
        out = np.zeros((N, T), dtype=np.int64)
        for n in range(N):
            for t in range(T):
                s = _seg_start(d, n, t)
                out[n, t] = sum(int(v) for v in xa[n, s:t + 1])
        return out
    xf = _f(xa)
    out = np.zeros((N, T))
    for n in range(N):
        for t in range(T):
            s = _seg_start(d, n, t)
            out[n, t] = float(sum(xf[n, s:t + 1]))
    return out


def affine(alpha, beta, reset=None, carry=None, reverse=False):
    """Generic segmented affine scan from its sum form:
        y_t = sum_{k in chain(t)} (prod of beta over the steps from t up to,
              not including, k) * alpha_k  [+ the same product over the whole
              chain times carry[n], when the chain reaches the row's start]
    where chain(t) walks from t against the scan order (t, t-1, ... forward;
    t, t+1, ... reverse) and stops after the first step whose reset is set.
    """
    a = np.asarray(alpha, dtype=np.float64)
    b = np.asarray(beta, dtype=np.float64)
    rs = np.zeros(a.shape, bool) if reset is None else (np.asarray(reset) != 0)
    c = np.zeros(a.shape[0]) if carry is None else np.asarray(carry, dtype=np.float64)
    N, T = a.shape
    step = 1 if reverse else -1
    out = np.zeros((N, T))
    for n in range(N):
        for t in range(T):
            total, w, k = 0.0, 1.0, t
            while True:
                total += w * a[n, k]
                if rs[n, k]:
                    break
                w *= b[n, k]
                k += step
                if k < 0 or k >= T:
                    total += w * c[n]
                    break
            out[n, t] = total
    return out
