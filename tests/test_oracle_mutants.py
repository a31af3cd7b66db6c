"""Mutation check of the oracle's pins (CPU only).

Plants plausible mistakes -- a dropped term, a wrong sign, a wrong index, a
transposed operand, a wrong reset rule -- into a copy of the oracle source,
compiles each copy, and requires that the brute-force / hand-worked pin
battery rejects every one.  The real oracle must pass the same battery.
"""
import numpy as np
import pytest

import bruteforce as bf
import oracle

MUTANTS = [
    # successor value and episode ends
    ("terminated ignored in successor", "if (term[i]) return 0.0;", ""),
    ("truncation bootstrap replaced by window bootstrap",
     "if (trunc && trunc[i]) return (double)trunc_val[i];",
     "if (trunc && trunc[i]) return boot ? (double)boot[n] : 0.0;"),
    ("window bootstrap dropped", "if (t == T - 1) return boot ? (double)boot[n] : 0.0;",
     "if (t == T - 1) return 0.0;"),
    ("window bootstrap of the wrong row", "return boot ? (double)boot[n] : 0.0;",
     "return boot ? (double)boot[0] : 0.0;"),
    ("truncation does not end the episode",
     "return term[i] || (trunc && trunc[i]) || t == T - 1;", "return term[i] || t == T - 1;"),
    # GAE
    ("GAE: gamma dropped on successor",
     "double delta = (double)rewards[i] + gamma * vn - (double)values[i];",
     "double delta = (double)rewards[i] + vn - (double)values[i];"),
    ("GAE: sign of V",
     "double delta = (double)rewards[i] + gamma * vn - (double)values[i];",
     "double delta = (double)rewards[i] + gamma * vn + (double)values[i];"),
    ("GAE: lambda dropped", "a += gamma * lambda * next_a;", "a += gamma * next_a;"),
    # TD(lambda)
    ("TD(lambda): lambda dropped on G", "(1.0 - lambda) * v1 + lambda * next_g",
     "(1.0 - lambda) * v1 + next_g"),
    ("TD(lambda): V_t instead of V_{t+1}", "double v1 = (double)values[i + 1];",
     "double v1 = (double)values[i];"),
    ("TD(lambda): mixing weights swapped", "(1.0 - lambda) * v1 + lambda * next_g",
     "lambda * v1 + (1.0 - lambda) * next_g"),
    # discounted returns
    ("returns: gamma dropped", "g = (double)rewards[i] + gamma * next_g;",
     "g = (double)rewards[i] + next_g;"),
    # V-trace
    ("V-trace: lambda dropped from c", "double c = lambda * fmin(c_bar, w);",
     "double c = fmin(c_bar, w);"),
    ("V-trace: rho clipped with c_bar", "double rho = fmin(rho_bar, w);",
     "double rho = fmin(c_bar, w);"),
    ("V-trace: pg target uses V_{t+1} only", "target_next = (double)values[i + 1] + next_a;",
     "target_next = (double)values[i + 1];"),
    ("V-trace: pg weighted by rho", "pg_adv[i] = rho_pg * (", "pg_adv[i] = rho * ("),
    ("V-trace: gamma dropped on trace", "a += gamma * c * next_a;", "a += c * next_a;"),
    # Retrace
    ("Retrace: trace of step t instead of t+1", "exp((double)log_rhos[i + 1])",
     "exp((double)log_rhos[i])"),
    ("Retrace: Q_t instead of Q_{t+1}", "c1 * (next_g - (double)q_values[i + 1])",
     "c1 * (next_g - (double)q_values[i])"),
    ("Retrace: Q and V transposed", "+ gamma * ((double)values[i + 1]",
     "+ gamma * ((double)q_values[i + 1]"),
    # forward estimators
    ("traces reset at the done step", "if (t > 0 && !done[i - 1]) e += gamma * lambda * prev;",
     "if (t > 0 && !done[i]) e += gamma * lambda * prev;"),
    ("traces: lambda dropped", "e += gamma * lambda * prev;", "e += gamma * prev;"),
    ("prefix f32 resets at the done step", "if (t == 0 || done[i - 1]) s = 0.0;",
     "if (t == 0 || done[i]) s = 0.0;"),
    ("prefix i32 resets at the done step", "if (t == 0 || done[i - 1]) s = 0;",
     "if (t == 0 || done[i]) s = 0;"),
    ("prefix i32 exclusive", "s += (int64_t)x[i];\n            out[i] = (int32_t)(uint32_t)(uint64_t)s;",
     "out[i] = (int32_t)(uint32_t)(uint64_t)s;\n            s += (int64_t)x[i];"),
    # generic affine scan
    ("affine: reset ignored", "if (!(reset && reset[i])) next += (double)beta[i] * y;",
     "next += (double)beta[i] * y;"),
    ("affine: carry dropped", "double y = carry ? (double)carry[n] : 0.0;", "double y = 0.0;"),
    ("affine: carry of the wrong row", "double y = carry ? (double)carry[n] : 0.0;",
     "double y = carry ? (double)carry[0] : 0.0;"),
    ("affine: direction flipped", "int64_t t = reverse ? T - 1 - k : k;",
     "int64_t t = reverse ? k : T - 1 - k;"),
    ("affine: alpha and beta transposed",
     "double next = (double)alpha[i];\n            if (!(reset && reset[i])) next += (double)beta[i] * y;",
     "double next = (double)beta[i];\n            if (!(reset && reset[i])) next += (double)alpha[i] * y;"),
    ("affine: reset also drops alpha",
     "if (!(reset && reset[i])) next += (double)beta[i] * y;",
     "if (!(reset && reset[i])) next += (double)beta[i] * y; else next = y;"),
]


def _cases():
    rng = np.random.default_rng(99)
    out = []
    for N, T, pt, pk in [(2, 9, 0.2, 0.2), (3, 17, 0.1, 0.1), (2, 12, 0.0, 0.0)]:
        out.append(dict(
            r=rng.standard_normal((N, T)).astype(np.float32),
            V=rng.standard_normal((N, T)).astype(np.float32),
            Q=rng.standard_normal((N, T)).astype(np.float32),
            lr=(0.7 * rng.standard_normal((N, T))).astype(np.float32),
            term=(rng.random((N, T)) < pt).astype(np.uint8),
            trunc=(rng.random((N, T)) < pk).astype(np.uint8),
            tv=rng.standard_normal((N, T)).astype(np.float32),
            boot=rng.standard_normal(N).astype(np.float32),
            x=rng.standard_normal((N, T)).astype(np.float32),
            xi=rng.integers(-50, 51, size=(N, T)).astype(np.int32),
        ))
    return out


CASES = _cases()


def battery_passes() -> bool:
    """True iff the current oracle matches every brute-force pin below."""
    g, lam = 0.9, 0.7
    for c in CASES:
        k = dict(truncateds=c["trunc"], trunc_values=c["tv"], bootstrap_value=c["boot"])
        t = dict(trunc=c["trunc"], tv=c["tv"], boot=c["boot"])
        pairs = [
            (oracle.gae(c["r"], c["V"], c["term"], g, lam, **k),
             bf.gae(c["r"], c["V"], c["term"], g, lam, **t)),
            (oracle.lambda_returns(c["r"], c["V"], c["term"], g, lam, **k),
             bf.lambda_returns(c["r"], c["V"], c["term"], g, lam, **t)),
            (oracle.discounted_returns(c["r"], c["term"], g, **k),
             bf.discounted(c["r"], c["term"], g, **t)),
            (oracle.retrace(c["lr"], c["r"], c["Q"], c["V"], c["term"], g, lam, c_bar=1.2, **k),
             bf.retrace(c["lr"], c["r"], c["Q"], c["V"], c["term"], g, lam, 1.2, **t)),
            (oracle.eligibility_traces(c["x"], c["term"], g, lam),
             bf.eligibility(c["x"], c["term"], g, lam)),
            (oracle.prefix_sum(c["x"], c["term"]), bf.prefix(c["x"], c["term"])),
            (oracle.prefix_sum(c["xi"], c["term"]), bf.prefix(c["xi"], c["term"])),
        ]
        vs, pg = oracle.vtrace(c["lr"], c["r"], c["V"], c["term"], g, lam, rho_bar=1.1,
                               c_bar=0.9, pg_rho_bar=1.3, **k)
        vs_b, pg_b = bf.vtrace(c["lr"], c["r"], c["V"], c["term"], g, lam, 1.1, 0.9, 1.3, **t)
        pairs += [(vs, vs_b), (pg, pg_b)]
        beta = (0.6 * c["V"]).astype(np.float32)
        for reverse in (False, True):
            pairs.append((oracle.affine_scan(c["x"], beta, reset=c["term"], carry_in=c["boot"],
                                             reverse=reverse),
                          bf.affine(c["x"], beta, c["term"], c["boot"], reverse)))
        for got, want in pairs:
            if not np.allclose(got, want, rtol=1e-10, atol=1e-10):
                return False
    return True


def test_real_oracle_passes_battery():
    assert battery_passes()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, tmp_path):
    src = oracle.source_text()
    assert src.count(old) >= 1, f"mutation site not found: {old!r}"
    mutated = src.replace(old, new, 1)
    lib = oracle.compile_variant(mutated, str(tmp_path / "mutant.so"))
    with oracle.use_library(lib):
        assert not battery_passes(), f"pins did not catch mutant: {name}"
