"""Calls captured into a HIP graph (torch.cuda.CUDAGraph) and replayed.

A graph freezes the kernel arguments, so a replay must get its launch tag
from the workspace header at run time and leave the header clean for the
next launch.  Each case captures one call, replays the graph several times
with eager calls of other sizes on the same stream (so on the same cached
workspace) between replays, and checks that every replay reproduces the
eager result bit for bit, and that the eager result matches the oracle.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import linear_recurrence_scan_env_amd as lrs  # noqa: E402
from linear_recurrence_scan_env_amd import workloads  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lrs.load()
    yield


def dev(a, tm=False):
    if a is None:
        return None
    if tm and a.ndim == 2:
        a = a.T
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def make(case, N, T, seed):
    """(call writing into fixed outputs, outputs, oracle results)."""
    tm = case.endswith("_tm")
    ro = workloads.rollout(N, T, seed=seed, term_p=0.002, trunc_p=0.002, done_p=0.002)
    a = ro.arrays
    D = {k: dev(v, tm) for k, v in a.items()}
    g, lam = ro.gamma, ro.lambda_
    shape = (T, N) if tm else (N, T)
    kg = dict(truncateds=D["truncateds"], trunc_values=D["trunc_values"],
              bootstrap_value=D["bootstrap_value"], time_major=tm)
    ko = dict(truncateds=a["truncateds"], trunc_values=a["trunc_values"],
              bootstrap_value=a["bootstrap_value"])
    if case.startswith("gae"):
        out = [torch.empty(shape, device="cuda")]
        fn = lambda: lrs.compute_gae(D["rewards"], D["values"], D["terminateds"], g, lam,  # noqa
                                     out=out[0], **kg)
        refs = [oracle.gae(a["rewards"], a["values"], a["terminateds"], g, lam, **ko)]
    elif case.startswith("vtrace"):
        out = [torch.empty(shape, device="cuda"), torch.empty(shape, device="cuda")]
        fn = lambda: lrs.compute_vtrace(D["log_rhos"], D["rewards"], D["values"],  # noqa
                                        D["terminateds"], g, lam, out=(out[0], out[1]), **kg)
        refs = list(oracle.vtrace(a["log_rhos"], a["rewards"], a["values"], a["terminateds"],
                                  g, lam, **ko))
    else:
        out = [torch.empty(shape, device="cuda", dtype=torch.int32)]
        fn = lambda: lrs.compute_episodic_prefix_sum(D["x_int"], D["dones"], out=out[0],  # noqa
                                                     time_major=tm)
        refs = [oracle.prefix_sum(a["x_int"], a["dones"])]
    return fn, out, refs, tm


# (case, num_envs, seq_len): rows that straddle tiles take the look-back
# path (row-major) or carry along time (time-major); 64 x 128 rows fit tiles.
CASES = [("gae", 5, 3001), ("vtrace", 3, 7001), ("prefix_i32", 4, 5003), ("gae", 64, 128),
         ("gae_tm", 5, 3001), ("prefix_i32_tm", 70, 1000)]


@pytest.mark.parametrize("case,N,T", CASES, ids=[f"{c}-{n}x{t}" for c, n, t in CASES])
def test_graph_replays_match_eager(case, N, T):
    s = torch.cuda.Stream()
    fn, out, refs, tm = make(case, N, T, seed=N + T)
    other, _, _, _ = make(case, N + 1, T + 777, seed=7)
    with torch.cuda.stream(s):
        fn()  # eager, on the capture stream (its workspace is allocated here)
        other()
        s.synchronize()
        eager = [o.clone() for o in out]
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            fn()
        for rep in range(5):
            for o in out:
                o.fill_(0)
            graph.replay()
            s.synchronize()
            for got, want in zip(out, eager):
                assert torch.equal(got, want), f"replay {rep} differs from the eager call"
            other()  # eager work of another size on the same workspace
            s.synchronize()
    for got, ref in zip(eager, refs):
        g = got.cpu().numpy()
        if tm:
            g = g.T
        if ref.dtype == np.int32:
            assert np.array_equal(g, ref)
        else:
            err = np.abs(g.astype(np.float64) - ref) / (1.0 + np.abs(ref))
            assert err.max() <= 1e-5
    for h in lrs.workspace_state():
        assert h["error"] == 0 and h["top"] == 0 and h["counters_nonzero"] == 0, h
        assert h["epochs_in_step"], h


def test_graph_keeps_its_workspace_when_the_cache_grows():
    """A call captured while the stream's cached workspace is small keeps
    replaying correctly after a larger call has replaced that workspace."""
    s = torch.cuda.Stream()
    fn, out, refs, _ = make("gae", 3, 3001, seed=11)
    big, _, _, _ = make("gae", 40, 30001, seed=12)
    with torch.cuda.stream(s):
        fn()
        s.synchronize()
        eager = out[0].clone()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            fn()
        big()  # grows the cached workspace
        s.synchronize()
        for rep in range(3):
            out[0].fill_(0)
            graph.replay()
            s.synchronize()
            assert torch.equal(out[0], eager)
            big()
            s.synchronize()
