"""Host logic of bench.py (no GPU): the algorithmic byte model, the graph
replay plan that keeps every call's inputs cold, and the one-GPU guard."""
import subprocess
import sys
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
import bench  # noqa: E402


@pytest.mark.parametrize("est,per_elem", [
    ("gae", 13), ("lambda_returns", 13), ("vtrace", 21), ("retrace", 21),
    ("discounted_returns", 9), ("eligibility_traces", 9), ("prefix_sum_f32", 9),
    ("prefix_sum_i32", 9), ("affine_fwd", 13),
])
def test_algorithmic_bytes(est, per_elem):
    """One read of every input and one write of every output, fp32 data and
    uint8 masks, plus one datum per env for backward calls (bootstrap) and the
    affine scan (carry)."""
    n, t = 7, 11
    per_env = 4 if est in bench.BACKWARD or est.startswith("affine") else 0
    assert bench.alg_bytes(est, False, n, t) == per_elem * n * t + per_env * n
    # 16-bit storage halves every data stream, not the masks
    rd, wr, masks = bench.STREAMS[est]
    assert bench.alg_bytes(est, False, n, t, width=2) == \
        (2 * (rd + wr) + masks) * n * t + per_env // 2 * n
    # the split into bytes read and written: outputs are the written streams
    r, w = bench.alg_bytes_rw(est, False, n, t)
    assert w == 4 * wr * n * t and r + w == bench.alg_bytes(est, False, n, t)
    assert wr == (2 if est == "vtrace" else 1)


def test_truncation_bytes():
    """Truncations add a mask byte per element and one trunc_values datum per
    truncation (the only ones the method reads)."""
    n, t = 4, 10
    base = bench.alg_bytes("gae", False, n, t)
    assert bench.alg_bytes("gae", True, n, t, n_trunc=3) == base + n * t + 4 * 3
    assert bench.alg_bytes("gae", True, n, t) == base + n * t + 4 * n * t


@pytest.mark.parametrize("R,G,K", [(25, 2, 400), (2560, 24, 400), (5, 8, 13), (1, 24, 7),
                                   (3, 1, 10), (6, 4, 9), (7, 3, 0), (228, 2, 400)])
@pytest.mark.parametrize("first", [0, 1, 20, 113])
def test_replay_plan_walks_replicas_in_order(R, G, K, first):
    """From any first graph (the one after the warm-up's last), the timed
    steps walk the replicas in order."""
    starts, _, _ = bench.replay_plan(R, G, K)
    first %= len(starts)
    starts, full, tail = bench.replay_plan(R, G, K, first)
    seq = []
    for k in range(full):
        seq += [(starts[(first + k) % len(starts)] + s) % R for s in range(G)]
    if tail is not None:
        seq += [(tail + s) % R for s in range(K % G)]
    assert seq == [(first * G + k) % R for k in range(K)]


def test_warmup_and_timed_steps_do_not_reuse_recent_replicas():
    """With the default 400 steps, 40 warm-up steps and the 4096 x 128
    replicas, the first timed step reads the replica after the warm-up's last
    one."""
    R, G, W = bench.replicas_for([4718592], bench.MIN_CYCLE_BYTES, 2), 2, 40
    starts, _, _ = bench.replay_plan(R, G, 400)
    first = -(-W // G) % len(starts)
    assert first * G == W % R


def test_replicas_cover_a_gib_per_call():
    """Every call cycles over >= 1 GiB of its own data, rounded up to whole
    graphs of steps."""
    for cb in ([4718592, 11566940], [117440512], [1 << 31], [5]):
        for G in (1, 2, 24):
            R = bench.replicas_for(cb, bench.MIN_CYCLE_BYTES, G)
            assert R % G == 0 and R >= 2
            assert min(cb) * R >= bench.MIN_CYCLE_BYTES or R == 2


def test_steps_per_graph():
    assert bench.steps_per_graph(12) == 2
    assert bench.steps_per_graph(1) == 24
    assert bench.steps_per_graph(24) == 1
    assert bench.steps_per_graph(100) == 1


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
