"""Host-side logic of bench.py, checked without a GPU.

- The position bookkeeping the benchmark's byte accounting and boundary schedule rest on
  (`n_slots_at`, `keys_at`, `is_boundary`, `first_boundary_after`) agrees with the oracle's
  key lists ([TR] §3.1 Eq. 4) and with the boundary steps t_m = S + W + m r ([TR] §3.2
  Algorithm 1 step 1) at the bench geometries.
- The headline's timed window holds ceil(steps / r) boundary steps for any step count.
- The Eq. 3 fit recovers an exact line.
- More than one GPU is refused before anything touches a device.
"""
import math
import os
import subprocess
import sys

import pytest

import bench
from oracle import masw_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEOMS = [(4, 2048, 64), (128, 128, 4), (128, 128, 8), (0, 1024, 0), (4, 2048, 0), (4, 32, 16)]


@pytest.mark.parametrize("S,W,r", GEOMS)
def test_key_counts_match_the_oracle(S, W, r):
    ts = sorted({1, S, S + 1, S + W, S + W + 1, S + W + max(r, 1), 3 * (S + W) + 5, 8192, 32768} - {0})
    for t in ts:
        n = len(O.keylist(t, S, W, r))
        assert bench.keys_at(t, S, W, r) == n, (t, S, W, r)
        assert bench.n_slots_at(t, S, W, r) == O.visible_slot_count(t, S, W, r)


@pytest.mark.parametrize("S,W,r", [g for g in GEOMS if g[2] > 0])
def test_boundaries_are_the_slot_steps(S, W, r):
    for t in range(1, S + W + 6 * r + 3):
        expect = t >= S + W + r and (t - S - W) % r == 0
        assert bench.is_boundary(t, S, W, r) == expect, t
        nxt = bench.first_boundary_after(t, S, W, r)
        assert nxt > t and bench.is_boundary(nxt, S, W, r)
        assert not any(bench.is_boundary(u, S, W, r) for u in range(t + 1, nxt))


@pytest.mark.parametrize("steps", [1, 5, 20, 63, 64, 65, 128, 256, 300])
def test_headline_window_holds_its_boundaries(steps):
    sh = bench.SHAPE
    S, W, r = sh.sink, sh.window, sh.interval
    warmup = 16
    b0 = bench.first_boundary_after(bench.T_HEAD, S, W, r)
    head_start = b0 - 1 - warmup
    # time_steps replays `warmup` steps from head_start, then times positions t0+1 .. t0+steps
    t0 = head_start + warmup
    timed = range(t0 + 1, t0 + steps + 1)
    assert timed[0] == b0
    assert sum(bench.is_boundary(t, S, W, r) for t in timed) == math.ceil(steps / r)


def test_eq3_fit_recovers_a_line():
    xs = [1024, 2048, 4096, 8192, 16384]
    a, b, r2 = bench.linear_fit(xs, [0.25 + 1.5e-4 * x for x in xs])
    assert abs(a - 0.25) < 1e-9 and abs(b - 1.5e-4) < 1e-12 and r2 > 1 - 1e-12


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, env={**os.environ, "HIP_VISIBLE_DEVICES": ""})
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
