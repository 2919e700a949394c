"""Host-side behaviour of bench.py that needs no GPU: the one-GPU guard and
the settle phase that runs before the timed steps."""
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def run_bench(args, env_extra=None):
    env = dict(os.environ, **(env_extra or {}))
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          env=env, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = run_bench(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_a_multi_rank_launch_is_refused():
    r = run_bench([], {"WORLD_SIZE": "2"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


class _Clock:
    """Stand-in for the torch module: synchronize() does nothing."""

    @staticmethod
    def synchronize():
        pass


def test_settle_repeats_the_step_for_the_requested_time():
    calls = []

    def step():
        calls.append(1)
        time.sleep(0.002)

    t0 = time.perf_counter()
    n = bench.settle(step, type("T", (), {"cuda": _Clock}), 40.0)
    took = (time.perf_counter() - t0) * 1e3
    assert n == len(calls) and n >= 5
    assert 30.0 <= took <= 400.0


def test_settle_of_zero_runs_nothing():
    calls = []
    assert bench.settle(lambda: calls.append(1), None, 0.0) == 0
    assert calls == []


def test_decode_algorithmic_bytes():
    """The roofline numerator: K/V bytes follow the pages' closed form
    2 x Hkv x D x s x (sum of lengths) per layer (the 8B shape's 8 x 2048
    tokens: 64 MiB), and the per-launch totals are the ones the profiles
    quote (bf16 and E4M3 70B fused steps)."""
    kv, _ = bench.decode_alg_bytes([2048] * 8, 32, 8, 128, 2, 16, False, True)
    assert kv == 2 * 8 * 128 * 2 * (8 * 2048) == 64 * 2 ** 20
    kv, launch = bench.decode_alg_bytes([4096] * 32, 64, 8, 128, 2, 16, False, True)
    assert kv == 536_870_912 and launch == 538_214_528
    _, split = bench.decode_alg_bytes([4096] * 32, 64, 8, 128, 2, 16, False, False)
    assert launch - split == 2 * 32 * 8 * 128 * 2 * 2  # the fused step's new rows, read and written
    kv8, launch8 = bench.decode_alg_bytes([4096] * 32, 64, 8, 128, 2, 16, True, True)
    assert kv8 == 2 * 8 * (128 + 4) * (32 * 4096) and launch8 == 278_104_192
    # ragged lengths: tables count each sequence's own blocks
    kv, launch = bench.decode_alg_bytes([1, 17, 0], 4, 2, 64, 2, 16, False, False)
    assert kv == 2 * 2 * 64 * 2 * 18
    assert launch == kv + 2 * 3 * 4 * 64 * 2 + 4 * (1 + 2 + 0) + 4 * 3
