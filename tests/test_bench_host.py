"""bench.py on the host: the one-GPU contract and its accounting (no GPU needed)."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_is_tied_to_the_kernel_sources():
    t = bench.measured_traffic()
    if bench.csrc_digest() == bench.TRAFFIC["sources"]:
        # FETCH_SIZE scaled by the copy factor plus WRITE_SIZE, in bytes, close to the
        # one-row launch's algorithmic bytes (8 experts of gate+up weights, x, logits, top-k, act)
        alg = 8 * 8912896 + 4096 * 2 + 8 * 2048 * 4 + 256 * 4 + 8 * 8
        assert 0.99 * alg < t < 1.05 * alg
    else:
        assert t is None
    f = bench.measured_traffic(bench.FP8_TRAFFIC, bench.FP8_SOURCES)
    if bench.csrc_digest(bench.FP8_SOURCES) == bench.FP8_TRAFFIC["sources"]:
        alg = 4096 * 4096 + 32 * 32 * 4       # weight bytes and scales of the 4096 x 4096 launch
        assert 0.99 * alg < f < 1.1 * alg
    else:
        assert f is None
    # prefill chunk (4,096 rows): at least the algorithmic bytes of the seeded layers
    # (about 2.58 GB gate/up, 1.94 GB down: each routed expert's weights once plus
    # the activations in and out), at most twice that
    for tr, alg in ((bench.PF_GU_TRAFFIC, 2.579e9), (bench.PF_DN_TRAFFIC, 1.944e9)):
        v = bench.measured_traffic(tr, bench.PREFILL_SOURCES)
        if bench.csrc_digest(bench.PREFILL_SOURCES) == tr["sources"]:
            assert 0.99 * alg < v < 2.0 * alg
        else:
            assert v is None


def test_sweep_sets_are_valid_pass_sizes():
    for gu, dn in bench.TIER_SWEEP:
        for t in (gu, dn):
            assert list(t) == sorted(set(t)) and all(2 <= v <= 8 for v in t)
