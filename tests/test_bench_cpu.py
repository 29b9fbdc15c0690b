"""Host logic of bench.py that the committed profiles depend on (no GPU): which dispatches of a
rocprofv3 trace belong to the timed steps, and the --gpus contract."""

import subprocess
import sys
import os

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_timed_dispatches_both_regions():
    # fused region: 3 warm-up + 10 timed + 10 event steps; call-by-call region: 3 warm-up + 10 timed
    sel = bench._timed_dispatches(36, 10, 3)
    assert sel == list(range(3, 23)) + list(range(26, 36))
    # four launches per step (the long prefix: its logits kernel once per chunk)
    sel4 = bench._timed_dispatches(4 * 36, 10, 3)
    assert sel4 == list(range(12, 92)) + list(range(104, 144))


def test_timed_dispatches_one_region_kernels():
    # a kernel only the fused entry launches (the paged top-k reading fragment maxima)
    assert bench._timed_dispatches(23, 10, 3) == list(range(3, 23))
    # a kernel only the call-by-call region launches (the top-k entry called alone)
    assert bench._timed_dispatches(13, 10, 3) == list(range(3, 13))
    # counter runs: 1 warm-up, 3 steps
    assert bench._timed_dispatches(11, 3, 1) == list(range(1, 7)) + list(range(8, 11))
    # outside the timed regions (a one-off copy)
    assert bench._timed_dispatches(1, 10, 3) is None
    assert bench._timed_dispatches(0, 10, 3) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr) or "1 GPU" in (r.stdout + r.stderr)
