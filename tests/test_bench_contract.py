"""The benchmark's work accounting and command-line contract (CPU only).

The roofline's `achieved` figure divides the layer's algorithmic work by the
attention kernel's time, so the work per head is pinned here to closed
forms: 4*d flops per (query, key) pair of a head's key set, and Q read + O
written + the key set's K and V read once, in bf16."""
import os
import subprocess
import sys

import pytest

import bench
from head_routed_kv_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def per_head(wl, lab):
    flops, nbytes = bench.algorithmic_work(wl, [lab])[lab]
    return flops, nbytes


def test_720p_work_per_head():
    wl = W.WORKLOADS["720p"]   # 45x80 grid, 3-frame blocks, 21-frame window, d = 128
    # Global: 10800 queries x 75600 keys; Sink and Dummy: 10800 x 10800
    assert per_head(wl, 3)[0] == 4 * 128 * 10800 * 75600 == 418_037_760_000
    assert per_head(wl, 0)[0] == per_head(wl, 1)[0] == 4 * 128 * 10800 * 10800
    # Spatial: 3 x 21 frames x (32 full 10x10 cells + 8 half cells of 5x10)^2 sizes
    assert per_head(wl, 2)[0] == 4 * 128 * 3 * 21 * (32 * 100 ** 2 + 8 * 50 ** 2)
    # bytes: Q + O = 2 * 10800 * 128 * 2; K + V of 75600 or 10800 keys
    qo = 2 * 10800 * 128 * 2
    assert per_head(wl, 3)[1] == per_head(wl, 2)[1] == qo + 2 * 75600 * 128 * 2
    assert per_head(wl, 0)[1] == qo + 2 * 10800 * 128 * 2


def test_layer_work_is_the_sum_over_heads():
    wl = W.WORKLOADS["720p"]
    labels = W.make_labels(wl)
    work = bench.algorithmic_work(wl, labels)
    counts = {lab: int(sum(1 for x in labels if int(x) == lab)) for lab in range(4)}
    assert counts == {3: 3, 2: 5, 0: 2, 1: 2}
    total = sum(f for f, _ in work.values())
    assert total == sum(counts[lab] * per_head(wl, lab)[0] for lab in range(4))
    assert abs(total / 1e12 - 1.548) < 5e-4


def test_cell_sizes_cover_the_frame():
    for name in ("480p", "720p", "1080p"):
        wl = W.WORKLOADS[name]
        assert sum(bench.cell_sizes(wl.grid_h, wl.grid_w)) == wl.grid_h * wl.grid_w


@pytest.mark.parametrize("n", [0, 2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
