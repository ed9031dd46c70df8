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


@pytest.mark.parametrize("name", ["480p", "720p", "1080p", "classifier720p"])
def test_threshold_study_flop_fraction_matches_oracle_key_sets(name):
    """The study's routed-FLOP fraction equals the oracle's key-set sizes
    (pinned by brute force in the oracle tests) summed over the heads'
    labels, over all heads Global."""
    from head_routed_kv_amd.threshold_study import layer_flop_fraction
    from oracle import headcast_oracle as O
    wl = W.WORKLOADS[name]
    g = O.Geometry(wl.grid_h, wl.grid_w, wl.block_frames, wl.window_frames, wl.cell_h, wl.cell_w)
    rng = __import__("numpy").random.default_rng(7)
    for _ in range(5):
        labels = rng.integers(0, 4, wl.heads)
        want = sum(O.keyset_sizes(g, int(x)) for x in labels) / (wl.heads * O.keyset_sizes(g, O.GLOBAL))
        assert layer_flop_fraction(wl, labels) == pytest.approx(want, rel=1e-15)
    assert layer_flop_fraction(wl, [3] * wl.heads) == 1.0


def test_threshold_table_from_the_oracles_diagnostics():
    """The rule and threshold table of the graded planted workload, computed
    from the oracle's stored diagnostics (the labels depend on the thresholds
    only through the rule, not through the diagnostics): the oracle's rule at
    every (theta, theta_sc), then the routed-FLOP fraction.  Rules 0 and 1
    agree here, since no head clears two proxies."""
    import json
    from head_routed_kv_amd.threshold_study import layer_flop_fraction
    from oracle import headcast_oracle as O
    gold = json.load(open(os.path.join(ROOT, "tests", "golden", "classifier720p_graded_seed0.json")))
    wl = W.WORKLOADS["classifier720p_graded"]
    table = {   # theta: (fractions at theta_sc 0.6, 0.755, 0.9), label counts at 0.755 (Sink, Dummy, Spatial, Global)
        0.85: ((0.557, 0.557, 0.606), (9, 6, 5, 20)),
        0.90: ((0.600, 0.600, 0.648), (7, 6, 5, 22)),
        0.95: ((0.624, 0.624, 0.648), (7, 6, 4, 23)),
        0.98: ((0.648, 0.648, 0.648), (7, 6, 3, 24)),
    }
    for theta, (fracs, counts) in table.items():
        for theta_sc, frac in zip((0.6, 0.755, 0.9), fracs):
            labs = {}
            for rule in (0, 1):
                p = O.ClassifyParams(theta_sink=theta, theta_dummy=theta, theta_spatial=theta,
                                     theta_score=theta_sc, rule=rule)
                labs[rule] = [O.decide_label(d, p) for d in gold["diag"]]
            assert labs[0] == labs[1]
            assert round(layer_flop_fraction(wl, labs[0]), 3) == frac, (theta, theta_sc)
            if theta_sc == 0.755:
                assert tuple(labs[0].count(k) for k in range(4)) == counts
    assert gold["planted"].count(0) == 9 and gold["planted"].count(1) == 6 and gold["planted"].count(2) == 12


def test_1080p_head_shards_over_8_gpus():
    """Longest-processing-time packing of the 1080p layer's 40 heads onto 8
    GPUs.  Every head lands on exactly one GPU.  With 10 Global heads on 8
    GPUs some GPU must hold two of them (pigeonhole), so no plan can do
    better than twice a Global head's cost; this one reaches that bound,
    and no GPU is left idle."""
    wl = W.WORKLOADS["1080p"]
    labels = W.make_labels(wl)
    counts = {lab: int(sum(1 for x in labels if int(x) == lab)) for lab in range(4)}
    assert counts == {3: 10, 2: 16, 0: 8, 1: 6}
    cost = bench.head_costs(wl)
    # Global and Sink/Dummy heads are priced by their flops, Spatial heads by their bytes
    assert cost[3] == bench.algorithmic_work(wl, [3])[3][0] / (bench.PEAK_BF16_TFLOPS * 1e12)
    assert cost[0] == cost[1] < cost[3]
    assert cost[2] == bench.algorithmic_work(wl, [2])[2][1] / (bench.PEAK_HBM_GBS * 1e9)
    shards = bench.shard_heads(labels, cost, 8)
    assert sorted(h for s in shards for h in s) == list(range(40))
    loads = [sum(cost[int(labels[h])] for h in s) for s in shards]
    assert max(loads) == pytest.approx(2 * cost[3])
    assert all(s for s in shards)
    assert sum(loads) / 8 < max(loads)


def test_head_shards_small_cases():
    cost = {0: 1.0, 1: 1.0, 2: 0.5, 3: 4.0}
    # one GPU takes everything, in head order
    assert bench.shard_heads([3, 0, 2], cost, 1) == [[0, 1, 2]]
    # heaviest first, each to the least-loaded GPU, ties to the lower GPU
    assert bench.shard_heads([0, 3, 1, 3], cost, 2) == [[0, 1], [2, 3]]
    # more GPUs than heads: the extra GPUs stay empty
    assert bench.shard_heads([2, 2], cost, 3) == [[0], [1], []]
