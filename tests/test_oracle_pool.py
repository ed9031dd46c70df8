"""The oracle's process pool (oracle/pool.py) against direct oracle calls:
assembling row chunks computed in worker processes gives the oracle's own
output for every (head, pathway) pair, and the sampled-rows mode gives those
rows.  CPU only (two spawned workers, a reduced workload)."""
import numpy as np

from head_routed_kv_amd import workloads as W
from oracle import headcast_oracle as O
from oracle import pool


def _direct(wl, seed, head, pathway, rows=None):
    data = W.window(wl, seed=seed, heads=[head], threads=1)
    q, k, v = (W.as_float(data[n], wl)[0] for n in ("q", "k", "v"))
    g = O.Geometry(wl.grid_h, wl.grid_w, wl.block_frames, wl.window_frames, wl.cell_h, wl.cell_w)
    return O.attend_head(q, k, v, pathway, g, rows=rows)


def test_pool_assembles_the_oracles_rows():
    wl = W.small(W.WORKLOADS["720p"], grid_h=13, grid_w=22, heads=3, window_frames=6, name="pool-test")
    pairs = [(0, O.GLOBAL), (1, O.SPATIAL), (2, O.SINK), (2, O.DUMMY)]
    res, cpu_s, wall = pool.run(wl, 5, pairs, rows_per_task=97, procs=2)   # ragged last chunk
    assert set(res) == set(pairs) and cpu_s > 0 and wall > 0
    for h, pw in pairs:
        want = _direct(wl, 5, h, pw)
        assert res[(h, pw)].shape == (wl.Nq, wl.head_dim)
        np.testing.assert_allclose(res[(h, pw)], want, rtol=0, atol=1e-12)


def test_pool_sampled_rows():
    wl = W.small(W.WORKLOADS["720p"], grid_h=13, grid_w=22, heads=2, window_frames=6, name="pool-test")
    rows = [0, 5, 200, wl.Nq - 1]
    res, _, _ = pool.run(wl, 3, [(1, O.SPATIAL), (0, O.GLOBAL)], rows=rows, procs=2)
    for (h, pw), got in res.items():
        np.testing.assert_allclose(got, _direct(wl, 3, h, pw, rows=np.asarray(rows)), rtol=0, atol=1e-12)


def test_chunks_cover_every_row_once():
    wl = W.WORKLOADS["720p"]
    tasks = pool.chunk_tasks(wl, 0, [(0, O.GLOBAL), (4, O.SPATIAL)], rows_per_task=1350)
    for h in (0, 4):
        spans = sorted((t[4], t[5]) for t in tasks if t[2] == h)
        assert spans[0][0] == 0 and sum(n for _, n in spans) == wl.Nq
        assert all(a + n == b for (a, n), (b, _) in zip(spans, spans[1:]))


def test_pool_fp8_cache_values():
    """kv_scales: the workers attend over the oracle's E4M3 quantise-then-decode
    of K and V, as an fp8 cache holds them."""
    wl = W.small(W.WORKLOADS["720p"], grid_h=13, grid_w=22, heads=2, window_frames=6, name="pool-test")
    ks, vs = 0.75, 1.5
    res, _, _ = pool.run(wl, 4, [(0, O.GLOBAL), (1, O.SPATIAL)], rows_per_task=200, procs=2, kv_scales=(ks, vs))
    g = O.Geometry(wl.grid_h, wl.grid_w, wl.block_frames, wl.window_frames, wl.cell_h, wl.cell_w)
    for h, pw in ((0, O.GLOBAL), (1, O.SPATIAL)):
        data = W.window(wl, seed=4, heads=[h], threads=1)
        q, k, v = (W.as_float(data[n], wl)[0] for n in ("q", "k", "v"))
        dk = O.dequantize_kv(O.quantize_kv(k, ks), ks)
        dv = O.dequantize_kv(O.quantize_kv(v, vs), vs)
        np.testing.assert_allclose(res[(h, pw)], O.attend_head(q, dk, dv, pw, g), rtol=0, atol=1e-12)
        assert not np.allclose(dk, k)   # the codes do change the values
