"""Helpers for the GPU parity tests: upload seeded inputs, run the library
through its C ABI, compare with the oracle."""
import sys

import numpy as np

import head_routed_kv_amd as hk
from head_routed_kv_amd import workloads as W
from oracle import headcast_oracle as O

BF16_TOL = 2e-2   # per query row and channel: |gpu - oracle| <= BF16_TOL * rms(oracle row) + u * |oracle|
FP32_TOL = 1e-5
BF16_U = 2.0 ** -8    # unit roundoff of the output format: a bf16 result is off by up to u * |o| by itself
FP32_U = 2.0 ** -24


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def torch():
    import torch as t
    return t


def upload(a, wl):
    """Storage-form numpy array -> device tensor (bf16 or fp32)."""
    t = torch()
    if wl.dtype == "fp32":
        return t.from_numpy(np.ascontiguousarray(a)).cuda()
    return t.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(t.bfloat16).cuda()


def download_bits(x):
    """Device tensor -> numpy storage form (uint16 bits for bf16)."""
    t = torch()
    if x.dtype == t.bfloat16:
        return x.view(t.int16).cpu().numpy().view(np.uint16)
    return x.cpu().numpy()


def to_float(x):
    t = torch()
    return x.float().cpu().numpy() if x.dtype != t.float32 else x.cpu().numpy()


def config_of(wl, dtype=None):
    return hk.make_config(wl.heads, wl.head_dim, wl.grid_h, wl.grid_w, wl.block_frames, wl.window_frames,
                          wl.cell_h, wl.cell_w, hk.HC_FP32 if wl.dtype == "fp32" else hk.HC_BF16)


def geometry_of(wl):
    return O.Geometry(wl.grid_h, wl.grid_w, wl.block_frames, wl.window_frames, wl.cell_h, wl.cell_w)


def fill_cache(wl, labels, k, v):
    """Restructure: create the cache and replay the window's blocks."""
    cache = hk.RoutedCache(config_of(wl), labels)
    BT = wl.Nq
    for b in range(wl.n_blocks):
        cache.append(k[:, b * BT:(b + 1) * BT], v[:, b * BT:(b + 1) * BT])
    return cache


def check_close(got, ref, tol, what=""):
    """got, ref [H, rows, d].  Every query row and channel c: |gpu - oracle|
    <= tol * RMS of the oracle's output row + u * |oracle_c|, u the unit
    roundoff of the output format (bf16 for BF16_TOL, fp32 for FP32_TOL).
    The second term is the output's own rounding, which no result in that
    format avoids; the first bounds the kernel's arithmetic.  (Against the
    RMS of a whole head, a correctly rounded bf16 output already misses 2e-2
    on Spatial heads, whose outputs are heavy-tailed: max|o|/RMS ~ 10.)
    Returns the worst ratio (|err| - u|o|) / RMS seen."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    u = BF16_U if tol == BF16_TOL else FP32_U
    rms = np.sqrt(np.mean(ref ** 2, axis=-1))
    excess = np.abs(got - ref) - u * np.abs(ref)
    err = excess.max(axis=-1)
    ratio = err / np.maximum(rms, 1e-30)
    h, r = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    assert ratio[h, r] <= tol, (f"{what} head {h} row {r}: max (abs err - u|o|) {err[h, r]:.3e} > {tol} * row rms "
                                f"{rms[h, r]:.3e}")
    return float(ratio.max())


def sample_rows(wl, n=48, seed=0):
    """Query rows to check at full size: both ends (ragged last q tile), the
    frame seams, border-cell rows, the last query of the first cell (in the
    cell's short remainder sub-tile when a cell holds more queries than one
    work group) and a seeded random spread."""
    rng = np.random.default_rng(seed)
    T, Nq, gw = wl.T, wl.Nq, wl.grid_w
    last_of_cell0 = (wl.block_frames - 1) * T + (min(wl.cell_h, wl.grid_h) - 1) * gw + min(wl.cell_w, gw) - 1
    fixed = [0, 1, 127, 128, Nq - 1, Nq - 2, T - 1, T, gw - 1, T - gw, Nq - gw, last_of_cell0]
    rows = set(r for r in fixed if 0 <= r < Nq)
    rows.update(rng.integers(0, Nq, n - len(rows)).tolist())
    return np.array(sorted(rows))
