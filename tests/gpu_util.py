"""Helpers for the GPU parity tests: upload seeded inputs, run the library
through its C ABI, compare with the oracle."""
import json
import os
import sys

import numpy as np

import head_routed_kv_amd as hk
from head_routed_kv_amd import workloads as W
from oracle import headcast_oracle as O

BF16_TOL = 2e-2   # per query row: max |gpu - oracle| <= BF16_TOL * RMS(oracle row)
FP32_TOL = 1e-5


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


def round_to_bf16(x):
    """float64 -> the nearest bf16 value (round half to even), as float64."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                       # x = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def parity_figures(got, ref, out_fmt):
    """Error figures of got against the oracle ref ([H, rows, d]):
      row_exact     max over query rows of max|gpu - oracle| / RMS(oracle row):
                    the asserted figure
      head          max over heads of max|gpu - oracle| / RMS(oracle head)
      tensor        max|gpu - oracle| / RMS(the whole oracle output)
    and, for results stored in bf16,
      row_rounded   as row_exact, against the oracle rounded to bf16
      floor_row, floor_head, floor_tensor
                    the row, head and tensor figures of the oracle rounded to
                    bf16 itself: what a correctly rounded bf16 result scores,
                    i.e. the part of each reading the output format takes
                    before any arithmetic error"""
    err = np.abs(got - ref)
    rms_row = np.maximum(np.sqrt(np.mean(ref ** 2, axis=-1)), 1e-30)
    rms_head = np.maximum(np.sqrt(np.mean(ref ** 2, axis=(-2, -1))), 1e-30)
    rms_all = max(np.sqrt(np.mean(ref ** 2)), 1e-30)
    fig = {"row_exact": float((err.max(axis=-1) / rms_row).max()),
           "head": float((err.max(axis=(-2, -1)) / rms_head).max()),
           "tensor": float(err.max() / rms_all)}
    if out_fmt == "bf16":
        rnd = round_to_bf16(ref)
        fig["row_rounded"] = float((np.abs(got - rnd).max(axis=-1) / rms_row).max())
        fl = np.abs(rnd - ref)
        fig["floor_row"] = float((fl.max(axis=-1) / rms_row).max())
        fig["floor_head"] = float((fl.max(axis=(-2, -1)) / rms_head).max())
        fig["floor_tensor"] = float(fl.max() / rms_all)
    return fig


def log_figures(what, fig, tol):
    """Print the figures and, when HEADCAST_PARITY_LOG names a file, append them
    to it as one JSON line."""
    rec = {"case": what, "tol": tol, **{k: round(v, 6) for k, v in fig.items()}}
    say("parity", json.dumps(rec))
    path = os.environ.get("HEADCAST_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(rec) + "\n")


def check_close(got, ref, tol, what="", out_fmt=None):
    """got, ref [H, rows, d]; asserts, for every query row,
        max_c |gpu - oracle| <= tol * RMS(oracle row),
    the bound read per query row: the output RMS is that of the row the
    error sits in.  out_fmt ("bf16" or "fp32", by default from the
    tolerance) only selects which figures are logged beside it
    (parity_figures): the per-head and whole-output readings, and for bf16
    results what correct rounding alone already scores under each reading.
    Returns the asserted figure."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    if out_fmt is None:
        out_fmt = "fp32" if tol == FP32_TOL else "bf16"
    fig = parity_figures(got, ref, out_fmt)
    log_figures(what, fig, tol)
    rms = np.sqrt(np.mean(ref ** 2, axis=-1))
    err = np.abs(got - ref).max(axis=-1)
    ratio = err / np.maximum(rms, 1e-30)
    h, r = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    assert ratio[h, r] <= tol, f"{what} head {h} row {r}: max abs err {err[h, r]:.3e} > {tol} * row rms {rms[h, r]:.3e}"
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
