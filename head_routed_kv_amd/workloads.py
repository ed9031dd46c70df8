"""Seeded synthetic workloads for head-routed attention.

This module only draws inputs: shapes, seeded normal draws, bf16 rounding,
label assignment and the planted structure of the classifier workload.  It
holds none of the attention or classification arithmetic, and both the GPU
tests and the CPU oracle take their inputs from here.

Workloads (all Q/K/V entries i.i.d. N(0,1) unless stated):
  tiny            fp32, 4 heads labelled Sink/Dummy/Spatial/Global, d=64,
                  grid 8x12, block 1 frame, window 4 frames
  480p            bf16, 12 heads, d=128, grid 30x52, block 3, window 21,
                  labels i.i.d. uniform per head
  720p            bf16, 12 heads, d=128, grid 45x80, block 3, window 21,
                  label mix Global 25% / Spatial 40% / Sink 20% / Dummy 15%
  1080p           bf16, 40 heads, d=128, grid 68x120, block 3, window 21, same mix
  classifier720p  bf16, 40 heads at the 720p shape with planted structure
                  (see `planted_window`)
  classifier720p_graded  the same, each planted head's key offset scaled by
                  a seeded strength u ~ U(0, 0.25): a full offset raises the
                  target keys' logits by about 34, so heads at u ~ 0.1 sit
                  near the cosine thresholds (threshold studies)

Random streams: numpy SeedSequence([seed, workload_id, head, tensor_id]) ->
PCG64 -> standard_normal(float32) -> bf16 by round-to-nearest-even, so any
head can be regenerated alone and every consumer sees identical bits.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

SINK, DUMMY, SPATIAL, GLOBAL = 0, 1, 2, 3


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int
    heads: int
    head_dim: int
    grid_h: int
    grid_w: int
    block_frames: int
    window_frames: int
    dtype: str          # "fp32" | "bf16"
    labels: str         # "fixed" | "uniform" | "mix" | "planted"
    cell_h: int = 10
    cell_w: int = 10

    @property
    def T(self):
        return self.grid_h * self.grid_w

    @property
    def Nq(self):
        return self.block_frames * self.T

    @property
    def Nk(self):
        return self.window_frames * self.T

    @property
    def n_blocks(self):
        return self.window_frames // self.block_frames


WORKLOADS = {
    "tiny": Workload("tiny", 0, 4, 64, 8, 12, 1, 4, "fp32", "fixed"),
    "480p": Workload("480p", 1, 12, 128, 30, 52, 3, 21, "bf16", "uniform"),
    "720p": Workload("720p", 2, 12, 128, 45, 80, 3, 21, "bf16", "mix"),
    "1080p": Workload("1080p", 3, 40, 128, 68, 120, 3, 21, "bf16", "mix"),
    "classifier720p": Workload("classifier720p", 4, 40, 128, 45, 80, 3, 21, "bf16", "planted"),
    "classifier720p_graded": Workload("classifier720p_graded", 5, 40, 128, 45, 80, 3, 21, "bf16", "graded"),
}

# tensor ids inside a (seed, workload, head) stream family
_T_Q, _T_PLANT, _T_LABEL, _T_STRENGTH = 0, 1, 2, 3
_T_BLOCK_K, _T_BLOCK_V = 16, 17        # + 2 * block index


def f32_to_bf16_bits(x, out=None, tmp=None):
    """float32 array -> bf16 bit patterns (uint16), round to nearest even.
    `out` (uint16) and `tmp` (uint32) may be given to avoid allocation."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if tmp is None:
        tmp = np.empty(u.shape, dtype=np.uint32)
    np.right_shift(u, 16, out=tmp)
    np.bitwise_and(tmp, 1, out=tmp)
    np.add(tmp, 0x7FFF, out=tmp)
    np.add(tmp, u, out=tmp)
    np.right_shift(tmp, 16, out=tmp)
    if out is None:
        return tmp.astype(np.uint16)
    np.copyto(out, tmp, casting="unsafe")
    return out


def bf16_bits_to_f32(b):
    """bf16 bit patterns (uint16) -> float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed, wl: Workload, head, tensor_id):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, wl.wid, head, tensor_id])))


def _normal(seed, wl, head, tensor_id, rows, d, out=None):
    if out is None:
        out = np.empty((rows, d), dtype=np.float32)
    _rng(seed, wl, head, tensor_id).standard_normal(out=out, dtype=np.float32)
    return out


def _encode(x, wl):
    """Storage form of a float32 array: float32 itself, or bf16 bits."""
    return x if wl.dtype == "fp32" else f32_to_bf16_bits(x)


def _store(x, dst, wl, tmp):
    """Write float32 x into the storage-form array dst."""
    if wl.dtype == "fp32":
        np.copyto(dst, x)
    else:
        f32_to_bf16_bits(x, dst, tmp)


def storage_dtype(wl):
    return np.float32 if wl.dtype == "fp32" else np.uint16


def as_float(x, wl):
    """Storage form -> float32 values."""
    return x if wl.dtype == "fp32" else bf16_bits_to_f32(x)


def make_labels(wl: Workload, seed: int = 0):
    """int8 [H] archetype labels for a routed-attention workload."""
    H = wl.heads
    if wl.labels == "fixed":
        return np.array([SINK, DUMMY, SPATIAL, GLOBAL][:H], dtype=np.int8)
    if wl.labels == "uniform":
        return _rng(seed, wl, 0, _T_LABEL).integers(0, 4, size=H).astype(np.int8)
    if wl.labels == "mix":
        # largest-remainder rounding of the 25/40/20/15 % mix, ties in the listed
        # order, then a seeded permutation over heads
        order = [GLOBAL, SPATIAL, SINK, DUMMY]
        pct = [25, 40, 20, 15]
        base = [H * p // 100 for p in pct]
        rem = [H * p % 100 for p in pct]
        left = H - sum(base)
        for i in sorted(range(4), key=lambda i: (-rem[i], i))[:left]:
            base[i] += 1
        labs = np.concatenate([np.full(n, lab, dtype=np.int8) for lab, n in zip(order, base)])
        return labs[_rng(seed, wl, 0, _T_LABEL).permutation(H)]
    raise ValueError(f"workload {wl.name} has planted labels; use planted_window")


def block_kv(wl: Workload, seed: int, block: int, head: int, out_k=None, out_v=None):
    """Float32 K and V of one block ([B*T, d] each) for one head, unplanted."""
    rows = wl.Nq
    k = _normal(seed, wl, head, _T_BLOCK_K + 2 * block, rows, wl.head_dim, out_k)
    v = _normal(seed, wl, head, _T_BLOCK_V + 2 * block, rows, wl.head_dim, out_v)
    return k, v


def _map_heads(fn, n, threads):
    if threads <= 1 or n <= 1:
        for i in range(n):
            fn(i)
        return
    with ThreadPoolExecutor(max_workers=min(threads, n)) as ex:
        list(ex.map(fn, range(n)))


def _fill_window(wl, seed, heads, threads, plant=None):
    """Allocate q [h,Nq,d], k/v [h,Nk,d] in storage form and fill them head by head."""
    H, d, BT = len(heads), wl.head_dim, wl.Nq
    sd = storage_dtype(wl)
    q = np.empty((H, wl.Nq, d), dtype=sd)
    k = np.empty((H, wl.Nk, d), dtype=sd)
    v = np.empty((H, wl.Nk, d), dtype=sd)

    def one(i):
        h = heads[i]
        tmp = np.empty((BT, d), dtype=np.uint32)
        if plant is None:
            fk = np.empty((BT, d), dtype=np.float32)
            fv = np.empty((BT, d), dtype=np.float32)
            for b in range(wl.n_blocks):
                block_kv(wl, seed, b, h, fk, fv)
                _store(fk, k[i, b * BT:(b + 1) * BT], wl, tmp)
                _store(fv, v[i, b * BT:(b + 1) * BT], wl, tmp)
            fq = _normal(seed, wl, h, _T_Q, BT, d, fk)
            _store(fq, q[i], wl, tmp)
        else:
            fk = np.empty((wl.Nk, d), dtype=np.float32)
            fv = np.empty((BT, d), dtype=np.float32)
            for b in range(wl.n_blocks):
                block_kv(wl, seed, b, h, fk[b * BT:(b + 1) * BT], fv)
                _store(fv, v[i, b * BT:(b + 1) * BT], wl, tmp)
            fq = _normal(seed, wl, h, _T_Q, BT, d, fv)
            plant(h, fq, fk)
            _store(fq, q[i], wl, tmp)
            ktmp = np.empty((wl.Nk, d), dtype=np.uint32)
            _store(fk, k[i], wl, ktmp)

    _map_heads(one, H, threads)
    return q, k, v


def window(wl: Workload, seed: int = 0, heads=None, threads: int = 8):
    """Routed-attention inputs at first window fill.

    Returns dict with q [h, Nq, d], k, v [h, Nk, d] in storage form (float32
    or bf16 bits), `labels` int8 [H] (all heads) and `heads` (the indices
    drawn).  The window is blocks 0 .. W/B-1; the queries are the last block."""
    if wl.labels in ("planted", "graded"):
        return planted_window(wl, seed, heads, threads)
    heads = list(range(wl.heads)) if heads is None else list(heads)
    q, k, v = _fill_window(wl, seed, heads, threads)
    return {"q": q, "k": k, "v": v, "heads": heads, "labels": make_labels(wl, seed)}


def stream_blocks(wl: Workload, seed: int, n_blocks: int, heads=None):
    """K/V of blocks 0..n_blocks-1 in storage form: lists of [h, B*T, d]."""
    heads = list(range(wl.heads)) if heads is None else list(heads)
    ks, vs = [], []
    for b in range(n_blocks):
        kb, vb = zip(*[block_kv(wl, seed, b, h) for h in heads])
        ks.append(_encode(np.stack(kb), wl))
        vs.append(_encode(np.stack(vb), wl))
    return ks, vs


def queries(wl: Workload, seed: int = 0, heads=None, tensor_id: int = _T_Q):
    heads = list(range(wl.heads)) if heads is None else list(heads)
    return _encode(np.stack([_normal(seed, wl, h, tensor_id, wl.Nq, wl.head_dim) for h in heads]), wl)


# ----------------------------------------------------------------------------
# Planted classifier workload.
#
# Each head draws a kind i.i.d. uniform over {Sink, Dummy, Spatial, none}.
# Planted heads get a shared query offset mu ~ N(0, I_d) (one per head for
# Sink/Dummy, one per 10x10 latent cell for Spatial); keys in the target region
# then get +3 * mean(q) over the relevant queries (all queries, or the cell's
# queries): first block (Sink), newest block (Dummy), the cell in every frame
# (Spatial).  "none" heads get neither and are expected to route Global.
# ----------------------------------------------------------------------------
NONE_KIND = GLOBAL


def planted_kinds(wl: Workload, seed: int = 0):
    r = _rng(seed, wl, 0, _T_LABEL).integers(0, 4, size=wl.heads)
    return np.array([[SINK, DUMMY, SPATIAL, NONE_KIND][i] for i in r], dtype=np.int8)


def _cell_index(wl, n_frames):
    """Latent 10x10 cell id of every token of n_frames frames (input recipe)."""
    t = np.arange(n_frames * wl.T)
    y = (t % wl.T) // wl.grid_w
    x = t % wl.grid_w
    ncx = -(-wl.grid_w // wl.cell_w)
    return (y // wl.cell_h) * ncx + x // wl.cell_w


def plant_strength(wl: Workload, seed: int = 0):
    """Per-head multiplier of the planted key offset: 1 for the planted
    workload, u ~ U(0, 0.25) per head for the graded one."""
    if wl.labels != "graded":
        return np.ones(wl.heads, dtype=np.float32)
    return np.array([0.25 * _rng(seed, wl, h, _T_STRENGTH).random() for h in range(wl.heads)], dtype=np.float32)


def _plant_head(wl, seed, h, kind, q, k, strength=1.0):
    """Add the planted structure to one head's float32 q [Nq,d], k [Nk,d] in place."""
    if kind == NONE_KIND:
        return
    B, T = wl.block_frames, wl.T
    rng = _rng(seed, wl, h, _T_PLANT)
    if kind in (SINK, DUMMY):
        mu = rng.standard_normal(wl.head_dim, dtype=np.float32)
        q += mu
        qm = as_float(_encode(q, wl), wl).mean(axis=0, dtype=np.float64).astype(np.float32)
        rows = slice(0, B * T) if kind == SINK else slice(wl.Nk - B * T, wl.Nk)
        k[rows] += np.float32(3.0 * strength) * qm
        return
    # Spatial: one offset per cell
    qcell = _cell_index(wl, B)
    kcell = _cell_index(wl, wl.window_frames)
    ncell = int(qcell.max()) + 1
    mus = rng.standard_normal((ncell, wl.head_dim), dtype=np.float32)
    q += mus[qcell]
    qs = as_float(_encode(q, wl), wl)
    for c in range(ncell):
        qm = qs[qcell == c].mean(axis=0, dtype=np.float64).astype(np.float32)
        k[kcell == c] += np.float32(3.0 * strength) * qm


def planted_window(wl: Workload, seed: int = 0, heads=None, threads: int = 8):
    heads = list(range(wl.heads)) if heads is None else list(heads)
    kinds = planted_kinds(wl, seed)
    strength = plant_strength(wl, seed)
    q, k, v = _fill_window(wl, seed, heads, threads,
                           plant=lambda h, fq, fk: _plant_head(wl, seed, h, int(kinds[h]), fq, fk,
                                                               float(strength[h])))
    return {"q": q, "k": k, "v": v, "heads": heads, "labels": kinds, "strength": strength}


def small(wl: Workload, grid_h=None, grid_w=None, heads=None, window_frames=None, name=None):
    """A reduced copy of a workload (same dtype, label recipe, block size)."""
    from dataclasses import replace
    return replace(wl, name=name or wl.name + "-small",
                   grid_h=grid_h or wl.grid_h, grid_w=grid_w or wl.grid_w,
                   heads=heads or wl.heads, window_frames=window_frames or wl.window_frames)
