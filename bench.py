"""Benchmark: head-routed attention query-heads/s per layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 720p]

One step = one steady-state denoising step of one layer: the block being
denoised gets new keys/values (hc_cache_append with REPLACE_NEWEST) and every
head attends over its archetype's keys (hc_attend).  Inputs are synthetic
N(0,1) bf16 of the workload's shape, resident in HBM before timing starts;
the cache is restructured (W/B block appends) before timing.  The GPU's
shader clock ramps up over the first ~100 ms of load, so untimed steps run
for --clock-warmup seconds before the W warm-up steps; the timed region is
still exactly K full steps.

Prints ONE JSON line with the metric, the roofline of the dominant kernel
(the attention kernel, timed with HIP events on the stream it runs on), the
same GPU's full-attention time (every head Global) and the CPU oracle timed
on a bounded sample."""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def cell_sizes(gh, gw, ch=10, cw=10):
    out = []
    for cy in range(-(-gh // ch)):
        for cx in range(-(-gw // cw)):
            out.append(min(ch, gh - cy * ch) * min(cw, gw - cx * cw))
    return out


def algorithmic_work(wl, labels):
    """Per pathway: (flops, bytes) a layer must compute / move.  Flops are
    4*d per (query, key) pair of each head's key set (QK^T and PV); bytes are
    Q read + O written + each head's K/V set read once (bf16)."""
    B, W, T, d, Nq = wl.block_frames, wl.window_frames, wl.T, wl.head_dim, wl.Nq
    pairs = {3: Nq * W * T, 0: Nq * B * T, 1: Nq * B * T,
             2: B * W * sum(c * c for c in cell_sizes(wl.grid_h, wl.grid_w))}
    keys = {3: W * T, 0: B * T, 1: B * T, 2: W * T}
    out = {}
    for lab in (0, 1, 2, 3):
        n = int(sum(1 for x in labels if int(x) == lab))
        out[lab] = (n * 4 * d * pairs[lab], n * (2 * 2 * Nq * d + 2 * 2 * keys[lab] * d))
    return out


def gen_inputs(wl, seed, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    mk = lambda n: torch.randn(wl.heads, n, wl.head_dim, generator=g, device=device,
                               dtype=torch.float32).to(torch.bfloat16)
    return mk(wl.Nq), mk(wl.Nk), mk(wl.Nk)


class Layer:
    """One layer's restructured cache plus its inputs."""

    def __init__(self, wl, labels, q, k, v, kv_format=0):
        import head_routed_kv_amd as hk
        self.hk = hk
        cfg = hk.make_config(wl.heads, wl.head_dim, wl.grid_h, wl.grid_w, wl.block_frames, wl.window_frames,
                             kv_format=kv_format)
        self.cache = hk.RoutedCache(cfg, [int(x) for x in labels])
        BT = wl.Nq
        for b in range(wl.n_blocks):
            self.cache.append(k[:, b * BT:(b + 1) * BT], v[:, b * BT:(b + 1) * BT])
        self.q = q
        self.k_new = k[:, (wl.n_blocks - 1) * BT:]
        self.v_new = v[:, (wl.n_blocks - 1) * BT:]
        import torch
        self.out = torch.empty_like(q)

    def append(self):
        self.cache.append(self.k_new, self.v_new, self.hk.HC_REPLACE_NEWEST)

    def attend(self):
        self.cache.attend(self.q, self.out)

    def step(self):
        self.append()
        self.attend()


def time_samples(fn, iters, flush=None):
    """ms of each of `iters` calls of fn(), between HIP events on the current stream."""
    import torch
    out = []
    for _ in range(iters):
        if flush is not None:
            flush()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        b.synchronize()
        out.append(a.elapsed_time(b))
    return out


def time_events(fn, iters, flush=None):
    """Average ms of fn() between HIP events on the current stream."""
    return statistics.fmean(time_samples(fn, iters, flush))


def summary(ms):
    return {"mean": round(statistics.fmean(ms), 4), "median": round(statistics.median(ms), 4),
            "min": round(min(ms), 4), "n": len(ms)}


def device_info(index=0):
    """Name, compute units and peak shader clock of the GPU (hipDeviceGetAttribute for the clock)."""
    import ctypes
    import torch
    p = torch.cuda.get_device_properties(index)
    info = {"name": p.name, "arch": p.gcnArchName.split(":")[0], "compute_units": p.multi_processor_count}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        khz = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(khz), 5, index) == 0:   # hipDeviceAttributeClockRate
            info["peak_sclk_mhz"] = khz.value // 1000
    except OSError:
        pass
    return info


def ceilings(device):
    """Achievable ceilings on this GPU, as context: a large bf16 GEMM (torch.matmul) and a device copy."""
    import torch
    n = 8192
    a = torch.randn(n, n, device=device, dtype=torch.float32).to(torch.bfloat16)
    b = torch.randn(n, n, device=device, dtype=torch.float32).to(torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    mm = statistics.median(time_samples(lambda: torch.matmul(a, b), 10))
    del a, b
    src = torch.ones(1 << 28, dtype=torch.float32, device=device)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    cp = statistics.median(time_samples(lambda: dst.copy_(src), 10))
    del src, dst
    torch.cuda.empty_cache()
    return {"matmul_bf16_8192": {"ms": round(mm, 4), "tflops": round(2 * n ** 3 / (mm / 1e3) / 1e12, 1)},
            "copy_1gib": {"ms": round(cp, 4), "gbs": round(2 * (1 << 30) / (cp / 1e3) / 1e9, 1)}}


def make_flush(device):
    import torch
    buf = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device=device)

    def flush():   # write 512 MiB so the 256 MB Infinity Cache holds none of the layer's K/V
        buf.fill_(1.0)
    return flush


def rollout_costs(wl, labels, q, k, v, full_ms, steps_per_block=4, lengths=(14, 40)):
    """Attention cost of one layer over a video rollout, phase by phase.

    Warm-up: while the first window fills, every head attends over the growing
    window (each block: one push and steps_per_block - 1 replacements, an
    attend after each).  At first fill: hc_classify on the window, then the
    window's blocks are replayed into the routed cache.  Afterwards each block's
    steps go through the routed cache.  The routed cache uses this layer's
    label mix (the classifier runs on the same random inputs only for its
    time).  Routed blocks are timed over 8 blocks; longer rollouts are
    extrapolated from that steady-state cost."""
    import torch
    import head_routed_kv_amd as hk
    from head_routed_kv_amd.session import LayerSession
    nb, BT = wl.window_frames // wl.block_frames, wl.Nq
    cfg = hk.make_config(wl.heads, wl.head_dim, wl.grid_h, wl.grid_w, wl.block_frames, wl.window_frames)
    out = torch.empty_like(q)

    def timed(fn):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        b.synchronize()
        return a.elapsed_time(b)

    def blk(kk, vv, b):
        return kk[:, b * BT:(b + 1) * BT], vv[:, b * BT:(b + 1) * BT]

    sess = LayerSession(cfg)
    ws = hk.classify(cfg, q, k, v)[2]          # workspace, allocated outside the timed region
    torch.cuda.synchronize()

    def block_steps(cache_push, cache_replace, attend, kb, vb):
        for s in range(steps_per_block):
            (cache_push if s == 0 else cache_replace)(kb, vb)
            attend(q, out)

    warm_ms = sum(timed(lambda b=b: block_steps(sess.push, sess.replace, sess.attend, *blk(k, v, b)))
                  for b in range(nb))
    kw, vw = sess.window_views()
    cls_ms = timed(lambda: hk.classify(cfg, q, kw, vw, workspace=ws))
    holder = {}

    def restructure():
        holder["c"] = hk.RoutedCache(cfg, [int(x) for x in labels])
        for b in range(nb):
            holder["c"].append(*blk(kw, vw, b))
    rest_ms = timed(restructure)
    routed = holder["c"]
    rep = lambda kb, vb: routed.append(kb, vb, hk.HC_REPLACE_NEWEST)
    n_timed = 8
    routed_ms = sum(timed(lambda b=b: block_steps(routed.append, rep, routed.attend, *blk(k, v, b % nb)))
                    for b in range(n_timed)) / n_timed
    sess.close()
    routed.close()
    full_block_ms = full_ms * steps_per_block
    res = {"steps_per_block": steps_per_block, "warmup_ms": round(warm_ms, 2), "classify_ms": round(cls_ms, 3),
           "restructure_ms": round(rest_ms, 3), "routed_block_ms": round(routed_ms, 3),
           "full_block_ms": round(full_block_ms, 3), "by_blocks": {}}
    for n in lengths:
        total = warm_ms + cls_ms + rest_ms + (n - nb) * routed_ms
        full_total = warm_ms + (n - nb) * full_block_ms
        res["by_blocks"][str(n)] = {"attention_ms": round(total, 1),
                                    "classification_share": round((cls_ms + rest_ms) / total, 4),
                                    "speedup_vs_full_attention": round(full_total / total, 3)}
    return res


def box_span(n, r):
    """Sum over positions 0..n-1 of the box extent [p-r, p+r] cut to [0, n)."""
    return sum(min(p + r, n - 1) - max(p - r, 0) + 1 for p in range(n))


def source_fingerprint(paths):
    """SHA-256 of the code in `paths` with comments and whitespace removed
    (// and /* */ in C/HIP sources, # in Python), so that a comment edit does
    not count as a kernel change and any code edit does."""
    import hashlib
    import re
    h = hashlib.sha256()
    for src in paths:
        text = open(os.path.join(ROOT, src), encoding="utf-8").read()
        if src.endswith(".py"):
            text = re.sub(r"#[^\n]*", " ", text)
        else:
            text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
            text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def counter_traffic(workload, kv="bf16"):
    """HBM bytes per launch of the attention kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE record, scaled by its copy calibration.
    None unless the record's source fingerprint matches the sources built now
    (the counters describe a kernel that no longer exists otherwise) and it
    was taken on this workload."""
    suffix = "" if kv == "bf16" else f"_{kv}"
    path = os.path.join(ROOT, "profiles", f"traffic_attn_bf16_{workload}_routed{suffix}.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
        if source_fingerprint(rec["sources"]) != rec["sources_fingerprint"]:
            return None
        return int(rec["traffic_bytes"])
    except (OSError, ValueError, KeyError, TypeError):
        return None


def cpu_baseline(wl, labels, seed, budget_s=20.0):
    """The oracle (fp64 numpy) on a bounded sample: every head, a seeded
    sample of query rows, timed on this host."""
    import numpy as np
    from head_routed_kv_amd import workloads as W
    from oracle import headcast_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = 1
    data = W.window(wl, seed=seed)
    fq, fk, fv = (W.as_float(data[n], wl) for n in ("q", "k", "v"))
    g = O.Geometry(wl.grid_h, wl.grid_w, wl.block_frames, wl.window_frames)
    rng = np.random.default_rng(seed)
    rows_per_head = 16
    done_rows, t0 = 0, time.perf_counter()
    while True:
        rows = np.sort(rng.choice(wl.Nq, rows_per_head, replace=False))
        O.routed_attention(fq, fk, fv, np.asarray(labels), g, rows=rows)
        done_rows += rows_per_head
        el = time.perf_counter() - t0
        if el > budget_s or done_rows >= 512:
            break
    qh = done_rows * wl.heads
    return {"value": qh / el, "unit": "query-heads/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{wl.name}: all {wl.heads} heads, {done_rows} seeded query rows per head "
                      f"({qh} query-heads) of the routed layer, fp64 numpy, {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--clock-warmup", type=float, default=0.3,
                    help="seconds of untimed steps before the warm-up steps, so the timed steps run at the "
                         "sustained shader clock")
    ap.add_argument("--workload", default="720p")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the 1080p and per-pathway figures")
    ap.add_argument("--theta", type=float, default=0.95, help="classifier cosine threshold (all three proxies)")
    ap.add_argument("--theta-sc", type=float, default=0.755, help="classifier Spatial score threshold")
    ap.add_argument("--gamma", type=float, default=5.0, help="classifier MSE weight")
    ap.add_argument("--percentile", type=float, default=5.0, help="classifier Spatial cosine percentile")
    ap.add_argument("--rule", type=int, default=0, choices=(0, 1), help="classifier rule")
    ap.add_argument("--radius", type=int, default=2, help="sliding-box proxy radius")
    ap.add_argument("--kv", default="bf16", choices=("bf16", "fp8"),
                    help="K/V cache format of the timed layer (fp8: OCP E4M3 codes, bf16 arithmetic)")
    ap.add_argument("--calibrate", action="store_true",
                    help="also run a plain 1 GiB device copy (known bytes) to scale HBM counters")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {a.gpus}). "
              "Heads shard across GPUs with no exchange in attention; run one process per GPU.", file=sys.stderr)
        sys.exit(2)

    import torch
    import head_routed_kv_amd as hk
    from head_routed_kv_amd import workloads as W

    dev = torch.device("cuda:0")
    if a.calibrate:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)     # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src, dst
    wl = W.WORKLOADS[a.workload]
    labels = W.make_labels(wl, a.seed)
    q, k, v = gen_inputs(wl, a.seed, dev)
    kvf = hk.HC_KV_FP8_E4M3 if a.kv == "fp8" else hk.HC_KV_SAME
    layer = Layer(wl, labels, q, k, v, kv_format=kvf)
    torch.cuda.synchronize()

    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < a.clock_warmup:
        for _ in range(10):
            layer.step()
        torch.cuda.synchronize()
    for _ in range(a.warmup):
        layer.step()
    torch.cuda.synchronize()
    # timed region: exactly K steps; HIP events on the same stream bracket each hc_attend
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(a.steps)]
    t0 = time.perf_counter()
    for i in range(a.steps):
        layer.append()
        evs[i][0].record()
        layer.attend()
        evs[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / a.steps
    attend_samples = [s.elapsed_time(e) for s, e in evs]
    attend_ms = statistics.fmean(attend_samples)

    work = algorithmic_work(wl, labels)
    flops = sum(f for f, _ in work.values())
    qo_bytes = 2 * 2 * wl.heads * wl.Nq * wl.head_dim
    alg_bytes = sum(b for _, b in work.values())
    if a.kv == "fp8":   # K/V read once at one byte per element
        alg_bytes = qo_bytes + (alg_bytes - qo_bytes) // 2
    value = wl.heads * wl.Nq / (ms_step / 1e3)
    achieved = flops / (attend_ms / 1e3) / 1e12

    flush = make_flush(dev)
    cold_samples = time_samples(layer.attend, 10, flush)
    cold_ms = statistics.fmean(cold_samples)
    # full-attention baseline on the same GPU: every head Global, same inputs
    full = Layer(wl, [3] * wl.heads, q, k, v, kv_format=kvf)
    for _ in range(3):
        full.attend()
    full_ms = time_events(full.attend, 10)
    full_cold_ms = time_events(full.attend, 5, flush)
    full_flops = wl.heads * 4 * wl.head_dim * wl.Nq * wl.Nk
    del full

    extra = {}
    if not a.no_extra:
        # each pathway group alone: a cache holding only that group's heads
        for lab, name in ((3, "global"), (0, "sink"), (1, "dummy"), (2, "spatial")):
            heads = [h for h in range(wl.heads) if int(labels[h]) == lab]
            if not heads:
                continue
            sub = W.small(wl, heads=len(heads))
            idx = torch.tensor(heads, device=dev)
            lay = Layer(sub, [lab] * len(heads), q[idx].contiguous(), k[idx].contiguous(), v[idx].contiguous())
            for _ in range(3):
                lay.attend()
            ms = time_events(lay.attend, 10, flush)
            f, by = work[lab]
            extra[name] = {"heads": len(heads), "ms_cold": round(ms, 4),
                           "tflops": round(f / (ms / 1e3) / 1e12, 1), "mfma_frac": round(f / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                           "hbm_gbs": round(by / (ms / 1e3) / 1e9, 1), "hbm_frac": round(by / (ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4)}
            del lay
        extra["rollout"] = rollout_costs(wl, labels, q, k, v, full_ms)
        # the same layer over an fp8 (E4M3) K/V cache: K/V bytes halve, the
        # attention arithmetic stays bf16
        l8 = Layer(wl, labels, q, k, v, kv_format=hk.HC_KV_FP8_E4M3)
        for _ in range(3):
            l8.step()
        ms8 = time_events(l8.attend, 20)
        ms8_cold = time_events(l8.attend, 10, flush)
        step8 = time_events(l8.step, 10)
        extra["fp8_kv"] = {"attend_ms": round(ms8, 4), "attend_cold_ms": round(ms8_cold, 4),
                           "ms_per_step": round(step8, 4),
                           "query_heads_per_s": round(wl.heads * wl.Nq / (step8 / 1e3)),
                           "tflops": round(flops / (ms8 / 1e3) / 1e12, 1),
                           "mfma_frac": round(flops / (ms8 / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                           "cache_bytes": l8.cache.nbytes, "cache_bytes_bf16": layer.cache.nbytes}
        del l8
        sp = [h for h in range(wl.heads) if int(labels[h]) == 2]
        if sp:
            idx = torch.tensor(sp, device=dev)
            sub = W.small(wl, heads=len(sp))
            ls8 = Layer(sub, [2] * len(sp), q[idx].contiguous(), k[idx].contiguous(), v[idx].contiguous(),
                        kv_format=hk.HC_KV_FP8_E4M3)
            for _ in range(3):
                ls8.attend()
            ms = time_events(ls8.attend, 10, flush)
            f, by = work[2]
            by8 = by - (by - 2 * 2 * sub.heads * sub.Nq * sub.head_dim) // 2   # K/V read once at 1 byte
            extra["fp8_kv"]["spatial"] = {"heads": len(sp), "ms_cold": round(ms, 4), "hbm_bytes": by8,
                                          "hbm_gbs": round(by8 / (ms / 1e3) / 1e9, 1),
                                          "hbm_frac": round(by8 / (ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4)}
            del ls8
        del layer, q, k, v
        torch.cuda.empty_cache()
        # 1080p layer
        wl2 = W.WORKLOADS["1080p"]
        lab2 = W.make_labels(wl2, a.seed)
        q2, k2, v2 = gen_inputs(wl2, a.seed + 1, dev)
        l2 = Layer(wl2, lab2, q2, k2, v2)
        for _ in range(2):
            l2.step()
        ms2 = time_events(l2.step, 5)
        at2 = time_events(l2.attend, 5)
        f2 = sum(f for f, _ in algorithmic_work(wl2, lab2).values())
        extra["1080p"] = {"ms_per_step": round(ms2, 3), "query_heads_per_s": round(wl2.heads * wl2.Nq / (ms2 / 1e3)),
                          "attend_ms": round(at2, 3), "tflops": round(f2 / (at2 / 1e3) / 1e12, 1),
                          "mfma_frac": round(f2 / (at2 / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del l2
        # each 1080p pathway group alone (10 Global, 8 Sink, 6 Dummy, 16 Spatial heads)
        work2 = algorithmic_work(wl2, lab2)
        alone = {}
        for lab, name in ((3, "global"), (0, "sink"), (1, "dummy"), (2, "spatial")):
            heads = [h for h in range(wl2.heads) if int(lab2[h]) == lab]
            if not heads:
                continue
            idx = torch.tensor(heads, device=dev)
            lay = Layer(W.small(wl2, heads=len(heads)), [lab] * len(heads), q2[idx].contiguous(),
                        k2[idx].contiguous(), v2[idx].contiguous())
            lay.attend()
            ms = time_events(lay.attend, 3, flush)
            f, by = work2[lab]
            alone[name] = {"heads": len(heads), "ms_cold": round(ms, 3),
                           "tflops": round(f / (ms / 1e3) / 1e12, 1),
                           "mfma_frac": round(f / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                           "hbm_gbs": round(by / (ms / 1e3) / 1e9, 1), "hbm_frac": round(by / (ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4)}
            del lay
            torch.cuda.empty_cache()
        extra["1080p"]["pathways"] = alone
        del q2, k2, v2
        torch.cuda.empty_cache()
        # one-shot classifier at the 720p shape, 40 heads (full + 3 proxy outputs, cosines, rule)
        wl3 = W.WORKLOADS["classifier720p"]
        q3, k3, v3 = gen_inputs(wl3, a.seed + 2, dev)
        cfg3 = hk.make_config(wl3.heads, wl3.head_dim, wl3.grid_h, wl3.grid_w, wl3.block_frames, wl3.window_frames)
        pg = hk.hc_default_classify_params()
        pg.theta_sink = pg.theta_dummy = pg.theta_spatial = a.theta
        pg.theta_score, pg.gamma, pg.percentile, pg.rule = a.theta_sc, a.gamma, a.percentile, a.rule
        ws = None
        for _ in range(2):
            _, _, ws = hk.classify(cfg3, q3, k3, v3, pg, workspace=ws)
        cls_ms = time_events(lambda: hk.classify(cfg3, q3, k3, v3, pg, workspace=ws), 3)
        # the Sink and Dummy proxies' keys are part of the full output's and are
        # attended once: the work is the full attention plus the Spatial proxy
        pairs = wl3.Nq * wl3.Nk + \
            wl3.block_frames * wl3.window_frames * sum(c * c for c in cell_sizes(wl3.grid_h, wl3.grid_w))
        f3 = wl3.heads * 4 * wl3.head_dim * pairs
        extra["classifier720p"] = {"heads": wl3.heads, "ms": round(cls_ms, 3), "tflops": round(f3 / (cls_ms / 1e3) / 1e12, 1),
                                   "mfma_frac": round(f3 / (cls_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        # the same with the pages' sliding 5x5 box as the Spatial proxy
        pb = hk.hc_default_classify_params()
        pb.theta_sink = pb.theta_dummy = pb.theta_spatial = a.theta
        pb.theta_score, pb.gamma, pb.percentile, pb.rule = a.theta_sc, a.gamma, a.percentile, a.rule
        pb.spatial_proxy, pb.radius = 1, a.radius
        for _ in range(2):
            hk.classify(cfg3, q3, k3, v3, pb, workspace=ws)
        box_ms = time_events(lambda: hk.classify(cfg3, q3, k3, v3, pb, workspace=ws), 3)
        pairs_b = wl3.Nq * wl3.Nk + \
            wl3.block_frames * wl3.window_frames * box_span(wl3.grid_h, a.radius) * box_span(wl3.grid_w, a.radius)
        fb = wl3.heads * 4 * wl3.head_dim * pairs_b
        extra["classifier720p_box"] = {"heads": wl3.heads, "ms": round(box_ms, 3),
                                       "tflops": round(fb / (box_ms / 1e3) / 1e12, 1),
                                       "mfma_frac": round(fb / (box_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del q3, k3, v3, ws
        torch.cuda.empty_cache()
        extra["ceilings"] = ceilings(dev)

    cpu = None
    if not a.no_cpu:
        cpu = cpu_baseline(wl, labels, a.seed)

    line = {
        "metric": "head-routed attention query-heads/sec per layer",
        "value": round(value, 1),
        "unit": "query-heads/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "clock_warmup_s": a.clock_warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic N(0,1) bf16 Q/K/V (seeded), labels by the 25/40/20/15% Global/Spatial/Sink/Dummy mix",
        "config": {"workload": f"{wl.name} routed layer", "heads": wl.heads, "head_dim": wl.head_dim,
                   "grid": [wl.grid_h, wl.grid_w], "block_frames": wl.block_frames,
                   "window_frames": wl.window_frames, "queries": wl.Nq, "keys": wl.Nk,
                   "labels": [int(x) for x in labels], "step": "append(REPLACE_NEWEST) + attend",
                   "kv_cache": "bf16" if a.kv == "bf16" else "fp8_e4m3"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": counter_traffic(a.workload, a.kv),
                     "kernel": "attn_bf16_kernel", "attend_ms": round(attend_ms, 4),
                     "traffic_unit": "bytes per launch (FETCH_SIZE x2.0 + WRITE_SIZE x1.0)",
                     "algorithmic_bytes": alg_bytes,
                     "algorithmic_flops": flops},
        "attend_cold_ms": round(cold_ms, 4),
        "attend_ms_stats": {"warm": summary(attend_samples), "cold": summary(cold_samples)},
        "device": device_info(0),
        "full_attention": {"ms": round(full_ms, 4), "ms_cold": round(full_cold_ms, 4),
                           "tflops": round(full_flops / (full_ms / 1e3) / 1e12, 1),
                           "speedup_vs_full": round(full_ms / attend_ms, 3)},
        "pathways": extra,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
