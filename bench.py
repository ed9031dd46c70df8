"""Benchmark: head-routed attention query-heads/s per layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 720p]

One step = one steady-state denoising step of one layer: the block being
denoised gets new keys/values (hc_cache_append with REPLACE_NEWEST) and every
head attends over its archetype's keys (hc_attend).  Inputs are synthetic
N(0,1) bf16 of the workload's shape, resident in HBM before timing starts;
the cache is restructured (W/B block appends) before timing.  The timed
region is exactly K steps, each preceded (untimed) by a 512 MiB write, so
that the layer's K/V come from HBM and not from the 256 MB Infinity Cache,
as in a model step where the other layers' work evicts them; HIP events on
the launch stream time each step and each hc_attend.  The same steps back to
back are reported as "warm".  The GPU's clocks settle to each pattern of
load over tens of milliseconds (ramping up at the start, and dipping for the
first ~20 steps when write-then-attend steps follow back-to-back ones), so
the untimed steps before each timed series run that series' own procedure:
--clock-warmup seconds of them, then the W warm-up steps.

Prints ONE JSON line with the metric, the roofline of the dominant kernel
(the attention kernel), the same GPU's full-attention time (every head
Global), the 480p and 1080p layers, per-pathway figures, the launch overhead
of a 30-layer step (eager against one HIP-graph replay), the classifier, the
same box's ceilings, and the CPU oracle timed on a bounded sample."""
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
    out = {"matmul_bf16_8192": {"ms": round(mm, 4), "tflops": round(2 * n ** 3 / (mm / 1e3) / 1e12, 1)},
           "copy_1gib": {"ms": round(cp, 4), "gbs": round(2 * (1 << 30) / (cp / 1e3) / 1e9, 1)}}
    out["sdpa_720p_full_attention"] = sdpa_ceiling(device)
    return out


def sdpa_ceiling(device):
    """torch's fused attention (bf16, d 128) at the 720p full-attention shape,
    12 heads x 10800 queries x 75600 keys, as a same-box dense-attention
    reference.  Only the fused backends are allowed: the unfused fallback
    would run batched bf16 products on transposed operands."""
    import torch
    try:
        from torch.nn.attention import SDPBackend, sdpa_kernel
        H, nq, nk, d = 12, 10800, 75600, 128
        q = torch.randn(1, H, nq, d, device=device, dtype=torch.float32).to(torch.bfloat16)
        k = torch.randn(1, H, nk, d, device=device, dtype=torch.float32).to(torch.bfloat16)
        v = torch.randn(1, H, nk, d, device=device, dtype=torch.float32).to(torch.bfloat16)
        res = {}
        for name, be in (("flash", SDPBackend.FLASH_ATTENTION), ("efficient", SDPBackend.EFFICIENT_ATTENTION)):
            try:
                with sdpa_kernel([be]):
                    fn = lambda: torch.nn.functional.scaled_dot_product_attention(q, k, v)
                    for _ in range(2):
                        fn()
                    ms = statistics.median(time_samples(fn, 5))
                res[name] = {"ms": round(ms, 4), "tflops": round(4 * d * H * nq * nk / (ms / 1e3) / 1e12, 1)}
            except Exception as e:   # backend not built for this GPU
                res[name] = {"error": str(e).splitlines()[0][:160]}
        del q, k, v
        torch.cuda.empty_cache()
        return res
    except Exception as e:
        return {"error": str(e).splitlines()[0][:160]}


def make_flush(device):
    import torch
    buf = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device=device)

    def flush():   # write 512 MiB so the 256 MB Infinity Cache holds none of the layer's K/V
        buf.fill_(1.0)
    return flush


def settle(fn, flush=None, seconds=0.1):
    """Untimed calls of fn (each preceded by flush(), if given) for `seconds`:
    the procedure about to be timed, so the clocks have settled to it."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(5):
            if flush is not None:
                flush()
            fn()
        torch.cuda.synchronize()


def layer_timing(layer, steps, flush, modes=("cold", "warm"), settle_s=0.1):
    """HIP-event times of `steps` steady-state steps (append, then attend) of
    one layer: cold (each step preceded, untimed, by the 512 MiB write) and
    warm (back to back), each series after settle_s seconds of its own
    untimed steps.  Returns per-step and per-attend samples in ms."""
    import torch
    res = {}
    for mode in modes:
        evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(steps)]
        settle(layer.step, flush if mode == "cold" else None, settle_s)
        for i in range(steps):
            if mode == "cold":
                flush()
            evs[i][0].record()
            layer.append()
            evs[i][1].record()
            layer.attend()
            evs[i][2].record()
        torch.cuda.synchronize()
        res[mode] = {"step": [a.elapsed_time(c) for a, _, c in evs], "attend": [b.elapsed_time(c) for _, b, c in evs]}
    return res


def pathway_alone(wl, labels, work, q, k, v, flush, dev, iters):
    """Each pathway group alone (a cache holding only that group's heads),
    timed cold: % of MFMA and HBM peak per group."""
    import torch
    from head_routed_kv_amd import workloads as W
    out = {}
    for lab, name in ((3, "global"), (0, "sink"), (1, "dummy"), (2, "spatial")):
        heads = [h for h in range(wl.heads) if int(labels[h]) == lab]
        if not heads:
            continue
        idx = torch.tensor(heads, device=dev)
        lay = Layer(W.small(wl, heads=len(heads)), [lab] * len(heads), q[idx].contiguous(), k[idx].contiguous(),
                    v[idx].contiguous())
        settle(lay.attend, flush, 0.05)
        ms = time_events(lay.attend, iters, flush)
        f, by = work[lab]
        out[name] = {"heads": len(heads), "ms_cold": round(ms, 4),
                     "tflops": round(f / (ms / 1e3) / 1e12, 1), "mfma_frac": round(f / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "hbm_gbs": round(by / (ms / 1e3) / 1e9, 1), "hbm_frac": round(by / (ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4)}
        del lay, idx
    torch.cuda.empty_cache()
    return out


def layer_line(wl, labels, seed, dev, flush, steps=10, alone=True):
    """Cold and warm timing of one routed layer of workload wl, its full
    attention baseline (every head Global) and, optionally, each pathway
    group alone."""
    import torch
    q, k, v = gen_inputs(wl, seed, dev)
    work = algorithmic_work(wl, labels)
    flops = sum(f for f, _ in work.values())
    lay = Layer(wl, labels, q, k, v)
    t = layer_timing(lay, steps, flush)
    del lay
    full = Layer(wl, [3] * wl.heads, q, k, v)
    settle(full.attend, flush)
    full_cold = time_events(full.attend, 5, flush)
    settle(full.attend)
    full_warm = time_events(full.attend, 5)
    del full
    torch.cuda.empty_cache()
    cold_step, cold_att = statistics.fmean(t["cold"]["step"]), statistics.fmean(t["cold"]["attend"])
    warm_step, warm_att = statistics.fmean(t["warm"]["step"]), statistics.fmean(t["warm"]["attend"])
    full_flops = wl.heads * 4 * wl.head_dim * wl.Nq * wl.Nk
    res = {"labels": [int(x) for x in labels],
           "ms_per_step": round(cold_step, 4), "query_heads_per_s": round(wl.heads * wl.Nq / (cold_step / 1e3)),
           "attend_ms": round(cold_att, 4), "tflops": round(flops / (cold_att / 1e3) / 1e12, 1),
           "mfma_frac": round(flops / (cold_att / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "warm": {"ms_per_step": round(warm_step, 4), "attend_ms": round(warm_att, 4),
                    "mfma_frac": round(flops / (warm_att / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
           "full_attention": {"ms_cold": round(full_cold, 4), "ms_warm": round(full_warm, 4),
                              "tflops": round(full_flops / (full_cold / 1e3) / 1e12, 1),
                              "speedup_vs_full": round(full_cold / cold_att, 3),
                              "flop_ratio": round(full_flops / flops, 3)}}
    if alone:
        res["pathways"] = pathway_alone(wl, labels, work, q, k, v, flush, dev, 5)
    del q, k, v
    torch.cuda.empty_cache()
    return res


def head_costs(wl):
    """Planned cost of one head per pathway label: its algorithmic flops at
    the matrix peak or its algorithmic bytes at the HBM peak, whichever takes
    longer (seconds)."""
    out = {}
    for lab in range(4):
        f, by = algorithmic_work(wl, [lab])[lab]
        out[lab] = max(f / (PEAK_BF16_TFLOPS * 1e12), by / (PEAK_HBM_GBS * 1e9))
    return out


def shard_heads(labels, cost, n_gpus):
    """Heads onto n_gpus by longest-processing-time packing: heads by
    decreasing cost (ties: lower head first), each onto the GPU with the
    least planned cost so far (ties: lower GPU first).  Returns the sorted
    head list of each GPU."""
    order = sorted(range(len(labels)), key=lambda h: (-cost[int(labels[h])], h))
    load = [0.0] * n_gpus
    shards = [[] for _ in range(n_gpus)]
    for h in order:
        g = min(range(n_gpus), key=lambda i: (load[i], i))
        shards[g].append(h)
        load[g] += cost[int(labels[h])]
    return [sorted(s) for s in shards]


def gpu_shares(wl, labels, seed, dev, flush, n_gpus=8, iters=5):
    """One GPU's share of the layer when its heads are sharded over n_gpus
    GPUs (attention needs no exchange between them): each share's heads as
    a cache of their own, timed cold on this GPU.  The layer's time on
    n_gpus GPUs is the slowest share's."""
    import torch
    from head_routed_kv_amd import workloads as W
    q, k, v = gen_inputs(wl, seed, dev)
    shares = []
    for heads in shard_heads(labels, head_costs(wl), n_gpus):
        if not heads:
            shares.append({"heads": [], "labels": [], "ms_cold": 0.0})
            continue
        idx = torch.tensor(heads, device=dev)
        labs = [int(labels[h]) for h in heads]
        lay = Layer(W.small(wl, heads=len(heads)), labs, q[idx].contiguous(), k[idx].contiguous(),
                    v[idx].contiguous())
        settle(lay.attend, flush, 0.05)
        shares.append({"heads": heads, "labels": labs, "ms_cold": round(time_events(lay.attend, iters, flush), 4)})
        del lay, idx
    del q, k, v
    torch.cuda.empty_cache()
    slowest = max(s["ms_cold"] for s in shares)
    return {"n_gpus": n_gpus, "shares": shares, "layer_ms": slowest,
            "query_heads_per_s": round(wl.heads * wl.Nq / (slowest / 1e3)),
            "balance": round(sum(s["ms_cold"] for s in shares) / n_gpus / slowest, 4)}


def launch_overhead(wl, labels, seed, dev, n_layers=30, reps=5):
    """A denoising step of an n_layers-deep model as far as this layer type
    goes: for each layer, append (REPLACE_NEWEST) then attend, each layer
    with its own cache (inputs shared).  Timed eagerly (one library call per
    kernel, from Python) and as one HIP-graph replay of the same sequence;
    the difference per layer is the launch overhead.  Routed and all-Global
    (full attention) alike."""
    import torch
    q, k, v = gen_inputs(wl, seed, dev)
    res = {"layers": n_layers}
    for name, labs in (("routed", labels), ("full", [3] * wl.heads)):
        layers = [Layer(wl, labs, q, k, v) for _ in range(n_layers)]

        def seq():
            for lay in layers:
                lay.step()
        for _ in range(2):
            seq()
        eager = statistics.median(time_samples(seq, reps))
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            seq()
        torch.cuda.synchronize()
        for _ in range(2):
            g.replay()
        graph = statistics.median(time_samples(g.replay, reps))
        res[name] = {"eager_ms": round(eager, 3), "graph_ms": round(graph, 3),
                     "eager_ms_per_layer": round(eager / n_layers, 4), "graph_ms_per_layer": round(graph / n_layers, 4),
                     "overhead_us_per_layer": round((eager - graph) / n_layers * 1e3, 2)}
        del g, layers
        torch.cuda.empty_cache()
    res["speedup_vs_full_eager"] = round(res["full"]["eager_ms"] / res["routed"]["eager_ms"], 3)
    res["speedup_vs_full_graph"] = round(res["full"]["graph_ms"] / res["routed"]["graph_ms"], 3)
    del q, k, v
    torch.cuda.empty_cache()
    return res


def rollout_costs(wl, labels, q, k, v, full_ms, steps_per_block=4, lengths=(14, 40)):
    """Attention cost of one layer over a video rollout, phase by phase.

    Warm-up: while the first window fills, every head attends over the growing
    window (each block: one push and steps_per_block - 1 replacements, an
    attend after each).  At first fill: hc_classify on the window, then the
    window's blocks are replayed into the routed cache, whose memory is
    allocated beforehand.  Afterwards each block's
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
    # the routed cache's memory is allocated before the timed region, like the
    # classifier workspace: restructuring is the window's block appends
    routed = hk.RoutedCache(cfg, [int(x) for x in labels])
    torch.cuda.synchronize()

    def restructure():
        for b in range(nb):
            routed.append(*blk(kw, vw, b))
    rest_ms = timed(restructure)
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


def cpu_baseline(wl, labels, seed, rows_per_head=2048, procs=None):
    """The oracle (fp64 numpy) on a bounded sample of the routed layer: every
    head, a seeded contiguous run of query rows, run process-parallel over
    (head, 512-row chunk) pieces with one BLAS thread per process.  Timed
    on this host's cores by wall clock, including each worker's regeneration
    of its head's seeded inputs; value = query-heads of the sample / seconds."""
    import numpy as np
    from oracle import pool
    procs = procs or pool.default_procs()
    rng = np.random.default_rng(seed)
    chunk = 512
    tasks = []
    for h in range(wl.heads):
        r0 = int(rng.integers(0, max(1, wl.Nq - rows_per_head)))
        for c in range(0, rows_per_head, chunk):
            tasks.append((h, int(labels[h]), r0 + c, min(chunk, rows_per_head - c)))
    from concurrent.futures import ProcessPoolExecutor
    import multiprocessing as mp
    t0 = time.perf_counter()
    with ProcessPoolExecutor(min(procs, len(tasks)), mp_context=mp.get_context("spawn"),
                             initializer=pool._init_worker) as ex:
        cpu_s = sum(sec for _, _, sec in ex.map(pool._run_task, [(wl, seed, h, lab, r0, n, 2, None)
                                                                  for h, lab, r0, n in tasks], chunksize=2))
    el = time.perf_counter() - t0
    qh = rows_per_head * wl.heads
    return {"value": qh / el, "unit": "query-heads/s", "cores": int(min(procs, len(tasks))), "kind": "oracle",
            "sample": f"{wl.name} routed layer: all {wl.heads} heads x {rows_per_head} contiguous seeded query "
                      f"rows ({qh} query-heads), fp64 numpy oracle in {min(procs, len(tasks))} processes of one "
                      f"thread each; {el:.1f} s wall ({cpu_s:.1f} s of oracle compute), the rate extrapolated "
                      f"to the layer from this sample"}


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
    ap.add_argument("--no-extra", action="store_true", help="skip every figure beyond the headline layer")
    ap.add_argument("--theta", type=float, default=0.95, help="classifier cosine threshold (all three proxies)")
    ap.add_argument("--theta-sc", type=float, default=0.755, help="classifier Spatial score threshold")
    ap.add_argument("--gamma", type=float, default=5.0, help="classifier MSE weight")
    ap.add_argument("--percentile", type=float, default=5.0, help="classifier Spatial cosine percentile")
    ap.add_argument("--rule", type=int, default=0, choices=(0, 1), help="classifier rule")
    ap.add_argument("--radius", type=int, default=2, help="sliding-box proxy radius")
    ap.add_argument("--kv", default="bf16", choices=("bf16", "fp8"),
                    help="K/V cache format of the timed layer (fp8: OCP E4M3 codes, bf16 arithmetic)")
    ap.add_argument("--pathway", choices=("global", "sink", "dummy", "spatial"),
                    help="profiling aid: time only this pathway's heads of the layer (no extras, no CPU leg); "
                         "the line's roofline is then that pathway's (HBM for Spatial)")
    ap.add_argument("--calibrate", action="store_true",
                    help="also run a plain 1 GiB device copy (known bytes) to scale HBM counters")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {a.gpus}). "
              "Heads shard across GPUs with no exchange in attention; run one process per GPU.", file=sys.stderr)
        sys.exit(2)

    from head_routed_kv_amd import workloads as W
    wl = W.WORKLOADS[a.workload]
    labels = W.make_labels(wl, a.seed)
    if a.pathway:
        a.no_cpu = a.no_extra = True
    # the CPU leg first, before this process touches the GPU
    cpu = None if a.no_cpu else cpu_baseline(wl, labels, a.seed)

    import torch
    import head_routed_kv_amd as hk

    dev = torch.device("cuda:0")
    if a.calibrate:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)     # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src, dst
    q, k, v = gen_inputs(wl, a.seed, dev)
    layer_name = f"{wl.name} routed layer"
    if a.pathway:
        lab = {"sink": 0, "dummy": 1, "spatial": 2, "global": 3}[a.pathway]
        heads = [h for h in range(wl.heads) if int(labels[h]) == lab]
        if not heads:
            sys.exit(f"the {wl.name} layer has no {a.pathway} heads")
        idx = torch.tensor(heads, device=dev)
        q, k, v = q[idx].contiguous(), k[idx].contiguous(), v[idx].contiguous()
        layer_name = f"{wl.name} {a.pathway} heads alone"
        wl, labels = W.small(wl, heads=len(heads), name=wl.name), [lab] * len(heads)
    kvf = hk.HC_KV_FP8_E4M3 if a.kv == "fp8" else hk.HC_KV_SAME
    layer = Layer(wl, labels, q, k, v, kv_format=kvf)
    flush = make_flush(dev)
    torch.cuda.synchronize()

    # untimed: the timed procedure itself (write, append, attend) for
    # --clock-warmup seconds, then the W warm-up steps
    settle(layer.step, flush, a.clock_warmup)
    for _ in range(a.warmup):
        flush()
        layer.step()
    torch.cuda.synchronize()
    # Timed region: exactly K steps, each preceded (untimed) by a 512 MiB write,
    # so that the 256 MB Infinity Cache holds none of the layer's K/V, as in a
    # model step, where the other layers' work evicts it between two calls of
    # one layer.  HIP events on the launch stream bracket each step and each
    # hc_attend.
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(a.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        flush()
        evs[i][0].record()
        layer.append()
        evs[i][1].record()
        layer.attend()
        evs[i][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_samples = [x.elapsed_time(z) for x, _, z in evs]
    attend_samples = [y.elapsed_time(z) for _, y, z in evs]
    ms_step = statistics.fmean(step_samples)
    attend_ms = statistics.fmean(attend_samples)
    # the same steps back to back (K/V partly served by the Infinity Cache)
    warm = layer_timing(layer, a.steps, flush, modes=("warm",))["warm"]
    warm_step, warm_attend = statistics.fmean(warm["step"]), statistics.fmean(warm["attend"])

    work = algorithmic_work(wl, labels)
    flops = sum(f for f, _ in work.values())
    qo_bytes = 2 * 2 * wl.heads * wl.Nq * wl.head_dim
    alg_bytes = sum(b for _, b in work.values())
    if a.kv == "fp8":   # K/V read once at one byte per element
        alg_bytes = qo_bytes + (alg_bytes - qo_bytes) // 2
    value = wl.heads * wl.Nq / (ms_step / 1e3)
    achieved = flops / (attend_ms / 1e3) / 1e12

    # full-attention baseline on the same GPU: every head Global, same inputs
    full = Layer(wl, [3] * wl.heads, q, k, v, kv_format=kvf)
    settle(full.attend, flush)
    full_cold_ms = time_events(full.attend, 10, flush)
    settle(full.attend)
    full_ms = time_events(full.attend, 10)
    full_flops = wl.heads * 4 * wl.head_dim * wl.Nq * wl.Nk
    full_splits = full.cache.layout().global_splits
    del full

    extra = {}
    if not a.no_extra:
        extra.update(pathway_alone(wl, labels, work, q, k, v, flush, dev, 10))
        extra["rollout"] = rollout_costs(wl, labels, q, k, v, full_ms)
        # the same layer over an fp8 (E4M3) K/V cache: K/V bytes halve, the
        # attention arithmetic stays bf16
        l8 = Layer(wl, labels, q, k, v, kv_format=hk.HC_KV_FP8_E4M3)
        t8 = layer_timing(l8, 10, flush)
        ms8, ms8_cold = statistics.fmean(t8["warm"]["attend"]), statistics.fmean(t8["cold"]["attend"])
        step8 = statistics.fmean(t8["cold"]["step"])
        extra["fp8_kv"] = {"attend_ms": round(ms8, 4), "attend_cold_ms": round(ms8_cold, 4),
                           "ms_per_step_cold": round(step8, 4),
                           "query_heads_per_s": round(wl.heads * wl.Nq / (step8 / 1e3)),
                           "tflops": round(flops / (ms8_cold / 1e3) / 1e12, 1),
                           "mfma_frac": round(flops / (ms8_cold / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                           "cache_bytes": l8.cache.nbytes, "cache_bytes_bf16": layer.cache.nbytes}
        del l8
        sp = [h for h in range(wl.heads) if int(labels[h]) == 2]
        if sp:
            idx = torch.tensor(sp, device=dev)
            sub = W.small(wl, heads=len(sp))
            ls8 = Layer(sub, [2] * len(sp), q[idx].contiguous(), k[idx].contiguous(), v[idx].contiguous(),
                        kv_format=hk.HC_KV_FP8_E4M3)
            settle(ls8.attend, flush, 0.05)
            ms = time_events(ls8.attend, 10, flush)
            f, by = work[2]
            by8 = by - (by - 2 * 2 * sub.heads * sub.Nq * sub.head_dim) // 2   # K/V read once at 1 byte
            extra["fp8_kv"]["spatial"] = {"heads": len(sp), "ms_cold": round(ms, 4), "hbm_bytes": by8,
                                          "hbm_gbs": round(by8 / (ms / 1e3) / 1e9, 1),
                                          "hbm_frac": round(by8 / (ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4)}
            del ls8
        del layer, q, k, v
        torch.cuda.empty_cache()
        # the 480p and 1080p layers, cold, each pathway group alone too
        for name, seed_off in (("480p", 3), ("1080p", 1)):
            wx = W.WORKLOADS[name]
            extra[name] = layer_line(wx, W.make_labels(wx, a.seed), a.seed + seed_off, dev, flush)
        # one GPU's share of the 1080p layer with its 40 heads sharded over 8 GPUs
        w10 = W.WORKLOADS["1080p"]
        extra["1080p"]["sharded"] = gpu_shares(w10, W.make_labels(w10, a.seed), a.seed + 1, dev, flush)
        # launch overhead of a 30-layer step, eager against one HIP-graph replay
        extra["launch_overhead"] = {name: launch_overhead(W.WORKLOADS[name], W.make_labels(W.WORKLOADS[name], a.seed),
                                                          a.seed, dev)
                                    for name in ("480p", "720p")}
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
        "config": {"workload": layer_name, "heads": wl.heads, "head_dim": wl.head_dim,
                   "grid": [wl.grid_h, wl.grid_w], "block_frames": wl.block_frames,
                   "window_frames": wl.window_frames, "queries": wl.Nq, "keys": wl.Nk,
                   "labels": [int(x) for x in labels], "step": "append(REPLACE_NEWEST) + attend",
                   "timing": "each step preceded (untimed) by a 512 MiB write: K/V come from HBM, not the "
                             "Infinity Cache; ms_per_step and attend_ms are HIP-event means over the K steps",
                   "kv_cache": "bf16" if a.kv == "bf16" else "fp8_e4m3"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": counter_traffic(a.workload, a.kv),
                     "kernel": "attn_bf16_kernel", "attend_ms": round(attend_ms, 4),
                     "traffic_unit": "bytes per launch (FETCH_SIZE x2.0 + WRITE_SIZE x1.0)",
                     "algorithmic_bytes": alg_bytes,
                     "algorithmic_flops": flops},
        "wall_ms_per_iteration": round(wall * 1e3 / a.steps, 4),
        "attend_ms_stats": {"cold": summary(attend_samples), "warm": summary(warm["attend"])},
        "warm": {"ms_per_step": round(warm_step, 4), "value": round(wl.heads * wl.Nq / (warm_step / 1e3), 1),
                 "attend_ms": round(warm_attend, 4),
                 "frac": round(flops / (warm_attend / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
        "device": device_info(0),
        "full_attention": {"ms_cold": round(full_cold_ms, 4), "ms_warm": round(full_ms, 4),
                           "global_splits": full_splits,
                           "tflops": round(full_flops / (full_cold_ms / 1e3) / 1e12, 1),
                           "speedup_vs_full": round(full_cold_ms / attend_ms, 3),
                           "speedup_vs_full_warm": round(full_ms / warm_attend, 3),
                           "flop_ratio": round(full_flops / flops, 3)},
        "pathways": extra,
        "cpu_baseline": cpu,
    }
    if a.pathway:
        line["roofline"]["traffic"] = None   # the stored counter record is the routed layer's
        if a.pathway == "spatial":           # an HBM-bound pathway: bytes against the HBM peak
            gbs = alg_bytes / (attend_ms / 1e3) / 1e9
            line["roofline"].update({"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)})
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
