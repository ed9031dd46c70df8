"""GPU parity of the restructured cache and routed attention (hc_cache_append,
hc_attend) against the CPU oracle."""
import numpy as np
import pytest

import head_routed_kv_amd as hk
from head_routed_kv_amd import workloads as W
from oracle import headcast_oracle as O
from oracle import pool
from tests.gpu_util import (BF16_TOL, FP32_TOL, check_close, config_of, download_bits, fill_cache, geometry_of,
                            sample_rows, say, to_float, torch, upload)

pytestmark = pytest.mark.gpu


def run_window(wl, labels, seed=0):
    data = W.window(wl, seed=seed)
    q, k, v = (upload(data[n], wl) for n in ("q", "k", "v"))
    cache = fill_cache(wl, labels, k, v)
    out = cache.attend(q)
    torch().cuda.synchronize()
    return data, cache, out


def oracle_routed(wl, data, labels, rows=None):
    fq, fk, fv = (W.as_float(data[n], wl) for n in ("q", "k", "v"))
    return O.routed_attention(fq, fk, fv, np.asarray(labels), geometry_of(wl), rows=rows)


def test_tiny_fp32_routed():
    wl = W.WORKLOADS["tiny"]
    labels = W.make_labels(wl)
    say("case tiny fp32", labels)
    data, cache, out = run_window(wl, labels)
    check_close(to_float(out), oracle_routed(wl, data, labels), FP32_TOL, "tiny")


@pytest.mark.parametrize("d", [128, 64])
def test_small_bf16_every_pathway(d):
    """Several q tiles and key tiles with ragged tails, uneven border cells."""
    wl = W.Workload("small", 9, 8, d, 23, 37, 2, 6, "bf16", "uniform")
    labels = [0, 1, 2, 3, 3, 2, 1, 0]
    say("case small bf16 d", d)
    data, cache, out = run_window(wl, labels, seed=5)
    assert cache.layout().global_splits >= 1
    check_close(to_float(out), oracle_routed(wl, data, labels), BF16_TOL, f"small d{d}")


def test_large_logits_and_late_max_jump():
    """Q and K scaled by 4 and the window's last frame of K by 16 more (powers
    of two: exact in bf16): scores reach a few hundred, the softmax is nearly
    one-hot, and the running max jumps by hundreds in the last key tiles, so
    the lazily rescaled accumulators are multiplied by exp2 of large negative
    numbers.  Every pathway, against the oracle."""
    wl = W.Workload("biglogit", 32, 4, 128, 23, 37, 2, 6, "bf16", "uniform")
    labels = [3, 0, 1, 2]
    say("case large logits")
    data = W.window(wl, seed=13)
    fq = W.as_float(data["q"], wl) * 4
    fk = W.as_float(data["k"], wl) * 4
    fk[:, -wl.T:] *= 4
    data = dict(data, q=W.f32_to_bf16_bits(fq), k=W.f32_to_bf16_bits(fk))
    q, k, v = (upload(data[n], wl) for n in ("q", "k", "v"))
    cache = fill_cache(wl, labels, k, v)
    out = cache.attend(q)
    torch().cuda.synchronize()
    check_close(to_float(out), oracle_routed(wl, data, labels), BF16_TOL, "large logits")


@pytest.mark.parametrize("d", [128, 64])
def test_fp32_long_key_sets(d):
    """fp32 layers with 8000-key Global sets and 1600-key Sink sets hold the
    1e-5 bound: the fp32 kernel sums each key tile before merging it into the
    running state, so rounding does not grow with one term per key."""
    wl = W.Workload("f32long", 33, 3, d, 20, 40, 2, 10, "fp32", "uniform")
    labels = [3, 0, 2]
    say("case fp32 long key sets d", d)
    data, cache, out = run_window(wl, labels, seed=21)
    check_close(to_float(out), oracle_routed(wl, data, labels), FP32_TOL, f"fp32 long d{d}")


def test_global_key_splits_merge():
    """Few queries over a long window: the cache plans several key-range
    splits for the Global head and merges them in the kernel."""
    wl = W.Workload("longwin", 10, 3, 128, 16, 16, 1, 64, "bf16", "uniform")
    labels = [3, 0, 3]
    say("case long window split merge")
    data, cache, out = run_window(wl, labels, seed=6)
    assert cache.layout().global_splits > 1
    check_close(to_float(out), oracle_routed(wl, data, labels), BF16_TOL, "split")
    # a second call reuses the self-resetting counters
    out2 = cache.attend(upload(data["q"], wl))
    torch().cuda.synchronize()
    assert torch().equal(out, out2)


def test_sink_dummy_key_splits_merge():
    """Sink and Dummy heads alone cannot fill the GPU: the cache splits their
    key sets too and the kernel merges the partials per category."""
    wl = W.Workload("sdsplit", 17, 4, 128, 16, 16, 4, 8, "bf16", "uniform")
    labels = [0, 1, 1, 0]
    say("case sink/dummy split merge")
    data, cache, out = run_window(wl, labels, seed=8)
    lay = cache.layout()
    assert lay.sink_splits > 1 and lay.dummy_splits > 1 and lay.global_splits == 1
    check_close(to_float(out), oracle_routed(wl, data, labels), BF16_TOL, "sink/dummy split")
    out2 = cache.attend(upload(data["q"], wl))
    torch().cuda.synchronize()
    assert torch().equal(out, out2)


def test_fp32_spatial_and_global_small():
    wl = W.Workload("small32", 11, 4, 128, 13, 21, 2, 6, "fp32", "uniform")
    labels = [2, 3, 1, 0]
    say("case small fp32 d128")
    data, cache, out = run_window(wl, labels, seed=7)
    check_close(to_float(out), oracle_routed(wl, data, labels), FP32_TOL, "small fp32")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_streaming_wrap_replace(dtype):
    """Push past the window (ring wrap), replace the newest block, attend after
    each step; the sink block stays the video's first block."""
    wl = W.Workload("stream", 12, 4, 64, 12, 17, 1, 3, dtype, "uniform")
    labels = [0, 1, 2, 3]
    g = geometry_of(wl)
    cache = hk.RoutedCache(config_of(wl), labels)
    model = O.CacheModel(g, labels)
    ks, vs = W.stream_blocks(wl, 8, 9)
    ks2, vs2 = W.stream_blocks(wl, 9, 9)
    q = W.queries(wl, 8)
    qd = upload(q, wl)
    for step in range(9):
        mode = hk.HC_REPLACE_NEWEST if step in (2, 6) else hk.HC_PUSH_BLOCK
        kb, vb = (ks2[step], vs2[step]) if mode == hk.HC_REPLACE_NEWEST else (ks[step], vs[step])
        cache.append(upload(kb, wl), upload(vb, wl), mode)
        model.append(kb, vb, mode)
        out = cache.attend(qd)
        torch().cuda.synchronize()
        wk, wv = model.window()
        nf = wk.shape[1] // g.T
        gq = O.Geometry(g.grid_h, g.grid_w, g.block_frames, nf, g.cell_h, g.cell_w)
        ref = O.routed_attention(W.as_float(q, wl), W.as_float(wk, wl), W.as_float(wv, wl), np.array(labels), gq,
                                 k_sink=W.as_float(model.sink_k, wl), v_sink=W.as_float(model.sink_v, wl))
        check_close(to_float(out), ref, BF16_TOL if dtype == "bf16" else FP32_TOL, f"step {step}")


def test_cache_buffers_bit_exact():
    """Every archetype buffer equals the oracle's index model byte for byte."""
    wl = W.Workload("bits", 13, 6, 64, 13, 23, 2, 6, "bf16", "uniform")
    labels = [2, 3, 0, 1, 3, 2]
    g = geometry_of(wl)
    cache = hk.RoutedCache(config_of(wl), labels)
    model = O.CacheModel(g, labels)
    ks, vs = W.stream_blocks(wl, 4, 6)
    ks2, vs2 = W.stream_blocks(wl, 5, 6)
    mem = cache.mem
    for step in range(6):
        mode = hk.HC_REPLACE_NEWEST if step == 4 else hk.HC_PUSH_BLOCK
        kb, vb = (ks2[step], vs2[step]) if mode else (ks[step], vs[step])
        cache.append(upload(kb, wl), upload(vb, wl), mode)
        model.append(kb, vb, mode)
        torch().cuda.synchronize()
        lay = cache.layout()
        raw = mem.cpu().numpy()
        for lab, (ok, ov) in {O.GLOBAL: (lay.off_global_k, lay.off_global_v),
                              O.SINK: (lay.off_sink_k, lay.off_sink_v),
                              O.DUMMY: (lay.off_dummy_k, lay.off_dummy_v),
                              O.SPATIAL: (lay.off_spatial_k, lay.off_spatial_v)}.items():
            for which, off in (("k", ok), ("v", ov)):
                exp, valid = model.expected_buffer(lab, which)
                n = exp.size * 2
                got = raw[off:off + n].view(np.uint16).reshape(exp.shape)
                assert np.array_equal(got[:, valid], exp[:, valid]), (step, lab, which)
        for h, lab in enumerate(labels):
            assert lay.head_slot[h] == sum(1 for x in labels[:h] if x == lab)


def test_strided_token_major_inputs():
    """[tokens][heads][d] views give bit-identical results to [heads][tokens][d]."""
    wl = W.Workload("strided", 14, 4, 128, 11, 19, 2, 4, "bf16", "uniform")
    labels = [3, 2, 1, 0]
    data = W.window(wl, seed=9)
    q, k, v = (upload(data[n], wl) for n in ("q", "k", "v"))
    ref_cache = fill_cache(wl, labels, k, v)
    ref = ref_cache.attend(q)
    tq, tk, tv = (x.transpose(0, 1).contiguous().transpose(0, 1) for x in (q, k, v))
    assert tq.stride(1) == wl.heads * wl.head_dim
    cache = fill_cache(wl, labels, tk, tv)
    out = torch().empty(wl.Nq, wl.heads, wl.head_dim, dtype=q.dtype, device=q.device).transpose(0, 1)
    cache.attend(tq, out)
    torch().cuda.synchronize()
    assert torch().equal(out, ref)


@pytest.mark.parametrize("name", ["480p", "720p"])
@pytest.mark.timeout(900)   # the oracle side runs every row, process-parallel
def test_full_size_every_row(name):
    """The full-size layer in the launch configuration the benchmark times:
    every query row of every head against the oracle (run process-parallel
    over heads and row chunks)."""
    wl = W.WORKLOADS[name]
    labels = W.make_labels(wl)
    say("case", name, "every row, labels", labels.tolist())
    data, cache, out = run_window(wl, labels)
    got = to_float(out)
    lay = cache.layout()
    say(name, "splits", lay.global_splits, lay.sink_splits, lay.dummy_splits)
    del data, cache, out
    res, cpu_s, wall = pool.run(wl, 0, [(h, int(labels[h])) for h in range(wl.heads)], rows_per_task=1350)
    say(name, f"oracle: {cpu_s:.0f} s of CPU in {wall:.0f} s")
    ref = np.stack([res[(h, int(labels[h]))] for h in range(wl.heads)])
    check_close(got, ref, BF16_TOL, f"{name} every row")


@pytest.mark.timeout(900)   # the oracle side runs every row, process-parallel
def test_1080p_every_head_sampled_rows():
    """The 1080p layer (40 heads): every head on sampled query rows, which
    include both ends, the frame seams and the rows of border cells."""
    wl = W.WORKLOADS["1080p"]
    labels = W.make_labels(wl)
    say("case 1080p, labels", labels.tolist())
    data, cache, out = run_window(wl, labels)
    rows = sample_rows(wl, 40)
    got = to_float(out)[:, rows]
    del data, cache, out
    res, cpu_s, wall = pool.run(wl, 0, [(h, int(labels[h])) for h in range(wl.heads)], rows=rows)
    say(f"1080p oracle: {cpu_s:.0f} s of CPU in {wall:.0f} s")
    ref = np.stack([res[(h, int(labels[h]))] for h in range(wl.heads)])
    check_close(got, ref, BF16_TOL, "1080p sampled rows, all heads")


@pytest.mark.timeout(900)   # the oracle side runs every row of four heads, process-parallel
def test_1080p_every_row_one_head_per_pathway():
    """The 1080p layer (40 heads) in its benchmark launch: every query row of
    the first head of each pathway (171,360 keys per Global query, the
    8-row border cells for Spatial) against the oracle."""
    wl = W.WORKLOADS["1080p"]
    labels = W.make_labels(wl)
    heads = [next(h for h in range(wl.heads) if int(labels[h]) == lab)
             for lab in (O.GLOBAL, O.SINK, O.DUMMY, O.SPATIAL)]
    say("case 1080p every row, heads", heads)
    data, cache, out = run_window(wl, labels)
    got = to_float(out[heads])
    del data, cache, out
    res, cpu_s, wall = pool.run(wl, 0, [(h, int(labels[h])) for h in heads], rows_per_task=1224)
    say(f"1080p oracle: {cpu_s:.0f} s of CPU in {wall:.0f} s")
    ref = np.stack([res[(h, int(labels[h]))] for h in heads])
    check_close(got, ref, BF16_TOL, "1080p every row, one head per pathway")


@pytest.mark.parametrize("lab", [O.GLOBAL, O.SINK, O.DUMMY, O.SPATIAL])
def test_720p_pathway_alone_sampled(lab):
    """Each pathway's heads of the 720p layer alone, as the benchmark's
    per-pathway figures run them: few heads, so ranged key sets are split
    (Global, Sink and Dummy alike) and merged in the kernel."""
    wl = W.WORKLOADS["720p"]
    heads = [h for h in range(wl.heads) if int(W.make_labels(wl)[h]) == lab]
    sub = W.small(wl, heads=len(heads))
    say("case 720p alone, pathway", lab, "heads", len(heads))
    data, cache, out = run_window(sub, [lab] * len(heads), seed=4)
    lay = cache.layout()
    if lab != O.SPATIAL:
        assert max(lay.global_splits, lay.sink_splits, lay.dummy_splits) > 1
    rows = sample_rows(sub, 48, seed=lab)
    fq, fk, fv = (W.as_float(data[n], sub) for n in ("q", "k", "v"))
    g = geometry_of(sub)
    ref = np.stack([O.attend_head(fq[h], fk[h], fv[h], lab, g, rows=rows) for h in range(len(heads))])
    check_close(to_float(out)[:, rows], ref, BF16_TOL, f"pathway {lab} alone")


def test_full_attention_baseline_720p_sampled():
    """All heads Global is the full-attention baseline the speedup is taken over."""
    wl = W.WORKLOADS["720p"]
    labels = np.full(wl.heads, O.GLOBAL)
    data, cache, out = run_window(wl, labels)
    rows = sample_rows(wl, 32, seed=3)
    fq, fk, fv = (W.as_float(data[n], wl) for n in ("q", "k", "v"))
    g = geometry_of(wl)
    heads = [0, 5, 11]
    ref = np.stack([O.attend_head(fq[h], fk[h], fv[h], O.GLOBAL, g, rows=rows) for h in heads])
    check_close(to_float(out)[heads][:, rows], ref, BF16_TOL, "full-attention baseline")


def test_spatial_cell_covering_frame_equals_global():
    """A Spatial head whose cell covers the frame reads the whole window."""
    wl = W.Workload("bigcell", 15, 2, 128, 9, 14, 1, 4, "bf16", "uniform", cell_h=9, cell_w=14)
    data = W.window(wl, seed=10)
    q, k, v = (upload(data[n], wl) for n in ("q", "k", "v"))
    a = fill_cache(wl, [2, 2], k, v).attend(q)
    b = fill_cache(wl, [3, 3], k, v).attend(q)
    torch().cuda.synchronize()
    ref = oracle_routed(wl, data, [3, 3])     # the Global pathway = full attention
    check_close(to_float(a), ref, BF16_TOL, "spatial, cell == frame")
    check_close(to_float(b), ref, BF16_TOL, "global")


def test_repeat_calls_deterministic():
    wl = W.Workload("det", 16, 6, 128, 20, 30, 3, 9, "bf16", "uniform")
    labels = [3, 3, 2, 1, 0, 2]
    data, cache, out = run_window(wl, labels, seed=12)
    out2 = cache.attend(upload(data["q"], wl))
    torch().cuda.synchronize()
    assert np.array_equal(download_bits(out), download_bits(out2))


def test_max_heads_every_pathway():
    """HC_MAX_HEADS = 128 heads, labels cycling through the four pathways: the
    per-category head tables hold every head at its slot."""
    wl = W.Workload("maxheads", 21, 128, 64, 8, 12, 1, 3, "bf16", "uniform")
    labels = [h % 4 for h in range(128)]
    say("case 128 heads")
    data, cache, out = run_window(wl, labels, seed=13)
    lay = cache.layout()
    assert (lay.n_sink, lay.n_dummy, lay.n_spatial, lay.n_global) == (32, 32, 32, 32)
    assert [lay.head_slot[h] for h in range(128)] == [h // 4 for h in range(128)]
    check_close(to_float(out), oracle_routed(wl, data, labels), BF16_TOL, "128 heads")


def test_two_caches_on_two_streams():
    """Two 480p caches attend at the same time on two streams.  Each
    persistent launch takes its units through its own cache's counters and
    merges key splits through its own partials, so both outputs equal those of
    the same calls made one after another, bit for bit, over three rounds."""
    wl = W.WORKLOADS["480p"]
    la = [int(x) for x in W.make_labels(wl)]
    lb = [3 - x for x in la]
    say("case two streams, labels", la, lb)
    da, ca, ref_a = run_window(wl, la, seed=14)
    db, cb, ref_b = run_window(wl, lb, seed=15)
    assert ca.layout().global_splits > 1 or cb.layout().global_splits > 1
    T = torch()
    qa, qb = upload(da["q"], wl), upload(db["q"], wl)
    sa, sb = T.cuda.Stream(), T.cuda.Stream()
    for _ in range(3):
        oa, ob = T.empty_like(qa), T.empty_like(qb)
        T.cuda.synchronize()
        with T.cuda.stream(sa):
            ca.attend(qa, oa)
        with T.cuda.stream(sb):
            cb.attend(qb, ob)
        T.cuda.synchronize()
        assert np.array_equal(download_bits(oa), download_bits(ref_a))
        assert np.array_equal(download_bits(ob), download_bits(ref_b))


def test_split_merges_repeat_bit_for_bit_under_load():
    """The three 720p Global heads alone: the planner splits each key range 8
    ways, so one launch has 1,032 units and 129 merges, each reading partials
    that other XCDs wrote with device-coherent stores.  Twenty launches back
    to back give the same bits; a merge that read a stale or partly written
    partial would not.  The first launch is also held to the oracle on
    sampled rows."""
    wl720 = W.WORKLOADS["720p"]
    heads = [h for h in range(wl720.heads) if int(W.make_labels(wl720)[h]) == O.GLOBAL]
    wl = W.small(wl720, heads=len(heads))
    say("case 720p Global heads alone, 20 launches")
    data, cache, out = run_window(wl, [O.GLOBAL] * len(heads), seed=21)
    assert cache.layout().global_splits == 8
    first = download_bits(out)
    q = upload(data["q"], wl)
    outs = [cache.attend(q) for _ in range(20)]
    torch().cuda.synchronize()
    for i, o in enumerate(outs):
        assert np.array_equal(download_bits(o), first), i
    rows = sample_rows(wl, 24, seed=3)
    check_close(to_float(out)[:, rows], oracle_routed(wl, data, [O.GLOBAL] * len(heads), rows=rows), BF16_TOL,
                "720p Global alone, 8 splits")
