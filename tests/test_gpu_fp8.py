"""GPU parity of the fp8 KV cache (OCP E4M3 codes, kv_format HC_KV_FP8_E4M3):
the cached codes against the oracle's quantiser byte for byte, and routed
attention on the decoded values against the oracle."""
import numpy as np
import pytest

import head_routed_kv_amd as hk
from head_routed_kv_amd import workloads as W
from oracle import headcast_oracle as O
from oracle import pool
from tests.gpu_util import BF16_TOL, check_close, geometry_of, sample_rows, say, to_float, torch, upload

pytestmark = pytest.mark.gpu

# Neither scale is a power of two, so the fp32 product x * (1/scale) rounds
# before the E4M3 rounding, on both sides.
K_SCALE, V_SCALE = 0.75, 1.5


def fp8_config(wl, k_scale=K_SCALE, v_scale=V_SCALE):
    return hk.make_config(wl.heads, wl.head_dim, wl.grid_h, wl.grid_w, wl.block_frames, wl.window_frames,
                          wl.cell_h, wl.cell_w, hk.HC_BF16, kv_format=hk.HC_KV_FP8_E4M3, k_scale=k_scale,
                          v_scale=v_scale)


def codes(x, wl, scale):
    return O.quantize_kv(W.as_float(x, wl), scale)


def fill(wl, labels, k, v, **kw):
    cache = hk.RoutedCache(fp8_config(wl, **kw), labels)
    BT = wl.Nq
    for b in range(wl.n_blocks):
        cache.append(k[:, b * BT:(b + 1) * BT], v[:, b * BT:(b + 1) * BT])
    return cache


def oracle_fp8(wl, data, labels, rows=None, heads=None, k_scale=K_SCALE, v_scale=V_SCALE):
    fq = W.as_float(data["q"], wl)
    dk = O.dequantize_kv(codes(data["k"], wl, k_scale), k_scale)
    dv = O.dequantize_kv(codes(data["v"], wl, v_scale), v_scale)
    g = geometry_of(wl)
    heads = range(wl.heads) if heads is None else heads
    return np.stack([O.attend_head(fq[h], dk[h], dv[h], int(labels[h]), g, rows=rows) for h in heads])


@pytest.mark.parametrize("d", [128, 64])
def test_fp8_cache_codes_bit_exact(d):
    """Every archetype buffer holds the oracle's E4M3 codes of the blocks, in
    the documented layout, through a ring wrap and a replacement; one block
    is scaled up so that codes saturate at +-448."""
    wl = W.Workload("bits8", 19, 6, d, 13, 23, 2, 6, "bf16", "uniform")
    labels = [2, 3, 0, 1, 3, 2]
    g = geometry_of(wl)
    cache = hk.RoutedCache(fp8_config(wl), labels)
    model = O.CacheModel(g, labels)
    ks, vs = W.stream_blocks(wl, 4, 6)
    ks2, vs2 = W.stream_blocks(wl, 5, 6)
    ks[3] = W.f32_to_bf16_bits(W.as_float(ks[3], wl) * 300.0)   # |x / 0.75| up to ~1500
    saturated = 0
    for step in range(6):
        mode = hk.HC_REPLACE_NEWEST if step == 4 else hk.HC_PUSH_BLOCK
        kb, vb = (ks2[step], vs2[step]) if mode else (ks[step], vs[step])
        say("fp8 append step", step, "mode", mode)
        cache.append(upload(kb, wl), upload(vb, wl), mode)
        kc, vc = codes(kb, wl, K_SCALE), codes(vb, wl, V_SCALE)
        saturated += int(np.sum((kc & 0x7F) == 0x7E))
        model.append(kc, vc, mode)
        torch().cuda.synchronize()
        lay = cache.layout()
        raw = cache.mem.cpu().numpy()
        for lab, (ok, ov) in {O.GLOBAL: (lay.off_global_k, lay.off_global_v),
                              O.SINK: (lay.off_sink_k, lay.off_sink_v),
                              O.DUMMY: (lay.off_dummy_k, lay.off_dummy_v),
                              O.SPATIAL: (lay.off_spatial_k, lay.off_spatial_v)}.items():
            for which, off in (("k", ok), ("v", ov)):
                exp, valid = model.expected_buffer(lab, which)
                got = raw[off:off + exp.size].reshape(exp.shape)
                assert np.array_equal(got[:, valid], exp[:, valid]), (step, lab, which)
    assert saturated > 0


@pytest.mark.parametrize("d", [128, 64])
def test_fp8_attend_every_pathway_small(d):
    """Several q tiles and key tiles with ragged tails, uneven border cells,
    all four pathways; repeat calls are bit-identical."""
    wl = W.Workload("small8", 20, 8, d, 23, 37, 2, 6, "bf16", "uniform")
    labels = [0, 1, 2, 3, 3, 2, 1, 0]
    say("case fp8 small, d", d)
    data = W.window(wl, seed=5)
    q, k, v = (upload(data[n], wl) for n in ("q", "k", "v"))
    cache = fill(wl, labels, k, v)
    out = cache.attend(q)
    out2 = cache.attend(q)
    torch().cuda.synchronize()
    check_close(to_float(out), oracle_fp8(wl, data, labels), BF16_TOL, "fp8 small")
    assert torch().equal(out, out2)


@pytest.mark.parametrize("lab", [O.GLOBAL, O.SINK, O.SPATIAL])
def test_fp8_720p_pathway_alone_sampled(lab):
    """One pathway's heads of the 720p layer alone: ranged key sets are split
    and merged in the kernel, where the V scale is applied at the merge."""
    wl = W.WORKLOADS["720p"]
    heads = [h for h in range(wl.heads) if int(W.make_labels(wl)[h]) == lab]
    sub = W.small(wl, heads=len(heads))
    say("case fp8 720p alone, pathway", lab, "heads", len(heads))
    data = W.window(sub, seed=4)
    q, k, v = (upload(data[n], sub) for n in ("q", "k", "v"))
    cache = fill(sub, [lab] * len(heads), k, v)
    out = cache.attend(q)
    torch().cuda.synchronize()
    lay = cache.layout()
    if lab != O.SPATIAL:
        assert max(lay.global_splits, lay.sink_splits) > 1
    rows = sample_rows(sub, 48, seed=lab)
    ref = oracle_fp8(sub, data, [lab] * len(heads), rows=rows)
    check_close(to_float(out)[:, rows], ref, BF16_TOL, f"fp8 pathway {lab} alone")


@pytest.mark.timeout(900)   # the oracle side runs every row, process-parallel
def test_fp8_720p_every_row():
    """The 720p routed layer over an fp8 cache with scales that are not
    powers of two, in the benchmark's launch configuration (its split plan
    for fp8 caches): every query row of every head against the oracle on the
    decoded K/V."""
    wl = W.WORKLOADS["720p"]
    labels = W.make_labels(wl)
    say("case fp8 720p every row")
    data = W.window(wl, seed=0)
    q, k, v = (upload(data[n], wl) for n in ("q", "k", "v"))
    cache = fill(wl, labels, k, v)
    lay = cache.layout()
    say("fp8 720p splits", lay.global_splits, lay.sink_splits, lay.dummy_splits)
    out = cache.attend(q)
    torch().cuda.synchronize()
    got = to_float(out)
    del q, k, v, out, cache
    res, cpu_s, wall = pool.run(wl, 0, [(h, int(labels[h])) for h in range(wl.heads)], rows_per_task=1350,
                                kv_scales=(K_SCALE, V_SCALE))
    say(f"fp8 720p oracle: {cpu_s:.0f} s of CPU in {wall:.0f} s")
    ref = np.stack([res[(h, int(labels[h]))] for h in range(wl.heads)])
    check_close(got, ref, BF16_TOL, "fp8 720p every row")


def test_fp8_720p_routed_sampled():
    """The full 720p routed layer in the launch configuration the benchmark
    times for the fp8 cache, on sampled rows of every head."""
    wl = W.WORKLOADS["720p"]
    labels = W.make_labels(wl)
    say("case fp8 720p routed")
    data = W.window(wl, seed=0)
    q, k, v = (upload(data[n], wl) for n in ("q", "k", "v"))
    cache = fill(wl, labels, k, v, k_scale=1.0, v_scale=1.0)
    out = cache.attend(q)
    torch().cuda.synchronize()
    rows = sample_rows(wl, 48, seed=2)
    ref = oracle_fp8(wl, data, labels, rows=rows, k_scale=1.0, v_scale=1.0)
    worst = check_close(to_float(out)[:, rows], ref, BF16_TOL, "fp8 720p")
    say("fp8 720p worst err/rms", worst)
