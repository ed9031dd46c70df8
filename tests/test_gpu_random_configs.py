"""Routed attention against the oracle on seeded random configurations.

Twelve configurations are drawn once, from a fixed seed, over the space the
API accepts: grids from one row or column up, cells from 1x1 to larger than
the frame, blocks of 1-3 frames, windows of 1-5 blocks, 1-6 heads with random
labels, d = 64 and 128, bf16 and fp32, and an fp8 cache.  Each case fills the
window, pushes up to two more blocks (the window slides; the Sink block stays
the first one), replaces the newest block once and attends; every output row
is compared with the oracle."""
import numpy as np
import pytest

import head_routed_kv_amd as hk
from head_routed_kv_amd import workloads as W
from oracle import headcast_oracle as O
from tests.gpu_util import BF16_TOL, FP32_TOL, check_close, say, to_float, torch, upload

pytestmark = pytest.mark.gpu

K_SCALE, V_SCALE = 0.75, 1.5


def draw_cases():
    rng = np.random.default_rng(2026)
    cases = []
    for i in range(12):
        d = (64, 128)[i % 2]
        dtype = "fp32" if i % 4 == 3 else "bf16"
        fp8 = dtype == "bf16" and d == 128 and i % 3 == 0
        gh, gw = int(rng.integers(1, 25)), int(rng.integers(1, 41))
        B, nb = int(rng.integers(1, 4)), int(rng.integers(1, 6))
        ch, cw = int(rng.integers(1, 13)), int(rng.integers(1, 13))
        H = int(rng.integers(1, 7))
        labels = [int(x) for x in rng.integers(0, 4, H)]
        extra = int(rng.integers(0, 3))
        wl = W.Workload(f"random{i}", 40 + i, H, d, gh, gw, B, B * nb, dtype, "uniform", ch, cw)
        cases.append(pytest.param(wl, labels, fp8, extra, id=f"{i}-{dtype}{'-fp8' if fp8 else ''}-d{d}-"
                                  f"{gh}x{gw}-B{B}W{B * nb}-c{ch}x{cw}-H{H}"))
    return cases


def config(wl, fp8):
    dt = hk.HC_FP32 if wl.dtype == "fp32" else hk.HC_BF16
    if fp8:
        return hk.make_config(wl.heads, wl.head_dim, wl.grid_h, wl.grid_w, wl.block_frames, wl.window_frames,
                              wl.cell_h, wl.cell_w, dt, kv_format=hk.HC_KV_FP8_E4M3, k_scale=K_SCALE,
                              v_scale=V_SCALE)
    return hk.make_config(wl.heads, wl.head_dim, wl.grid_h, wl.grid_w, wl.block_frames, wl.window_frames,
                          wl.cell_h, wl.cell_w, dt)


@pytest.mark.parametrize("wl,labels,fp8,extra", draw_cases())
def test_random_configuration(wl, labels, fp8, extra):
    say("random case", wl.name, "labels", labels, "fp8", fp8, "extra blocks", extra)
    geo = O.Geometry(wl.grid_h, wl.grid_w, wl.block_frames, wl.window_frames, wl.cell_h, wl.cell_w)
    cache = hk.RoutedCache(config(wl, fp8), labels)
    model = O.CacheModel(geo, labels)
    n = wl.n_blocks + extra
    ks, vs = W.stream_blocks(wl, 1, n)
    for b in range(n):
        cache.append(upload(ks[b], wl), upload(vs[b], wl))
        if fp8:
            model.append(O.quantize_kv(W.as_float(ks[b], wl), K_SCALE), O.quantize_kv(W.as_float(vs[b], wl), V_SCALE),
                         hk.HC_PUSH_BLOCK)
        else:
            model.append(ks[b], vs[b], hk.HC_PUSH_BLOCK)
    # a later denoising step of the newest block replaces its keys and values
    rk, rv = W.stream_blocks(wl, 3, 1)
    cache.append(upload(rk[0], wl), upload(rv[0], wl), hk.HC_REPLACE_NEWEST)
    if fp8:
        model.append(O.quantize_kv(W.as_float(rk[0], wl), K_SCALE), O.quantize_kv(W.as_float(rv[0], wl), V_SCALE),
                     hk.HC_REPLACE_NEWEST)
    else:
        model.append(rk[0], rv[0], hk.HC_REPLACE_NEWEST)
    q = W.queries(wl, 2)
    out = cache.attend(upload(q, wl))
    torch().cuda.synchronize()

    wk, wv = model.window()
    if fp8:
        fk, fv = O.dequantize_kv(wk, K_SCALE), O.dequantize_kv(wv, V_SCALE)
        sk, sv = O.dequantize_kv(model.sink_k, K_SCALE), O.dequantize_kv(model.sink_v, V_SCALE)
    else:
        fk, fv = W.as_float(wk, wl), W.as_float(wv, wl)
        sk, sv = W.as_float(model.sink_k, wl), W.as_float(model.sink_v, wl)
    ref = O.routed_attention(W.as_float(q, wl), fk, fv, np.array(labels), geo, k_sink=sk, v_sink=sv)
    check_close(to_float(out), ref, FP32_TOL if wl.dtype == "fp32" else BF16_TOL, wl.name)


def label_comparable(o_diag, op, dtol, n_blocks):
    """Whether the GPU's label must equal the oracle's.  The diagnostics are
    asserted within dtol of the oracle's, so a decision margin above 2*dtol
    fixes the label (the margin's own guarantee).  A one-block window is the
    exact tie the rule breaks by order: the full output and the Sink and
    Dummy proxies are the same output on both sides, so both pick Sink,
    unless the Spatial proxy could win or lose its own comparison."""
    if O.decision_margin(o_diag, op) > 2 * dtol:
        return True
    if n_blocks == 1:
        sp_clear_gap = min(abs(o_diag[2] - op.theta_spatial), abs(o_diag[3] - op.theta_score))
        sp_out = o_diag[2] < op.theta_spatial or o_diag[3] < op.theta_score
        return sp_out and sp_clear_gap > 2 * dtol and O.decide_label(o_diag, op) == O.SINK
    return False


def draw_classifier_cases():
    rng = np.random.default_rng(2027)
    cases = []
    for i in range(8):
        d = (128, 64)[i % 2]
        dtype = "fp32" if i % 4 == 2 else "bf16"
        gh, gw = int(rng.integers(1, 21)), int(rng.integers(1, 33))
        B, nb = int(rng.integers(1, 4)), int(rng.integers(1, 5))
        ch, cw = int(rng.integers(1, 13)), int(rng.integers(1, 13))
        H = int(rng.integers(1, 6))
        proxy = i % 2                       # 0: the deployed cell, 1: the sliding box
        radius = int(rng.integers(1, 4))
        wl = W.Workload(f"rcls{i}", 60 + i, H, d, gh, gw, B, B * nb, dtype, "uniform", ch, cw)
        cases.append(pytest.param(wl, proxy, radius, id=f"{i}-{dtype}-d{d}-{gh}x{gw}-B{B}W{B * nb}-c{ch}x{cw}-H{H}-"
                                  + ("cell" if proxy == 0 else f"box{radius}")))
    return cases


@pytest.mark.parametrize("wl,proxy,radius", draw_classifier_cases())
def test_random_classifier_configuration(wl, proxy, radius):
    """hc_classify on a random configuration: the four outputs, the per-query
    cosines and the per-head diagnostics against the oracle; labels where the
    oracle's decision margin is clear of the diagnostics' tolerance."""
    say("random classifier case", wl.name, "proxy", proxy, "radius", radius)
    fp32 = wl.dtype == "fp32"
    tol, dtol = (FP32_TOL, 1e-5) if fp32 else (BF16_TOL, 1e-2)
    data = W.window(wl, seed=5)
    t = torch()
    q, k, v = (upload(data[n], wl) for n in ("q", "k", "v"))
    p = hk.hc_default_classify_params()
    p.spatial_proxy, p.radius = proxy, radius
    labels, diag, ws = hk.classify(config(wl, False), q, k, v, p)
    t.cuda.synchronize()
    H, Nq, d = wl.heads, wl.Nq, wl.head_dim
    outs = ws[:4 * H * Nq * d * 4].view(t.float32).view(4, H, Nq, d).cpu().numpy()
    off = ((4 * H * Nq * d * 4 + 255) // 256) * 256
    cos = ws[off:off + H * 4 * Nq * 4].view(t.float32).view(H, 4, Nq).cpu().numpy()
    labels, diag = labels.cpu().numpy(), diag.cpu().numpy()

    op = O.ClassifyParams(spatial_proxy=proxy, radius=radius)
    geo = O.Geometry(wl.grid_h, wl.grid_w, wl.block_frames, wl.window_frames, wl.cell_h, wl.cell_w)
    sp = O.SPATIAL if proxy == 0 else O.SLIDING
    for h in range(H):
        fq, fk, fv = (W.as_float(data[n], wl)[h] for n in ("q", "k", "v"))
        o_outs = [O.attend_head(fq, fk, fv, pw, geo, radius=radius) for pw in (O.GLOBAL, O.SINK, O.DUMMY, sp)]
        o_diag, o_cos, _ = O.head_scores(*o_outs, op)
        for j in range(4):
            check_close(outs[j, h][None], o_outs[j][None], tol, f"{wl.name} head {h} output {j}", out_fmt="fp32")
        np.testing.assert_allclose(cos[h, :3], o_cos, atol=dtol)
        np.testing.assert_allclose(diag[h], o_diag, atol=dtol)
        assert label_comparable(o_diag, op, dtol, wl.n_blocks) is False or \
            labels[h] == O.decide_label(o_diag, op), (h, labels[h], o_diag)


def draw_planted_cases():
    """Random geometries with the planted classifier structure (Sink, Dummy,
    Spatial and unplanted heads), windows of 2-5 blocks."""
    rng = np.random.default_rng(2028)
    cases = []
    for i in range(6):
        d = (128, 64)[i % 2]
        dtype = "fp32" if i % 3 == 2 else "bf16"
        gh, gw = int(rng.integers(10, 25)), int(rng.integers(10, 41))
        B, nb = int(rng.integers(1, 4)), int(rng.integers(2, 6))
        ch, cw = int(rng.integers(4, 13)), int(rng.integers(4, 13))
        H = int(rng.integers(4, 9))
        cases.append(W.Workload(f"rplant{i}", 80 + i, H, d, gh, gw, B, B * nb, dtype, "planted", ch, cw))
    return cases


def test_random_planted_classifier_labels():
    """hc_classify on six random planted geometries: diagnostics against the
    oracle, and labels wherever the oracle's margin is clear.  Every label
    (Sink, Dummy, Spatial, Global) must be among the compared ones, so label
    parity is exercised beyond the Global heads that unplanted random data
    give."""
    t = torch()
    compared = {lab: 0 for lab in range(4)}
    for wl in draw_planted_cases():
        say("random planted classifier case", wl)
        fp32 = wl.dtype == "fp32"
        dtol = 1e-5 if fp32 else 1e-2
        data = W.window(wl, seed=5)
        q, k, v = (upload(data[n], wl) for n in ("q", "k", "v"))
        labels, diag, _ = hk.classify(config(wl, False), q, k, v)
        t.cuda.synchronize()
        labels, diag = labels.cpu().numpy(), diag.cpu().numpy()
        geo = O.Geometry(wl.grid_h, wl.grid_w, wl.block_frames, wl.window_frames, wl.cell_h, wl.cell_w)
        fq, fk, fv = (W.as_float(data[n], wl) for n in ("q", "k", "v"))
        op = O.ClassifyParams()
        for h in range(wl.heads):
            o_lab, o_diag, _, _ = O.classify_head(fq[h], fk[h], fv[h], geo, op)
            np.testing.assert_allclose(diag[h], o_diag, atol=dtol)
            if label_comparable(o_diag, op, dtol, wl.n_blocks):
                assert labels[h] == o_lab, (wl.name, h, labels[h], o_lab, o_diag)
                compared[o_lab] += 1
    say("labels compared per kind (sink, dummy, spatial, global):", compared)
    assert all(n >= 1 for n in compared.values()), compared
    assert sum(compared.values()) >= 30, compared
