"""Routed attention against the oracle on seeded random configurations.

Twelve configurations are drawn once, from a fixed seed, over the space the
API accepts: grids from one row or column up, cells from 1x1 to larger than
the frame, blocks of 1-3 frames, windows of 1-5 blocks, 1-6 heads with random
labels, d = 64 and 128, bf16 and fp32, and an fp8 cache.  Each case fills the
window, pushes up to two more blocks (the window slides; the Sink block stays
the first one) and attends; every output row is compared with the oracle."""
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
