"""The per-step work of denoising one block (HC_REPLACE_NEWEST append, then
routed attention) recorded into a HIP graph and replayed: each replay, with
new block data copied into the recorded inputs and eager work and
synchronisation between replays, must equal the same calls made eagerly,
bit for bit (output and cache buffers); the last replay is also checked
against the oracle."""
import numpy as np
import pytest

import head_routed_kv_amd as hk
from head_routed_kv_amd import workloads as W
from oracle import headcast_oracle as O
from tests.gpu_util import BF16_TOL, check_close, geometry_of, sample_rows, say, to_float, torch, upload

pytestmark = pytest.mark.gpu

K_SCALE, V_SCALE = 0.75, 1.5
REPLAYS = 4


def graph_config(wl, kv):
    if kv == "fp8":
        return hk.make_config(wl.heads, wl.head_dim, wl.grid_h, wl.grid_w, wl.block_frames, wl.window_frames,
                              wl.cell_h, wl.cell_w, hk.HC_BF16, kv_format=hk.HC_KV_FP8_E4M3, k_scale=K_SCALE,
                              v_scale=V_SCALE)
    return hk.make_config(wl.heads, wl.head_dim, wl.grid_h, wl.grid_w, wl.block_frames, wl.window_frames,
                          wl.cell_h, wl.cell_w, hk.HC_BF16)


def stored(x, wl, kv, scale):
    """The values attention sees for cached storage-form x."""
    f = W.as_float(x, wl)
    return O.dequantize_kv(O.quantize_kv(f, scale), scale) if kv == "fp8" else f


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_graph_replays_of_the_block_step(kv):
    t = torch()
    # d = 128, every pathway, a full window of 4 blocks, Global heads split
    # five ways (so the split counters and merges run inside the graph).
    wl = W.Workload("graph", 30, 6, 128, 23, 37, 2, 8, "bf16", "uniform")
    labels = [3, 0, 1, 2, 3, 2]
    cfg = graph_config(wl, kv)
    eager, graphed = hk.RoutedCache(cfg, labels), hk.RoutedCache(cfg, labels)
    ks, vs = W.stream_blocks(wl, 3, wl.n_blocks)
    for b in range(wl.n_blocks):
        kb, vb = upload(ks[b], wl), upload(vs[b], wl)
        eager.append(kb, vb)
        graphed.append(kb, vb)
    lay = eager.layout()
    assert lay.global_splits > 1
    new_k, new_v = W.stream_blocks(wl, 4, REPLAYS)
    new_q = [W.queries(wl, 10 + r) for r in range(REPLAYS)]

    # recorded inputs; recording runs nothing, so their contents do not matter
    k_in, v_in, q_in = (upload(x, wl) for x in (new_k[0], new_v[0], new_q[0]))
    t.cuda.synchronize()
    say("recording the block step,", kv)
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        graphed.append(k_in, v_in, hk.HC_REPLACE_NEWEST)
        out_g = graphed.attend(q_in)
    t.cuda.synchronize()

    end = lay.off_scratch   # K/V buffers; the scratch region holds split partials
    for r in range(REPLAYS):
        say("replay", r, kv)
        kr, vr, qr = upload(new_k[r], wl), upload(new_v[r], wl), upload(new_q[r], wl)
        k_in.copy_(kr)
        v_in.copy_(vr)
        q_in.copy_(qr)
        g.replay()
        eager.append(kr, vr, hk.HC_REPLACE_NEWEST)
        ref = eager.attend(qr)
        t.cuda.synchronize()
        assert t.equal(out_g, ref), f"replay {r}: output differs from the eager calls"
        assert t.equal(graphed.mem[:end], eager.mem[:end]), f"replay {r}: cache buffers differ"

    # oracle: the window is blocks 0..2 as pushed and the last replay's block
    # as the newest; no wrap, so the Sink block is the window's first block
    last = REPLAYS - 1
    wk = np.concatenate([*ks[:-1], new_k[last]], axis=1)
    wv = np.concatenate([*vs[:-1], new_v[last]], axis=1)
    dk = stored(wk, wl, kv, K_SCALE if kv == "fp8" else 1.0)
    dv = stored(wv, wl, kv, V_SCALE if kv == "fp8" else 1.0)
    fq = W.as_float(new_q[last], wl)
    geo = geometry_of(wl)
    rows = sample_rows(wl, 64, seed=7)
    ref = np.stack([O.attend_head(fq[h], dk[h], dv[h], labels[h], geo, rows=rows) for h in range(wl.heads)])
    check_close(to_float(out_g)[:, rows], ref, BF16_TOL, f"graph replay {last} ({kv})")


def test_graph_replays_of_the_classifier():
    """hc_classify recorded once and replayed on new windows copied into the
    recorded inputs: labels, diagnostics, the four outputs and the per-query
    cosines equal an eager call on the same data, bit for bit."""
    t = torch()
    wl = W.Workload("graphcls", 31, 5, 128, 19, 29, 2, 6, "bf16", "uniform")
    cfg = graph_config(wl, "bf16")
    draws = [W.window(wl, seed=20 + r) for r in range(3)]
    q_in, k_in, v_in = (upload(draws[0][n], wl) for n in ("q", "k", "v"))
    params = hk.hc_default_classify_params()
    ws = t.empty(hk.hc_classify_workspace_bytes(cfg), dtype=t.uint8, device="cuda")
    hk.classify(cfg, q_in, k_in, v_in, params, ws)   # eager first call outside the recording
    t.cuda.synchronize()
    say("recording the classifier")
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        labels_g, diag_g, ws_g = hk.classify(cfg, q_in, k_in, v_in, params, ws)
    t.cuda.synchronize()
    for r, data in enumerate(draws):
        say("classifier replay", r)
        q, k, v = (upload(data[n], wl) for n in ("q", "k", "v"))
        q_in.copy_(q)
        k_in.copy_(k)
        v_in.copy_(v)
        g.replay()
        t.cuda.synchronize()
        got = (labels_g.clone(), diag_g.clone(), ws_g.clone())
        labels_e, diag_e, ws_e = hk.classify(cfg, q, k, v, params)
        t.cuda.synchronize()
        assert t.equal(got[0], labels_e), r
        assert t.equal(got[1], diag_e), r
        H, Nq, d = wl.heads, wl.Nq, wl.head_dim
        n_out = 4 * H * Nq * d * 4                      # four fp32 outputs
        off = (n_out + 255) // 256 * 256                 # then the cosines, 256-byte aligned
        n_cos = H * 4 * Nq * 4
        assert t.equal(got[2][:n_out], ws_e[:n_out]), r
        assert t.equal(got[2][off:off + n_cos], ws_e[off:off + n_cos]), r
