"""GPU test of the streaming driver (head_routed_kv_amd.session): all-Global
warm-up, classification at the first full window, restructuring by replay,
then routed rollout with pushes and replacements.  Every attention output is
checked against the oracle."""
import numpy as np
import pytest

import head_routed_kv_amd as hk
from head_routed_kv_amd import workloads as W
from head_routed_kv_amd.session import LayerSession
from oracle import headcast_oracle as O
from tests.gpu_util import BF16_TOL, check_close, config_of, geometry_of, say, to_float, torch, upload

pytestmark = pytest.mark.gpu


K8, V8 = 0.5, 1.25   # scales of the fp8 routed cache


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_layer_session_rollout(kv):
    """With kv = fp8 the warm-up cache stays bf16 (the classifier reads it) and
    the restructured cache stores E4M3 codes."""
    # planted window (blocks 0..2, queries of block 2) whose kinds the classifier recovers
    wl = W.small(W.WORKLOADS["classifier720p"], grid_h=20, grid_w=30, heads=12, window_frames=9)
    fp8 = kv == "fp8"
    cfg = config_of(wl)
    if fp8:
        cfg.kv_format, cfg.k_scale, cfg.v_scale = hk.HC_KV_FP8_E4M3, K8, V8

    def enc(kb, vb):   # what the routed cache stores
        if not fp8:
            return kb, vb
        return O.quantize_kv(W.as_float(kb, wl), K8), O.quantize_kv(W.as_float(vb, wl), V8)

    def dec(x, scale):
        return O.dequantize_kv(x, scale) if fp8 else W.as_float(x, wl)
    data = W.window(wl, seed=2)
    g = geometry_of(wl)
    H, BT, B = wl.heads, wl.Nq, wl.block_frames
    nb = wl.window_frames // B
    win_k = [data["k"][:, b * BT:(b + 1) * BT] for b in range(nb)]
    win_v = [data["v"][:, b * BT:(b + 1) * BT] for b in range(nb)]
    later_k, later_v = W.stream_blocks(wl, 21, 3)     # blocks after the first window
    step2_k, step2_v = W.stream_blocks(wl, 22, 3)     # their second denoising step
    sess = LayerSession(cfg)
    model = None

    def expect(q):
        fq = W.as_float(q, wl)
        if model is None:   # warm-up: every head over the blocks pushed so far
            wk, wv = np.concatenate(pushed_k, axis=1), np.concatenate(pushed_v, axis=1)
            gq = O.Geometry(g.grid_h, g.grid_w, B, wk.shape[1] // g.T, g.cell_h, g.cell_w)
            return O.routed_attention(fq, W.as_float(wk, wl), W.as_float(wv, wl), np.full(H, O.GLOBAL), gq)
        wk, wv = model.window()
        gq = O.Geometry(g.grid_h, g.grid_w, B, wk.shape[1] // g.T, g.cell_h, g.cell_w)
        return O.routed_attention(fq, dec(wk, K8), dec(wv, V8), np.array(sess.labels), gq,
                                  k_sink=dec(model.sink_k, K8), v_sink=dec(model.sink_v, V8))

    pushed_k, pushed_v = [], []
    for b in range(nb + 3):
        kb, vb = (win_k[b], win_v[b]) if b < nb else (later_k[b - nb], later_v[b - nb])
        sess.push(upload(kb, wl), upload(vb, wl))
        pushed_k.append(kb)
        pushed_v.append(vb)
        q = data["q"] if b == nb - 1 else W.queries(wl, 30 + b)
        qd = upload(q, wl)
        say("session", kv, "block", b, "routed" if sess.routed else "warm-up")
        if sess.classify_due():
            labels = sess.classify(qd)
            np.testing.assert_array_equal(labels, data["labels"])
            model = O.CacheModel(g, labels)
            for bb in range(nb):
                model.append(*enc(win_k[bb], win_v[bb]), hk.HC_PUSH_BLOCK)
        elif model is not None:
            model.append(*enc(kb, vb), hk.HC_PUSH_BLOCK)
        out = sess.attend(qd)
        torch().cuda.synchronize()
        check_close(to_float(out), expect(q), BF16_TOL, f"block {b} first step")
        if b >= nb:   # a second denoising step replaces the newest block
            sess.replace(upload(step2_k[b - nb], wl), upload(step2_v[b - nb], wl))
            model.append(*enc(step2_k[b - nb], step2_v[b - nb]), hk.HC_REPLACE_NEWEST)
            out = sess.attend(qd)
            torch().cuda.synchronize()
            check_close(to_float(out), expect(q), BF16_TOL, f"block {b} second step")
    assert sess.routed and not sess.classify_due()
    with pytest.raises(hk.HeadcastError):
        sess.classify(qd)
    sess.close()
