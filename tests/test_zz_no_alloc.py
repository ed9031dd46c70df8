"""hc_classify_static, the allocation-free classifier, against hc_classify
through the C ABI: labels and diagnostics bit for bit (the same kernels run
on a different workspace), on two calls in a row, the second on a smaller
layer, so the second call reuses the static scratch the first one filled."""
import numpy as np
import pytest

import head_routed_kv_amd as hk
from head_routed_kv_amd import workloads as W
from tests.gpu_util import config_of, say, torch, upload

pytestmark = pytest.mark.gpu


def test_static_classifier_matches_workspace_classifier():
    t = torch()
    cases = [
        (W.small(W.WORKLOADS["classifier720p"], grid_h=20, grid_w=30, heads=12, window_frames=9), 2),
        (W.Workload("static2", 70, 5, 64, 13, 17, 2, 6, "bf16", "uniform"), 5),
    ]
    for wl, seed in cases:
        cfg = config_of(wl)
        need = hk.hc_classify_workspace_bytes(cfg)
        assert need <= hk._native.HC_STATIC_SCRATCH_BYTES
        say("static classifier case", wl.name, "workspace bytes", need)
        data = W.window(wl, seed=seed)
        q, k, v = (upload(data[n], wl) for n in ("q", "k", "v"))
        ref_labels, ref_diag, _ = hk.classify(cfg, q, k, v)
        labels = t.full((wl.heads,), -1, dtype=t.int8, device="cuda")
        diag = t.full((wl.heads, 4), float("nan"), dtype=t.float32, device="cuda")
        t.cuda.synchronize()
        hk.classify_static(cfg, q, k, v, labels=labels, diag=diag)
        t.cuda.synchronize()
        assert t.equal(labels, ref_labels), (wl.name, labels.cpu().numpy(), ref_labels.cpu().numpy())
        assert t.equal(diag, ref_diag), wl.name
        say(wl.name, "labels", labels.cpu().numpy().tolist())
        if wl.labels == "planted":   # and they are the planted kinds
            assert np.array_equal(labels.cpu().numpy(), data["labels"])
