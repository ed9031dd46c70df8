"""Classifier rule and threshold study on the planted synthetic workload.

For each (rule, theta, theta_sc) the one-shot classifier (hc_classify, on
the GPU) labels every head of a planted 40-head 720p workload, by default
the graded one, whose heads carry their planted structure at strengths
spread so that some sit near each threshold.  Reported
per setting: label counts, heads whose label differs from the default
setting, heads whose label differs from the planted kind, and the layer's
routed attention FLOPs as a fraction of full attention.  This is the speed
side of the threshold ablation ([Pith] Fig. 5 caption: lowering either
threshold routes more heads to sparse paths; Referee Report comment 3 asks
for such sweeps); the quality side needs trained weights and is not here.
theta is applied to all three cosine thresholds.

    python -m head_routed_kv_amd.threshold_study [--proxy 0|1] [--json out.json]
"""
from __future__ import annotations

import argparse
import json
import time

import numpy as np

from . import _torch, classify, hc_default_classify_params, make_config
from . import workloads as W

THETAS = (0.85, 0.90, 0.95, 0.98)
THETA_SCS = (0.60, 0.70, 0.755, 0.80, 0.90)


def layer_flop_fraction(wl, labels):
    """Routed attention FLOPs of the layer / full attention FLOPs (QK and PV
    over each head's key set: Global Nq*Nk, Sink and Dummy Nq*B*T, Spatial
    B*W*sum of squared cell sizes)."""
    T = wl.grid_h * wl.grid_w
    cells = [min(wl.cell_h, wl.grid_h - y) * min(wl.cell_w, wl.grid_w - x)
             for y in range(0, wl.grid_h, wl.cell_h) for x in range(0, wl.grid_w, wl.cell_w)]
    pairs = {0: wl.Nq * wl.block_frames * T, 1: wl.Nq * wl.block_frames * T,
             2: wl.block_frames * wl.window_frames * sum(c * c for c in cells), 3: wl.Nq * wl.Nk}
    return sum(pairs[int(x)] for x in labels) / (len(labels) * pairs[3])


def run(proxy=0, seed=0, workload="classifier720p_graded", return_diag=False):
    torch = _torch()
    wl = W.WORKLOADS[workload]
    t0 = time.time()
    data = W.window(wl, seed=seed)
    dev = torch.device("cuda")

    def up(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v = up(data["q"]), up(data["k"]), up(data["v"])
    cfg = make_config(wl.heads, wl.head_dim, wl.grid_h, wl.grid_w, wl.block_frames, wl.window_frames)
    planted = np.asarray(data["labels"])
    ws = None
    rows = []
    default = None
    for rule in (0, 1):
        for th in THETAS:
            for ts in THETA_SCS:
                p = hc_default_classify_params()
                p.rule, p.spatial_proxy = rule, proxy
                p.theta_sink = p.theta_dummy = p.theta_spatial = th
                p.theta_score = ts
                labels, diag, ws = classify(cfg, q, k, v, p, workspace=ws)
                lab = labels.cpu().numpy().astype(int)
                if rule == 0 and th == 0.95 and ts == 0.755:
                    default = lab
                    default_diag = diag.cpu().numpy()
                rows.append({"rule": rule, "theta": th, "theta_sc": ts, "labels": lab.tolist()})
    for r in rows:
        lab = np.array(r["labels"])
        r["counts"] = {n: int((lab == i).sum()) for i, n in enumerate(("sink", "dummy", "spatial", "global"))}
        r["flips_vs_default"] = int((lab != default).sum())
        r["differs_from_planted"] = int((lab != planted).sum())
        r["flop_fraction"] = round(layer_flop_fraction(wl, lab), 4)
    out = {"workload": f"{workload}, 40 heads, seed {seed}", "spatial_proxy": proxy,
           "strength": [round(float(x), 3) for x in data["strength"]],
           "planted_counts": {n: int((planted == i).sum()) for i, n in enumerate(("sink", "dummy", "spatial", "global"))},
           "seconds": round(time.time() - t0, 1), "rows": rows}
    if return_diag:   # the default setting's [H, 4] diagnostics (they do not depend on the thresholds)
        out["diag"] = default_diag.tolist()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--proxy", type=int, default=0, choices=(0, 1))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--workload", default="classifier720p_graded")
    ap.add_argument("--json", default=None)
    a = ap.parse_args()
    res = run(a.proxy, a.seed, a.workload)
    print("rule theta theta_sc | sink dummy spatial global | flips differs_from_planted flop_fraction")
    for r in res["rows"]:
        c = r["counts"]
        print(f"{r['rule']} {r['theta']:.3f} {r['theta_sc']:.3f} | {c['sink']:2d} {c['dummy']:2d} {c['spatial']:2d} "
              f"{c['global']:2d} | {r['flips_vs_default']:2d} {r['differs_from_planted']:2d} {r['flop_fraction']:.4f}")
    if a.json:
        with open(a.json, "w") as f:
            json.dump(res, f, indent=1)


if __name__ == "__main__":
    main()
