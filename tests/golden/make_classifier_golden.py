"""Write the oracle's expected labels and diagnostics for a planted
classifier workload (40 heads at the 720p shape, seed 0): the planted one
(default) or the graded one (--workload classifier720p_graded, whose
diagnostics fix every cell of the rule and threshold study, since the
diagnostics do not depend on the thresholds), with the deployed grid-cell
Spatial proxy (default) or the sliding (2r+1)^2 box proxy (--spatial-proxy 1,
file suffix _box).

Calls only the CPU oracle and the seeded input generator.  Run from the
repository root:  python tests/golden/make_classifier_golden.py [--procs N]
[--spatial-proxy 1 --radius 2].  Takes about 45 minutes on 6 cores."""
import argparse
import json
import os
import sys
import time
from concurrent.futures import ProcessPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
os.environ.setdefault("OMP_NUM_THREADS", "1")
os.environ.setdefault("OPENBLAS_NUM_THREADS", "1")


def one_head(args):
    name, seed, h, proxy, radius = args
    from head_routed_kv_amd import workloads as W
    from oracle import headcast_oracle as O
    wl = W.WORKLOADS[name]
    data = W.window(wl, seed=seed, heads=[h], threads=1)
    q, k, v = (W.as_float(data[n], wl)[0] for n in ("q", "k", "v"))
    g = O.Geometry(wl.grid_h, wl.grid_w, wl.block_frames, wl.window_frames)
    prm = O.ClassifyParams(spatial_proxy=proxy, radius=radius)
    lab, diag, cos, mse = O.classify_head(q, k, v, g, prm)
    return h, int(lab), [float(x) for x in diag], float(mse), float(O.decision_margin(diag, prm)), \
        int(data["labels"][h])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="classifier720p")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--procs", type=int, default=6)
    ap.add_argument("--spatial-proxy", type=int, default=0, choices=(0, 1))
    ap.add_argument("--radius", type=int, default=2)
    a = ap.parse_args()
    from head_routed_kv_amd import workloads as W
    wl = W.WORKLOADS[a.workload]
    t0 = time.time()
    rows = {}
    with ProcessPoolExecutor(a.procs) as ex:
        for h, lab, diag, mse, margin, planted in ex.map(one_head, [(a.workload, a.seed, h, a.spatial_proxy, a.radius)
                                                                       for h in range(wl.heads)]):
            rows[h] = dict(label=lab, diag=diag, mse=mse, margin=margin, planted=planted)
            print(f"head {h}: label {lab} planted {planted} diag {diag} margin {margin:.4f}", flush=True)
    out = {
        "_source": "CPU oracle (oracle/headcast_oracle.py, fp64) on the seeded planted workload; "
                   "written by tests/golden/make_classifier_golden.py",
        "workload": a.workload, "seed": a.seed, "spatial_proxy": a.spatial_proxy, "radius": a.radius,
        "labels": [rows[h]["label"] for h in range(wl.heads)],
        "planted": [rows[h]["planted"] for h in range(wl.heads)],
        "diag": [rows[h]["diag"] for h in range(wl.heads)],
        "mse": [rows[h]["mse"] for h in range(wl.heads)],
        "margin": [rows[h]["margin"] for h in range(wl.heads)],
        "seconds": round(time.time() - t0, 1),
    }
    suffix = "" if a.spatial_proxy == 0 else ("_box" if a.radius == 2 else f"_box_r{a.radius}")
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), f"{a.workload}{suffix}_seed{a.seed}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path, "in", out["seconds"], "s")


if __name__ == "__main__":
    main()
