"""Pins for the CPU oracle: closed forms, invariants, library routines and
brute force on tiny inputs (no GPU).  Each test names what fixes the value."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import headcast_oracle as O
from head_routed_kv_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TINY = O.Geometry(8, 12, 1, 4)


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def sdpa_f64(q, k, v, mask, scale):
    """torch's library attention in float64 on the CPU."""
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        attn_mask=torch.from_numpy(mask)[None], scale=scale)
    return out[0].numpy()


# ----------------------------------------------------------------------------- geometry
@pytest.mark.parametrize("gh,gw,cells,sizes", [
    (8, 12, 2, {80: 1, 16: 1}),               # tiny: one 8x10 and one 8x2 cell
    (30, 52, 18, {100: 15, 20: 3}),           # 480p: last column of cells is 10x2
    (45, 80, 40, {100: 32, 50: 8}),           # 720p: last row of cells is 5x10
    (68, 120, 84, {100: 72, 80: 12}),         # 1080p: last row of cells is 8x10
])
def test_cells_partition_frame(gh, gw, cells, sizes):
    """Non-overlapping 10x10 cells anchored at the origin, truncated at the
    frame edge (ledger 'deployed spatial grid cell')."""
    g = O.Geometry(gh, gw, 3, 21)
    assert g.n_cells == cells
    got = {}
    for c in range(g.n_cells):
        got[g.cell_size(c)] = got.get(g.cell_size(c), 0) + 1
    assert got == sizes
    assert sum(g.cell_size(c) for c in range(g.n_cells)) == g.T
    # every token belongs to exactly the cell whose box contains it
    t = np.arange(g.T)
    _, y, x = g.split_token(t)
    cid = g.cell_of(y, x)
    for c in range(g.n_cells):
        y0, y1, x0, x1 = g.cell_box(c)
        inside = (y >= y0) & (y < y1) & (x >= x0) & (x < x1)
        assert np.array_equal(inside, cid == c)


def test_free_parameters_match_pages():
    fx = json.load(open(os.path.join(GOLDEN, "free_parameters.json")))
    p = O.ClassifyParams()
    for key in ("theta_sink", "theta_dummy", "theta_spatial", "theta_score", "gamma", "percentile", "radius"):
        assert getattr(p, key) == fx[key], key
    g = O.Geometry(45, 80, 3, 21)
    assert (g.cell_h, g.cell_w) == (fx["cell_h"], fx["cell_w"])


# ----------------------------------------------------------------------------- key sets
@pytest.mark.parametrize("pathway", [O.SINK, O.DUMMY, O.SPATIAL, O.GLOBAL, O.SLIDING])
@pytest.mark.parametrize("geom", [TINY, O.Geometry(13, 23, 2, 6), O.Geometry(9, 7, 1, 3, 4, 3)])
def test_keyset_mask_equals_keylist(pathway, geom):
    mask = O.key_mask(geom, pathway)
    for i in range(geom.Nq):
        assert np.array_equal(np.flatnonzero(mask[i]), np.sort(O.key_list(geom, pathway, i))), i


def test_keyset_mask_rows_subset():
    g = O.Geometry(13, 23, 2, 6)
    rows = np.array([5, 0, 597, 300, 1])
    for p in (O.SINK, O.DUMMY, O.SPATIAL, O.GLOBAL, O.SLIDING):
        assert np.array_equal(O.key_mask(g, p, rows=rows), O.key_mask(g, p)[rows])


def test_keyset_brute_force_tiny():
    """Brute force over (frame, y, x) on the tiny grid, straight from the
    archetype descriptions."""
    g = TINY
    for i in range(g.Nq):
        qy, qx = divmod(i, g.grid_w)
        sets = {p: set() for p in (O.SINK, O.DUMMY, O.SPATIAL, O.GLOBAL)}
        for f in range(g.window_frames):
            for y in range(g.grid_h):
                for x in range(g.grid_w):
                    t = f * g.T + y * g.grid_w + x
                    sets[O.GLOBAL].add(t)
                    if f == 0:
                        sets[O.SINK].add(t)
                    if f == g.window_frames - 1:
                        sets[O.DUMMY].add(t)
                    if y // 10 == qy // 10 and x // 10 == qx // 10:
                        sets[O.SPATIAL].add(t)
        for p, s in sets.items():
            assert set(O.key_list(g, p, i).tolist()) == s
    # the spatial set of a query in the narrow border cell: x in {10, 11}, every y, every frame
    assert len(O.key_list(g, O.SPATIAL, 11)) == 4 * 8 * 2
    assert len(O.key_list(g, O.SPATIAL, 0)) == 4 * 8 * 10


def test_keyset_sizes_closed_form():
    for g in (TINY, O.Geometry(45, 80, 3, 21), O.Geometry(30, 52, 3, 21)):
        for p in (O.SINK, O.DUMMY, O.SPATIAL, O.GLOBAL):
            if g.Nq * g.Nk > 5e7:
                continue
            assert O.keyset_sizes(g, p) == int(O.key_mask(g, p).sum())
    g = O.Geometry(45, 80, 3, 21)
    assert O.keyset_sizes(g, O.GLOBAL) == 10800 * 75600
    assert O.keyset_sizes(g, O.SINK) == 10800 * 10800
    assert O.keyset_sizes(g, O.SPATIAL) == 3 * 21 * (32 * 100 * 100 + 8 * 50 * 50)


# ----------------------------------------------------------------------------- attention
@pytest.mark.parametrize("pathway", [O.SINK, O.DUMMY, O.SPATIAL, O.GLOBAL, O.SLIDING])
def test_attention_matches_torch_sdpa_f64(pathway):
    """Library routine (torch SDPA, float64, CPU, explicit boolean mask)."""
    g = O.Geometry(9, 13, 2, 6, 4, 5)
    d = 16
    q, k, v = rnd((g.Nq, d), 1), rnd((g.Nk, d), 2), rnd((g.Nk, 24), 3)
    s = O.default_scale(d)
    got = O.attend_head(q, k, v, pathway, g, radius=1)
    ref = sdpa_f64(q, k, v, O.key_mask(g, pathway, radius=1), s)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("pathway", [O.SINK, O.DUMMY, O.SPATIAL, O.GLOBAL])
def test_attention_two_formulations_agree(pathway):
    g = TINY
    d = 64
    q, k, v = rnd((g.Nq, d), 4), rnd((g.Nk, d), 5), rnd((g.Nk, d), 6)
    s = O.default_scale(d)
    a = O.attention_masked(q, k, v, O.key_mask(g, pathway), s)
    b = O.attention_keylist(q, k, v, [(i, O.key_list(g, pathway, i)) for i in range(g.Nq)], s)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_scale_is_inverse_sqrt_d():
    assert O.default_scale(128) == 1 / math.sqrt(128)
    g = TINY
    q, k, v = rnd((g.Nq, 64), 7), rnd((g.Nk, 64), 8), rnd((g.Nk, 64), 9)
    ref = sdpa_f64(q, k, v, np.ones((g.Nq, g.Nk), bool), None)   # torch default scale
    np.testing.assert_allclose(O.attend_head(q, k, v, O.GLOBAL, g), ref, atol=1e-12)


@pytest.mark.parametrize("pathway", [O.SINK, O.DUMMY, O.SPATIAL, O.GLOBAL])
def test_constant_values_reproduced_exactly(pathway):
    """Softmax weights sum to one: if every value row is v, the output is v."""
    g = O.Geometry(12, 21, 2, 6)
    q, k = rnd((g.Nq, 32), 10), rnd((g.Nk, 32), 11) * 3
    vrow = rnd((1, 32), 12)
    out = O.attend_head(q, k, np.repeat(vrow, g.Nk, 0), pathway, g)
    np.testing.assert_allclose(out, np.repeat(vrow, g.Nq, 0), rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("pathway", [O.SINK, O.DUMMY, O.SPATIAL, O.GLOBAL])
def test_zero_keys_give_mean_of_keyset(pathway):
    """K = 0 -> uniform weights -> output is the plain mean of V over S(i)."""
    g = O.Geometry(11, 23, 2, 6)
    q, v = rnd((g.Nq, 8), 13), rnd((g.Nk, 8), 14)
    out = O.attend_head(q, np.zeros((g.Nk, 8)), v, pathway, g)
    for i in range(0, g.Nq, 7):
        np.testing.assert_allclose(out[i], v[O.key_list(g, pathway, i)].mean(0), atol=1e-13)


def test_identity_values_expose_weights():
    """V = identity: output row i is the weight vector, >= 0, sums to 1, zero
    outside S(i), and proportional to exp(s q.k) inside."""
    g = TINY
    q, k = rnd((g.Nq, 64), 15), rnd((g.Nk, 64), 16)
    for p in (O.SINK, O.DUMMY, O.SPATIAL, O.GLOBAL):
        P = O.attend_head(q, k, np.eye(g.Nk), p, g)
        m = O.key_mask(g, p)
        assert np.all(P >= 0) and np.all(P[~m] == 0)
        np.testing.assert_allclose(P.sum(1), 1.0, atol=1e-13)
        i = 5
        keys = O.key_list(g, p, i)
        lg = (k[keys] @ q[i]) / 8.0
        ratio = P[i, keys] / np.exp(lg - lg.max())
        np.testing.assert_allclose(ratio / ratio[0], 1.0, rtol=1e-12)


def test_global_is_full_attention_and_routing():
    g = O.Geometry(10, 14, 2, 6)
    H, d = 4, 16
    q, k, v = rnd((H, g.Nq, d), 17), rnd((H, g.Nk, d), 18), rnd((H, g.Nk, d), 19)
    labels = np.array([O.GLOBAL, O.SPATIAL, O.SINK, O.DUMMY])
    out = O.routed_attention(q, k, v, labels, g)
    full = np.ones((g.Nq, g.Nk), bool)
    np.testing.assert_allclose(out[0], sdpa_f64(q[0], k[0], v[0], full, None), atol=1e-12)
    for h, p in enumerate(labels):
        np.testing.assert_allclose(out[h], sdpa_f64(q[h], k[h], v[h], O.key_mask(g, p), 0.25), atol=1e-12)
    # explicit sink block equals frames [0,B) at first fill
    ks, vs = k[:, :g.Nq], v[:, :g.Nq]
    out2 = O.routed_attention(q, k, v, labels, g, k_sink=ks, v_sink=vs)
    np.testing.assert_allclose(out2, out, atol=1e-13)


def test_spatial_with_cell_covering_frame_is_global():
    g_cell = O.Geometry(8, 12, 1, 4, cell_h=8, cell_w=12)
    g_big = O.Geometry(8, 12, 1, 4, cell_h=50, cell_w=50)
    q, k, v = rnd((96, 64), 20), rnd((384, 64), 21), rnd((384, 64), 22)
    ref = O.attend_head(q, k, v, O.GLOBAL, g_cell)
    np.testing.assert_allclose(O.attend_head(q, k, v, O.SPATIAL, g_cell), ref, atol=1e-13)
    np.testing.assert_allclose(O.attend_head(q, k, v, O.SPATIAL, g_big), ref, atol=1e-13)


def test_one_block_window_collapses_pathways():
    g = O.Geometry(7, 9, 2, 2)     # W = B
    q, k, v = rnd((g.Nq, 16), 23), rnd((g.Nk, 16), 24), rnd((g.Nk, 16), 25)
    ref = O.attend_head(q, k, v, O.GLOBAL, g)
    for p in (O.SINK, O.DUMMY):
        np.testing.assert_allclose(O.attend_head(q, k, v, p, g), ref, atol=1e-13)


def test_key_permutation_invariance():
    """Reordering keys (with their values) leaves Global unchanged, and
    reordering whole frames leaves Spatial unchanged: the cache may store keys
    in ring or cell-major order."""
    g = O.Geometry(12, 15, 2, 6)
    q, k, v = rnd((g.Nq, 16), 26), rnd((g.Nk, 16), 27), rnd((g.Nk, 16), 28)
    perm = np.random.default_rng(0).permutation(g.Nk)
    np.testing.assert_allclose(O.attend_head(q, k[perm], v[perm], O.GLOBAL, g),
                               O.attend_head(q, k, v, O.GLOBAL, g), atol=1e-13)
    fperm = np.array([3, 0, 5, 1, 2, 4])
    tok = (fperm[:, None] * g.T + np.arange(g.T)[None]).ravel()
    np.testing.assert_allclose(O.attend_head(q, k[tok], v[tok], O.SPATIAL, g),
                               O.attend_head(q, k, v, O.SPATIAL, g), atol=1e-13)


# ----------------------------------------------------------------------------- classifier
def test_cosine_properties():
    a = rnd((50, 16), 29)
    np.testing.assert_allclose(O.cosine_rows(a, a), 1.0, atol=1e-15)
    np.testing.assert_allclose(O.cosine_rows(a, 3.5 * a), 1.0, atol=1e-15)
    np.testing.assert_allclose(O.cosine_rows(a, -a), -1.0, atol=1e-15)
    b = rnd((50, 16), 30)
    c = O.cosine_rows(a, b)
    assert np.all(np.abs(c) <= 1)
    ref = torch.nn.functional.cosine_similarity(torch.from_numpy(a), torch.from_numpy(b), dim=1).numpy()
    np.testing.assert_allclose(c, ref, atol=1e-14)
    e = np.zeros((2, 4)); e[0, 0] = 1; e[1, 1] = 1
    f = np.zeros((2, 4)); f[0, 1] = 1
    np.testing.assert_array_equal(O.cosine_rows(e, f), [0.0, 0.0])   # orthogonal; zero row -> 0


@pytest.mark.parametrize("n", [1, 2, 7, 100, 10800])
@pytest.mark.parametrize("p", [0.0, 5.0, 37.5, 50.0, 100.0])
def test_percentile_matches_numpy(n, p):
    x = rnd(n, n)
    assert O.percentile_linear(x, p) == pytest.approx(float(np.percentile(x, p)), abs=1e-15)


def test_percentile_hand_values():
    x = np.array([5.0, 1.0, 4.0, 2.0, 3.0])          # sorted 1..5, rank 0.05*4 = 0.2
    assert O.percentile_linear(x, 5) == pytest.approx(1.2)
    assert O.percentile_linear(np.arange(21.0), 5) == pytest.approx(1.0)


def test_head_scores_closed_form():
    of = rnd((40, 8), 31)
    diag, cos, mse = O.head_scores(of, 2 * of, -of, of + 0.1)
    assert diag[0] == pytest.approx(1.0) and diag[1] == pytest.approx(-1.0)
    assert mse == pytest.approx(0.01, rel=1e-12)
    expected_p5 = float(np.percentile(O.cosine_rows(of, of + 0.1), 5))
    assert diag[3] == pytest.approx(expected_p5 - 5 * 0.01, abs=1e-14)
    assert diag[2] == pytest.approx(O.cosine_rows(of, of + 0.1).mean(), abs=1e-15)
    d2, _, m2 = O.head_scores(of, of, of, of)   # a head equal to its proxy scores 1
    np.testing.assert_allclose(d2, [1, 1, 1, 1], atol=1e-15)
    assert m2 == 0


@pytest.mark.parametrize("diag,rule,label", [
    ([0.10, 0.20, 0.30, 0.0], 0, O.GLOBAL),
    ([0.96, 0.20, 0.30, 0.0], 0, O.SINK),
    ([0.20, 0.951, 0.30, 0.0], 0, O.DUMMY),
    ([0.20, 0.30, 0.97, 0.80], 0, O.SPATIAL),
    ([0.20, 0.30, 0.97, 0.70], 0, O.GLOBAL),      # Spatial needs the score gate too
    ([0.20, 0.30, 0.90, 0.90], 0, O.GLOBAL),      # ... and the cosine gate
    ([0.96, 0.98, 0.30, 0.0], 0, O.DUMMY),        # argmax among cleared
    ([0.96, 0.98, 0.30, 0.0], 1, O.SINK),         # first cleared
    ([0.96, 0.97, 0.99, 0.80], 0, O.SPATIAL),
    ([0.96, 0.97, 0.99, 0.80], 1, O.SINK),
    ([0.97, 0.97, 0.97, 0.90], 0, O.SINK),        # ties resolve Sink < Dummy < Spatial
    ([0.50, 0.97, 0.97, 0.90], 0, O.DUMMY),
    ([0.95, 0.0, 0.0, 0.0], 0, O.SINK),           # threshold is inclusive
    ([0.0, 0.0, 0.95, 0.755], 0, O.SPATIAL),
])
def test_rule_table(diag, rule, label):
    assert O.decide_label(diag, O.ClassifyParams(rule=rule)) == label


# decision_margin: hand-built diagnostics, each row built so that one gap is
# the smallest; the expected value is that gap, worked out by hand.
@pytest.mark.parametrize("diag,rule,margin", [
    ([0.10, 0.20, 0.30, 0.00], 0, 0.65),    # every proxy far below: the Spatial cosine gap (0.95 - 0.30)
    ([0.96, 0.20, 0.30, 0.00], 0, 0.01),    # the Sink threshold gap
    ([0.20, 0.93, 0.30, 0.00], 0, 0.02),    # the Dummy threshold gap, from below
    ([0.20, 0.30, 0.97, 0.80], 0, 0.02),    # the Spatial cosine gap, from above
    ([0.20, 0.30, 0.99, 0.76], 0, 0.005),   # the S_sc gap, from above
    ([0.20, 0.30, 0.99, 0.745], 0, 0.01),   # the S_sc gap, from below (Spatial does not clear)
    ([0.99, 0.98, 0.30, 0.00], 0, 0.01),    # rule 0: Sink and Dummy both clear, top-two gap
    ([0.99, 0.98, 0.30, 0.00], 1, 0.03),    # rule 1 ignores the top-two gap: Dummy threshold gap
    ([0.99, 0.30, 0.995, 0.90], 0, 0.005),  # rule 0: Sink and Spatial clear, top-two gap
    ([0.99, 0.30, 0.995, 0.90], 1, 0.04),   # rule 1: Sink threshold gap
    ([0.30, 0.985, 0.999, 0.90], 0, 0.014), # rule 0: Dummy and Spatial clear, top-two gap
    ([0.99, 0.30, 0.999, 0.70], 0, 0.04),   # Spatial fails its score gate: no top-two gap with it
    ([0.999, 0.99, 0.98, 0.90], 0, 0.009),  # three cleared: the top two decide (0.999 - 0.99)
    ([0.97, 0.97, 0.30, 0.00], 0, 0.0),     # an exact tie between cleared proxies
    ([0.95, 0.10, 0.10, 0.10], 0, 0.0),     # a cosine exactly at its (inclusive) threshold
])
def test_decision_margin_table(diag, rule, margin):
    assert O.decision_margin(diag, O.ClassifyParams(rule=rule)) == pytest.approx(margin, abs=1e-12)


def test_decision_margin_custom_thresholds():
    p = O.ClassifyParams(theta_sink=0.5, theta_dummy=0.6, theta_spatial=0.7, theta_score=0.2)
    assert O.decision_margin([0.55, 0.0, 0.0, 0.0], p) == pytest.approx(0.05)
    assert O.decision_margin([0.0, 0.61, 0.0, 0.0], p) == pytest.approx(0.01)
    assert O.decision_margin([0.0, 0.0, 0.0, 0.23], p) == pytest.approx(0.03)


def _margin_holds(margin_fn, n=400, seed=41):
    """Brute force: for diagnostics drawn near the thresholds, shifting every
    component by any of -eps, 0, +eps with eps just under margin/2 never
    changes the label (the guarantee decision_margin states)."""
    rng = np.random.default_rng(seed)
    shifts = np.array(np.meshgrid(*[[-1.0, 0.0, 1.0]] * 4)).reshape(4, -1).T
    for i in range(n):
        rule = i % 2
        p = O.ClassifyParams(rule=rule)
        diag = np.array([0.95, 0.95, 0.95, 0.755]) + rng.uniform(-0.05, 0.05, 4)
        m = margin_fn(diag, p)
        eps = 0.499 * m
        base = O.decide_label(diag, p)
        for s in shifts:
            if O.decide_label(diag + eps * s, p) != base:
                return False
    return True


def test_decision_margin_brute_force():
    assert _margin_holds(O.decision_margin)


def test_decision_margin_pins_catch_mistakes():
    """Each plausible mistake in decision_margin fails a pin above."""
    def no_score_gap(diag, p=O.ClassifyParams()):
        c = [float(x) for x in diag]
        return min(abs(c[0] - p.theta_sink), abs(c[1] - p.theta_dummy), abs(c[2] - p.theta_spatial))

    def no_top_two(diag, p=O.ClassifyParams()):
        return O.decision_margin(diag, O.ClassifyParams(rule=1))

    assert not _margin_holds(no_score_gap)     # a missing gap lets the label flip inside the margin
    assert not _margin_holds(no_top_two)

    def shrunk(diag, p=O.ClassifyParams()):
        return 0.5 * O.decision_margin(diag, p)
    assert shrunk([0.96, 0.20, 0.30, 0.00]) != pytest.approx(0.01)   # a shrunk margin fails the table


def test_one_block_window_classifies_sink():
    """W = B: every proxy equals the full output, cosines are 1, rule picks Sink."""
    g = O.Geometry(7, 9, 2, 2, 4, 4)
    q, k, v = rnd((g.Nq, 16), 32), rnd((g.Nk, 16), 33), rnd((g.Nk, 16), 34)
    for rule in (0, 1):
        lab, diag, _, mse = O.classify_head(q, k, v, g, O.ClassifyParams(rule=rule))
        assert lab == O.SINK
        np.testing.assert_allclose(diag[:2], [1, 1], atol=1e-14)


def test_planted_structure_is_recovered():
    """Planted Sink / Dummy / Spatial / none heads (reduced 720p-like shape)
    classify as planted, with wide margins.  A sanity pin of the classifier
    arithmetic end to end."""
    wl = W.small(W.WORKLOADS["classifier720p"], grid_h=20, grid_w=30, heads=12, window_frames=9)
    data = W.window(wl, seed=2)
    g = O.Geometry(wl.grid_h, wl.grid_w, wl.block_frames, wl.window_frames)
    q, k, v = (W.as_float(data[n], wl) for n in ("q", "k", "v"))
    labels, diag = O.classify(q, k, v, g)
    np.testing.assert_array_equal(labels, data["labels"])
    assert set(data["labels"].tolist()) == {0, 1, 2, 3}
    for h in range(wl.heads):
        assert O.decision_margin(diag[h]) > 0.03


def test_sliding_proxy_variant():
    """r = 2 sliding box: |S(i)| = frames * (clipped 5) * (clipped 5)."""
    g = O.Geometry(9, 11, 1, 3)
    for i in (0, 1, 2, 50, 98):
        y, x = divmod(i, 11)
        ny = min(8, y + 2) - max(0, y - 2) + 1
        nx = min(10, x + 2) - max(0, x - 2) + 1
        assert O.key_list(g, O.SLIDING, i).size == 3 * ny * nx


# ----------------------------------------------------------------------------- cache model
def test_cache_model_ring_and_cells():
    """Brute-force replay: decode every buffer row back to (block, token) with
    arithmetic written here, independently of the model's construction."""
    g = O.Geometry(13, 23, 2, 6)          # 3 block slots, 6 cells of uneven size
    labels = np.array([O.SPATIAL, O.GLOBAL, O.SINK, O.DUMMY, O.GLOBAL, O.SPATIAL])
    H, d, BT, nb = 6, 2, g.Nq, 3
    rng = np.random.default_rng(35)
    m = O.CacheModel(g, labels)
    history = []
    for step in range(9):
        kb = rng.integers(0, 2**15, (H, BT, d)).astype(np.uint16)
        vb = rng.integers(0, 2**15, (H, BT, d)).astype(np.uint16)
        mode = O.REPLACE_NEWEST if step in (3, 4, 8) else O.PUSH_BLOCK
        m.append(kb, vb, mode)
        if mode == O.PUSH_BLOCK:
            history.append((kb, vb))
        else:
            history[-1] = (kb, vb)
        n = len(history)
        # logical window: last nb blocks in order
        wk, _ = m.window()
        assert np.array_equal(wk, np.concatenate([h[0] for h in history[-nb:]], axis=1))
        gk, gvalid = m.expected_buffer(O.GLOBAL, "k")
        for row in np.flatnonzero(gvalid):
            slot, tok = divmod(row, BT)
            b = max(b for b in range(n) if b % nb == slot)
            for s, h in enumerate([1, 4]):
                assert np.array_equal(gk[s, row], history[b][0][h, tok])
        assert gvalid.sum() == min(n, nb) * BT
        sk, _ = m.expected_buffer(O.SINK, "v")
        assert np.array_equal(sk[0], history[0][1][2])
        dk, _ = m.expected_buffer(O.DUMMY, "k")
        assert np.array_equal(dk[0], history[-1][0][3])
        pk, pvalid = m.expected_buffer(O.SPATIAL, "k")
        assert pvalid.sum() == min(n, nb) * BT
        # decode spatial rows: walk cells in order, W frame slots each
        sizes = [g.cell_size(c) for c in range(g.n_cells)]
        starts = np.cumsum([0] + [g.window_frames * s for s in sizes])
        for row in np.flatnonzero(pvalid)[::5]:
            c = int(np.searchsorted(starts, row, side="right") - 1)
            fs, r = divmod(row - starts[c], sizes[c])
            y0, y1, x0, x1 = g.cell_box(c)
            yy, xx = y0 + r // (x1 - x0), x0 + r % (x1 - x0)
            slot, i = divmod(fs, g.block_frames)
            b = max(b for b in range(n) if b % nb == slot)
            tok = i * g.T + yy * g.grid_w + xx
            assert np.array_equal(pk[1, row], history[b][0][5, tok])


def test_cache_window_attention_after_slide():
    """After the window slides, routed attention over the model's window plus
    the kept sink block equals attention over explicitly assembled key sets."""
    g = O.Geometry(6, 11, 1, 3, 4, 4)
    labels = np.array([O.SINK, O.GLOBAL, O.SPATIAL, O.DUMMY])
    rng = np.random.default_rng(36)
    m = O.CacheModel(g, labels)
    blocks = [(rng.standard_normal((4, g.Nq, 8)), rng.standard_normal((4, g.Nq, 8))) for _ in range(5)]
    for kb, vb in blocks:
        m.append(kb, vb)
    q = rng.standard_normal((4, g.Nq, 8))
    wk, wv = m.window()
    out = O.routed_attention(q, wk, wv, labels, g, k_sink=m.sink_k, v_sink=m.sink_v)
    s = O.default_scale(8)
    full = np.ones((g.Nq, g.Nq), bool)
    np.testing.assert_allclose(out[0], sdpa_f64(q[0], blocks[0][0][0], blocks[0][1][0], full, s), atol=1e-12)
    kk = np.concatenate([b[0][1] for b in blocks[2:]])
    vv = np.concatenate([b[1][1] for b in blocks[2:]])
    np.testing.assert_allclose(out[1], sdpa_f64(q[1], kk, vv, np.ones((g.Nq, 3 * g.Nq), bool), s), atol=1e-12)
    np.testing.assert_allclose(out[3], sdpa_f64(q[3], blocks[4][0][3], blocks[4][1][3], full, s), atol=1e-12)


# ----------------------------------------------------------------------------- fp8 KV codes
def _torch_e4m3(x):
    """torch's float32 -> float8_e4m3fn conversion (round to nearest even)."""
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_decode_matches_torch_on_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = O.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref)) and np.isnan(got).sum() == 2   # 0x7F, 0xFF
    assert np.array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])
    # closed forms of the format: 1.0, the largest finite, the smallest normal and subnormal
    assert O.e4m3_decode(np.uint8(0x38)) == 1.0 and O.e4m3_decode(np.uint8(0x7E)) == 448.0
    assert O.e4m3_decode(np.uint8(0x08)) == 2.0 ** -6 and O.e4m3_decode(np.uint8(0x01)) == 2.0 ** -9


def test_e4m3_encode_round_trips_and_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    vals = O.e4m3_decode(codes)
    fin = ~np.isnan(vals)
    assert np.array_equal(O.e4m3_encode(vals[fin]), codes[fin])           # exact values (and -0) round-trip
    grid = np.unique(vals[fin])
    mids = (grid[:-1] + grid[1:]) / 2                                      # ties: round to even code
    rng = np.random.default_rng(7)
    x = np.concatenate([mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf),
                        rng.uniform(-448, 448, 20000), rng.standard_normal(20000),
                        rng.uniform(-2.0 ** -5, 2.0 ** -5, 5000)]).astype(np.float32)
    assert np.array_equal(O.e4m3_encode(x), _torch_e4m3(x))


def test_e4m3_encode_saturates_and_is_monotone():
    big = np.array([448.0, 449.0, 463.9, 464.0, 1e4, 3e38], np.float32)
    assert np.all(O.e4m3_encode(big) == 0x7E) and np.all(O.e4m3_encode(-big) == 0xFE)
    x = np.sort(np.random.default_rng(3).uniform(-600, 600, 50000)).astype(np.float32)
    assert np.all(np.diff(O.e4m3_decode(O.e4m3_encode(x))) >= 0)
    # round to nearest: the error is at most half a grid step of the value's binade
    y = x[np.abs(x) <= 448]
    err = np.abs(O.e4m3_decode(O.e4m3_encode(y)) - y)
    step = np.exp2(np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -6))) - 3)
    assert np.all(err <= step / 2 + 1e-12)
    with pytest.raises(ValueError):
        O.e4m3_encode(np.array([np.nan], np.float32))


def test_quantize_kv_scales():
    x = (np.random.default_rng(5).standard_normal((3, 50, 16)) * 3).astype(np.float32)
    assert np.array_equal(O.quantize_kv(x, 1.0), _torch_e4m3(x))
    assert np.array_equal(O.quantize_kv(x, 4.0), _torch_e4m3(x / 4))     # power of two: exact scaling
    c = O.quantize_kv(x, 0.3)
    assert np.array_equal(c, _torch_e4m3(x * (np.float32(1) / np.float32(0.3))))
    d = O.dequantize_kv(c, 0.3)
    assert np.all(np.abs(d - x) <= np.abs(x) * 2.0 ** -4 + 2.0 ** -10 * 0.3 + 1e-7)   # relative half-step


# ----------------------------------------------------------------------------- planted mistakes
def test_pins_catch_planted_mistakes(monkeypatch):
    """Plant plausible mistakes in the oracle and check a pin notices each."""
    g = O.Geometry(9, 13, 2, 6, 4, 5)
    q, k, v = rnd((g.Nq, 16), 1), rnd((g.Nk, 16), 2), rnd((g.Nk, 16), 3)
    ref = sdpa_f64(q, k, v, O.key_mask(g, O.SPATIAL), 0.25)
    # wrong softmax scale
    monkeypatch.setattr(O, "default_scale", lambda d: 1.0 / d)
    assert not np.allclose(O.attend_head(q, k, v, O.SPATIAL, g), ref, atol=1e-6)
    monkeypatch.undo()
    # wrong cell anchoring (cells of width 5 instead of 10 along x)
    g2 = O.Geometry(9, 13, 2, 6, 4, 4)
    assert not np.array_equal(O.key_mask(g2, O.SPATIAL), O.key_mask(g, O.SPATIAL))
    # transposed operand in the value product
    monkeypatch.setattr(O, "attention_masked",
                        lambda q_, k_, v_, m_, s_, rows=None: (np.ones((q_.shape[0], k_.shape[0])) @ v_) / k_.shape[0])
    assert not np.allclose(O.attend_head(q, k, v, O.SPATIAL, g), ref, atol=1e-6)
    monkeypatch.undo()
    # wrong percentile rank convention (nearest-rank instead of interpolation)
    x = rnd(10800, 4)
    s = np.sort(x)
    assert abs(s[int(0.05 * 10800)] - np.percentile(x, 5)) > 0 and \
        O.percentile_linear(x, 5) == pytest.approx(np.percentile(x, 5), abs=1e-15)
    # wrong sign of the MSE penalty would flip the closed form
    of = rnd((40, 8), 31)
    diag, _, _ = O.head_scores(of, of, of, of + 0.1)
    assert diag[3] < float(np.percentile(O.cosine_rows(of, of + 0.1), 5))
