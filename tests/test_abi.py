"""C ABI tests that need no GPU: the library loads, exports every function
declared in include/headcast.h, and rejects bad arguments before any launch
(host-only paths; device pointers here are never dereferenced)."""
import ctypes as C
import os
import re

import pytest

from head_routed_kv_amd import _native as N

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "headcast.h")
FAKE = 1 << 40          # 256-byte aligned, never dereferenced


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(hc_[a-z_]+)\s*\(", src)))


def cfg(**kw):
    base = dict(num_heads=4, head_dim=128, grid_h=8, grid_w=12, block_frames=1, window_frames=4, cell_h=10,
                cell_w=10, dtype=N.HC_BF16, softmax_scale=0.0)
    base.update(kw)
    return N.hc_config(**base)


def status(fn, *args):
    return fn(*args)


def test_every_declared_symbol_is_exported():
    L = N.lib()
    names = declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(N.EXPORTS)


def test_status_strings():
    L = N.lib()
    for s, name in [(0, b"HC_OK"), (-1, b"HC_ERR_INVALID_ARG"), (-6, b"HC_ERR_STATE"), (-8, b"HC_ERR_UNSUPPORTED")]:
        assert L.hc_status_string(s) == name


@pytest.mark.parametrize("kw,err", [
    (dict(dtype=7), N.HC_ERR_DTYPE),
    (dict(num_heads=0), N.HC_ERR_SHAPE),
    (dict(num_heads=129), N.HC_ERR_SHAPE),
    (dict(head_dim=96), N.HC_ERR_SHAPE),
    (dict(window_frames=5, block_frames=2), N.HC_ERR_SHAPE),
    (dict(grid_h=0), N.HC_ERR_SHAPE),
    (dict(cell_w=0), N.HC_ERR_SHAPE),
    (dict(softmax_scale=-1.0), N.HC_ERR_INVALID_ARG),
    (dict(kv_format=2), N.HC_ERR_INVALID_ARG),
    (dict(kv_format=N.HC_KV_FP8_E4M3, dtype=N.HC_FP32), N.HC_ERR_DTYPE),
    (dict(kv_format=N.HC_KV_FP8_E4M3, k_scale=-1.0), N.HC_ERR_INVALID_ARG),
    (dict(kv_format=N.HC_KV_FP8_E4M3, v_scale=float("inf")), N.HC_ERR_INVALID_ARG),
])
def test_bad_configs(kw, err):
    c = cfg(**kw)
    assert N.lib().hc_validate_config(C.byref(c)) == err
    assert N.hc_last_error_message()


def test_cache_bytes_and_layout():
    c = cfg()
    labels = [3, 2, 0, 1]
    n = N.hc_cache_bytes(c, labels)
    T, d = 96, 128
    assert n >= 2 * 2 * (2 * 4 * T * d) + 2 * 2 * (2 * T * d)
    h = N.hc_cache_create(c, labels, FAKE, n)
    lay = N.hc_cache_get_layout(h)
    assert lay.total_bytes == n
    assert (lay.n_global, lay.n_sink, lay.n_dummy, lay.n_spatial) == (1, 1, 1, 1)
    offs = [lay.off_global_k, lay.off_global_v, lay.off_sink_k, lay.off_sink_v, lay.off_dummy_k, lay.off_dummy_v,
            lay.off_spatial_k, lay.off_spatial_v]
    assert all(o % 256 == 0 for o in offs)
    assert lay.off_global_v - lay.off_global_k >= 4 * T * d * 2
    assert lay.blocks_appended == 0
    N.hc_cache_destroy(h)


def test_fp8_cache_layout_halves_kv_bytes():
    """An fp8 K/V cache stores one byte per element; the scales are ignored
    unless kv_format asks for fp8, and 0 selects 1."""
    labels = [3, 2, 0, 1]
    c16 = cfg(k_scale=-5.0)                     # ignored: kv_format is HC_KV_SAME
    assert N.lib().hc_validate_config(C.byref(c16)) == N.HC_OK
    c8 = cfg(kv_format=N.HC_KV_FP8_E4M3)
    assert N.lib().hc_validate_config(C.byref(c8)) == N.HC_OK
    h16 = N.hc_cache_create(c16, labels, FAKE, N.hc_cache_bytes(c16, labels))
    h8 = N.hc_cache_create(c8, labels, FAKE, N.hc_cache_bytes(c8, labels))
    a, b = N.hc_cache_get_layout(h16), N.hc_cache_get_layout(h8)
    T, d = 96, 128
    assert a.off_global_v - a.off_global_k == 4 * T * d * 2
    assert b.off_global_v - b.off_global_k == 4 * T * d
    assert b.off_sink_v - b.off_sink_k == T * d
    N.hc_cache_destroy(h16)
    N.hc_cache_destroy(h8)
    # the 720p routed layer: the K/V region (everything before the split
    # scratch) halves exactly; the scratch (fp32 partials of the key splits,
    # counters) follows each cache's own split plan
    c720 = dict(num_heads=12, head_dim=128, grid_h=45, grid_w=80, block_frames=3, window_frames=21)
    lab720 = [2, 0, 3, 1, 3, 2, 2, 3, 2, 2, 0, 1]
    lays = []
    for kvf in (N.HC_KV_SAME, N.HC_KV_FP8_E4M3):
        c = cfg(**c720, kv_format=kvf)
        h = N.hc_cache_create(c, lab720, FAKE, N.hc_cache_bytes(c, lab720))
        lays.append(N.hc_cache_get_layout(h))
        N.hc_cache_destroy(h)
    assert lays[1].off_scratch * 2 == lays[0].off_scratch == 331_776_000
    assert lays[0].scratch_bytes > 0 and lays[1].scratch_bytes > 0


def test_cache_create_errors():
    c = cfg()
    L = N.lib()
    labs = (C.c_int8 * 4)(3, 2, 0, 1)
    out = C.c_void_p()
    n = N.hc_cache_bytes(c, [3, 2, 0, 1])
    assert L.hc_cache_create(C.byref(c), labs, C.c_void_p(FAKE + 16), n, C.byref(out)) == N.HC_ERR_ALIGN
    assert L.hc_cache_create(C.byref(c), labs, C.c_void_p(FAKE), n - 1, C.byref(out)) == N.HC_ERR_WORKSPACE
    assert L.hc_cache_create(C.byref(c), labs, None, n, C.byref(out)) == N.HC_ERR_INVALID_ARG
    bad = (C.c_int8 * 4)(3, 2, 4, 1)
    assert L.hc_cache_create(C.byref(c), bad, C.c_void_p(FAKE), n, C.byref(out)) == N.HC_ERR_INVALID_ARG
    assert "label" in N.hc_last_error_message()
    assert L.hc_cache_bytes(C.byref(c), None, C.byref(C.c_size_t())) == N.HC_ERR_INVALID_ARG


def test_misuse_is_rejected_before_launch():
    c = cfg()
    n = N.hc_cache_bytes(c, [3, 2, 0, 1])
    h = N.hc_cache_create(c, [3, 2, 0, 1], FAKE, n)
    L = N.lib()
    q = N.hc_tensor(FAKE, 96 * 128, 128)
    o = N.hc_out_tensor(FAKE + (1 << 30), 96 * 128, 128)
    assert L.hc_attend(h, q, o, None) == N.HC_ERR_STATE                 # nothing appended yet
    kv = N.hc_tensor(FAKE, 96 * 128, 128)
    assert L.hc_cache_append(h, kv, kv, N.HC_REPLACE_NEWEST, None) == N.HC_ERR_STATE
    assert L.hc_cache_append(h, kv, kv, 5, None) == N.HC_ERR_INVALID_ARG
    assert L.hc_cache_append(h, N.hc_tensor(FAKE + 8, 96 * 128, 128), kv, 0, None) == N.HC_ERR_ALIGN
    assert L.hc_cache_append(h, N.hc_tensor(FAKE, 96 * 128, 100), kv, 0, None) == N.HC_ERR_SHAPE
    assert L.hc_cache_append(h, N.hc_tensor(None, 96 * 128, 128), kv, 0, None) == N.HC_ERR_INVALID_ARG
    assert L.hc_cache_append(h, N.hc_tensor(FAKE, 96 * 128 + 4, 128), kv, 0, None) == N.HC_ERR_ALIGN
    assert L.hc_attend(h, q, N.hc_out_tensor(FAKE, 96 * 128, 128), None) == N.HC_ERR_INVALID_ARG  # aliases q
    N.hc_cache_destroy(h)
    assert L.hc_cache_destroy(None) == N.HC_ERR_INVALID_ARG


def test_launch_failure_is_reported_as_hip_error():
    """A valid call whose kernel launch fails returns HC_ERR_HIP and names the
    step.  Forced here by the absence of a GPU, so it runs only on a host
    without one (elsewhere the call would really launch on a fake pointer)."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible: this call would launch")
    c = cfg()
    h = N.hc_cache_create(c, [0, 1, 2, 3], FAKE, N.hc_cache_bytes(c, [0, 1, 2, 3]))
    kv = N.hc_tensor(FAKE, 96 * 128, 128)
    assert N.lib().hc_cache_append(h, kv, kv, N.HC_PUSH_BLOCK, None) == N.HC_ERR_HIP
    assert b"append" in N.lib().hc_last_error_message()
    N.hc_cache_destroy(h)


def test_classify_argument_checks():
    c = cfg()
    L = N.lib()
    p = N.hc_default_classify_params()
    assert (round(p.theta_sink, 6), round(p.theta_score, 6), p.gamma, p.percentile, p.rule, p.radius) == \
        (0.95, 0.755, 5.0, 5.0, 0, 2)
    need = N.hc_classify_workspace_bytes(c)
    assert need >= 4 * 4 * 96 * 128 * 4
    t = N.hc_tensor(FAKE, 384 * 128, 128)
    args = lambda prm, ws, wsb: (C.byref(c), C.byref(prm), t, t, t, C.c_void_p(ws), wsb, C.c_void_p(FAKE),
                                 C.c_void_p(FAKE), None)
    assert L.hc_classify(*args(p, FAKE, need - 1)) == N.HC_ERR_WORKSPACE
    assert L.hc_classify(*args(p, FAKE + 16, need)) == N.HC_ERR_ALIGN
    p2 = N.hc_default_classify_params()
    p2.spatial_proxy = 2
    assert L.hc_classify(*args(p2, FAKE, need)) == N.HC_ERR_INVALID_ARG
    for r in (-1, 9):   # the sliding-box proxy takes radius 0..8
        p2 = N.hc_default_classify_params()
        p2.spatial_proxy, p2.radius = 1, r
        assert L.hc_classify(*args(p2, FAKE, need)) == N.HC_ERR_INVALID_ARG
    p3 = N.hc_default_classify_params()
    p3.rule = 3
    assert L.hc_classify(*args(p3, FAKE, need)) == N.HC_ERR_INVALID_ARG
    p4 = N.hc_default_classify_params()
    p4.percentile = 101
    assert L.hc_classify(*args(p4, FAKE, need)) == N.HC_ERR_INVALID_ARG


def test_static_classifier_rejects_layers_beyond_its_scratch():
    """hc_classify_static checks its arguments like hc_classify and rejects a
    layer whose workspace would not fit the static scratch, before touching
    the GPU."""
    L = N.lib()
    p = N.hc_default_classify_params()
    big = cfg(num_heads=40, grid_h=45, grid_w=80, block_frames=3, window_frames=21)   # 40-head 720p layer
    assert N.hc_classify_workspace_bytes(big) > N.HC_STATIC_SCRATCH_BYTES
    t = N.hc_tensor(FAKE, 75600 * 128, 128)
    assert L.hc_classify_static(C.byref(big), C.byref(p), t, t, t, C.c_void_p(FAKE), C.c_void_p(FAKE), None) == \
        N.HC_ERR_WORKSPACE
    assert "static scratch" in N.hc_last_error_message()
    small = cfg()
    assert N.hc_classify_workspace_bytes(small) <= N.HC_STATIC_SCRATCH_BYTES
    t = N.hc_tensor(FAKE, 384 * 128, 128)
    p3 = N.hc_default_classify_params()
    p3.rule = 3
    assert L.hc_classify_static(C.byref(small), C.byref(p3), t, t, t, C.c_void_p(FAKE), C.c_void_p(FAKE), None) == \
        N.HC_ERR_INVALID_ARG
    assert L.hc_classify_static(C.byref(small), C.byref(p), t, t, t, None, C.c_void_p(FAKE), None) == \
        N.HC_ERR_INVALID_ARG
    # the header's figure and the binding's agree
    hdr = open(HEADER).read()
    assert re.search(r"#define HC_STATIC_SCRATCH_BYTES \(64u << 20\)", hdr)
    assert N.HC_STATIC_SCRATCH_BYTES == 64 << 20


def test_split_plan_for_benchmark_layers():
    """The host plans key-range splits for Global heads when their q tiles
    alone cannot fill the chip (720p: 3 Global heads x 43 q tiles)."""
    c = N.make_config(12, 128, 45, 80, 3, 21)
    labels = [2, 0, 3, 1, 3, 2, 2, 3, 2, 2, 0, 1]
    h = N.hc_cache_create(c, labels, FAKE, N.hc_cache_bytes(c, labels))
    lay = N.hc_cache_get_layout(h)
    assert lay.global_splits > 1 and lay.scratch_bytes > 0
    N.hc_cache_destroy(h)
    h = N.hc_cache_create(cfg(), [0, 1, 2, 3], FAKE, N.hc_cache_bytes(cfg(), [0, 1, 2, 3]))
    assert N.hc_cache_get_layout(h).global_splits == 1
    N.hc_cache_destroy(h)
    # two Sink heads alone: 2 x 43 q tiles; their key sets are split as well
    c = N.make_config(2, 128, 45, 80, 3, 21)
    h = N.hc_cache_create(c, [0, 0], FAKE, N.hc_cache_bytes(c, [0, 0]))
    lay = N.hc_cache_get_layout(h)
    assert lay.sink_splits > 1 and lay.global_splits == 1 and lay.scratch_bytes > 0
    N.hc_cache_destroy(h)
    # fp32 layers are never split
    c = N.make_config(2, 128, 45, 80, 3, 21, dtype=N.HC_FP32)
    h = N.hc_cache_create(c, [0, 3], FAKE, N.hc_cache_bytes(c, [0, 3]))
    lay = N.hc_cache_get_layout(h)
    assert (lay.global_splits, lay.sink_splits, lay.dummy_splits, lay.scratch_bytes) == (1, 1, 1, 0)
    N.hc_cache_destroy(h)


def test_split_plan_models_the_dispatch():
    """The split planner simulates hc_attend's persistent launch (one work
    group per compute unit, each XCD's 32 taking the units of its own list
    as they come free) with unit costs measured on MI355X.  On the benchmark
    layers it picks the counts that measured fastest there among 1-8 (or
    within 1% of it): 4 Global splits for the 720p routed layer (2 measured
    37% slower), 3 for the 480p routed layer, 4 for the 480p and 1080p
    Global heads alone, 8 for the 720p Global heads alone, and no split for
    the 1080p routed layer, which fills the GPU by itself."""
    from head_routed_kv_amd import workloads as W

    def plan(name, labels):
        wl = W.WORKLOADS[name]
        c = N.make_config(len(labels), 128, wl.grid_h, wl.grid_w, 3, 21)
        h = N.hc_cache_create(c, labels, FAKE, N.hc_cache_bytes(c, labels))
        lay = N.hc_cache_get_layout(h)
        N.hc_cache_destroy(h)
        return lay.global_splits, lay.sink_splits, lay.dummy_splits
    lab = {n: [int(x) for x in W.make_labels(W.WORKLOADS[n])] for n in ("480p", "720p", "1080p")}
    assert plan("720p", lab["720p"])[0] == 4
    assert plan("480p", lab["480p"])[0] == 3
    assert plan("480p", [3] * lab["480p"].count(3))[0] == 4
    assert plan("1080p", [3] * lab["1080p"].count(3))[0] == 4
    assert plan("720p", [3] * lab["720p"].count(3))[0] == 8
    assert plan("1080p", lab["1080p"]) == (1, 1, 1)


def test_binding_checks_tensors_against_the_config():
    """The torch conveniences refuse tensors the library would read out of
    bounds (too few tokens or heads), of the wrong dtype, or in host memory."""
    import torch
    import head_routed_kv_amd as hk
    c = hk.make_config(4, 64, 8, 12, 1, 4)          # B*T = 96 rows per block
    ok = torch.zeros(4, 96, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="shape"):
        hk.check_tensor(torch.zeros(4, 95, 64, dtype=torch.bfloat16), c, hk.block_rows(c), "k_block")
    with pytest.raises(ValueError, match="shape"):
        hk.check_tensor(torch.zeros(3, 96, 64, dtype=torch.bfloat16), c, 96, "k_block")
    with pytest.raises(ValueError, match="dtype"):
        hk.check_tensor(ok.float(), c, 96, "q_block")
    with pytest.raises(ValueError, match="device"):
        hk.check_tensor(ok, c, 96, "q_block")
    with pytest.raises(ValueError, match="contiguous channels"):
        hk.tensor_arg(torch.zeros(4, 64, 96, dtype=torch.bfloat16).transpose(1, 2))


def test_c_program_against_the_header_and_library(tmp_path):
    """tests/c/abi_host.c, compiled as C11 with gcc against include/headcast.h
    and linked to libheadcast.so, runs the host-only entry points and agrees
    with the Python binding."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    lib = os.path.join(ROOT, "head_routed_kv_amd", "libheadcast.so")   # the plain build, also under HEADCAST_LIB
    if not os.path.exists(lib):
        pytest.skip("libheadcast.so is not built")
    libdir = os.path.dirname(lib)
    exe = tmp_path / "abi_host"
    cmd = [gcc, "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(rocm, "include"), os.path.join(ROOT, "tests", "c", "abi_host.c"), "-o", str(exe),
           "-L", libdir, "-l:libheadcast.so", "-Wl,-rpath," + libdir]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True, timeout=60).stdout
    got = dict(line.split(" ", 1) for line in out.strip().splitlines())
    labels = [2, 0, 3, 1, 3, 2, 2, 3, 2, 2, 0, 1]
    c = N.make_config(12, 128, 45, 80, 3, 21)
    assert int(got["validate"]) == 0 and int(got["create"]) == 0 and int(got["destroy"]) == 0
    assert int(got["cache_bytes"]) == N.hc_cache_bytes(c, labels)
    h = N.hc_cache_create(c, labels, FAKE, N.hc_cache_bytes(c, labels))
    lay = N.hc_cache_get_layout(h)
    N.hc_cache_destroy(h)
    assert (int(got["n_global"]), int(got["n_spatial"]), int(got["n_sink"]), int(got["n_dummy"])) == (3, 5, 2, 2)
    assert int(got["global_splits"]) == lay.global_splits
    assert int(got["workspace"]) == N.hc_classify_workspace_bytes(c)
    assert float(got["theta_score"]) == pytest.approx(0.755) and float(got["gamma"]) == pytest.approx(5.0)
    code, name = got["bad"].split()
    assert int(code) != 0 and name.startswith("HC_ERR") and got["message_nonempty"] == "1"
