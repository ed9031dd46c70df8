"""ctypes binding of libheadcast.so.  Argument marshalling only: every
computation runs in the library's HIP kernels.  Function names match the C
declarations in include/headcast.h.  Tensors are passed as
(pointer, stride_head, stride_token) with strides in elements."""
from __future__ import annotations

import ctypes as C
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# HEADCAST_LIB selects another build of the same library (e.g. the host-ASan one).
LIB_PATH = os.environ.get("HEADCAST_LIB") or os.path.join(_PKG, "libheadcast.so")

HC_MAX_HEADS = 128
HC_OK, HC_ERR_INVALID_ARG, HC_ERR_SHAPE, HC_ERR_DTYPE, HC_ERR_ALIGN = 0, -1, -2, -3, -4
HC_ERR_WORKSPACE, HC_ERR_STATE, HC_ERR_HIP, HC_ERR_UNSUPPORTED = -5, -6, -7, -8
HC_SINK, HC_DUMMY, HC_SPATIAL, HC_GLOBAL = 0, 1, 2, 3
HC_BF16, HC_FP32 = 0, 1
HC_KV_SAME, HC_KV_FP8_E4M3 = 0, 1
HC_PUSH_BLOCK, HC_REPLACE_NEWEST = 0, 1


class hc_config(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("num_heads", "head_dim", "grid_h", "grid_w", "block_frames",
                                         "window_frames", "cell_h", "cell_w", "dtype")] + \
               [("softmax_scale", C.c_float), ("kv_format", C.c_int32), ("k_scale", C.c_float), ("v_scale", C.c_float)]


class hc_tensor(C.Structure):
    _fields_ = [("ptr", C.c_void_p), ("stride_head", C.c_int64), ("stride_token", C.c_int64)]


class hc_out_tensor(C.Structure):
    _fields_ = [("ptr", C.c_void_p), ("stride_head", C.c_int64), ("stride_token", C.c_int64)]


class hc_classify_params(C.Structure):
    _fields_ = [(n, C.c_float) for n in ("theta_sink", "theta_dummy", "theta_spatial", "theta_score", "gamma",
                                         "percentile")] + [(n, C.c_int32) for n in ("rule", "spatial_proxy", "radius")]


class hc_cache_layout(C.Structure):
    _fields_ = [(n, C.c_uint64) for n in ("total_bytes", "off_global_k", "off_global_v", "off_sink_k", "off_sink_v",
                                          "off_dummy_k", "off_dummy_v", "off_spatial_k", "off_spatial_v",
                                          "off_scratch", "scratch_bytes")] + \
               [(n, C.c_int32) for n in ("n_global", "n_sink", "n_dummy", "n_spatial", "blocks_appended",
                                         "global_splits", "sink_splits", "dummy_splits")] + \
               [("head_slot", C.c_int32 * HC_MAX_HEADS)]


EXPORTS = {
    "hc_default_classify_params": (None, [C.POINTER(hc_classify_params)]),
    "hc_validate_config": (C.c_int, [C.POINTER(hc_config)]),
    "hc_cache_bytes": (C.c_int, [C.POINTER(hc_config), C.c_void_p, C.POINTER(C.c_size_t)]),
    "hc_cache_create": (C.c_int, [C.POINTER(hc_config), C.c_void_p, C.c_void_p, C.c_size_t, C.POINTER(C.c_void_p)]),
    "hc_cache_destroy": (C.c_int, [C.c_void_p]),
    "hc_cache_get_layout": (C.c_int, [C.c_void_p, C.POINTER(hc_cache_layout)]),
    "hc_cache_append": (C.c_int, [C.c_void_p, hc_tensor, hc_tensor, C.c_int32, C.c_void_p]),
    "hc_attend": (C.c_int, [C.c_void_p, hc_tensor, hc_out_tensor, C.c_void_p]),
    "hc_classify_workspace_bytes": (C.c_int, [C.POINTER(hc_config), C.POINTER(C.c_size_t)]),
    "hc_classify": (C.c_int, [C.POINTER(hc_config), C.POINTER(hc_classify_params), hc_tensor, hc_tensor, hc_tensor,
                              C.c_void_p, C.c_size_t, C.c_void_p, C.c_void_p, C.c_void_p]),
    "hc_classify_static": (C.c_int, [C.POINTER(hc_config), C.POINTER(hc_classify_params), hc_tensor, hc_tensor,
                                     hc_tensor, C.c_void_p, C.c_void_p, C.c_void_p]),
    "hc_status_string": (C.c_char_p, [C.c_int]),
    "hc_last_error_message": (C.c_char_p, []),
}

_lib = None


class HeadcastError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


def _status_name(s):
    return {0: "HC_OK", -1: "HC_ERR_INVALID_ARG", -2: "HC_ERR_SHAPE", -3: "HC_ERR_DTYPE", -4: "HC_ERR_ALIGN",
            -5: "HC_ERR_WORKSPACE", -6: "HC_ERR_STATE", -7: "HC_ERR_HIP", -8: "HC_ERR_UNSUPPORTED"}.get(s, str(s))


def lib():
    """The loaded library.  Raises if it has not been built: there is no
    fallback implementation."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status):
    if status != HC_OK:
        raise HeadcastError(status, lib().hc_last_error_message().decode())


def make_config(num_heads, head_dim, grid_h, grid_w, block_frames, window_frames, cell_h=10, cell_w=10,
                dtype=HC_BF16, softmax_scale=0.0, kv_format=HC_KV_SAME, k_scale=0.0, v_scale=0.0):
    return hc_config(num_heads, head_dim, grid_h, grid_w, block_frames, window_frames, cell_h, cell_w, dtype,
                     softmax_scale, kv_format, k_scale, v_scale)


def _labels_buf(labels):
    arr = (C.c_int8 * len(labels))(*[int(x) for x in labels])
    return arr


def hc_default_classify_params():
    p = hc_classify_params()
    lib().hc_default_classify_params(C.byref(p))
    return p


def hc_validate_config(cfg):
    _check(lib().hc_validate_config(C.byref(cfg)))


def hc_cache_bytes(cfg, labels):
    n = C.c_size_t()
    _check(lib().hc_cache_bytes(C.byref(cfg), _labels_buf(labels), C.byref(n)))
    return n.value


def hc_cache_create(cfg, labels, device_ptr, nbytes):
    h = C.c_void_p()
    _check(lib().hc_cache_create(C.byref(cfg), _labels_buf(labels), C.c_void_p(device_ptr), nbytes, C.byref(h)))
    return h


def hc_cache_destroy(handle):
    _check(lib().hc_cache_destroy(handle))


def hc_cache_get_layout(handle):
    lay = hc_cache_layout()
    _check(lib().hc_cache_get_layout(handle, C.byref(lay)))
    return lay


def hc_cache_append(handle, k, v, mode, stream):
    _check(lib().hc_cache_append(handle, hc_tensor(*k), hc_tensor(*v), mode, C.c_void_p(stream)))


def hc_attend(handle, q, out, stream):
    _check(lib().hc_attend(handle, hc_tensor(*q), hc_out_tensor(*out), C.c_void_p(stream)))


def hc_classify_workspace_bytes(cfg):
    n = C.c_size_t()
    _check(lib().hc_classify_workspace_bytes(C.byref(cfg), C.byref(n)))
    return n.value


def hc_classify(cfg, params, q, k, v, workspace, ws_bytes, labels_dev, diag_dev, stream):
    _check(lib().hc_classify(C.byref(cfg), C.byref(params), hc_tensor(*q), hc_tensor(*k), hc_tensor(*v),
                             C.c_void_p(workspace), ws_bytes, C.c_void_p(labels_dev), C.c_void_p(diag_dev),
                             C.c_void_p(stream)))


def hc_classify_static(cfg, params, q, k, v, labels_dev, diag_dev, stream):
    _check(lib().hc_classify_static(C.byref(cfg), C.byref(params), hc_tensor(*q), hc_tensor(*k), hc_tensor(*v),
                                    C.c_void_p(labels_dev), C.c_void_p(diag_dev), C.c_void_p(stream)))


HC_STATIC_SCRATCH_BYTES = 64 << 20


def hc_status_string(s):
    return lib().hc_status_string(s).decode()


def hc_last_error_message():
    return lib().hc_last_error_message().decode()
