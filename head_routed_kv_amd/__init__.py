"""Head-routed attention (HeadCast) for AMD MI355X.

The compute lives in libheadcast.so (HIP kernels for gfx950) behind the C ABI
declared in include/headcast.h.  This package is its Python face:
  * `_native`     ctypes binding, one function per C entry point, same names;
  * `RoutedCache`, `classify`, `tensor_arg`   torch conveniences that only
    allocate device memory with torch and pass pointers, strides and the
    current HIP stream to the library;
  * `workloads`   seeded synthetic inputs.
"""
from __future__ import annotations

from . import _native
from ._native import (HC_BF16, HC_DUMMY, HC_FP32, HC_GLOBAL, HC_KV_FP8_E4M3, HC_KV_SAME, HC_PUSH_BLOCK,
                      HC_REPLACE_NEWEST, HC_SINK, HC_SPATIAL, HeadcastError, hc_attend, hc_cache_append, hc_cache_bytes, hc_cache_create,
                      hc_cache_destroy, hc_cache_get_layout, hc_classify, hc_classify_static, hc_classify_workspace_bytes,
                      hc_default_classify_params, hc_last_error_message, hc_status_string, hc_validate_config,
                      make_config)

__all__ = ["RoutedCache", "classify", "classify_static", "tensor_arg", "make_config", "HeadcastError", "HC_BF16", "HC_FP32",
           "HC_SINK", "HC_DUMMY", "HC_SPATIAL", "HC_GLOBAL", "HC_PUSH_BLOCK", "HC_REPLACE_NEWEST", "HC_KV_SAME",
           "HC_KV_FP8_E4M3"]


def _torch():
    import torch
    return torch


def tensor_arg(t):
    """(pointer, stride_head, stride_token) of a [H, N, d] tensor with
    contiguous channels."""
    if t.dim() != 3 or t.stride(2) != 1:
        raise ValueError("expected a [heads, tokens, channels] tensor with contiguous channels")
    return (t.data_ptr(), t.stride(0), t.stride(1))


def _stream():
    return _torch().cuda.current_stream().cuda_stream


def check_tensor(t, cfg, rows, name):
    """The library reads num_heads x rows x head_dim elements of cfg's dtype
    through a tensor's pointer and strides; anything smaller would be read
    out of bounds, so shape, dtype and device are checked here first."""
    want = (cfg.num_heads, rows, cfg.head_dim)
    if tuple(t.shape) != want:
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {want} (heads, tokens, channels)")
    if t.dtype != torch_dtype(cfg):
        raise ValueError(f"{name}: dtype {t.dtype}, expected {torch_dtype(cfg)}")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: a device tensor is needed, got one on {t.device}")
    return tensor_arg(t)


def block_rows(cfg):
    return cfg.block_frames * cfg.grid_h * cfg.grid_w


def torch_dtype(cfg):
    torch = _torch()
    return torch.bfloat16 if cfg.dtype == HC_BF16 else torch.float32


class RoutedCache:
    """A restructured KV cache for one layer: device memory from torch, all
    work in the library."""

    def __init__(self, cfg, labels, device="cuda"):
        torch = _torch()
        self.cfg = cfg
        self.labels = [int(x) for x in labels]
        self.nbytes = hc_cache_bytes(cfg, self.labels)
        self.mem = torch.empty(max(self.nbytes, 256), dtype=torch.uint8, device=device)
        self.handle = hc_cache_create(cfg, self.labels, self.mem.data_ptr(), self.mem.numel())

    def append(self, k_block, v_block, mode=HC_PUSH_BLOCK):
        n = block_rows(self.cfg)
        hc_cache_append(self.handle, check_tensor(k_block, self.cfg, n, "k_block"),
                        check_tensor(v_block, self.cfg, n, "v_block"), mode, _stream())

    def attend(self, q_block, out=None):
        n = block_rows(self.cfg)
        q = check_tensor(q_block, self.cfg, n, "q_block")
        if out is None:
            out = _torch().empty_like(q_block)
        hc_attend(self.handle, q, check_tensor(out, self.cfg, n, "out"), _stream())
        return out

    def layout(self):
        return hc_cache_get_layout(self.handle)

    def close(self):
        if self.handle is not None:
            hc_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def classify(cfg, q_block, k_window, v_window, params=None, workspace=None):
    """One-shot classifier.  Returns (labels int8 [H], diag fp32 [H,4],
    workspace) as device tensors; the workspace holds the four outputs and
    the per-query cosines (layout in include/headcast.h)."""
    torch = _torch()
    params = params or hc_default_classify_params()
    H = cfg.num_heads
    need = hc_classify_workspace_bytes(cfg)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_block.device)
    labels = torch.empty(H, dtype=torch.int8, device=q_block.device)
    diag = torch.empty(H, 4, dtype=torch.float32, device=q_block.device)
    nw = cfg.window_frames * cfg.grid_h * cfg.grid_w
    hc_classify(cfg, params, check_tensor(q_block, cfg, block_rows(cfg), "q_block"),
                check_tensor(k_window, cfg, nw, "k_window"), check_tensor(v_window, cfg, nw, "v_window"),
                workspace.data_ptr(), workspace.numel(), labels.data_ptr(), diag.data_ptr(), _stream())
    return labels, diag, workspace


def classify_static(cfg, q_block, k_window, v_window, params=None, labels=None, diag=None):
    """hc_classify_static: the classifier with the library's static scratch
    as its workspace.  labels (int8 [H]) and diag (fp32 [H, 4]) device tensors
    may be given, so that the call allocates nothing; returns them."""
    torch = _torch()
    params = params or hc_default_classify_params()
    H = cfg.num_heads
    if labels is None:
        labels = torch.empty(H, dtype=torch.int8, device=q_block.device)
    if diag is None:
        diag = torch.empty(H, 4, dtype=torch.float32, device=q_block.device)
    if labels.dtype != torch.int8 or labels.numel() < H or diag.dtype != torch.float32 or diag.numel() < 4 * H:
        raise ValueError("labels must be int8 [num_heads] and diag fp32 [num_heads, 4]")
    nw = cfg.window_frames * cfg.grid_h * cfg.grid_w
    hc_classify_static(cfg, params, check_tensor(q_block, cfg, block_rows(cfg), "q_block"),
                       check_tensor(k_window, cfg, nw, "k_window"), check_tensor(v_window, cfg, nw, "v_window"),
                       labels.data_ptr(), diag.data_ptr(), _stream())
    return labels, diag
