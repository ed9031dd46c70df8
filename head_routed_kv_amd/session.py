"""Streaming driver for one attention layer: the steps on either side of the
routed hot path.

  warm-up      while the first window fills, every head attends over the whole
               (growing) window, i.e. the cache holds all heads as Global;
  classify     once, when the sliding window first fills ([Pith] "What
               carries the argument"), at the newest block's first denoising
               step, the noisiest one ([Pith] "The pith"; ledger entry
               "classification denoising timestep t = 1000"): hc_classify
               compares each head's full output with its Sink, Dummy and
               Spatial proxies;
  restructure  the window's blocks are replayed, oldest first, into a cache
               laid out by the labels (Sink = the video's first block, which at
               first fill is the window's first block);
  rollout      every later block is pushed, its denoising steps replace it, and
               each step attends through the routed cache.

Orchestration only: every step is a library call.  Periodic re-classification
is not offered: after restructuring, Sink and Dummy heads no longer keep the
window that a classifier pass reads.
"""
from __future__ import annotations

import copy

from . import (HC_GLOBAL, HC_KV_SAME, HC_PUSH_BLOCK, HC_REPLACE_NEWEST, HeadcastError, RoutedCache, _torch,
               classify, torch_dtype)
from ._native import HC_ERR_STATE


class LayerSession:
    """One layer's KV cache across a video rollout."""

    def __init__(self, cfg, device="cuda", params=None):
        self.cfg = cfg
        self.device = device
        self.params = params
        self.blocks_per_window = cfg.window_frames // cfg.block_frames
        self.labels = None        # host list once classified
        self.diag = None          # device [H, 4] once classified
        self.blocks = 0           # blocks pushed so far
        # the warm-up cache keeps K/V in the layer's dtype, since the classifier
        # reads its window; an fp8 layout (cfg.kv_format) applies from the
        # restructure on
        self.warm_cfg = copy.copy(cfg)
        self.warm_cfg.kv_format = HC_KV_SAME
        self.cache = RoutedCache(self.warm_cfg, [HC_GLOBAL] * cfg.num_heads, device)

    @property
    def routed(self) -> bool:
        return self.labels is not None

    def push(self, k_block, v_block):
        """A new block enters the window (its first denoising step)."""
        self.cache.append(k_block, v_block, HC_PUSH_BLOCK)
        self.blocks += 1

    def replace(self, k_block, v_block):
        """A later denoising step of the newest block."""
        self.cache.append(k_block, v_block, HC_REPLACE_NEWEST)

    def classify_due(self) -> bool:
        """True exactly while the first window is full and not yet classified."""
        return not self.routed and self.blocks == self.blocks_per_window

    def window_views(self):
        """K and V of the current window as [H, W*T, d] views of the warm-up
        cache's Global ring.  At first fill ring slot b holds block b, so the
        rows are in time order."""
        if self.routed:
            raise HeadcastError(HC_ERR_STATE, "the window is no longer held once the cache is restructured")
        torch = _torch()
        cfg, lay = self.warm_cfg, self.cache.layout()
        dt = torch_dtype(cfg)
        n = cfg.num_heads * cfg.window_frames * cfg.grid_h * cfg.grid_w * cfg.head_dim
        esz = torch.tensor([], dtype=dt).element_size()
        shape = (cfg.num_heads, cfg.window_frames * cfg.grid_h * cfg.grid_w, cfg.head_dim)
        k = self.cache.mem[lay.off_global_k:lay.off_global_k + n * esz].view(dt).view(shape)
        v = self.cache.mem[lay.off_global_v:lay.off_global_v + n * esz].view(dt).view(shape)
        return k, v

    def classify(self, q_block):
        """Classify every head on the first full window and restructure the
        cache.  q_block are the newest block's queries at this step.  Returns
        the host labels."""
        if not self.classify_due():
            raise HeadcastError(HC_ERR_STATE, f"classification runs once, at the first full window "
                                f"({self.blocks} of {self.blocks_per_window} blocks pushed, routed={self.routed})")
        torch = _torch()
        k_win, v_win = self.window_views()
        labels, diag, _ = classify(self.cfg, q_block, k_win, v_win, self.params)
        self.labels = [int(x) for x in labels.cpu()]
        self.diag = diag
        new = RoutedCache(self.cfg, self.labels, self.device)
        bt = self.cfg.block_frames * self.cfg.grid_h * self.cfg.grid_w
        for b in range(self.blocks_per_window):
            new.append(k_win[:, b * bt:(b + 1) * bt], v_win[:, b * bt:(b + 1) * bt], HC_PUSH_BLOCK)
        # the replay reads the warm-up cache's memory on the stream: release it
        # only after those copies have run
        torch.cuda.current_stream().synchronize()
        self.cache.close()
        self.cache = new
        return self.labels

    def attend(self, q_block, out=None):
        """Attention of the newest block's queries through the current cache."""
        return self.cache.attend(q_block, out)

    def close(self):
        self.cache.close()
