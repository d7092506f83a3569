"""Ranking against a cached history as a sequence of library calls
("DLRMv4 Brings Sequence-Based Recommendation Training to MLPerf", "Model
Architecture": candidates appended to the history and compared with it).

A history row never attends to a candidate, so the history is run through
the layers once (hstu_layer_fwd keeping each layer's U|V|Q|K) and each
layer's K and V blocks are kept; every later batch of candidates then runs
through the layers alone (hstu_layer_fwd_cached).  This module only orders
the calls and holds the cached tensors.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import torch

from . import binding as B


class HistoryCache:
    """Per-layer keys and values of a batch of users' histories."""

    def __init__(self, layers: List[B.History], zh: List[torch.Tensor]):
        self.layers = layers
        self._zh = zh   # owners of the K/V views


def build_history_cache(x_hist, layers: Sequence, hist_offsets, hist_ts, cfg: B.LayerConfig,
                        workspace: Optional[B.LayerWorkspace] = None) -> HistoryCache:
    """Run the histories through the stack once, keeping each layer's K, V.
    Layers are (W1, W2, rab_pos, rab_time) tuples of device tensors."""
    ws = workspace if workspace is not None else B.LayerWorkspace()
    T = x_hist.shape[0]
    x = x_hist
    kv, zhs = [], []
    for (W1, W2, rp, rt) in layers:
        zh = torch.empty((T, cfg.f1), dtype=x.dtype, device=x.device)
        x = B.hstu_layer_fwd(x, W1, W2, rp, rt, hist_offsets, hist_ts, cfg, keep_zh=zh,
                             workspace=ws)
        zhs.append(zh)
        kv.append(B.history_from_zh(zh, cfg, hist_offsets, hist_ts))
    return HistoryCache(kv, zhs)


def cached_stack_fwd(x_cand, layers: Sequence, cache: HistoryCache, cand_offsets, cand_ts,
                     cfg: B.LayerConfig, workspace: Optional[B.LayerWorkspace] = None,
                     out_bufs=None):
    """Candidate rows through the stack against the cached histories."""
    ws = workspace if workspace is not None else B.LayerWorkspace()
    x = x_cand
    for li, ((W1, W2, rp, rt), hist) in enumerate(zip(layers, cache.layers)):
        y = None if out_bufs is None else out_bufs[li % len(out_bufs)]
        x = B.hstu_layer_fwd_cached(x, W1, W2, rp, rt, cand_offsets, cand_ts, hist, cfg, y=y,
                                    workspace=ws)
    return x
