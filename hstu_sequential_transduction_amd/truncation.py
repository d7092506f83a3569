"""Attention truncation as a sequence of library calls ("Bending the Scaling
Law Curve in Large-Scale Recommendation Systems", Attention Truncation):
N layers over the whole sequences, the segment gather (each history's last
`keep` events plus the candidates), M layers over the segments; the
backward runs the same calls in reverse with the gradient scatter between
the two groups.  Every step is a libhstu.so entry point; this module only
orders the calls and holds the tensors a training step keeps.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import torch

from . import binding as B


@dataclasses.dataclass
class TruncRecord:
    """What the backward needs from a training forward."""
    full_in: List[torch.Tensor]      # input of each full layer
    full_saved: List[B.Saved]
    tail_in: List[torch.Tensor]      # input of each tail layer (segment rows)
    tail_saved: List[B.Saved]
    seg_offsets: torch.Tensor
    ts_seg: torch.Tensor
    T: int
    T_seg: int


def truncated_stack_fwd(x, full_layers: Sequence, tail_layers: Sequence, seq_offsets, timestamps,
                        cfg_full: B.LayerConfig, cfg_tail: B.LayerConfig, keep: int,
                        num_candidates=None, T_seg: Optional[int] = None, training: bool = False,
                        workspace: Optional[B.LayerWorkspace] = None):
    """(y_seg [T_seg, D], seg_offsets, TruncRecord or None).

    Layers are (W1, W2, rab_pos, rab_time) tuples of device tensors.  T_seg,
    when the caller knows it, saves reading it back from the device."""
    ws = workspace if workspace is not None else B.LayerWorkspace()
    T = x.shape[0]
    full_in, full_saved, tail_in, tail_saved = [], [], [], []
    for (W1, W2, rp, rt) in full_layers:
        sv = B.Saved(T, cfg_full, x.dtype, x.device) if training else None
        full_in.append(x)
        full_saved.append(sv)
        x = B.hstu_layer_fwd(x, W1, W2, rp, rt, seq_offsets, timestamps, cfg_full,
                             num_candidates=num_candidates, saved=sv, workspace=ws)
    seg, T_seg = B.hstu_truncate_offsets(seq_offsets, keep, num_candidates, T_seg)
    x, ts_seg = B.hstu_truncate_gather(x, seq_offsets, seg, T_seg, timestamps)
    for (W1, W2, rp, rt) in tail_layers:
        sv = B.Saved(T_seg, cfg_tail, x.dtype, x.device) if training else None
        tail_in.append(x)
        tail_saved.append(sv)
        x = B.hstu_layer_fwd(x, W1, W2, rp, rt, seg, ts_seg, cfg_tail,
                             num_candidates=num_candidates, saved=sv, workspace=ws)
    rec = (TruncRecord(full_in, full_saved, tail_in, tail_saved, seg, ts_seg, T, T_seg)
           if training else None)
    return x, seg, rec


def truncated_stack_bwd(dy_seg, full_layers: Sequence, tail_layers: Sequence, seq_offsets,
                        timestamps, cfg_full: B.LayerConfig, cfg_tail: B.LayerConfig,
                        rec: TruncRecord, num_candidates=None,
                        workspace: Optional[B.LayerWorkspace] = None):
    """(dx [T, D], grads of the full layers, grads of the tail layers)."""
    ws = workspace if workspace is not None else B.LayerWorkspace()
    g = dy_seg
    g_tail = [None] * len(tail_layers)
    for l in range(len(tail_layers) - 1, -1, -1):
        W1, W2, rp, rt = tail_layers[l]
        g, g_tail[l] = B.hstu_layer_bwd(rec.tail_in[l], W1, W2, rp, rt, rec.seg_offsets,
                                        rec.ts_seg, cfg_tail, rec.tail_saved[l], g,
                                        num_candidates=num_candidates, workspace=ws)
    g = B.hstu_truncate_scatter(g, seq_offsets, rec.seg_offsets, rec.T)
    g_full = [None] * len(full_layers)
    for l in range(len(full_layers) - 1, -1, -1):
        W1, W2, rp, rt = full_layers[l]
        g, g_full[l] = B.hstu_layer_bwd(rec.full_in[l], W1, W2, rp, rt, seq_offsets, timestamps,
                                        cfg_full, rec.full_saved[l], g,
                                        num_candidates=num_candidates, workspace=ws)
    return g, g_full, g_tail
