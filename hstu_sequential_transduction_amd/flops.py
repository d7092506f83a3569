"""Algorithmic FLOP and byte counts of the HSTU layer (host-side cost model).

The counting convention is the one of the DLRMv4 page ("DLRMv4 Brings
Sequence-Based Recommendation Training to MLPerf", section "Computation Cost
Analysis", Tables 6 and 7): a weight GEMM costs 2*M*N*K in the forward pass
and three times that for forward plus backward; causal attention counts S^2/2
query-key pairs, 2*(d_qk + d_v) FLOP per pair and head in the forward pass,
and 3.5 times that for forward plus backward.

For jagged batches the per-sequence S^2/2 becomes n_b^2/2.  A sequence whose
last c tokens are candidates (history n_h = n - c) contributes the causal
history triangle n_h^2/2 plus c*n_h candidate-history pairs plus c
self-pairs.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np


def table7(B: int, L: int, h: int, d_qk: int, d_v: int, D: int, S: int,
           outproj_width_mult: int = 3) -> Dict[str, float]:
    """Per-GPU-step FLOPs of the page's cost table (fwd+bwd, every sequence of length S).

    The output-projection row of that table uses an input width of
    3*h*d_v; outproj_width_mult=1 gives the width of the layer built here
    (h*d_v), the page's printed total needs 3.
    """
    uvqk = B * L * 3 * 2 * S * D * (2 * d_qk + 2 * d_v) * h
    outp = B * L * 3 * 2 * S * (outproj_width_mult * h * d_v) * D
    attn = B * L * 3.5 * 2 * (S ** 2 / 2) * h * (d_qk + d_v)
    return {"uvqk": float(uvqk), "outproj": float(outp), "attn": float(attn),
            "total": float(uvqk + outp + attn)}


def attn_pairs(lengths: Sequence[int], num_candidates: Optional[Sequence[int]] = None) -> float:
    """Query-key pairs per head under the page's S^2/2 causal convention."""
    n = np.asarray(lengths, dtype=np.float64)
    if num_candidates is None:
        return float((n ** 2 / 2).sum())
    c = np.asarray(num_candidates, dtype=np.float64)
    nh = n - c
    return float((nh ** 2 / 2 + c * nh + c).sum())


def _tri_min(K: int, cap: int) -> int:
    """sum_{t=1..K} min(t, cap) for K >= 0."""
    if K <= 0:
        return 0
    if K <= cap:
        return K * (K + 1) // 2
    return cap * (cap + 1) // 2 + (K - cap) * cap


def attn_pairs_window(lengths: Sequence[int], num_candidates: Optional[Sequence[int]],
                      win_local: int, win_global: int) -> float:
    """Exact allowed query-key pairs per head under semi-local attention (a local
    window of win_local positions and the first win_global tokens; "Bending the
    Scaling Law Curve in Large-Scale Recommendation Systems", Semi-Local
    Attention).  With win_local = 0 (no window) the exact causal count."""
    total = 0
    cands = [0] * len(lengths) if num_candidates is None else list(num_candidates)
    for n, c in zip(lengths, cands):
        n, c = int(n), int(c)
        nh = n - c
        if win_local <= 0:
            total += nh * (nh + 1) // 2 + c * (nh + 1)
            continue
        # history row i: local keys min(i+1, W_l); global keys below the band
        # min(W_g, max(0, i - W_l + 1))
        total += _tri_min(nh, win_local) + _tri_min(nh - win_local, win_global)
        # candidate row: history keys within W_l of position n_h, global keys
        # below them, and itself
        band = max(0, nh - win_local + 1)
        total += c * ((nh - band) + min(win_global, band) + 1)
    return float(total)


def attn_fwd_flops(lengths, num_candidates, H: int, d_qk: int, d_v: int) -> float:
    return 2.0 * attn_pairs(lengths, num_candidates) * H * (d_qk + d_v)


def layer_flops(lengths, num_candidates, D: int, H: int, d_qk: int, d_v: int,
                backward: bool, window=None) -> Dict[str, float]:
    """Algorithmic FLOPs of one layer over a jagged batch (fwd, or fwd+bwd);
    window = (win_local, win_global) counts the semi-local pairs exactly."""
    T = float(np.sum(lengths))
    w = 3.0 if backward else 1.0
    uvqk = w * 2 * T * D * H * (2 * d_qk + 2 * d_v)
    outp = w * 2 * T * H * d_v * D
    if window is not None and window[0] > 0:
        af = 2.0 * attn_pairs_window(lengths, num_candidates, window[0], window[1]) * H * (d_qk + d_v)
    else:
        af = attn_fwd_flops(lengths, num_candidates, H, d_qk, d_v)
    attn = 3.5 * af if backward else af
    return {"uvqk": uvqk, "outproj": outp, "attn": attn, "attn_fwd": af,
            "attn_bwd": (2.5 * af if backward else 0.0), "total": uvqk + outp + attn}


def attn_min_bytes(T: int, H: int, d_qk: int, d_v: int, elem: int = 2) -> float:
    """Compulsory HBM bytes of the fused attention forward: read Q, K, V, write O."""
    return float(T * H * (2 * d_qk + 2 * d_v) * elem)


def ln_gate_fwd_bytes(T: int, width: int, elem: int = 2, stats: bool = True) -> float:
    """Compulsory bytes of the LayerNorm + gating epilogue: read O and U, write G (+ mu, rstd)."""
    return float(T * (3 * width * elem + (8 if stats else 0)))
