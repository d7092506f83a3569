"""Seeded input generators (no layer arithmetic here).

Draw order, fixed so that every consumer sees the same values for a seed:
lengths -> timestamps (sequence by sequence) -> X -> per layer (W1, W2,
rab_pos, rab_time) -> dY.

* lengths: ("uniform", lo, hi) draws integers in [lo, hi]; ("zipf", a, lo, hi)
  draws numpy's Zipf(a) and clips it to [lo, hi]; ("fixed", n) gives every
  sequence n history tokens.  Candidates (if any) are appended after the
  history.
* timestamps: per sequence t_0 ~ U{1.6e9 .. 1.7e9} seconds, then exponential
  gaps (mean 60 s) accumulated and floored: t_k = t_0 + floor(sum of the first
  k gaps).  Candidate timestamps equal the last history timestamp.
* X ~ N(0, x_std) with x_std = 1/sqrt(D) by default; W1 ~ N(0, 1/sqrt(D)),
  W2 ~ N(0, 1/sqrt(H*d_v)) (the fan-in of each); rab tables ~ N(0, rab_std);
  dY ~ N(0, 1).  The second argument of N(.,.) is the standard deviation.
* bf16 workloads round X, W1, W2 and dY to bf16 (round to nearest even) here,
  so the oracle and the GPU consume identical values; rab tables stay fp32.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

from .configs import Config


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 value (ties to even); result is float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def make_lengths(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    kind = cfg.lengths[0]
    if kind == "uniform":
        _, lo, hi = cfg.lengths
        n = rng.integers(lo, hi + 1, size=cfg.B)
    elif kind == "zipf":
        _, a, lo, hi = cfg.lengths
        n = np.clip(rng.zipf(a, size=cfg.B), lo, hi)
    elif kind == "fixed":
        n = np.full(cfg.B, cfg.lengths[1], dtype=np.int64)
    elif kind == "list":
        n = np.asarray(cfg.lengths[1], dtype=np.int64)
        assert n.shape == (cfg.B,)
    else:
        raise ValueError(kind)
    return n.astype(np.int64) + cfg.num_candidates


@dataclasses.dataclass
class LayerWeights:
    W1: np.ndarray          # [D, H*(2*d_v + 2*d_qk)]  float32 (bf16-representable for bf16)
    W2: np.ndarray          # [H*d_v, D]
    rab_pos: np.ndarray     # [H, n_pos_buckets] float32
    rab_time: np.ndarray    # [H, n_time_buckets] float32


@dataclasses.dataclass
class Inputs:
    cfg: Config
    lengths: np.ndarray         # [B] int64 (history + candidates)
    seq_offsets: np.ndarray     # [B+1] int64
    num_candidates: Optional[np.ndarray]   # [B] int64 or None
    timestamps: np.ndarray      # [T] int64 seconds
    X: np.ndarray               # [T, D] float32
    layers: List[LayerWeights]
    dY: Optional[np.ndarray]    # [T, D] float32 (training workloads)
    norm_len: int

    @property
    def T(self) -> int:
        return int(self.seq_offsets[-1])


def _timestamps(rng: np.random.Generator, n_hist: int, n_cand: int, cfg: Config) -> np.ndarray:
    t0 = rng.integers(cfg.t0_range[0], cfg.t0_range[1] + 1)
    gaps = rng.exponential(cfg.gap_mean_s, size=max(n_hist - 1, 0))
    t = t0 + np.floor(np.concatenate([[0.0], np.cumsum(gaps)])[:n_hist]).astype(np.int64)
    if n_cand:
        last = t[-1] if n_hist > 0 else t0
        t = np.concatenate([t, np.full(n_cand, last, dtype=np.int64)])
    return t.astype(np.int64)


def make_inputs(cfg: Config, seed: Optional[int] = None, with_dy: Optional[bool] = None) -> Inputs:
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    lengths = make_lengths(cfg, rng)
    offs = np.zeros(cfg.B + 1, dtype=np.int64)
    offs[1:] = np.cumsum(lengths)
    T = int(offs[-1])
    c = cfg.num_candidates
    ts = [_timestamps(rng, int(n) - c, c, cfg) for n in lengths]
    timestamps = np.concatenate(ts) if ts else np.zeros(0, dtype=np.int64)

    rnd = bf16_round if cfg.dtype == "bf16" else (lambda a: a.astype(np.float32))
    x_std = cfg.x_std if cfg.x_std is not None else 1.0 / np.sqrt(cfg.D)
    X = rnd(rng.standard_normal((T, cfg.D)) * x_std)
    layers = []
    for _ in range(cfg.n_layers):
        W1 = rnd(rng.standard_normal((cfg.D, cfg.f1_width)) / np.sqrt(cfg.D))
        W2 = rnd(rng.standard_normal((cfg.H * cfg.d_v, cfg.D)) / np.sqrt(cfg.H * cfg.d_v))
        rp = (rng.standard_normal((cfg.H, cfg.n_pos_buckets)) * cfg.rab_std).astype(np.float32)
        rt = (rng.standard_normal((cfg.H, cfg.n_time_buckets)) * cfg.rab_std).astype(np.float32)
        layers.append(LayerWeights(W1, W2, rp, rt))
    want_dy = cfg.backward if with_dy is None else with_dy
    dY = rnd(rng.standard_normal((T, cfg.D))) if want_dy else None
    nc = np.full(cfg.B, c, dtype=np.int64) if c else None
    return Inputs(cfg, lengths, offs, nc, timestamps, X, layers, dY, cfg.norm_len)


def sub_batch(inp: Inputs, seqs) -> Inputs:
    """The same inputs restricted to the listed sequences (sequences are independent)."""
    seqs = list(seqs)
    rows = np.concatenate([np.arange(inp.seq_offsets[b], inp.seq_offsets[b + 1]) for b in seqs]) \
        if seqs else np.zeros(0, dtype=np.int64)
    lengths = inp.lengths[seqs]
    offs = np.zeros(len(seqs) + 1, dtype=np.int64)
    offs[1:] = np.cumsum(lengths)
    return Inputs(inp.cfg, lengths, offs,
                  None if inp.num_candidates is None else inp.num_candidates[seqs],
                  inp.timestamps[rows], inp.X[rows], inp.layers,
                  None if inp.dY is None else inp.dY[rows], inp.norm_len)


@dataclasses.dataclass
class AttnInputs:
    """Direct inputs of the attention step alone (no projection)."""
    lengths: np.ndarray
    seq_offsets: np.ndarray
    num_candidates: Optional[np.ndarray]
    timestamps: np.ndarray
    q: np.ndarray        # [T, H, d_qk] float32 (bf16-representable for bf16)
    k: np.ndarray
    v: np.ndarray        # [T, H, d_v]
    rab_pos: np.ndarray  # [H, P] float32
    rab_time: np.ndarray
    d_out: np.ndarray    # [T, H, d_v]
    norm_len: int


def make_attn_inputs(cfg: Config, seed: Optional[int] = None, qk_std: Optional[float] = None,
                     rab_std: float = 1.0) -> AttnInputs:
    """Q, K, V, bias tables and an output gradient for the attention step.

    Lengths and timestamps follow `make_inputs`; q, k ~ N(0, d_qk^-1/4) so that
    q.k has unit scale, v ~ N(0, 1), rab ~ N(0, rab_std), d_out ~ N(0, 1).
    """
    rng = np.random.default_rng(cfg.seed + 1000 if seed is None else seed)
    lengths = make_lengths(cfg, rng)
    offs = np.zeros(cfg.B + 1, dtype=np.int64)
    offs[1:] = np.cumsum(lengths)
    T = int(offs[-1])
    c = cfg.num_candidates
    ts = [_timestamps(rng, int(n) - c, c, cfg) for n in lengths]
    timestamps = np.concatenate(ts) if ts else np.zeros(0, dtype=np.int64)
    rnd = bf16_round if cfg.dtype == "bf16" else (lambda a: a.astype(np.float32))
    s = cfg.d_qk ** -0.25 if qk_std is None else qk_std
    q = rnd(rng.standard_normal((T, cfg.H, cfg.d_qk)) * s)
    k = rnd(rng.standard_normal((T, cfg.H, cfg.d_qk)) * s)
    v = rnd(rng.standard_normal((T, cfg.H, cfg.d_v)))
    rp = (rng.standard_normal((cfg.H, cfg.n_pos_buckets)) * rab_std).astype(np.float32)
    rt = (rng.standard_normal((cfg.H, cfg.n_time_buckets)) * rab_std).astype(np.float32)
    dO = rnd(rng.standard_normal((T, cfg.H, cfg.d_v)))
    nc = np.full(cfg.B, c, dtype=np.int64) if c else None
    return AttnInputs(lengths, offs, nc, timestamps, q, k, v, rp, rt, dO, cfg.norm_len)
