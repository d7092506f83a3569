"""Thin torch-facing binding of libhstu.so: argument marshalling only.

Each function takes device tensors, allocates outputs and the workspace with
torch (device memory only), and calls the C entry point of the same name on
torch's current HIP stream.  No computation happens here.
"""
from __future__ import annotations

import ctypes as C
import dataclasses
from typing import Optional

import torch

from . import _lib
from ._lib import (AttnDesc, HistoryKV, LayerDesc, LayerGrads, LayerSaved, LayerWeights,
                   MxIO, MxWeights, check)

_DT = {torch.float32: _lib.HSTU_F32, torch.bfloat16: _lib.HSTU_BF16}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _dev(t: Optional[torch.Tensor], name: str) -> None:
    if t is not None and not t.is_cuda:
        raise ValueError(f"{name} must be a device (cuda/hip) tensor")


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


@dataclasses.dataclass
class AttnConfig:
    H: int
    d_qk: int
    d_v: int
    norm_len: int = 1
    norm_mode: int = 0
    n_pos_buckets: int = 128
    n_time_buckets: int = 128
    win_local: int = 0    # semi-local attention windows (0: full causal)
    win_global: int = 0
    max_len: int = 0      # longest sequence, if known (lets the backward keep dS)
    reuse_plan: int = 0   # forward: the workspace already holds this batch's plan
    key_splits: int = 0   # forward: 0 auto, 1 never, k >= 2 split long query blocks' keys


def set_check_mode(on: bool) -> None:
    """Debug mode of the library: wait for the device and read the launch
    error after every launch (see hstu_set_check_mode in include/hstu.h)."""
    check("hstu_set_check_mode", _lib.lib().hstu_set_check_mode(1 if on else 0))


def check_mode() -> bool:
    return bool(_lib.lib().hstu_check_mode())


def attn_desc(cfg: AttnConfig, B: int, T: int, dtype: torch.dtype, rab_stride: int) -> AttnDesc:
    return AttnDesc(B, T, cfg.H, cfg.d_qk, cfg.d_v, cfg.n_pos_buckets, cfg.n_time_buckets,
                    cfg.norm_mode, cfg.norm_len, _DT[dtype], rab_stride, cfg.win_local,
                    cfg.win_global, cfg.max_len, cfg.reuse_plan, cfg.key_splits)


def _rab_stride(rab_pos: torch.Tensor, rab_time: torch.Tensor) -> int:
    if rab_pos.dim() == 1:
        if rab_time.dim() != 1:
            raise ValueError("rab_pos and rab_time must both be shared or both per head")
        return 0
    if rab_pos.stride(0) != rab_time.stride(0) or rab_pos.stride(1) != 1 or rab_time.stride(1) != 1:
        raise ValueError("per-head rab tables must share one contiguous head stride")
    return rab_pos.stride(0)


def hstu_attn_fwd(q, k, v, seq_offsets, timestamps, rab_pos, rab_time, cfg: AttnConfig,
                  num_candidates=None, out=None, stream=None,
                  workspace: Optional["LayerWorkspace"] = None):
    """O [T, H*d_v] of the pointwise attention (see include/hstu.h).  With
    cfg.reuse_plan = 1 the call needs the `workspace` of an earlier planning
    call on the same batch."""
    for n_, t_ in (("q", q), ("k", k), ("v", v), ("seq_offsets", seq_offsets),
                   ("timestamps", timestamps), ("rab_pos", rab_pos), ("rab_time", rab_time),
                   ("num_candidates", num_candidates)):
        _dev(t_, n_)
    T = q.shape[0]
    B = seq_offsets.shape[0] - 1
    if out is None:
        out = torch.empty((T, cfg.H * cfg.d_v), dtype=q.dtype, device=q.device)
    d = attn_desc(cfg, B, T, q.dtype, _rab_stride(rab_pos, rab_time))
    L = _lib.lib()
    nb = L.hstu_attn_fwd_workspace_size(C.byref(d))
    ws = _layer_ws(workspace, nb, q.device, cfg.reuse_plan)
    st = L.hstu_attn_fwd(C.byref(d), _ptr(q), _ptr(k), q.stride(0), _ptr(v), v.stride(0),
                         _ptr(seq_offsets), _ptr(timestamps), _ptr(rab_pos), _ptr(rab_time),
                         _ptr(num_candidates), _ptr(out), out.stride(0), _ptr(ws), ws.numel(),
                         _stream(stream))
    check("hstu_attn_fwd", st)
    return out


def hstu_attn_fwd_noalloc(q, k, v, seq_offsets, timestamps, rab_pos, rab_time, cfg: AttnConfig,
                          num_candidates=None, out=None, stream=None):
    """hstu_attn_fwd without a workspace: the library's per-GPU scratch holds
    the plan (see include/hstu.h).  `out` is allocated here unless given."""
    for n_, t_ in (("q", q), ("k", k), ("v", v), ("seq_offsets", seq_offsets),
                   ("timestamps", timestamps), ("rab_pos", rab_pos), ("rab_time", rab_time),
                   ("num_candidates", num_candidates), ("out", out)):
        _dev(t_, n_)
    T = q.shape[0]
    B = seq_offsets.shape[0] - 1
    if out is None:
        out = torch.empty((T, cfg.H * cfg.d_v), dtype=q.dtype, device=q.device)
    d = attn_desc(cfg, B, T, q.dtype, _rab_stride(rab_pos, rab_time))
    st = _lib.lib().hstu_attn_fwd_noalloc(
        C.byref(d), _ptr(q), _ptr(k), q.stride(0), _ptr(v), v.stride(0), _ptr(seq_offsets),
        _ptr(timestamps), _ptr(rab_pos), _ptr(rab_time), _ptr(num_candidates), _ptr(out),
        out.stride(0), _stream(stream))
    check("hstu_attn_fwd_noalloc", st)
    return out


def hstu_attn_bwd(q, k, v, seq_offsets, timestamps, rab_pos, rab_time, d_out, cfg: AttnConfig,
                  num_candidates=None, stream=None):
    """(dq, dk, dv, d_rab_pos, d_rab_time) for the output gradient d_out."""
    T = q.shape[0]
    B = seq_offsets.shape[0] - 1
    dev = q.device
    dq = torch.empty((T, cfg.H * cfg.d_qk), dtype=q.dtype, device=dev)
    dk = torch.empty_like(dq)
    dv = torch.empty((T, cfg.H * cfg.d_v), dtype=q.dtype, device=dev)
    drp = torch.empty_like(rab_pos, dtype=torch.float32)
    drt = torch.empty_like(rab_time, dtype=torch.float32)
    d = attn_desc(cfg, B, T, q.dtype, _rab_stride(rab_pos, rab_time))
    L = _lib.lib()
    ws = _ws(L.hstu_attn_bwd_workspace_size(C.byref(d)), dev)
    st = L.hstu_attn_bwd(C.byref(d), _ptr(q), _ptr(k), q.stride(0), _ptr(v), v.stride(0),
                         _ptr(seq_offsets), _ptr(timestamps), _ptr(rab_pos), _ptr(rab_time),
                         _ptr(num_candidates), _ptr(d_out), d_out.stride(0), _ptr(dq), _ptr(dk),
                         _ptr(dv), _ptr(drp), _ptr(drt), _ptr(ws), ws.numel(), _stream(stream))
    check("hstu_attn_bwd", st)
    return dq, dk, dv, drp, drt


@dataclasses.dataclass
class LayerConfig:
    D: int
    attn: AttnConfig
    proj_silu: bool = True
    residual: bool = True
    ln_eps: float = 1e-6

    @property
    def f1(self) -> int:
        return self.attn.H * (2 * self.attn.d_v + 2 * self.attn.d_qk)


def layer_desc(cfg: LayerConfig, B: int, T: int, dtype, rab_stride: int) -> LayerDesc:
    return LayerDesc(attn_desc(cfg.attn, B, T, dtype, rab_stride), cfg.D, int(cfg.proj_silu),
                     int(cfg.residual), cfg.ln_eps)


def _weights(W1, W2, rab_pos, rab_time, b1=None, b2=None, gamma=None, beta=None):
    return LayerWeights(_ptr(W1), _ptr(W2), _ptr(b1), _ptr(b2), _ptr(gamma), _ptr(beta),
                        _ptr(rab_pos), _ptr(rab_time))


class Saved:
    """Forward intermediates of a training step (device tensors)."""

    def __init__(self, T: int, cfg: LayerConfig, dtype, device):
        W = cfg.attn.H * cfg.attn.d_v
        self.Z = torch.empty((T, cfg.f1), dtype=dtype, device=device)
        self.Zh = torch.empty((T, cfg.f1), dtype=dtype, device=device)
        self.O = torch.empty((T, W), dtype=torch.float32, device=device)
        self.G = torch.empty((T, W), dtype=dtype, device=device)
        self.mu = torch.empty((T,), dtype=torch.float32, device=device)
        self.rstd = torch.empty((T,), dtype=torch.float32, device=device)

    def c(self) -> LayerSaved:
        return LayerSaved(_ptr(self.Z), _ptr(self.Zh), _ptr(self.O), _ptr(self.G),
                          _ptr(self.mu), _ptr(self.rstd))


class LayerWorkspace:
    """Reusable workspace for repeated layer calls of one shape."""

    def __init__(self):
        self.buf = None

    def get(self, nbytes: int, device, reuse_plan: int = 0) -> torch.Tensor:
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != device:
            if reuse_plan:
                raise ValueError("reuse_plan=1 needs the workspace an earlier forward call on "
                                 "the same batch planned into; this one would be reallocated")
            self.buf = _ws(nbytes, device)
        return self.buf


def _layer_ws(workspace: Optional[LayerWorkspace], nbytes: int, device, reuse_plan: int = 0):
    if workspace is None:
        if reuse_plan:
            raise ValueError("reuse_plan=1 needs the persistent workspace of the planning call")
        return _ws(nbytes, device)
    return workspace.get(nbytes, device, reuse_plan)


def hstu_layer_fwd(x, W1, W2, rab_pos, rab_time, seq_offsets, timestamps, cfg: LayerConfig,
                   num_candidates=None, b1=None, b2=None, gamma=None, beta=None,
                   saved: Optional[Saved] = None, y=None, workspace: Optional[LayerWorkspace] = None,
                   stream=None, keep_zh: Optional[torch.Tensor] = None):
    """Y = HSTU layer(x); fills `saved` when given (training), or only the
    U|V|Q|K tensor `keep_zh` [T, F1] (inference that keeps the projections)."""
    T = x.shape[0]
    B = seq_offsets.shape[0] - 1
    if y is None:
        y = torch.empty_like(x)
    d = layer_desc(cfg, B, T, x.dtype, _rab_stride(rab_pos, rab_time))
    L = _lib.lib()
    nb = L.hstu_layer_fwd_workspace_size(C.byref(d), 1 if saved is not None else 0)
    ws = _layer_ws(workspace, nb, x.device, cfg.attn.reuse_plan)
    w = _weights(W1, W2, rab_pos, rab_time, b1, b2, gamma, beta)
    sv = saved.c() if saved is not None else None
    if keep_zh is not None:
        if saved is not None:
            raise ValueError("keep_zh and saved are exclusive")
        sv = LayerSaved(None, _ptr(keep_zh), None, None, None, None)
    st = L.hstu_layer_fwd(C.byref(d), _ptr(x), C.byref(w), _ptr(seq_offsets), _ptr(timestamps),
                          _ptr(num_candidates), _ptr(y), C.byref(sv) if sv is not None else None,
                          _ptr(ws), ws.numel(), _stream(stream))
    check("hstu_layer_fwd", st)
    return y


@dataclasses.dataclass
class Grads:
    dW1: torch.Tensor
    dW2: torch.Tensor
    drab_pos: torch.Tensor
    drab_time: torch.Tensor
    db1: Optional[torch.Tensor] = None
    db2: Optional[torch.Tensor] = None
    dgamma: Optional[torch.Tensor] = None
    dbeta: Optional[torch.Tensor] = None


def hstu_layer_bwd(x, W1, W2, rab_pos, rab_time, seq_offsets, timestamps, cfg: LayerConfig,
                   saved: Saved, dy, num_candidates=None, b1=None, b2=None, gamma=None,
                   beta=None, dx=None, grads: Optional[Grads] = None,
                   workspace: Optional[LayerWorkspace] = None, stream=None, mx: bool = False):
    """(dx, Grads) of the layer for the output gradient dy.  mx: the backward
    of hstu_layer_fwd_mx (hstu_layer_bwd_mx: dG, dX, dW2 and dW1 as MXFP8 products)."""
    T = x.shape[0]
    B = seq_offsets.shape[0] - 1
    dev = x.device
    if dx is None:
        dx = torch.empty_like(x)
    if grads is None:
        f32 = dict(dtype=torch.float32, device=dev)
        grads = Grads(torch.empty(W1.shape, **f32), torch.empty(W2.shape, **f32),
                      torch.empty(rab_pos.shape, **f32), torch.empty(rab_time.shape, **f32),
                      None if b1 is None else torch.empty(b1.shape, **f32),
                      None if b2 is None else torch.empty(b2.shape, **f32),
                      None if gamma is None else torch.empty(gamma.shape, **f32),
                      None if beta is None else torch.empty(beta.shape, **f32))
    d = layer_desc(cfg, B, T, x.dtype, _rab_stride(rab_pos, rab_time))
    L = _lib.lib()
    nb = (L.hstu_layer_bwd_mx_workspace_size if mx else L.hstu_layer_bwd_workspace_size)(
        C.byref(d))
    ws = workspace.get(nb, dev) if workspace is not None else _ws(nb, dev)
    w = _weights(W1, W2, rab_pos, rab_time, b1, b2, gamma, beta)
    g = LayerGrads(_ptr(grads.dW1), _ptr(grads.dW2), _ptr(grads.db1), _ptr(grads.db2),
                   _ptr(grads.dgamma), _ptr(grads.dbeta), _ptr(grads.drab_pos),
                   _ptr(grads.drab_time))
    sv = saved.c()
    fn = L.hstu_layer_bwd_mx if mx else L.hstu_layer_bwd
    st = fn(C.byref(d), _ptr(x), C.byref(w), _ptr(seq_offsets), _ptr(timestamps),
            _ptr(num_candidates), C.byref(sv), _ptr(dy), _ptr(dx), C.byref(g),
            _ptr(ws), ws.numel(), _stream(stream))
    check("hstu_layer_bwd_mx" if mx else "hstu_layer_bwd", st)
    return dx, grads


@dataclasses.dataclass
class History:
    """One layer's cached history keys and values (device tensors; k and v
    may be strided column views, e.g. of the Zh a history forward kept)."""
    k: torch.Tensor           # [T_hist, H*d_qk]
    v: torch.Tensor           # [T_hist, H*d_v]
    offsets: torch.Tensor     # [B+1] int32
    timestamps: torch.Tensor  # [T_hist] int64

    def c(self) -> HistoryKV:
        return HistoryKV(_ptr(self.k), _ptr(self.v), self.k.stride(0), self.v.stride(0),
                         _ptr(self.offsets), _ptr(self.timestamps), self.k.shape[0])


def history_from_zh(Zh: torch.Tensor, cfg: LayerConfig, offsets, timestamps) -> History:
    """The K and V column blocks of a history forward's U|V|Q|K output."""
    W, HQ = cfg.attn.H * cfg.attn.d_v, cfg.attn.H * cfg.attn.d_qk
    return History(Zh[:, 2 * W + HQ:2 * W + 2 * HQ], Zh[:, W:2 * W], offsets, timestamps)


def hstu_attn_cached_fwd(q, k, v, cand_offsets, cand_ts, hist: History, rab_pos, rab_time,
                         cfg: AttnConfig, out=None, stream=None):
    """O [T_c, H*d_v] of candidates against a cached history (see include/hstu.h)."""
    T = q.shape[0]
    B = cand_offsets.shape[0] - 1
    if out is None:
        out = torch.empty((T, cfg.H * cfg.d_v), dtype=q.dtype, device=q.device)
    d = attn_desc(cfg, B, T, q.dtype, _rab_stride(rab_pos, rab_time))
    L = _lib.lib()
    h = hist.c()
    ws = _ws(L.hstu_attn_cached_workspace_size(C.byref(d), h.T), q.device)
    st = L.hstu_attn_cached_fwd(C.byref(d), _ptr(q), _ptr(k), q.stride(0), _ptr(v), v.stride(0),
                                _ptr(cand_offsets), _ptr(cand_ts), C.byref(h), _ptr(rab_pos),
                                _ptr(rab_time), _ptr(out), out.stride(0), _ptr(ws), ws.numel(),
                                _stream(stream))
    check("hstu_attn_cached_fwd", st)
    return out


def hstu_layer_fwd_cached(x, W1, W2, rab_pos, rab_time, cand_offsets, cand_ts, hist: History,
                          cfg: LayerConfig, b1=None, b2=None, gamma=None, beta=None, y=None,
                          workspace: Optional[LayerWorkspace] = None, stream=None):
    """Y of one layer over candidate rows against this layer's cached history."""
    T = x.shape[0]
    B = cand_offsets.shape[0] - 1
    if y is None:
        y = torch.empty_like(x)
    d = layer_desc(cfg, B, T, x.dtype, _rab_stride(rab_pos, rab_time))
    L = _lib.lib()
    h = hist.c()
    nb = L.hstu_layer_cached_workspace_size(C.byref(d), h.T)
    ws = workspace.get(nb, x.device) if workspace is not None else _ws(nb, x.device)
    w = _weights(W1, W2, rab_pos, rab_time, b1, b2, gamma, beta)
    st = L.hstu_layer_fwd_cached(C.byref(d), _ptr(x), C.byref(w), _ptr(cand_offsets),
                                 _ptr(cand_ts), C.byref(h), _ptr(y), _ptr(ws), ws.numel(),
                                 _stream(stream))
    check("hstu_layer_fwd_cached", st)
    return y


def hstu_mx_quantize(x, stream=None):
    """(codes uint8 [rows, K], scales uint8 [rows, K/32]) of bf16 rows (MXFP8)."""
    rows, K = x.shape
    codes = torch.empty((rows, K), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, K // 32), dtype=torch.uint8, device=x.device)
    st = _lib.lib().hstu_mx_quantize(rows, K, _ptr(x), x.stride(0), _ptr(codes), _ptr(scales),
                                     _stream(stream))
    check("hstu_mx_quantize", st)
    return codes, scales


def hstu_mx_quantize_heads(x, H, d, stream=None):
    """MXFP8 of an attention operand x [T, >= H*d] (bf16, e.g. q or k) along each
    head's d channels: (codes uint8 [T, H*d], head-major scale words int32
    [H, T], byte b of a word = the scale of channels 32b..32b+31)."""
    T = x.shape[0]
    codes = torch.empty((T, H * d), dtype=torch.uint8, device=x.device)
    scales = torch.empty((H, T), dtype=torch.int32, device=x.device)
    st = _lib.lib().hstu_mx_quantize_heads(T, H, d, _ptr(x), x.stride(0), _ptr(codes), H * d,
                                           _ptr(scales), _stream(stream))
    check("hstu_mx_quantize_heads", st)
    return codes, scales


def hstu_attn_fwd_mx(q_codes, q_scales, k_codes, k_scales, v, seq_offsets, timestamps, rab_pos,
                     rab_time, cfg: AttnConfig, num_candidates=None, out=None, stream=None,
                     workspace: Optional["LayerWorkspace"] = None):
    """hstu_attn_fwd with the score product in MXFP8: q and k as written by
    hstu_mx_quantize_heads (codes [T, ld] with one row stride, scale words [H, T])."""
    for n_, t_ in (("q_codes", q_codes), ("k_codes", k_codes), ("q_scales", q_scales),
                   ("k_scales", k_scales), ("v", v), ("seq_offsets", seq_offsets),
                   ("timestamps", timestamps), ("rab_pos", rab_pos), ("rab_time", rab_time),
                   ("num_candidates", num_candidates)):
        _dev(t_, n_)
    if q_codes.stride(0) != k_codes.stride(0):
        raise ValueError("q_codes and k_codes need one row stride")
    T = v.shape[0]
    B = seq_offsets.shape[0] - 1
    if out is None:
        out = torch.empty((T, cfg.H * cfg.d_v), dtype=v.dtype, device=v.device)
    d = attn_desc(cfg, B, T, v.dtype, _rab_stride(rab_pos, rab_time))
    L = _lib.lib()
    nb = L.hstu_attn_fwd_workspace_size(C.byref(d))
    ws = _layer_ws(workspace, nb, v.device, cfg.reuse_plan)
    qk = _lib.AttnMxQK(_ptr(q_codes), _ptr(k_codes), q_codes.stride(0), _ptr(q_scales),
                       _ptr(k_scales))
    st = L.hstu_attn_fwd_mx(C.byref(d), C.byref(qk), _ptr(v), v.stride(0), _ptr(seq_offsets),
                            _ptr(timestamps), _ptr(rab_pos), _ptr(rab_time),
                            _ptr(num_candidates), _ptr(out), out.stride(0), _ptr(ws), ws.numel(),
                            _stream(stream))
    check("hstu_attn_fwd_mx", st)
    return out


def hstu_mx_quantize_weight(w, stream=None):
    """(codes [N, K], scales [N, K/32]) of a bf16 [K, N] weight, blocks along K."""
    K, N = w.shape
    w = w.contiguous()
    codes = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    scales = torch.empty((N, K // 32), dtype=torch.uint8, device=w.device)
    st = _lib.lib().hstu_mx_quantize_weight(K, N, _ptr(w), _ptr(codes), _ptr(scales),
                                            _stream(stream))
    check("hstu_mx_quantize_weight", st)
    return codes, scales


def hstu_mx_gemm(a, a_scales, b, b_scales, stream=None):
    """C [M, N] fp32 = A B^T of MXFP8 A [M, K] and B [N, K]."""
    M, K = a.shape
    N = b.shape[0]
    ldc = (N + 3) // 4 * 4           # fp32 rows are written four values at a time
    c = torch.empty((M, ldc), dtype=torch.float32, device=a.device)
    st = _lib.lib().hstu_mx_gemm(M, N, K, _ptr(a), _ptr(a_scales), _ptr(b), _ptr(b_scales),
                                 _ptr(c), ldc, _stream(stream))
    check("hstu_mx_gemm", st)
    return c[:, :N]


@dataclasses.dataclass
class MxLayerWeights:
    """A layer's MXFP8 weights (codes transposed, blocks along the contraction)."""
    W1: torch.Tensor
    W1_scales: torch.Tensor
    W2: torch.Tensor
    W2_scales: torch.Tensor

    @staticmethod
    def from_bf16(W1, W2, stream=None) -> "MxLayerWeights":
        c1, s1 = hstu_mx_quantize_weight(W1, stream)
        c2, s2 = hstu_mx_quantize_weight(W2, stream)
        return MxLayerWeights(c1, s1, c2, s2)

    def c(self) -> MxWeights:
        return MxWeights(_ptr(self.W1), _ptr(self.W1_scales), _ptr(self.W2), _ptr(self.W2_scales))


def hstu_layer_fwd_mx(x, wm: MxLayerWeights, rab_pos, rab_time, seq_offsets, timestamps,
                      cfg: LayerConfig, num_candidates=None, b1=None, b2=None, gamma=None,
                      beta=None, y=None, workspace: Optional[LayerWorkspace] = None, stream=None,
                      g_out=None, x_mx=None, y_mx=None, saved: Optional["Saved"] = None,
                      mx_scores: bool = False):
    """Y of one layer with MXFP8 projection and output products.
    Optional (codes, scales) pairs: x_mx holds x already in MXFP8 (e.g. the
    previous layer's y_mx), y_mx receives y in MXFP8, g_out the quantized
    gated output the output product used.  saved (training): receives the
    intermediates for hstu_layer_bwd(..., mx=True).  mx_scores (inference):
    the attention's score product in MXFP8 too."""
    T = x.shape[0]
    B = seq_offsets.shape[0] - 1
    if y is None:
        y = torch.empty_like(x)
    d = layer_desc(cfg, B, T, x.dtype, _rab_stride(rab_pos, rab_time))
    L = _lib.lib()
    nb = L.hstu_layer_fwd_mx_workspace_size(C.byref(d))
    ws = _layer_ws(workspace, nb, x.device, cfg.attn.reuse_plan)
    w = _weights(None, None, rab_pos, rab_time, b1, b2, gamma, beta)
    m = wm.c()
    pair = lambda p: (None, None) if p is None else (_ptr(p[0]), _ptr(p[1]))
    io = MxIO(*pair(x_mx), *pair(y_mx), *pair(g_out), 1 if mx_scores else 0)
    sv = saved.c() if saved is not None else None
    st = L.hstu_layer_fwd_mx(C.byref(d), _ptr(x), C.byref(w), C.byref(m), _ptr(seq_offsets),
                             _ptr(timestamps), _ptr(num_candidates), _ptr(y), C.byref(io),
                             C.byref(sv) if sv is not None else None,
                             _ptr(ws), ws.numel(), _stream(stream))
    check("hstu_layer_fwd_mx", st)
    return y


def hstu_truncate_offsets(seq_offsets, keep: int, num_candidates=None, T_seg: Optional[int] = None,
                          stream=None):
    """(seg_offsets [B+1] int32, T_seg) of attention truncation's segments.
    When T_seg is not given it is read back from the device (a synchronisation)."""
    B = seq_offsets.shape[0] - 1
    seg = torch.empty((B + 1,), dtype=torch.int32, device=seq_offsets.device)
    st = _lib.lib().hstu_truncate_offsets(B, _ptr(seq_offsets), _ptr(num_candidates), int(keep),
                                          _ptr(seg), _stream(stream))
    check("hstu_truncate_offsets", st)
    if T_seg is None:
        T_seg = int(seg[B].item())
    return seg, T_seg


def hstu_truncate_gather(x, seq_offsets, seg_offsets, T_seg: int, timestamps=None, stream=None):
    """(x_seg [T_seg, D], ts_seg [T_seg] or None): the rows of the truncated batch."""
    B = seq_offsets.shape[0] - 1
    T, D = x.shape
    xs = torch.empty((T_seg, D), dtype=x.dtype, device=x.device)
    tss = None if timestamps is None else torch.empty((T_seg,), dtype=torch.int64,
                                                       device=x.device)
    st = _lib.lib().hstu_truncate_gather(B, T, T_seg, D, _DT[x.dtype], _ptr(x), _ptr(seq_offsets),
                                         _ptr(seg_offsets), _ptr(timestamps), _ptr(xs), _ptr(tss),
                                         _stream(stream))
    check("hstu_truncate_gather", st)
    return xs, tss


def hstu_truncate_scatter(dx_seg, seq_offsets, seg_offsets, T: int, stream=None):
    """dx [T, D]: dx_seg's rows back at their full-batch rows, zeros elsewhere."""
    B = seq_offsets.shape[0] - 1
    T_seg, D = dx_seg.shape
    dx = torch.empty((T, D), dtype=dx_seg.dtype, device=dx_seg.device)
    st = _lib.lib().hstu_truncate_scatter(B, T, T_seg, D, _DT[dx_seg.dtype], _ptr(dx_seg),
                                          _ptr(seq_offsets), _ptr(seg_offsets), _ptr(dx),
                                          _stream(stream))
    check("hstu_truncate_scatter", st)
    return dx


def hstu_bias_buckets(seq_offsets, timestamps, pair_seq, pair_i, pair_j, cfg: AttnConfig,
                      num_candidates=None, stream=None):
    """(bp, bt) int32 device tensors for the listed (sequence, query row, key row) pairs."""
    T = timestamps.shape[0]
    B = seq_offsets.shape[0] - 1
    n = pair_seq.shape[0]
    dev = timestamps.device
    bp = torch.empty((n,), dtype=torch.int32, device=dev)
    bt = torch.empty((n,), dtype=torch.int32, device=dev)
    d = attn_desc(cfg, B, T, torch.bfloat16, 0)
    L = _lib.lib()
    ws = _ws(L.hstu_attn_fwd_workspace_size(C.byref(d)), dev)
    st = L.hstu_bias_buckets(C.byref(d), _ptr(seq_offsets), _ptr(timestamps),
                             _ptr(num_candidates), _ptr(pair_seq), _ptr(pair_i), _ptr(pair_j), n,
                             _ptr(bp), _ptr(bt), _ptr(ws), ws.numel(), _stream(stream))
    check("hstu_bias_buckets", st)
    return bp, bt


def hstu_schedule(seq_offsets, T: int, block_rows: int, reverse: bool = False, stream=None):
    """(items [n, 2] int32, n) of the device-built jagged work list."""
    B = seq_offsets.shape[0] - 1
    dev = seq_offsets.device
    L = _lib.lib()
    cap = L.hstu_schedule_capacity(T, B, block_rows)
    items = torch.full((cap, 2), -1, dtype=torch.int32, device=dev)
    n = torch.zeros((1,), dtype=torch.int32, device=dev)
    ws = _ws(L.hstu_schedule_workspace_size(B, T, block_rows), dev)
    st = L.hstu_schedule(B, T, _ptr(seq_offsets), block_rows, int(reverse), _ptr(items), _ptr(n),
                         _ptr(ws), ws.numel(), _stream(stream))
    check("hstu_schedule", st)
    return items, n


def hstu_validate_inputs(seq_offsets, T: int, num_candidates=None, stream=None) -> int:
    """Status code of the synchronous device-contract check (0 = ok)."""
    B = seq_offsets.shape[0] - 1
    flag = torch.zeros((1,), dtype=torch.int32, device=seq_offsets.device)
    return _lib.lib().hstu_validate_inputs(B, T, _ptr(seq_offsets), _ptr(num_candidates),
                                           _ptr(flag), _stream(stream))
