"""fp64 CPU oracle of the HSTU layer -- TEST INFRASTRUCTURE, NOT PRODUCT CODE.

Only the test suite, the package entry's smoke check and the benchmark's CPU
baseline leg may import this module.  The HIP library never calls it and
shares no code with it; both only consume the seeded inputs made by `synth`.

Pages cited (their text, not line numbers):
  [GR]     NVIDIA generative-recommenders summary (quantumzeitgeist.com),
           section "HSTU Architecture: Efficient Attention for User History".
  [DLRMv4] "DLRMv4 Brings Sequence-Based Recommendation Training to MLPerf"
           (xfinit.ro), sections "Model Architecture", "HSTU Hyperparameters",
           "Computation Cost Analysis" (Tables 6 and 7).
  [ULTRA]  Telegram summary of "Bending the Scaling Law Curve in Large-Scale
           Recommendation Systems" (ULTRA-HSTU), items "Semi-Local Attention",
           "Mixed precision" and "Attention Truncation".
  [MX]     OCP Microscaling Formats (MX) Specification v1.0: FP8 E4M3 element
           encoding, E8M0 shared block scales, the block-scale choice.

What is computed (every array is float64; integer work is exact):

1. Projection ([DLRMv4] "Model Architecture", first bullet; width from
   Table 7's UVQK row): Z = X W1 (+ b1), Zh = SiLU(Z) when proj_silu, split
   column-wise into U | V | Q | K blocks of widths H*d_v, H*d_v, H*d_qk,
   H*d_qk; inside a block head h owns columns h*d .. h*d+d-1.
2. Pointwise attention ([GR]: SiLU weighting instead of softmax plus a
   relative bias; [DLRMv4] "Model Architecture", second bullet: the bias
   comes from positional and temporal distance; Table 7 note: only the lower
   triangle is evaluated; "Model Architecture": candidates appended and
   compared with the history in one pass).  Per sequence of n tokens of which
   the last c are candidates (n_h = n - c), for each head:
       s_ij = q_i . k_j + rab_pos[h, bp(i,j)] + rab_time[h, bt(i,j)]
       a_ij = SiLU(s_ij) / N   if allowed(i, j), else 0
       O_i  = sum_j a_ij v_j
   allowed(i, j): history row i sees history j <= i; a candidate row sees all
   history and itself only.  Semi-local attention ([ULTRA]: a local and a
   global window instead of the full causal mask; window sizes not given, so
   they are parameters W_l, W_g): when W_l > 0 a pair is also required to
   satisfy p(i) - p(j) < W_l (the W_l most recent positions) or j < W_g (the
   first W_g tokens of the sequence).  p(i) = min(i, n_h); bp = min(p(i) - p(j), P-1);
   dt = min(max(ts_i - ts_j, 0), 2^31 - 1); bt = min(floor(log2(dt + 1)), Tb-1).
   N = norm_len (norm_mode 0) or the sequence's own n (norm_mode 1).
3. Gated output ([GR]: elementwise gating before the output projection;
   [DLRMv4] third bullet): LayerNorm over the H*d_v vector of each token
   (biased variance, eps; optional gamma/beta), G = LN(O) * U.
4. Y = G W2 (+ b2) (+ X when residual).  Layers stack Y -> next X.
   Attention truncation ([ULTRA]: after N layers over whole sequences, M
   further layers see only a segment of length L' of each history, taken
   from its most recent events): the segment is read as the last
   min(n_h, L') history tokens followed by the sequence's c candidates, a
   contiguous tail of the sequence that keeps its own timestamps; it is
   attended as a sequence of its own (positions restart, which changes no
   bucket since buckets depend on position differences only).
   Ranking against a cached history: a history row never attends to a
   candidate, so each layer's history keys and values, and the history's
   layer outputs, do not depend on the candidates ([DLRMv4] "Model
   Architecture": candidates appended and compared with the history in one
   pass).  Computed once per history, the per-layer K and V let a batch of
   candidates run through the layers alone: candidate rows at position n_h
   attend to the cached keys and to themselves.  This equals the candidate
   rows of the full target-aware stack when N is a fixed norm_len.
   FP8 matmuls ([ULTRA] "Mixed precision": BF16 for most operations, FP8
   for the matrix products; no scaling recipe given): the projection and
   output matrices are multiplied as MXFP8 ([MX]): every 32 consecutive
   values along the contraction share a power-of-two scale
   2^(floor(log2 amax) - 8) and are rounded to E4M3 (nearest, ties to even,
   saturating at 448); the product of two such operands is computed exactly
   here.  Attention and everything else stay as above, except in
   attn_fwd_mx, where the attention's score product q_i . k_j is an MXFP8
   product too: q and k rounded along their contraction (the d_qk channels
   of each head, in blocks of 32), the rest of step 2 unchanged.
5. Backward: the chain rule of 1-4 written out by hand (no autograd).

Readings where the pages are silent (each is a flag here):
  proj_silu=True, residual=True, no 1/sqrt(d) on q.k, LayerNorm eps=1e-6 with
  no affine by default, clamp-style position buckets, integer log2 time
  buckets, dt = t_query - t_key clamped at 0, per-head bias tables.

Parity status: every function below is pinned by tests in tests/ (brute-force
loops on tiny inputs, closed forms, invariants, finite differences, the
page's Table 7 FLOP totals for the cost model).  The numeric choices listed
as readings above cannot be pinned by any value the pages print; they are
pinned only to their own definitions.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

INT31_MAX = (1 << 31) - 1


# ----------------------------------------------------------------------------
# Elementwise pieces
# ----------------------------------------------------------------------------

def bf16_round(x) -> np.ndarray:
    """x rounded to float32 and then to bfloat16 (8 significant bits), both
    to nearest with ties to even, returned as float64: a finite value
    m 2^e with m in [0.5, 1) becomes rint(256 m) 2^(e - 8)."""
    f = np.asarray(x, np.float64).astype(np.float32).astype(np.float64)
    m, e = np.frexp(f)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def sigmoid(x: np.ndarray) -> np.ndarray:
    """Logistic function via the exact identity 1/(1+e^-x) = (1 + tanh(x/2)) / 2."""
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def silu(x: np.ndarray) -> np.ndarray:
    """SiLU(x) = x * sigmoid(x) ([GR]: the weighting that replaces softmax)."""
    return x * sigmoid(x)


def silu_grad(x: np.ndarray) -> np.ndarray:
    """d/dx SiLU(x) = sigmoid(x) * (1 + x * (1 - sigmoid(x)))."""
    s = sigmoid(x)
    return s * (1.0 + x * (1.0 - s))


# ----------------------------------------------------------------------------
# Relative-bias buckets ([DLRMv4] "Model Architecture": positional and temporal distance)
# ----------------------------------------------------------------------------

def time_bucket(dt: np.ndarray, n_buckets: int = 128) -> np.ndarray:
    """floor(log2(dt + 1)) with dt clamped to [0, 2^31-1], capped at n_buckets-1.

    Computed exactly: frexp of an integer below 2^53 returns its bit length.
    """
    dt = np.clip(np.asarray(dt, dtype=np.int64), 0, INT31_MAX)
    _, e = np.frexp((dt + 1).astype(np.float64))
    return np.minimum(e.astype(np.int64) - 1, n_buckets - 1)


def pos_bucket(dp: np.ndarray, n_buckets: int = 128) -> np.ndarray:
    """Clamp of the (non-negative) position distance to n_buckets-1."""
    return np.minimum(np.maximum(np.asarray(dp, dtype=np.int64), 0), n_buckets - 1)


def positions(n: int, c: int) -> np.ndarray:
    """p(i) = min(i, n_h): candidates all sit at the position after the history."""
    return np.minimum(np.arange(n, dtype=np.int64), n - c)


def allowed_mask(n: int, c: int, rows: Optional[np.ndarray] = None,
                 win_local: int = 0, win_global: int = 0) -> np.ndarray:
    """Boolean [len(rows), n]: causal for history rows, history+self for candidates;
    with win_local > 0 also the semi-local window ([ULTRA] "Semi-Local Attention")."""
    n_h = n - c
    i = np.arange(n) if rows is None else np.asarray(rows)
    j = np.arange(n)
    hist_row = (i < n_h)[:, None]
    causal = j[None, :] <= i[:, None]
    cand = (j[None, :] < n_h) | (j[None, :] == i[:, None])
    M = np.where(hist_row, causal, cand)
    if win_local > 0:
        p = positions(n, c)
        local = (p[i][:, None] - p[None, :]) < win_local
        glob = (j < win_global)[None, :]
        M = M & (local | glob)
    return M


def bias_buckets(ts: np.ndarray, c: int, rows: np.ndarray, n_pos: int, n_time: int):
    """(bp, bt) integer arrays [len(rows), n] for one sequence."""
    n = ts.shape[0]
    p = positions(n, c)
    bp = pos_bucket(p[rows][:, None] - p[None, :], n_pos)
    bt = time_bucket(ts[rows][:, None] - ts[None, :], n_time)
    return bp, bt


# ----------------------------------------------------------------------------
# Attention
# ----------------------------------------------------------------------------

def _norm(n: int, norm_mode: int, norm_len: int) -> float:
    return float(norm_len) if norm_mode == 0 else float(n)


def _seq_iter(seq_offsets, num_candidates):
    B = len(seq_offsets) - 1
    for b in range(B):
        o0, o1 = int(seq_offsets[b]), int(seq_offsets[b + 1])
        c = 0 if num_candidates is None else int(num_candidates[b])
        yield b, o0, o1, c


def _rab(tab: np.ndarray, H: int) -> np.ndarray:
    tab = np.asarray(tab, dtype=np.float64)
    return np.broadcast_to(tab, (H, tab.shape[-1])) if tab.ndim == 1 else tab


def attn_fwd(q, k, v, seq_offsets, timestamps, rab_pos, rab_time,
             num_candidates=None, norm_mode=0, norm_len=1, row_block=1024,
             return_rows=None, win_local=0, win_global=0):
    """O[T, H, d_v] of the pointwise attention (step 2 above).

    q, k: [T, H, d_qk]; v: [T, H, d_v]; rab_pos/rab_time: [H, P] or [P].
    return_rows: optional per-sequence list of local query rows to compute
    (others stay zero) -- used for sampled checks at full size.
    """
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64); v = np.asarray(v, np.float64)
    T, H, _ = q.shape
    dv = v.shape[2]
    rp, rt = _rab(rab_pos, H), _rab(rab_time, H)
    O = np.zeros((T, H, dv))
    for b, o0, o1, c in _seq_iter(seq_offsets, num_candidates):
        n = o1 - o0
        if n == 0:
            continue
        N = _norm(n, norm_mode, norm_len)
        ts = np.asarray(timestamps[o0:o1], np.int64)
        all_rows = np.arange(n) if return_rows is None else np.asarray(return_rows[b], np.int64)
        for r0 in range(0, len(all_rows), row_block):
            rows = all_rows[r0:r0 + row_block]
            M = allowed_mask(n, c, rows, win_local, win_global)
            bp, bt = bias_buckets(ts, c, rows, rp.shape[1], rt.shape[1])
            for h in range(H):
                s = q[o0 + rows, h, :] @ k[o0:o1, h, :].T + rp[h][bp] + rt[h][bt]
                a = np.where(M, silu(s), 0.0) / N
                O[o0 + rows, h, :] = a @ v[o0:o1, h, :]
    return O


def attn_bwd(q, k, v, seq_offsets, timestamps, rab_pos, rab_time, d_out,
             num_candidates=None, norm_mode=0, norm_len=1, row_block=1024,
             win_local=0, win_global=0):
    """(dq, dk, dv, d_rab_pos[H,P], d_rab_time[H,Tb]) for attn_fwd's output gradient."""
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64); v = np.asarray(v, np.float64)
    dO = np.asarray(d_out, np.float64)
    T, H, _ = q.shape
    rp, rt = _rab(rab_pos, H), _rab(rab_time, H)
    P, Tb = rp.shape[1], rt.shape[1]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    drp, drt = np.zeros((H, P)), np.zeros((H, Tb))
    for b, o0, o1, c in _seq_iter(seq_offsets, num_candidates):
        n = o1 - o0
        if n == 0:
            continue
        N = _norm(n, norm_mode, norm_len)
        ts = np.asarray(timestamps[o0:o1], np.int64)
        for r0 in range(0, n, row_block):
            rows = np.arange(r0, min(n, r0 + row_block))
            M = allowed_mask(n, c, rows, win_local, win_global)
            bp, bt = bias_buckets(ts, c, rows, P, Tb)
            for h in range(H):
                s = q[o0 + rows, h, :] @ k[o0:o1, h, :].T + rp[h][bp] + rt[h][bt]
                a = np.where(M, silu(s), 0.0) / N                 # A = SiLU(S) M / N
                dv[o0:o1, h, :] += a.T @ dO[o0 + rows, h, :]      # dV = A^T dO
                da = dO[o0 + rows, h, :] @ v[o0:o1, h, :].T       # dA = dO V^T
                ds = np.where(M, da * silu_grad(s), 0.0) / N      # dS = dA SiLU'(S) M / N
                dq[o0 + rows, h, :] += ds @ k[o0:o1, h, :]        # dQ = dS K
                dk[o0:o1, h, :] += ds.T @ q[o0 + rows, h, :]      # dK = dS^T Q
                drp[h] += np.bincount(bp.ravel(), weights=ds.ravel(), minlength=P)
                drt[h] += np.bincount(bt.ravel(), weights=ds.ravel(), minlength=Tb)
    return dq, dk, dv, drp, drt


# ----------------------------------------------------------------------------
# LayerNorm + gating (step 3)
# ----------------------------------------------------------------------------

def layernorm_fwd(x, eps=1e-6, gamma=None, beta=None):
    """Returns (y, mu, rstd, xhat); normalises over the last axis with biased variance."""
    x = np.asarray(x, np.float64)
    mu = x.mean(axis=-1)
    var = ((x - mu[..., None]) ** 2).mean(axis=-1)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (x - mu[..., None]) * rstd[..., None]
    y = xhat
    if gamma is not None:
        y = y * np.asarray(gamma, np.float64)
    if beta is not None:
        y = y + np.asarray(beta, np.float64)
    return y, mu, rstd, xhat


def layernorm_bwd(dy, xhat, rstd, gamma=None):
    """(dx, dgamma, dbeta) of layernorm_fwd."""
    dy = np.asarray(dy, np.float64)
    dgamma = (dy * xhat).sum(axis=0)
    dbeta = dy.sum(axis=0)
    dxh = dy * np.asarray(gamma, np.float64) if gamma is not None else dy
    m1 = dxh.mean(axis=-1, keepdims=True)
    m2 = (dxh * xhat).mean(axis=-1, keepdims=True)
    dx = rstd[..., None] * (dxh - m1 - xhat * m2)
    return dx, dgamma, dbeta


# ----------------------------------------------------------------------------
# Whole layer
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class LayerFlags:
    H: int
    d_qk: int
    d_v: int
    norm_mode: int = 0
    norm_len: int = 1
    proj_silu: bool = True
    residual: bool = True
    eps: float = 1e-6
    win_local: int = 0     # semi-local attention windows (0: full causal)
    win_global: int = 0


def split_uvqk(Zh: np.ndarray, f: LayerFlags):
    T = Zh.shape[0]
    a, bq = f.H * f.d_v, f.H * f.d_qk
    U = Zh[:, 0:a]
    V = Zh[:, a:2 * a].reshape(T, f.H, f.d_v)
    Q = Zh[:, 2 * a:2 * a + bq].reshape(T, f.H, f.d_qk)
    K = Zh[:, 2 * a + bq:2 * a + 2 * bq].reshape(T, f.H, f.d_qk)
    return U, V, Q, K


def layer_fwd(X, W1, W2, rab_pos, rab_time, seq_offsets, timestamps, num_candidates,
              f: LayerFlags, b1=None, b2=None, gamma=None, beta=None):
    """Y and the saved intermediates of one HSTU layer (steps 1-4)."""
    X = np.asarray(X, np.float64)
    Z = X @ np.asarray(W1, np.float64)
    if b1 is not None:
        Z = Z + np.asarray(b1, np.float64)
    Zh = silu(Z) if f.proj_silu else Z
    U, V, Q, K = split_uvqk(Zh, f)
    O = attn_fwd(Q, K, V, seq_offsets, timestamps, rab_pos, rab_time, num_candidates,
                 f.norm_mode, f.norm_len, win_local=f.win_local, win_global=f.win_global)
    T = X.shape[0]
    O2 = O.reshape(T, f.H * f.d_v)
    Yn, mu, rstd, xhat = layernorm_fwd(O2, f.eps, gamma, beta)
    G = Yn * U
    Y = G @ np.asarray(W2, np.float64)
    if b2 is not None:
        Y = Y + np.asarray(b2, np.float64)
    if f.residual:
        Y = Y + X
    saved = dict(Z=Z, Zh=Zh, O=O2, mu=mu, rstd=rstd, xhat=xhat, Yn=Yn, G=G)
    return Y, saved


def layer_bwd(dY, X, W1, W2, rab_pos, rab_time, seq_offsets, timestamps, num_candidates,
              f: LayerFlags, saved: Dict, b1=None, b2=None, gamma=None, beta=None,
              act_matmul=None, wgt_matmul=None):
    """All gradients of one layer, by the chain rule written out (step 5).
    act_matmul (default: the exact product) computes the two products that
    carry the activation gradients back, dG = dY W2^T and dX = dZ W1^T;
    wgt_matmul (default: exact) the two weight gradients dW2 = G^T dY and
    dW1 = X^T dZ, contracted over the tokens (layer_bwd_mx passes the MXFP8
    product for all four)."""
    mm = act_matmul if act_matmul is not None else (lambda a, b: a @ b)
    wm = wgt_matmul if wgt_matmul is not None else (lambda a, b: a @ b)
    dY = np.asarray(dY, np.float64)
    X = np.asarray(X, np.float64)
    W1 = np.asarray(W1, np.float64); W2 = np.asarray(W2, np.float64)
    T = X.shape[0]
    U, V, Q, K = split_uvqk(saved["Zh"], f)
    # Y = G W2 + b2 (+ X)
    dG = mm(dY, W2.T)
    dW2 = wm(saved["G"].T, dY)
    db2 = dY.sum(axis=0)
    # G = Yn * U
    dU = dG * saved["Yn"]
    dYn = dG * U
    # Yn = LN(O)
    dO2, dgamma, dbeta = layernorm_bwd(dYn, saved["xhat"], saved["rstd"], gamma)
    dO = dO2.reshape(T, f.H, f.d_v)
    dQ, dK, dV, drp, drt = attn_bwd(Q, K, V, seq_offsets, timestamps, rab_pos, rab_time, dO,
                                    num_candidates, f.norm_mode, f.norm_len,
                                    win_local=f.win_local, win_global=f.win_global)
    dZh = np.concatenate([dU, dV.reshape(T, -1), dQ.reshape(T, -1), dK.reshape(T, -1)], axis=1)
    dZ = dZh * silu_grad(saved["Z"]) if f.proj_silu else dZh
    dW1 = wm(X.T, dZ)
    db1 = dZ.sum(axis=0)
    dX = mm(dZ, W1.T)
    if f.residual:
        dX = dX + dY
    return dict(dX=dX, dW1=dW1, dW2=dW2, db1=db1, db2=db2, dgamma=dgamma, dbeta=dbeta,
                drab_pos=drp, drab_time=drt, dZ=dZ, dO=dO2, dG=dG)


def stack_fwd(X, layers: List, seq_offsets, timestamps, num_candidates, f: LayerFlags):
    """Layers stacked: the output of layer l is the input of layer l+1.

    `layers` holds objects with W1, W2, rab_pos, rab_time attributes.
    Returns the list of per-layer outputs.
    """
    outs = []
    x = np.asarray(X, np.float64)
    for w in layers:
        x, _ = layer_fwd(x, w.W1, w.W2, w.rab_pos, w.rab_time, seq_offsets, timestamps,
                         num_candidates, f)
        outs.append(x)
    return outs


# ----------------------------------------------------------------------------
# Attention truncation ([ULTRA] "Attention Truncation")
# ----------------------------------------------------------------------------

def truncate_rows(seq_offsets, num_candidates, keep: int):
    """(seg_offsets [B+1], rows [T_seg]) of the truncated batch: sequence b's
    segment is its last min(n_h, keep) history rows followed by its c_b
    candidate rows; rows[r] is the source row of segment row r."""
    offs = np.asarray(seq_offsets, np.int64)
    B = len(offs) - 1
    seg = np.zeros(B + 1, np.int64)
    parts = []
    for b in range(B):
        n = int(offs[b + 1] - offs[b])
        c = 0 if num_candidates is None else int(num_candidates[b])
        m = min(n - c, keep) + c
        parts.append(np.arange(offs[b + 1] - m, offs[b + 1], dtype=np.int64))
        seg[b + 1] = seg[b] + m
    rows = np.concatenate(parts) if parts else np.zeros(0, np.int64)
    return seg, rows


def truncated_stack_fwd(X, full_layers: List, tail_layers: List, seq_offsets, timestamps,
                        num_candidates, f_full: LayerFlags, f_tail: LayerFlags, keep: int):
    """N layers over the whole sequences, then M layers over the truncated
    segments.  Returns (Y_seg [T_seg, D], record for truncated_stack_bwd)."""
    x = np.asarray(X, np.float64)
    ts = np.asarray(timestamps, np.int64)
    full = []
    for w in full_layers:
        y, sv = layer_fwd(x, w.W1, w.W2, w.rab_pos, w.rab_time, seq_offsets, ts,
                          num_candidates, f_full)
        full.append((x, sv))
        x = y
    seg, rows = truncate_rows(seq_offsets, num_candidates, keep)
    ts_seg = ts[rows]
    x = x[rows]
    tail = []
    for w in tail_layers:
        y, sv = layer_fwd(x, w.W1, w.W2, w.rab_pos, w.rab_time, seg, ts_seg, num_candidates,
                          f_tail)
        tail.append((x, sv))
        x = y
    rec = dict(full=full, tail=tail, seg_offsets=seg, rows=rows, ts_seg=ts_seg,
               T=int(np.asarray(X).shape[0]))
    return x, rec


def truncated_stack_bwd(dY_seg, full_layers: List, tail_layers: List, seq_offsets, timestamps,
                        num_candidates, f_full: LayerFlags, f_tail: LayerFlags, rec: Dict):
    """Gradients of truncated_stack_fwd for the segment-output gradient dY_seg:
    (dX [T, D], per-layer gradient dicts of the full layers, of the tail layers).
    Rows outside the segments receive no gradient from the tail layers."""
    g = np.asarray(dY_seg, np.float64)
    g_tail = [None] * len(tail_layers)
    for l in range(len(tail_layers) - 1, -1, -1):
        w = tail_layers[l]
        x, sv = rec["tail"][l]
        r = layer_bwd(g, x, w.W1, w.W2, w.rab_pos, w.rab_time, rec["seg_offsets"],
                      rec["ts_seg"], num_candidates, f_tail, sv)
        g_tail[l] = r
        g = r["dX"]
    dx = np.zeros((rec["T"], g.shape[1]), np.float64)
    dx[rec["rows"]] = g
    g_full = [None] * len(full_layers)
    for l in range(len(full_layers) - 1, -1, -1):
        w = full_layers[l]
        x, sv = rec["full"][l]
        r = layer_bwd(dx, x, w.W1, w.W2, w.rab_pos, w.rab_time, seq_offsets, timestamps,
                      num_candidates, f_full, sv)
        g_full[l] = r
        dx = r["dX"]
    return dx, g_full, g_tail


# ----------------------------------------------------------------------------
# Ranking against a cached history ([DLRMv4] "Model Architecture": appended
# candidates compared with the history; the history part computed once)
# ----------------------------------------------------------------------------

def attn_fwd_cached(q, k, v, cand_offsets, cand_ts, k_hist, v_hist, hist_offsets, hist_ts,
                    rab_pos, rab_time, norm_len=1, win_local=0, win_global=0):
    """O[T_c, H, d_v] of candidate rows scored against a cached history.

    User b's candidates (rows cand_offsets[b] .. cand_offsets[b+1]) sit at
    position n_h = hist_offsets[b+1] - hist_offsets[b] and attend to each
    history key j of the user (when W_l > 0 only if n_h - j < W_l or
    j < W_g) and to their own key, never to another candidate.
    q, k, v: the candidates' own rows [T_c, H, d]; k_hist, v_hist: [T_h, H, d].
    """
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64); v = np.asarray(v, np.float64)
    kh = np.asarray(k_hist, np.float64); vh = np.asarray(v_hist, np.float64)
    Tc, H, _ = q.shape
    rp, rt = _rab(rab_pos, H), _rab(rab_time, H)
    P, Tb = rp.shape[1], rt.shape[1]
    O = np.zeros((Tc, H, v.shape[2]))
    N = float(norm_len)
    bp_self = pos_bucket(np.array(0), P)
    bt_self = time_bucket(np.array(0), Tb)
    for b in range(len(cand_offsets) - 1):
        c0, c1 = int(cand_offsets[b]), int(cand_offsets[b + 1])
        h0, h1 = int(hist_offsets[b]), int(hist_offsets[b + 1])
        if c1 == c0:
            continue
        nh = h1 - h0
        j = np.arange(nh)
        keep = np.ones(nh, bool) if win_local <= 0 else (nh - j < win_local) | (j < win_global)
        bp = pos_bucket(nh - j, P)                                            # [n_h]
        bt = time_bucket(np.asarray(cand_ts[c0:c1], np.int64)[:, None]
                         - np.asarray(hist_ts[h0:h1], np.int64)[None, :], Tb)  # [c, n_h]
        for h in range(H):
            s_hist = q[c0:c1, h, :] @ kh[h0:h1, h, :].T + rp[h][bp][None, :] + rt[h][bt]
            a_hist = np.where(keep[None, :], silu(s_hist), 0.0) / N
            s_self = np.sum(q[c0:c1, h, :] * k[c0:c1, h, :], axis=1) + rp[h][bp_self] + rt[h][bt_self]
            O[c0:c1, h, :] = a_hist @ vh[h0:h1, h, :] + (silu(s_self) / N)[:, None] * v[c0:c1, h, :]
    return O


def layer_fwd_cached(Xc, W1, W2, rab_pos, rab_time, k_hist, v_hist, hist_offsets, hist_ts,
                     cand_offsets, cand_ts, f: LayerFlags, b1=None, b2=None, gamma=None,
                     beta=None):
    """One layer over candidate rows only, attention against this layer's
    cached history keys and values (steps 1-4 with attn_fwd_cached)."""
    Xc = np.asarray(Xc, np.float64)
    Z = Xc @ np.asarray(W1, np.float64)
    if b1 is not None:
        Z = Z + np.asarray(b1, np.float64)
    Zh = silu(Z) if f.proj_silu else Z
    U, V, Q, K = split_uvqk(Zh, f)
    O = attn_fwd_cached(Q, K, V, cand_offsets, cand_ts, k_hist, v_hist, hist_offsets, hist_ts,
                        rab_pos, rab_time, f.norm_len, f.win_local, f.win_global)
    Yn, _, _, _ = layernorm_fwd(O.reshape(Xc.shape[0], f.H * f.d_v), f.eps, gamma, beta)
    Y = (Yn * U) @ np.asarray(W2, np.float64)
    if b2 is not None:
        Y = Y + np.asarray(b2, np.float64)
    if f.residual:
        Y = Y + Xc
    return Y


def history_cache(Xh, layers: List, hist_offsets, hist_ts, f: LayerFlags):
    """Per layer (K_hist, V_hist) of the history run through the stack alone."""
    caches = []
    x = np.asarray(Xh, np.float64)
    for w in layers:
        y, sv = layer_fwd(x, w.W1, w.W2, w.rab_pos, w.rab_time, hist_offsets, hist_ts, None, f)
        _, V, _, K = split_uvqk(sv["Zh"], f)
        caches.append((K, V))
        x = y
    return caches


def cached_stack_fwd(Xc, layers: List, caches: List, hist_offsets, hist_ts, cand_offsets,
                     cand_ts, f: LayerFlags):
    """Candidate rows through the stack against the per-layer history caches."""
    x = np.asarray(Xc, np.float64)
    for w, (K, V) in zip(layers, caches):
        x = layer_fwd_cached(x, w.W1, w.W2, w.rab_pos, w.rab_time, K, V, hist_offsets, hist_ts,
                             cand_offsets, cand_ts, f)
    return x


# ----------------------------------------------------------------------------
# MXFP8 matmuls ([ULTRA] "Mixed precision"; [MX] element and scale formats)
# ----------------------------------------------------------------------------

E4M3_MAX = 448.0
MX_BLOCK = 32
E4M3_EMAX = 8          # exponent of the largest power of two in E4M3 (256)


def e4m3_decode(codes) -> np.ndarray:
    """Values of FP8 E4M3 codes ([MX] element format: 1 sign bit, 4 exponent
    bits with bias 7, 3 mantissa bits, subnormals at exponent 0, no
    infinities, S.1111.111 is NaN)."""
    c = np.asarray(codes, np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


_E4M3_POS = e4m3_decode(np.arange(0x7F))    # the 127 non-negative finite values, increasing


def e4m3_encode(x) -> np.ndarray:
    """Codes of x rounded to the nearest E4M3 value, ties to the even code
    (even mantissa), magnitudes above 448 saturated to 448."""
    x = np.asarray(x, np.float64)
    ax = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, ax)            # first value >= |x|
    hi = np.minimum(hi, len(_E4M3_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = ax - _E4M3_POS[lo]
    dhi = _E4M3_POS[hi] - ax
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(_E4M3_POS[hi] == ax, hi, np.where(pick_hi, hi, lo))
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def mx_quantize(x, axis=-1):
    """MXFP8 of x along `axis` (its length a multiple of 32): (codes uint8
    like x, E8M0 scale bytes with one entry per block of 32 along the axis).
    Block scale X = 2^(floor(log2(amax)) - 8) ([MX]: shared exponent from the
    largest magnitude minus the element format's largest exponent); an
    all-zero block gets the smallest scale 2^-127 and zero codes."""
    x = np.asarray(x, np.float64)
    xm = np.moveaxis(x, axis, -1)
    n = xm.shape[-1]
    assert n % MX_BLOCK == 0
    blk = xm.reshape(xm.shape[:-1] + (n // MX_BLOCK, MX_BLOCK))
    amax = np.max(np.abs(blk), axis=-1)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))      # amax = f * 2^ex, f in [0.5, 1)
    shared = np.where(amax > 0, (ex - 1) - E4M3_EMAX, -127)
    shared = np.clip(shared, -127, 127)
    codes = e4m3_encode(blk / np.exp2(shared)[..., None])
    codes = np.moveaxis(codes.reshape(xm.shape), -1, axis)
    scales = np.moveaxis((shared + 127).astype(np.uint8), -1, axis)
    return codes, scales


def mx_dequantize(codes, scales, axis=-1):
    """Values of MXFP8 data (inverse of mx_quantize's encoding)."""
    c = np.moveaxis(np.asarray(codes), axis, -1)
    s = np.moveaxis(np.asarray(scales, np.int64), axis, -1)
    v = e4m3_decode(c).reshape(c.shape[:-1] + (s.shape[-1], MX_BLOCK))
    v = v * np.exp2(s - 127.0)[..., None]
    return np.moveaxis(v.reshape(c.shape), -1, axis)


def mx_matmul(a, b):
    """a @ b with both operands rounded to MXFP8 along the contraction (a's
    rows, b's columns), the products summed exactly.  A contraction whose
    length is not a multiple of 32 ends in a short block, read as padded
    with zeros (zeros change neither a block's largest magnitude nor the
    product)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    k = a.shape[1]
    kp = -(-k // MX_BLOCK) * MX_BLOCK
    if kp != k:
        a = np.pad(a, ((0, 0), (0, kp - k)))
        b = np.pad(b, ((0, kp - k), (0, 0)))
    qa, sa = mx_quantize(a, axis=1)
    qb, sb = mx_quantize(b, axis=0)
    return mx_dequantize(qa, sa, axis=1) @ mx_dequantize(qb, sb, axis=0)


def layer_fwd_mx(X, W1, W2, rab_pos, rab_time, seq_offsets, timestamps, num_candidates,
                 f: LayerFlags, b1=None, b2=None, gamma=None, beta=None, return_g=False,
                 return_saved=False, mx_scores=False):
    """One layer with MXFP8 projection and output matmuls (steps 1 and 4);
    attention, LayerNorm and gating as in layer_fwd.  return_g: also the
    gated output G before its quantization; return_saved: also the
    intermediates layer_bwd_mx needs (as layer_fwd's).  mx_scores: the
    attention's score product in MXFP8 as well (attn_fwd_mx; no windows).
    Reading: q and k are quantized from the layer's stored bf16 U|V|Q|K
    (bf16_round of Zh), the precision in which the kernels decide those
    codes; in training (return_saved) the saved Zh holds q and k as those
    MXFP8 values, so layer_bwd_mx differentiates the scores the forward
    computed, the quantizer counting as the identity (as O31's)."""
    X = np.asarray(X, np.float64)
    Z = mx_matmul(X, W1)
    if b1 is not None:
        Z = Z + np.asarray(b1, np.float64)
    Zh = silu(Z) if f.proj_silu else Z
    U, V, Q, K = split_uvqk(Zh, f)
    if mx_scores:
        assert f.win_local == 0
        qc, qs = mx_quantize(bf16_round(Q), axis=2)
        kc, ks = mx_quantize(bf16_round(K), axis=2)
        Qm, Km = mx_dequantize(qc, qs, axis=2), mx_dequantize(kc, ks, axis=2)
        O = attn_fwd(Qm, Km, V, seq_offsets, timestamps, rab_pos, rab_time, num_candidates,
                     f.norm_mode, f.norm_len)
        T = X.shape[0]
        Zh = np.concatenate([U.reshape(T, -1), V.reshape(T, -1), Qm.reshape(T, -1),
                             Km.reshape(T, -1)], axis=1)
    else:
        O = attn_fwd(Q, K, V, seq_offsets, timestamps, rab_pos, rab_time, num_candidates,
                     f.norm_mode, f.norm_len, win_local=f.win_local, win_global=f.win_global)
    O2 = O.reshape(X.shape[0], f.H * f.d_v)
    Yn, mu, rstd, xhat = layernorm_fwd(O2, f.eps, gamma, beta)
    G = Yn * U
    Y = mx_matmul(G, W2)
    if b2 is not None:
        Y = Y + np.asarray(b2, np.float64)
    if f.residual:
        Y = Y + X
    if return_saved:
        return Y, dict(Z=Z, Zh=Zh, O=O2, mu=mu, rstd=rstd, xhat=xhat, Yn=Yn, G=G)
    return (Y, G) if return_g else Y


def layer_bwd_mx(dY, X, W1, W2, rab_pos, rab_time, seq_offsets, timestamps, num_candidates,
                 f: LayerFlags, saved: Dict, b1=None, b2=None, gamma=None, beta=None):
    """Gradients of layer_fwd_mx for training with FP8 matmuls ([ULTRA] "Mixed
    precision": the matrix products in FP8, the rest in BF16).  Reading:
    all four products of the backward are MXFP8 products, each operand
    rounded along its own contraction (the forward's recipe): dG = dY W2^T
    and dX = dZ W1^T (blocks along D and along F1), and the weight gradients
    dW2 = G^T dY and dW1 = X^T dZ (blocks of 32 tokens along the token
    index, a short last block read as zero-padded); the quantizers count as
    the identity in the chain rule (the forward's rounding is not
    differentiated).  `saved` from layer_fwd_mx(..., return_saved=True)."""
    return layer_bwd(dY, X, W1, W2, rab_pos, rab_time, seq_offsets, timestamps,
                     num_candidates, f, saved, b1, b2, gamma, beta, act_matmul=mx_matmul,
                     wgt_matmul=mx_matmul)


def attn_fwd_mx(q, k, v, seq_offsets, timestamps, rab_pos, rab_time,
                num_candidates=None, norm_mode=0, norm_len=1, return_rows=None):
    """attn_fwd with the score product in MXFP8 ([ULTRA] "Mixed precision":
    the matrix products in FP8).  q and k [T, H, d_qk] are rounded to MXFP8
    along their contraction index, the d_qk channels of one head (d_qk a
    multiple of 32: whole blocks per head), and their products summed
    exactly; bias, SiLU, mask, normalisation and the product with v follow
    attn_fwd unchanged.  Reading: of the attention's two products only the
    score product q_i . k_j is taken in FP8 (v keeps the precision of the
    rest of the layer)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    assert q.shape[2] % MX_BLOCK == 0
    qc, qs = mx_quantize(q, axis=2)
    kc, ks = mx_quantize(k, axis=2)
    return attn_fwd(mx_dequantize(qc, qs, axis=2), mx_dequantize(kc, ks, axis=2), v,
                    seq_offsets, timestamps, rab_pos, rab_time, num_candidates,
                    norm_mode, norm_len, return_rows=return_rows)
