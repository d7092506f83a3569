"""Per-pair Python loops written from the layer's prose definition.

They serve only as an independent check of the vectorised oracle on tiny
inputs: every index, mask and bucket is spelled out element by element, with
the integer log2 taken by repeated halving.
"""
import math

import numpy as np


def _floor_log2(x: int) -> int:
    r = 0
    while x > 1:
        x >>= 1
        r += 1
    return r


def _silu(s: float) -> float:
    if s < -700.0:
        return 0.0
    return s / (1.0 + math.exp(-s))


def _silu_prime(s: float) -> float:
    sg = 1.0 / (1.0 + math.exp(-s)) if s > -700.0 else 0.0
    return sg + s * sg * (1.0 - sg)


def _pair_ok(i, j, n_h, win_local=0, win_global=0):
    if i < n_h:            # history token: itself and everything before it
        ok = j <= i
    else:
        ok = j < n_h or j == i   # candidate: whole history plus itself
    if ok and win_local > 0:
        # semi-local: the key is one of the win_local most recent positions
        # seen from the query, or one of the first win_global tokens
        pi = i if i < n_h else n_h
        pj = j if j < n_h else n_h
        in_local = (pi - pj) < win_local
        in_global = j < win_global
        ok = in_local or in_global
    return ok


def _bias(i, j, n_h, ts, h, rp, rt):
    pi = i if i < n_h else n_h
    pj = j if j < n_h else n_h
    dp = pi - pj
    if dp > rp.shape[1] - 1:
        dp = rp.shape[1] - 1
    dt = int(ts[i]) - int(ts[j])
    if dt < 0:
        dt = 0
    if dt > 2 ** 31 - 1:
        dt = 2 ** 31 - 1
    bt = _floor_log2(dt + 1)
    if bt > rt.shape[1] - 1:
        bt = rt.shape[1] - 1
    return rp[h, dp] + rt[h, bt], dp, bt


def brute_attn_fwd(q, k, v, offs, ts, rp, rt, cands, norm_mode, norm_len, win_local=0,
                   win_global=0):
    T, H, dqk = q.shape
    dv = v.shape[2]
    out = np.zeros((T, H, dv))
    for b in range(len(offs) - 1):
        o0, o1 = int(offs[b]), int(offs[b + 1])
        n = o1 - o0
        c = 0 if cands is None else int(cands[b])
        n_h = n - c
        N = norm_len if norm_mode == 0 else n
        for i in range(n):
            for h in range(H):
                acc = [0.0] * dv
                for j in range(n):
                    if not _pair_ok(i, j, n_h, win_local, win_global):
                        continue
                    s = 0.0
                    for cc in range(dqk):
                        s += q[o0 + i, h, cc] * k[o0 + j, h, cc]
                    bias, _, _ = _bias(i, j, n_h, ts[o0:o1], h, rp, rt)
                    w = _silu(s + bias) / N
                    for cc in range(dv):
                        acc[cc] += w * v[o0 + j, h, cc]
                out[o0 + i, h, :] = acc
    return out


def brute_attn_bwd(q, k, v, offs, ts, rp, rt, dO, cands, norm_mode, norm_len, win_local=0,
                   win_global=0):
    """Gradients accumulated pair by pair: dV_j += a dO_i, dq_i += ds k_j, ..."""
    T, H, dqk = q.shape
    dv_ = v.shape[2]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    drp, drt = np.zeros_like(rp), np.zeros_like(rt)
    for b in range(len(offs) - 1):
        o0, o1 = int(offs[b]), int(offs[b + 1])
        n = o1 - o0
        c = 0 if cands is None else int(cands[b])
        n_h = n - c
        N = norm_len if norm_mode == 0 else n
        for i in range(n):
            for j in range(n):
                if not _pair_ok(i, j, n_h, win_local, win_global):
                    continue
                for h in range(H):
                    s = sum(q[o0 + i, h, cc] * k[o0 + j, h, cc] for cc in range(dqk))
                    bias, bp, bt = _bias(i, j, n_h, ts[o0:o1], h, rp, rt)
                    s += bias
                    a = _silu(s) / N
                    da = sum(dO[o0 + i, h, cc] * v[o0 + j, h, cc] for cc in range(dv_))
                    ds = da * _silu_prime(s) / N
                    for cc in range(dv_):
                        dv[o0 + j, h, cc] += a * dO[o0 + i, h, cc]
                    for cc in range(dqk):
                        dq[o0 + i, h, cc] += ds * k[o0 + j, h, cc]
                        dk[o0 + j, h, cc] += ds * q[o0 + i, h, cc]
                    drp[h, bp] += ds
                    drt[h, bt] += ds
    return dq, dk, dv, drp, drt


def brute_layernorm(x, eps):
    out = np.zeros_like(x)
    for t in range(x.shape[0]):
        row = [float(a) for a in x[t]]
        m = sum(row) / len(row)
        var = sum((a - m) ** 2 for a in row) / len(row)
        out[t] = [(a - m) / math.sqrt(var + eps) for a in row]
    return out


def brute_matmul(a, b):
    M, K = a.shape
    K2, N = b.shape
    assert K == K2
    out = np.zeros((M, N))
    for i in range(M):
        for j in range(N):
            s = 0.0
            for kk in range(K):
                s += a[i, kk] * b[kk, j]
            out[i, j] = s
    return out
