"""Pins of the oracle's ranking against a cached history (CPU only).

The cached path must reproduce the candidate rows of the full target-aware
computation on the concatenated sequence [history; candidates]; it is also
checked against a per-pair loop written from the definition (each candidate
sees the whole history at its own position n_h, and itself).
"""
import types

import numpy as np
import pytest

from oracle import hstu as orc
from tests.brute import _floor_log2, _silu


def _users(rng, n_hist, n_cand, H=2, dqk=3, dv=4, D=8):
    """History and candidate rows of each user, and the same users laid out as
    concatenated sequences [history; candidates] with num_candidates."""
    hist_off = np.concatenate([[0], np.cumsum(n_hist)]).astype(np.int64)
    cand_off = np.concatenate([[0], np.cumsum(n_cand)]).astype(np.int64)
    hts, cts = [], []
    for nh, nc in zip(n_hist, n_cand):
        t = 1_600_000_000 + np.floor(np.cumsum(rng.exponential(9.0, size=nh))).astype(np.int64)
        last = t[-1] if nh else 1_600_000_000
        hts.append(t)
        cts.append(last + rng.integers(0, 40, size=nc))   # candidates at or after the history
    hist_ts = np.concatenate(hts).astype(np.int64) if hts else np.zeros(0, np.int64)
    cand_ts = np.concatenate(cts).astype(np.int64) if cts else np.zeros(0, np.int64)
    Xh = rng.standard_normal((int(hist_off[-1]), D))
    Xc = rng.standard_normal((int(cand_off[-1]), D))
    # concatenated layout
    rows_h, rows_c, off = [], [], [0]
    for b in range(len(n_hist)):
        base = off[-1]
        rows_h.append(np.arange(base, base + n_hist[b]))
        rows_c.append(np.arange(base + n_hist[b], base + n_hist[b] + n_cand[b]))
        off.append(base + n_hist[b] + n_cand[b])
    cat = types.SimpleNamespace(
        offsets=np.asarray(off, np.int64), num_candidates=np.asarray(n_cand),
        rows_h=np.concatenate(rows_h).astype(np.int64),
        rows_c=np.concatenate(rows_c).astype(np.int64))
    T = off[-1]
    cat.ts = np.zeros(T, np.int64)
    cat.ts[cat.rows_h] = hist_ts
    cat.ts[cat.rows_c] = cand_ts
    cat.X = np.zeros((T, D))
    cat.X[cat.rows_h] = Xh
    cat.X[cat.rows_c] = Xc
    return hist_off, cand_off, hist_ts, cand_ts, Xh, Xc, cat


CASES = [([7, 0, 12, 3], [2, 3, 1, 0], 0, 0),
         ([9, 5, 200], [3, 1, 4], 0, 0),
         ([9, 5, 200], [3, 1, 4], 4, 2),
         ([30, 1], [5, 2], 1, 0)]


@pytest.mark.parametrize("n_hist,n_cand,wl,wg", CASES)
def test_cached_attention_equals_candidate_rows_of_the_full_pass(n_hist, n_cand, wl, wg):
    rng = np.random.default_rng(sum(n_hist) + wl)
    H, dqk, dv = 2, 3, 4
    hist_off, cand_off, hist_ts, cand_ts, _, _, cat = _users(rng, n_hist, n_cand, H, dqk, dv)
    T = len(cat.ts)
    q = rng.standard_normal((T, H, dqk))
    k = rng.standard_normal((T, H, dqk))
    v = rng.standard_normal((T, H, dv))
    rp, rt = rng.standard_normal((H, 128)), rng.standard_normal((H, 128))
    full = orc.attn_fwd(q, k, v, cat.offsets, cat.ts, rp, rt, cat.num_candidates, 0, 37,
                        win_local=wl, win_global=wg)
    got = orc.attn_fwd_cached(q[cat.rows_c], k[cat.rows_c], v[cat.rows_c], cand_off, cand_ts,
                              k[cat.rows_h], v[cat.rows_h], hist_off, hist_ts, rp, rt, 37, wl, wg)
    np.testing.assert_allclose(got, full[cat.rows_c], rtol=1e-12, atol=1e-13)


def test_cached_attention_matches_a_pair_loop():
    rng = np.random.default_rng(5)
    H, dqk, dv, N = 2, 3, 2, 9.0
    n_hist, n_cand = [6, 0, 140], [2, 2, 3]
    hist_off, cand_off, hist_ts, cand_ts, _, _, _ = _users(rng, n_hist, n_cand, H, dqk, dv)
    Tc, Th = int(cand_off[-1]), int(hist_off[-1])
    q, k, v = (rng.standard_normal((Tc, H, dqk)), rng.standard_normal((Tc, H, dqk)),
               rng.standard_normal((Tc, H, dv)))
    kh, vh = rng.standard_normal((Th, H, dqk)), rng.standard_normal((Th, H, dv))
    rp, rt = rng.standard_normal((H, 128)), rng.standard_normal((H, 128))
    got = orc.attn_fwd_cached(q, k, v, cand_off, cand_ts, kh, vh, hist_off, hist_ts, rp, rt, N)
    want = np.zeros_like(got)
    for b in range(3):
        nh = n_hist[b]
        for r in range(cand_off[b], cand_off[b + 1]):
            for h in range(H):
                acc = np.zeros(dv)
                for j in range(nh):
                    g = hist_off[b] + j
                    dp = min(nh - j, 127)
                    dt = min(max(int(cand_ts[r]) - int(hist_ts[g]), 0), 2 ** 31 - 1)
                    bt = min(_floor_log2(dt + 1), 127)
                    s = float(np.dot(q[r, h], kh[g, h])) + rp[h, dp] + rt[h, bt]
                    acc += _silu(s) * vh[g, h]
                s = float(np.dot(q[r, h], k[r, h])) + rp[h, 0] + rt[h, 0]   # itself
                acc += _silu(s) * v[r, h]
                want[r, h] = acc / N
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("wl,wg", [(0, 0), (5, 2)])
def test_cached_stack_equals_the_target_aware_stack(wl, wg):
    rng = np.random.default_rng(7 + wl)
    H, dqk, dv, D = 2, 3, 4, 8
    n_hist, n_cand = [11, 0, 25, 4], [3, 2, 1, 0]
    hist_off, cand_off, hist_ts, cand_ts, Xh, Xc, cat = _users(rng, n_hist, n_cand, H, dqk, dv, D)
    layers = [types.SimpleNamespace(
        W1=rng.standard_normal((D, H * (2 * dv + 2 * dqk))) / np.sqrt(D),
        W2=rng.standard_normal((H * dv, D)) / np.sqrt(H * dv),
        rab_pos=rng.standard_normal((H, 128)), rab_time=rng.standard_normal((H, 128)))
        for _ in range(3)]
    f = orc.LayerFlags(H=H, d_qk=dqk, d_v=dv, norm_mode=0, norm_len=20, eps=1e-3,
                       win_local=wl, win_global=wg)
    outs = orc.stack_fwd(cat.X, layers, cat.offsets, cat.ts, cat.num_candidates, f)
    caches = orc.history_cache(Xh, layers, hist_off, hist_ts, f)
    got = orc.cached_stack_fwd(Xc, layers, caches, hist_off, hist_ts, cand_off, cand_ts, f)
    np.testing.assert_allclose(got, outs[-1][cat.rows_c], rtol=1e-11, atol=1e-12)
    # the history rows of the full pass are the history-only stack's rows
    hist_only = orc.stack_fwd(Xh, layers, hist_off, hist_ts, None, f)
    np.testing.assert_allclose(outs[-1][cat.rows_h], hist_only[-1], rtol=1e-11, atol=1e-12)
