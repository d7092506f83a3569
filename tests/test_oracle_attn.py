"""Pins of the oracle's attention (CPU only).

Each check compares the vectorised fp64 oracle with something that is not the
oracle: per-pair Python loops written from the definition, a dense closed
form, a closed form for one token, or an invariant of the method (causality,
jagged == padded, candidate isolation and equivalence).
"""
import math
import os

import numpy as np
import pytest

from oracle import hstu as orc
from tests.brute import brute_attn_fwd

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _read_pairs(name):
    out = []
    with open(os.path.join(GOLD, name)) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b = line.split()
            out.append((int(a), int(b)))
    return out


def _rand_case(rng, lengths, H=2, dqk=4, dv=3, cands=None, scale=1.0, P=128, Tb=128,
               gap=60.0):
    lengths = np.asarray(lengths)
    offs = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(offs[-1])
    q = rng.standard_normal((T, H, dqk)) * scale
    k = rng.standard_normal((T, H, dqk)) * scale
    v = rng.standard_normal((T, H, dv))
    ts = []
    for b, n in enumerate(lengths):
        c = 0 if cands is None else cands[b]
        t = 1_650_000_000 + np.floor(np.cumsum(rng.exponential(gap, size=n - c))).astype(np.int64)
        if c:
            t = np.concatenate([t, np.full(c, t[-1] if n - c else 1_650_000_000)])
        ts.append(t)
    ts = np.concatenate(ts).astype(np.int64)
    rp = rng.standard_normal((H, P))
    rt = rng.standard_normal((H, Tb))
    return q, k, v, offs, ts, rp, rt


def test_time_bucket_golden():
    pairs = _read_pairs("time_buckets.txt")
    dt = np.array([p[0] for p in pairs], dtype=np.int64)
    want = np.array([p[1] for p in pairs])
    np.testing.assert_array_equal(orc.time_bucket(dt, 128), want)


def test_time_bucket_small_table_cap():
    # a table with fewer buckets caps the index at its last entry
    assert orc.time_bucket(np.array([10 ** 9]), 8)[0] == 7


def test_pos_bucket_golden():
    pairs = _read_pairs("pos_buckets.txt")
    dp = np.array([p[0] for p in pairs], dtype=np.int64)
    want = np.array([p[1] for p in pairs])
    np.testing.assert_array_equal(orc.pos_bucket(dp, 128), want)


def test_time_bucket_exhaustive_boundaries():
    # every power-of-two boundary up to 2^31: 2^k - 1 -> k, 2^k - 2 -> k - 1
    for kk in range(1, 32):
        x = (1 << kk)
        assert orc.time_bucket(np.array([x - 1]))[0] == kk
        assert orc.time_bucket(np.array([x - 2]))[0] == kk - 1


@pytest.mark.parametrize("cands", [None, [0, 2, 3]])
def test_attention_matches_brute_force(cands):
    rng = np.random.default_rng(11)
    lengths = [5, 7, 9]
    q, k, v, offs, ts, rp, rt = _rand_case(rng, lengths, cands=cands, scale=0.7, gap=3.0)
    for norm_mode, N in [(0, 13), (1, 0)]:
        got = orc.attn_fwd(q, k, v, offs, ts, rp, rt, cands, norm_mode, N)
        want = brute_attn_fwd(q, k, v, offs, ts, rp, rt, cands, norm_mode, N)
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_attention_long_distances_hit_clamped_buckets():
    # sequences longer than the position table and timestamps far apart
    rng = np.random.default_rng(5)
    lengths = [140, 3]
    q, k, v, offs, ts, rp, rt = _rand_case(rng, lengths, H=1, dqk=2, dv=2, scale=0.5,
                                           gap=3.0e7)
    got = orc.attn_fwd(q, k, v, offs, ts, rp, rt, None, 0, 200)
    want = brute_attn_fwd(q, k, v, offs, ts, rp, rt, None, 0, 200)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_zero_bias_is_plain_silu_attention():
    rng = np.random.default_rng(3)
    n = 11
    q, k, v, offs, ts, rp, rt = _rand_case(rng, [n], H=1, dqk=6, dv=5)
    rp[:] = 0.0
    rt[:] = 0.0
    got = orc.attn_fwd(q, k, v, offs, ts, rp, rt, None, 0, 17)[:, 0, :]
    S = q[:, 0, :] @ k[:, 0, :].T
    M = np.tril(np.ones((n, n)))
    dense = (S / (1.0 + np.exp(-S))) * M @ v[:, 0, :] / 17
    np.testing.assert_allclose(got, dense, rtol=1e-13, atol=1e-14)


def test_single_token_closed_form():
    rng = np.random.default_rng(4)
    q, k, v, offs, ts, rp, rt = _rand_case(rng, [1], H=2, dqk=3, dv=4)
    got = orc.attn_fwd(q, k, v, offs, ts, rp, rt, None, 0, 7)
    for h in range(2):
        s = float(q[0, h] @ k[0, h]) + rp[h, 0] + rt[h, 0]
        w = s / (1.0 + math.exp(-s)) / 7
        np.testing.assert_allclose(got[0, h], w * v[0, h], rtol=1e-14)


def test_causality_exact():
    rng = np.random.default_rng(6)
    n = 24
    q, k, v, offs, ts, rp, rt = _rand_case(rng, [n], H=2, dqk=4, dv=4)
    base = orc.attn_fwd(q, k, v, offs, ts, rp, rt, None, 0, 32)
    for cut in (0, 5, 17):
        q2, k2, v2, ts2 = q.copy(), k.copy(), v.copy(), ts.copy()
        q2[cut + 1:] += 1.0
        k2[cut + 1:] -= 2.0
        v2[cut + 1:] *= 3.0
        ts2[cut + 1:] += 10_000
        pert = orc.attn_fwd(q2, k2, v2, offs, ts2, rp, rt, None, 0, 32)
        assert np.array_equal(pert[:cut + 1], base[:cut + 1])
        assert not np.allclose(pert[cut + 1:], base[cut + 1:])


def test_jagged_equals_padded():
    rng = np.random.default_rng(7)
    lengths = np.array([3, 8, 1, 6])
    cands = [0, 3, 0, 2]
    H, dqk, dv = 2, 4, 3
    q, k, v, offs, ts, rp, rt = _rand_case(rng, lengths, H, dqk, dv, cands=cands)
    N = 10
    jag = orc.attn_fwd(q, k, v, offs, ts, rp, rt, cands, 0, N)
    B, nmax = len(lengths), int(lengths.max())
    Qp = np.zeros((B, nmax, H, dqk)); Kp = np.zeros_like(Qp); Vp = np.zeros((B, nmax, H, dv))
    Tp = np.zeros((B, nmax), dtype=np.int64)
    for b in range(B):
        o0, o1 = offs[b], offs[b + 1]
        Qp[b, :o1 - o0] = q[o0:o1]; Kp[b, :o1 - o0] = k[o0:o1]; Vp[b, :o1 - o0] = v[o0:o1]
        Tp[b, :o1 - o0] = ts[o0:o1]
    idx = np.arange(nmax)
    n_b = lengths[:, None, None]
    nh_b = (lengths - np.asarray(cands))[:, None, None]
    I, J = idx[None, :, None], idx[None, None, :]
    valid = (I < n_b) & (J < n_b)
    mask = valid & np.where(I < nh_b, J <= I, (J < nh_b) | (J == I))
    pI, pJ = np.minimum(I, nh_b), np.minimum(J, nh_b)
    bp = np.minimum(np.maximum(pI - pJ, 0), 127)
    dt = np.clip(Tp[:, :, None] - Tp[:, None, :], 0, 2 ** 31 - 1)
    bt = np.minimum(np.floor(np.log2(dt + 1.0)).astype(np.int64), 127)
    out = np.zeros((B, nmax, H, dv))
    for h in range(H):
        S = np.einsum("bic,bjc->bij", Qp[:, :, h], Kp[:, :, h]) + rp[h][bp] + rt[h][bt]
        A = np.where(mask, S / (1 + np.exp(-S)), 0.0) / N
        out[:, :, h] = np.einsum("bij,bjc->bic", A, Vp[:, :, h])
    for b in range(B):
        np.testing.assert_allclose(jag[offs[b]:offs[b + 1]], out[b, :lengths[b]],
                                   rtol=1e-12, atol=1e-14)


def test_candidates_do_not_attend_to_each_other():
    rng = np.random.default_rng(8)
    n, c = 12, 4
    q, k, v, offs, ts, rp, rt = _rand_case(rng, [n], cands=[c])
    base = orc.attn_fwd(q, k, v, offs, ts, rp, rt, [c], 0, 16)
    for cand in range(n - c, n):
        k2, v2 = k.copy(), v.copy()
        k2[cand] += 5.0
        v2[cand] -= 4.0
        pert = orc.attn_fwd(q, k2, v2, offs, ts, rp, rt, [c], 0, 16)
        diff = np.abs(pert - base).reshape(n, -1).max(axis=1)
        changed = set(np.nonzero(diff > 0)[0].tolist())
        assert changed == {cand}


def test_candidate_equals_last_row_of_causal_sequence():
    rng = np.random.default_rng(9)
    n_h, c = 9, 3
    n = n_h + c
    q, k, v, offs, ts, rp, rt = _rand_case(rng, [n], cands=[c])
    got = orc.attn_fwd(q, k, v, offs, ts, rp, rt, [c], 0, 20)
    for m in range(c):
        rows = list(range(n_h)) + [n_h + m]
        o1 = np.array([0, n_h + 1])
        alone = orc.attn_fwd(q[rows], k[rows], v[rows], o1, ts[rows], rp, rt, None, 0, 20)
        np.testing.assert_allclose(got[n_h + m], alone[-1], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(got[:n_h], alone[:n_h], rtol=0, atol=0)


def test_all_candidates_sequence_is_self_only():
    rng = np.random.default_rng(10)
    n = 5
    q, k, v, offs, ts, rp, rt = _rand_case(rng, [n], cands=[n])
    got = orc.attn_fwd(q, k, v, offs, ts, rp, rt, [n], 0, 3)
    for i in range(n):
        for h in range(q.shape[1]):
            s = q[i, h] @ k[i, h] + rp[h, 0] + rt[h, 0]
            np.testing.assert_allclose(got[i, h], s / (1 + math.exp(-s)) / 3 * v[i, h], rtol=1e-13)


def test_empty_sequences_and_sampled_rows():
    rng = np.random.default_rng(12)
    lengths = [0, 6, 0, 4]
    q, k, v, offs, ts, rp, rt = _rand_case(rng, lengths)
    full = orc.attn_fwd(q, k, v, offs, ts, rp, rt, None, 0, 8)
    rows = [[], [1, 5], [], [0, 3]]
    part = orc.attn_fwd(q, k, v, offs, ts, rp, rt, None, 0, 8, return_rows=rows)
    for b, rr in enumerate(rows):
        for r in rr:
            np.testing.assert_array_equal(part[offs[b] + r], full[offs[b] + r])


def test_row_blocking_does_not_change_result():
    rng = np.random.default_rng(13)
    q, k, v, offs, ts, rp, rt = _rand_case(rng, [37, 20], cands=[5, 0])
    a = orc.attn_fwd(q, k, v, offs, ts, rp, rt, [5, 0], 0, 40, row_block=1024)
    b = orc.attn_fwd(q, k, v, offs, ts, rp, rt, [5, 0], 0, 40, row_block=7)
    np.testing.assert_allclose(a, b, rtol=1e-14, atol=1e-16)


# ----------------------------------------------------------------------------
# Semi-local attention ([ULTRA] "Semi-Local Attention": a local and a global
# window instead of the full causal mask; the window sizes are parameters)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("cands", [None, [0, 3, 2]])
@pytest.mark.parametrize("wl,wg", [(1, 0), (3, 0), (2, 2), (4, 1), (6, 3)])
def test_semilocal_matches_brute_force(cands, wl, wg):
    rng = np.random.default_rng(21)
    lengths = [7, 9, 6]
    q, k, v, offs, ts, rp, rt = _rand_case(rng, lengths, cands=cands, scale=0.7, gap=3.0)
    got = orc.attn_fwd(q, k, v, offs, ts, rp, rt, cands, 0, 11, win_local=wl, win_global=wg)
    want = brute_attn_fwd(q, k, v, offs, ts, rp, rt, cands, 0, 11, win_local=wl, win_global=wg)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_semilocal_window_covering_the_sequence_is_full_causal():
    rng = np.random.default_rng(22)
    lengths = [9, 13]
    cands = [0, 4]
    q, k, v, offs, ts, rp, rt = _rand_case(rng, lengths, cands=cands, gap=5.0)
    full = orc.attn_fwd(q, k, v, offs, ts, rp, rt, cands, 0, 16)
    for wl, wg in [(13, 0), (40, 0), (13, 5)]:
        got = orc.attn_fwd(q, k, v, offs, ts, rp, rt, cands, 0, 16, win_local=wl,
                           win_global=wg)
        assert np.array_equal(got, full)


def test_semilocal_self_only_closed_form():
    # W_l = 1, W_g = 0: every token attends to itself only
    rng = np.random.default_rng(23)
    q, k, v, offs, ts, rp, rt = _rand_case(rng, [6], H=2, dqk=3, dv=4)
    got = orc.attn_fwd(q, k, v, offs, ts, rp, rt, None, 0, 5, win_local=1)
    for i in range(6):
        for h in range(2):
            s = float(q[i, h] @ k[i, h]) + rp[h, 0] + rt[h, 0]
            w = s / (1.0 + math.exp(-s)) / 5
            np.testing.assert_allclose(got[i, h], w * v[i, h], rtol=1e-12, atol=1e-15)


def test_semilocal_keys_outside_both_windows_do_not_matter():
    rng = np.random.default_rng(24)
    n, wl, wg = 20, 4, 3
    q, k, v, offs, ts, rp, rt = _rand_case(rng, [n], H=1, dqk=4, dv=3)
    base = orc.attn_fwd(q, k, v, offs, ts, rp, rt, None, 0, 8, win_local=wl, win_global=wg)
    i = 15
    outside = [j for j in range(n) if j <= i and not (i - j < wl or j < wg)]
    assert outside == list(range(3, 12))
    k2, v2 = k.copy(), v.copy()
    k2[outside] += 5.0
    v2[outside] *= -3.0
    pert = orc.attn_fwd(q, k2, v2, offs, ts, rp, rt, None, 0, 8, win_local=wl, win_global=wg)
    np.testing.assert_array_equal(pert[i], base[i])
    # rows 12.. have some of those keys in their local window
    assert not np.allclose(pert[12:i], base[12:i])
    # and a key inside the global window does matter to the last row
    k3 = k.copy()
    k3[1] += 5.0
    pert3 = orc.attn_fwd(q, k3, v, offs, ts, rp, rt, None, 0, 8, win_local=wl, win_global=wg)
    assert not np.allclose(pert3[n - 1], base[n - 1])
