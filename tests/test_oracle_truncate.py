"""Pins of the oracle's attention truncation (CPU only).

[ULTRA] "Attention Truncation": N layers over the whole sequences, then M
layers over a segment of each history made of its most recent events.  The
segment is read as the last min(n_h, L') history rows followed by the
candidates; these tests tie that composition to things fixed independently
of it: a list-built segment, the plain stack when nothing is cut, sequences
run one at a time, the full-sequence layer where a local window already
hides everything before the segment, and finite differences.
"""
import types

import numpy as np
import pytest

from oracle import hstu as orc


def _case(rng, lengths, cands, n_full, n_tail, D=6, H=2, dqk=3, dv=3):
    lengths = np.asarray(lengths)
    offs = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(offs[-1])
    X = rng.standard_normal((T, D))
    ts = []
    for b, n in enumerate(lengths):
        c = 0 if cands is None else cands[b]
        t = 1_600_000_000 + np.floor(np.cumsum(rng.exponential(7.0, size=n - c))).astype(np.int64)
        if c:
            t = np.concatenate([t, np.full(c, t[-1] if n - c else 1_600_000_000)])
        ts.append(t.astype(np.int64))
    ts = np.concatenate(ts) if ts else np.zeros(0, np.int64)

    def layer():
        return types.SimpleNamespace(
            W1=rng.standard_normal((D, H * (2 * dv + 2 * dqk))) / np.sqrt(D),
            W2=rng.standard_normal((H * dv, D)) / np.sqrt(H * dv),
            rab_pos=rng.standard_normal((H, 128)), rab_time=rng.standard_normal((H, 128)))
    full = [layer() for _ in range(n_full)]
    tail = [layer() for _ in range(n_tail)]
    f = orc.LayerFlags(H=H, d_qk=dqk, d_v=dv, norm_mode=0, norm_len=16, eps=1e-3)
    return X, offs, ts, full, tail, f


def _segment_by_lists(offs, cands, keep):
    """The segment built from Python lists: history rows, cut to the last
    `keep` (none when keep = 0), then the candidate rows."""
    seg_rows, seg_lens = [], []
    for b in range(len(offs) - 1):
        rows = list(range(int(offs[b]), int(offs[b + 1])))
        c = 0 if cands is None else cands[b]
        hist, cand = rows[:len(rows) - c], rows[len(rows) - c:]
        kept = hist[len(hist) - keep:] if keep < len(hist) else hist
        seg_rows += kept + cand
        seg_lens.append(len(kept) + len(cand))
    return seg_lens, seg_rows


@pytest.mark.parametrize("keep", [0, 1, 3, 8, 100])
def test_truncate_rows_matches_list_segments(keep):
    rng = np.random.default_rng(11)
    lengths = [9, 0, 4, 12, 6, 1]
    cands = [2, 0, 4, 0, 1, 1]
    offs = np.concatenate([[0], np.cumsum(lengths)])
    seg, rows = orc.truncate_rows(offs, cands, keep)
    lens, want = _segment_by_lists(offs, cands, keep)
    assert list(np.diff(seg)) == lens and seg[0] == 0
    assert list(rows) == want
    # without candidates
    seg, rows = orc.truncate_rows(offs, None, keep)
    lens, want = _segment_by_lists(offs, None, keep)
    assert list(np.diff(seg)) == lens and list(rows) == want
    del rng


def test_nothing_cut_equals_the_plain_stack():
    rng = np.random.default_rng(12)
    cands = [2, 0, 3]
    X, offs, ts, full, tail, f = _case(rng, [7, 5, 9], cands, 2, 2)
    y, rec = orc.truncated_stack_fwd(X, full, tail, offs, ts, cands, f, f, keep=50)
    assert list(rec["rows"]) == list(range(X.shape[0]))
    want = orc.stack_fwd(X, full + tail, offs, ts, cands, f)[-1]
    np.testing.assert_array_equal(y, want)


def test_tail_layers_treat_each_segment_as_its_own_sequence():
    """N = 0: the batched truncated layers equal each sequence's tail, cut by
    slicing, run alone with its own timestamps."""
    rng = np.random.default_rng(13)
    lengths, cands, keep = [11, 3, 8, 0], [2, 1, 0, 0], 4
    X, offs, ts, _, tail, f = _case(rng, lengths, cands, 0, 2)
    y, rec = orc.truncated_stack_fwd(X, [], tail, offs, ts, cands, f, f, keep=keep)
    seg = rec["seg_offsets"]
    for b, n in enumerate(lengths):
        c = cands[b]
        m = min(n - c, keep) + c
        a, e = int(offs[b + 1]) - m, int(offs[b + 1])
        one = orc.stack_fwd(X[a:e], tail, np.array([0, m]), ts[a:e], [c], f)[-1]
        np.testing.assert_allclose(y[seg[b]:seg[b + 1]], one, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("cands", [None, [3, 1, 2]])
def test_local_window_inside_the_segment_matches_the_full_sequence(cands):
    """With a local window W_l <= L' and no global window, a segment row
    whose window lies inside the segment sees exactly the keys it sees in the
    whole sequence, with the same position differences and timestamps; so the
    truncated layer reproduces the full-sequence layer on those rows."""
    rng = np.random.default_rng(14)
    lengths, keep, wl = [15, 9, 20], 6, 4
    X, offs, ts, _, tail, f = _case(rng, lengths, cands, 0, 1)
    fw = orc.LayerFlags(**{**f.__dict__, "win_local": wl, "win_global": 0})
    y_seg, rec = orc.truncated_stack_fwd(X, [], tail, offs, ts, cands, fw, fw, keep=keep)
    y_full = orc.stack_fwd(X, tail, offs, ts, cands, fw)[-1]
    rows, seg = rec["rows"], rec["seg_offsets"]
    checked = 0
    for b, n in enumerate(lengths):
        c = 0 if cands is None else cands[b]
        n_h = n - c
        start = n_h - min(n_h, keep)          # first kept history index
        for r in range(seg[b], seg[b + 1]):
            i = int(rows[r] - offs[b])
            p = min(i, n_h)
            if p - wl + 1 >= start:           # window [p - W_l + 1, p] inside the segment
                np.testing.assert_allclose(y_seg[r], y_full[rows[r]], rtol=1e-12, atol=1e-13)
                checked += 1
    assert checked >= 8
    # and a row whose window reaches before the segment does differ
    r0 = seg[0]
    assert not np.allclose(y_seg[r0], y_full[rows[r0]])


def _loss(X, full, tail, offs, ts, cands, f, keep, dY):
    y, _ = orc.truncated_stack_fwd(X, full, tail, offs, ts, cands, f, f, keep=keep)
    return float(np.sum(y * dY))


def test_truncated_backward_finite_differences():
    rng = np.random.default_rng(15)
    cands, keep = [2, 0, 3], 3
    X, offs, ts, full, tail, f = _case(rng, [7, 5, 9], cands, 1, 1)
    y, rec = orc.truncated_stack_fwd(X, full, tail, offs, ts, cands, f, f, keep=keep)
    dY = rng.standard_normal(y.shape)
    dX, gf, gt = orc.truncated_stack_bwd(dY, full, tail, offs, ts, cands, f, f, rec)
    h = 1e-6
    rows = set(int(r) for r in rec["rows"])
    # X entries inside and outside the segments
    for (i, j) in [(0, 1), (3, 0), (6, 5), (8, 2), (12, 4), (20, 3), (14, 0)]:
        Xp, Xm = X.copy(), X.copy()
        Xp[i, j] += h
        Xm[i, j] -= h
        num = (_loss(Xp, full, tail, offs, ts, cands, f, keep, dY)
               - _loss(Xm, full, tail, offs, ts, cands, f, keep, dY)) / (2 * h)
        assert abs(num - dX[i, j]) <= 1e-6 * max(1.0, abs(num)), (i, j, i in rows)
    # parameters of the full layer and of the tail layer
    for lay, grads in ((full[0], gf[0]), (tail[0], gt[0])):
        for name, gname, idx in (("W1", "dW1", (2, 5)), ("W2", "dW2", (4, 1)),
                                 ("rab_time", "drab_time", (1, 0)),
                                 ("rab_pos", "drab_pos", (0, 2))):
            arr = getattr(lay, name)
            old = arr[idx]
            arr[idx] = old + h
            lp = _loss(X, full, tail, offs, ts, cands, f, keep, dY)
            arr[idx] = old - h
            lm = _loss(X, full, tail, offs, ts, cands, f, keep, dY)
            arr[idx] = old
            num = (lp - lm) / (2 * h)
            assert abs(num - grads[gname][idx]) <= 1e-6 * max(1.0, abs(num)), name


def test_rows_outside_the_segments_get_no_gradient_without_full_layers():
    rng = np.random.default_rng(16)
    cands, keep = [1, 2], 2
    X, offs, ts, _, tail, f = _case(rng, [8, 6], cands, 0, 2)
    y, rec = orc.truncated_stack_fwd(X, [], tail, offs, ts, cands, f, f, keep=keep)
    dX, _, _ = orc.truncated_stack_bwd(rng.standard_normal(y.shape), [], tail, offs, ts, cands,
                                       f, f, rec)
    outside = np.setdiff1d(np.arange(X.shape[0]), rec["rows"])
    assert outside.size == 14 - 7
    assert np.all(dX[outside] == 0)
    assert np.all(np.any(dX[rec["rows"]] != 0, axis=1))
