"""GPU parity of the attention entry points against the fp64 oracle.

Every call goes through libhstu.so's C ABI (via the ctypes binding).  Inputs
come from `synth`; expected values only from `oracle`.
"""
import dataclasses

import numpy as np
import pytest

import synth
from oracle import hstu as orc
from tests.gpu_util import check_close, dev, host, say, torch_dtype

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from hstu_sequential_transduction_amd import binding
    return binding


def _cfgobj(binding, cfg, norm_len=None):
    return binding.AttnConfig(H=cfg.H, d_qk=cfg.d_qk, d_v=cfg.d_v,
                              norm_len=cfg.norm_len if norm_len is None else norm_len,
                              n_pos_buckets=cfg.n_pos_buckets, n_time_buckets=cfg.n_time_buckets)


def _upload(a, cfg):
    td = torch_dtype(cfg.dtype)
    T = a.q.shape[0]
    return dict(
        q=dev(a.q.reshape(T, -1), td), k=dev(a.k.reshape(T, -1), td),
        v=dev(a.v.reshape(T, -1), td), offs=dev(a.seq_offsets.astype(np.int32)),
        ts=dev(a.timestamps.astype(np.int64)), rp=dev(a.rab_pos), rt=dev(a.rab_time),
        nc=None if a.num_candidates is None else dev(a.num_candidates.astype(np.int32)),
        dO=dev(a.d_out.reshape(T, -1), td))


def _fwd(binding, a, cfg, ac):
    u = _upload(a, cfg)
    out = binding.hstu_attn_fwd(u["q"], u["k"], u["v"], u["offs"], u["ts"], u["rp"], u["rt"], ac,
                                num_candidates=u["nc"])
    return host(out).reshape(a.v.shape)


SMALL = {
    1: [1, 16, 65, 128, 0, 37],
    2: [1, 64, 130, 257, 0, 700],
    3: [32, 33, 520, 2048, 95],
    4: [300, 1100, 129],
    5: [100, 300, 0, 64],
}


# key_splits 0: the library default, which for these small bf16 batches runs
# 64-row work items whose key tiles two waves share; 1: 128-row items
@pytest.mark.parametrize("ks", [0, 1])
@pytest.mark.parametrize("ci", [1, 2, 3, 4, 5])
def test_attn_fwd_small(B, ci, ks):
    base = synth.get_config(ci)
    hist = SMALL[ci]
    cfg = base.shrunk(B=len(hist), lengths=("list", hist))
    say(f"attn fwd small cfg{ci} key_splits={ks} lengths={hist} c={cfg.num_candidates}")
    a = synth.make_attn_inputs(cfg, seed=100 + ci)
    ac = _cfgobj(B, cfg)
    ac.key_splits = ks
    got = _fwd(B, a, cfg, ac)
    want = orc.attn_fwd(a.q, a.k, a.v, a.seq_offsets, a.timestamps, a.rab_pos, a.rab_time,
                        a.num_candidates, 0, cfg.norm_len)
    check_close(got, want, cfg.dtype, f"O cfg{ci}")


@pytest.mark.parametrize("ks", [0, 1])
@pytest.mark.parametrize("ci", [2, 3, 4, 5])
def test_attn_fwd_literal_scale(B, ci, ks):
    """Small q, k and rab tables of std 0.02 as in the workloads' literal scales."""
    base = synth.get_config(ci)
    hist = SMALL[ci]
    cfg = base.shrunk(B=len(hist), lengths=("list", hist))
    a = synth.make_attn_inputs(cfg, seed=200 + ci, qk_std=0.15, rab_std=0.02)
    ac = _cfgobj(B, cfg)
    ac.key_splits = ks
    got = _fwd(B, a, cfg, ac)
    want = orc.attn_fwd(a.q, a.k, a.v, a.seq_offsets, a.timestamps, a.rab_pos, a.rab_time,
                        a.num_candidates, 0, cfg.norm_len)
    check_close(got, want, cfg.dtype, f"O literal cfg{ci}")


def test_attn_fwd_norm_mode_1_and_shared_tables(B):
    cfg = synth.get_config(2).shrunk(B=3, lengths=("list", [5, 200, 77]))
    a = synth.make_attn_inputs(cfg, seed=7)
    ac = _cfgobj(B, cfg)
    ac.norm_mode = 1
    u = _upload(a, cfg)
    rp1, rt1 = a.rab_pos[1], a.rab_time[2]
    out = B.hstu_attn_fwd(u["q"], u["k"], u["v"], u["offs"], u["ts"], dev(rp1), dev(rt1), ac)
    got = host(out).reshape(a.v.shape)
    want = orc.attn_fwd(a.q, a.k, a.v, a.seq_offsets, a.timestamps, rp1, rt1, None, 1, 0)
    check_close(got, want, "bf16", "O norm_mode=1 shared")


@pytest.mark.parametrize("ks", [0, 1])
def test_attn_fwd_all_candidates_and_edge_sequences(B, ks):
    cfg = synth.get_config(5).shrunk(B=4, lengths=("list", [0, 1, 127, 128]), num_candidates=3)
    a = synth.make_attn_inputs(cfg, seed=8)
    ac = _cfgobj(B, cfg)
    ac.key_splits = ks
    got = _fwd(B, a, cfg, ac)
    want = orc.attn_fwd(a.q, a.k, a.v, a.seq_offsets, a.timestamps, a.rab_pos, a.rab_time,
                        a.num_candidates, 0, cfg.norm_len)
    check_close(got, want, "bf16", "O all-candidate/edge")


def test_attn_fwd_unsorted_and_wide_timestamps(B):
    """Negative time distances clamp to bucket 0; a span beyond 2^31 s takes the 64-bit path."""
    cfg = synth.get_config(2).shrunk(B=3, lengths=("list", [150, 90, 200]))
    a = synth.make_attn_inputs(cfg, seed=9)
    rng = np.random.default_rng(9)
    ts = a.timestamps.copy()
    o = a.seq_offsets
    ts[o[0]:o[1]] = ts[o[0]] + rng.integers(-5000, 5000, size=150)          # unsorted
    ts[o[1]:o[2]] = np.sort(rng.integers(0, 1 << 40, size=90))               # wide span
    a = dataclasses.replace(a, timestamps=ts)
    for ks in (0, 1):
        ac = _cfgobj(B, cfg)
        ac.key_splits = ks
        got = _fwd(B, a, cfg, ac)
        want = orc.attn_fwd(a.q, a.k, a.v, a.seq_offsets, a.timestamps, a.rab_pos, a.rab_time,
                            None, 0, cfg.norm_len)
        check_close(got, want, "bf16", f"O unsorted/wide key_splits={ks}")


SPLIT_CASES = {
    3: [2048, 33, 1500, 520, 1],
    5: [1900, 700, 64, 0],
    4: [1300, 129],
}


@pytest.mark.parametrize("ci", [3, 5, 4])
@pytest.mark.parametrize("splits", [1, 2, 3, 8])
def test_attn_fwd_key_splits(B, ci, splits):
    """Long query blocks' keys cut into `splits` runs (1: never): the same O."""
    hist = SPLIT_CASES[ci]
    cfg = synth.get_config(ci).shrunk(B=len(hist), lengths=("list", hist))
    say(f"attn fwd key_splits={splits} cfg{ci} lengths={hist} c={cfg.num_candidates}")
    a = synth.make_attn_inputs(cfg, seed=300 + ci)
    ac = _cfgobj(B, cfg)
    ac.key_splits = splits
    got = _fwd(B, a, cfg, ac)
    want = orc.attn_fwd(a.q, a.k, a.v, a.seq_offsets, a.timestamps, a.rab_pos, a.rab_time,
                        a.num_candidates, 0, cfg.norm_len)
    check_close(got, want, cfg.dtype, f"O cfg{ci} splits={splits}")


def test_attn_fwd_key_splits_reused_plan(B):
    """The split counters return to zero after each call: a stack of calls on
    one plan gives the first call's output every time."""
    import torch
    hist = SPLIT_CASES[3]
    cfg = synth.get_config(3).shrunk(B=len(hist), lengths=("list", hist))
    a = synth.make_attn_inputs(cfg, seed=310)
    u = _upload(a, cfg)
    ac = _cfgobj(B, cfg)
    ac.key_splits = 4
    ws = B.LayerWorkspace()
    first = B.hstu_attn_fwd(u["q"], u["k"], u["v"], u["offs"], u["ts"], u["rp"], u["rt"], ac,
                            workspace=ws)
    ac.reuse_plan = 1
    for _ in range(3):
        again = B.hstu_attn_fwd(u["q"], u["k"], u["v"], u["offs"], u["ts"], u["rp"], u["rt"],
                                ac, workspace=ws)
        assert torch.equal(again, first)
    want = orc.attn_fwd(a.q, a.k, a.v, a.seq_offsets, a.timestamps, a.rab_pos, a.rab_time,
                        None, 0, cfg.norm_len)
    check_close(host(first).reshape(a.v.shape), want, "bf16", "O split reused plan")


@pytest.mark.parametrize("ci", [2, 3, 4, 5])
def test_attn_fwd_full_size_sampled_rows(B, ci):
    cfg = synth.get_config(ci)
    say(f"attn fwd full cfg{ci}")
    a = synth.make_attn_inputs(cfg)
    ac = _cfgobj(B, cfg)
    got = _fwd(B, a, cfg, ac)
    rng = np.random.default_rng(ci)
    rows = []
    for b in range(cfg.B):
        n = int(a.lengths[b])
        r = {0, n - 1, n // 2} | set(rng.integers(0, n, size=6).tolist())
        if cfg.num_candidates:
            r |= {n - cfg.num_candidates - 1, n - cfg.num_candidates, n - 2}
        rows.append(sorted(x for x in r if 0 <= x < n))
    want = orc.attn_fwd(a.q, a.k, a.v, a.seq_offsets, a.timestamps, a.rab_pos, a.rab_time,
                        a.num_candidates, 0, cfg.norm_len, return_rows=rows)
    sel = np.concatenate([a.seq_offsets[b] + np.asarray(rows[b], dtype=np.int64)
                          for b in range(cfg.B)])
    check_close(got[sel], want[sel], cfg.dtype, f"O full cfg{ci} sampled", scale_ref=want[sel])


def test_bias_buckets_bit_exact(B):
    import torch
    rng = np.random.default_rng(11)
    lens = [300, 90, 50, 7]
    cands = [20, 0, 50, 3]
    ts = []
    for n, c in zip(lens, cands):
        t = 1_650_000_000 + np.cumsum(rng.exponential(400.0, size=n - c)).astype(np.int64)
        ts.append(np.concatenate([t, np.full(c, t[-1] if n > c else 0)]))
    ts[1] = np.sort(rng.integers(-(1 << 41), 1 << 41, size=90))            # wide span
    ts[3] = rng.integers(0, 10 ** 6, size=7)                                 # unsorted
    timestamps = np.concatenate(ts).astype(np.int64)
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    ps, pi, pj = [], [], []
    for b, n in enumerate(lens):
        for _ in range(400):
            ps.append(b); pi.append(rng.integers(0, n)); pj.append(rng.integers(0, n))
        for i in range(n):
            ps.append(b); pi.append(i); pj.append(0)
    ps, pi, pj = (np.asarray(x, np.int32) for x in (ps, pi, pj))
    for nP, nT in [(128, 128), (37, 9)]:
        ac = B.AttnConfig(H=1, d_qk=64, d_v=64, norm_len=1, n_pos_buckets=nP, n_time_buckets=nT)
        bp, bt = B.hstu_bias_buckets(dev(offs), dev(timestamps), dev(ps), dev(pi), dev(pj), ac,
                                     num_candidates=dev(np.asarray(cands, np.int32)))
        torch.cuda.synchronize()
        bp, bt = bp.cpu().numpy(), bt.cpu().numpy()
        wp = np.zeros_like(bp)
        wt = np.zeros_like(bt)
        for k in range(len(ps)):
            b = ps[k]
            o0 = offs[b]
            n = lens[b]
            p = orc.positions(n, cands[b])
            wp[k] = orc.pos_bucket(np.array([p[pi[k]] - p[pj[k]]]), nP)[0]
            wt[k] = orc.time_bucket(np.array([timestamps[o0 + pi[k]] - timestamps[o0 + pj[k]]]),
                                    nT)[0]
        np.testing.assert_array_equal(bp, wp)
        np.testing.assert_array_equal(bt, wt)


@pytest.mark.parametrize("reverse", [False, True])
def test_schedule_covers_every_block_once(B, reverse):
    import torch
    rng = np.random.default_rng(12)
    lens = np.concatenate([[0, 1, 128, 129, 4096], rng.integers(0, 3000, size=60)])
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(offs[-1])
    for bm in (64, 128):
        items, n = B.hstu_schedule(dev(offs), T, bm, reverse)
        torch.cuda.synchronize()
        items, n = items.cpu().numpy(), int(n.cpu().numpy()[0])
        nb = (lens + bm - 1) // bm
        assert n == int(nb.sum())
        got = sorted(map(tuple, items[:n].tolist()))
        want = sorted((b, m) for b in range(len(lens)) for m in range(nb[b]))
        assert got == want
        cost = [(nb[b] - 1 - m) if reverse else m for b, m in items[:n].tolist()]
        assert all(cost[i] >= cost[i + 1] for i in range(n - 1)), "not longest-first"


@pytest.mark.parametrize("bm", [64, 128])
def test_schedule_in_global_memory(B, bm):
    """More than 3 070 entries: the work-list builder keeps its arrays in the
    workspace instead of LDS (T = 260k rows at 64-row blocks)."""
    import torch
    rng = np.random.default_rng(13)
    lens = np.concatenate([[0, 1, 64, 65], rng.integers(0, 2600, size=200)])
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(offs[-1])
    from hstu_sequential_transduction_amd import _lib
    cap = _lib.lib().hstu_schedule_capacity(T, len(lens), bm)
    if bm == 64:
        assert cap + 2 > 3072, cap
    items, n = B.hstu_schedule(dev(offs), T, bm, False)
    torch.cuda.synchronize()
    items, n = items.cpu().numpy(), int(n.cpu().numpy()[0])
    nb = (lens + bm - 1) // bm
    assert n == int(nb.sum())
    got = sorted(map(tuple, items[:n].tolist()))
    want = sorted((b, m) for b in range(len(lens)) for m in range(nb[b]))
    assert got == want
    cost = [m for _, m in items[:n].tolist()]
    assert all(cost[i] >= cost[i + 1] for i in range(n - 1)), "not longest-first"


def test_attn_fwd_plan_in_global_memory(B):
    """A forward whose work list exceeds the LDS-resident builder (T = 400k
    rows at 128-row blocks), against the oracle on sampled rows."""
    rng = np.random.default_rng(14)
    lens = rng.integers(1000, 5600, size=120)
    cfg = synth.get_config(2).shrunk(B=len(lens), lengths=("list", lens.tolist()))
    cfg = dataclasses.replace(cfg, H=1, d_qk=32, d_v=32)
    say(f"attn fwd global-memory plan: T={int(lens.sum())}")
    a = synth.make_attn_inputs(cfg, seed=15)
    from hstu_sequential_transduction_amd import _lib
    assert _lib.lib().hstu_schedule_capacity(int(lens.sum()), len(lens), 128) + 2 > 3072
    ac = _cfgobj(B, cfg)
    got = _fwd(B, a, cfg, ac)
    sub = [0, 7, 55, 119]
    rows = [[0, int(lens[b]) // 2, int(lens[b]) - 1] for b in sub]
    offs = a.seq_offsets
    keep = np.concatenate([np.arange(offs[b], offs[b + 1]) for b in sub])
    sub_offs = np.concatenate([[0], np.cumsum([lens[b] for b in sub])])
    want = orc.attn_fwd(a.q[keep], a.k[keep], a.v[keep], sub_offs, a.timestamps[keep],
                        a.rab_pos, a.rab_time, None, 0, cfg.norm_len, return_rows=rows)
    sel = np.concatenate([offs[b] + np.asarray(r) for b, r in zip(sub, rows)])
    wsel = np.concatenate([sub_offs[i] + np.asarray(r) for i, r in enumerate(rows)])
    check_close(got[sel], want[wsel], "bf16", "O global-memory plan", scale_ref=want[wsel])


def test_validate_inputs(B):
    offs = dev(np.array([0, 5, 9], np.int32))
    assert B.hstu_validate_inputs(offs, 9) == 0
    assert B.hstu_validate_inputs(offs, 10) != 0
    assert B.hstu_validate_inputs(dev(np.array([0, 5, 3], np.int32)), 3) != 0
    assert B.hstu_validate_inputs(offs, 9, dev(np.array([0, 6], np.int32))) != 0
    assert B.hstu_validate_inputs(offs, 9, dev(np.array([5, 4], np.int32))) == 0


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------
def _bwd(binding, a, cfg, ac):
    u = _upload(a, cfg)
    dq, dk, dv, drp, drt = binding.hstu_attn_bwd(u["q"], u["k"], u["v"], u["offs"], u["ts"],
                                                 u["rp"], u["rt"], u["dO"], ac,
                                                 num_candidates=u["nc"])
    T = a.q.shape[0]
    return (host(dq).reshape(a.q.shape), host(dk).reshape(a.k.shape), host(dv).reshape(a.v.shape),
            host(drp), host(drt))


BWD_CASES = [
    (4, [300, 1100, 129], 0),
    (2, [1, 64, 130, 257, 0, 700], 0),
    (5, [100, 300, 0, 64], 40),
    (3, [32, 2048, 95], 0),
]


@pytest.mark.parametrize("ci,hist,c", BWD_CASES)
def test_attn_bwd_small(B, ci, hist, c):
    cfg = synth.get_config(ci).shrunk(B=len(hist), lengths=("list", hist), num_candidates=c)
    say(f"attn bwd small cfg{ci} lengths={hist} c={c}")
    a = synth.make_attn_inputs(cfg, seed=300 + ci)
    ac = _cfgobj(B, cfg)
    got = _bwd(B, a, cfg, ac)
    want = orc.attn_bwd(a.q, a.k, a.v, a.seq_offsets, a.timestamps, a.rab_pos, a.rab_time,
                        a.d_out, a.num_candidates, 0, cfg.norm_len)
    for name, g, w in zip(("dq", "dk", "dv", "drab_pos", "drab_time"), got, want):
        check_close(g, w, "bf16", f"{name} cfg{ci}")


def test_attn_bwd_full_size_config4_sampled_sequence(B):
    """Full training batch on the GPU; one sequence through the oracle; bias
    gradients checked by additivity over sequences (a property at any size)."""
    import torch
    cfg = synth.get_config(4)
    a = synth.make_attn_inputs(cfg)
    ac = _cfgobj(B, cfg)
    say("attn bwd full cfg4")
    got = _bwd(B, a, cfg, ac)
    b = int(np.argmin(a.lengths))
    o0, o1 = a.seq_offsets[b], a.seq_offsets[b + 1]
    sub = dataclasses.replace(
        a, lengths=a.lengths[[b]], seq_offsets=np.array([0, o1 - o0]), q=a.q[o0:o1], k=a.k[o0:o1],
        v=a.v[o0:o1], d_out=a.d_out[o0:o1], timestamps=a.timestamps[o0:o1])
    want = orc.attn_bwd(sub.q, sub.k, sub.v, sub.seq_offsets, sub.timestamps, sub.rab_pos,
                        sub.rab_time, sub.d_out, None, 0, cfg.norm_len)
    for name, g, w in zip(("dq", "dk", "dv"), got[:3], want[:3]):
        check_close(g[o0:o1], w, "bf16", f"{name} full cfg4 seq{b}")
    # additivity of the table gradients over sequences
    tot_p = np.zeros_like(got[3])
    tot_t = np.zeros_like(got[4])
    for bb in range(cfg.B):
        p0, p1 = a.seq_offsets[bb], a.seq_offsets[bb + 1]
        s1 = dataclasses.replace(
            a, lengths=a.lengths[[bb]], seq_offsets=np.array([0, p1 - p0]), q=a.q[p0:p1],
            k=a.k[p0:p1], v=a.v[p0:p1], d_out=a.d_out[p0:p1], timestamps=a.timestamps[p0:p1])
        r = _bwd(B, s1, cfg, ac)
        if bb == b:
            check_close(r[3], want[3], "bf16", "drab_pos seq")
            check_close(r[4], want[4], "bf16", "drab_time seq")
        tot_p += r[3]
        tot_t += r[4]
    torch.cuda.synchronize()
    check_close(got[3], tot_p, "bf16", "drab_pos additivity")
    check_close(got[4], tot_t, "bf16", "drab_time additivity")


# Every (d_qk, d_v) the bf16 kernels instantiate, including mixed ones, with
# candidates; forward with both item shapes (key_splits 0: 64-row key-half
# items for this small batch; 1: 128-row items) and the backward.
HEAD_SIZES = [(32, 32), (32, 128), (128, 32), (64, 128), (128, 64), (32, 64)]


@pytest.mark.parametrize("dqk,dv", HEAD_SIZES)
def test_attn_mixed_head_sizes(B, dqk, dv):
    cfg = dataclasses.replace(synth.get_config(5), H=2, d_qk=dqk, d_v=dv)
    hist = [70, 260, 1, 140]
    cfg = cfg.shrunk(B=len(hist), lengths=("list", hist), num_candidates=9)
    say(f"attn mixed head sizes d_qk={dqk} d_v={dv} lengths={hist} c=9")
    a = synth.make_attn_inputs(cfg, seed=900 + dqk + dv)
    want = orc.attn_fwd(a.q, a.k, a.v, a.seq_offsets, a.timestamps, a.rab_pos, a.rab_time,
                        a.num_candidates, 0, cfg.norm_len)
    for ks in (0, 1):
        ac = _cfgobj(B, cfg)
        ac.key_splits = ks
        check_close(_fwd(B, a, cfg, ac), want, "bf16", f"O d=({dqk},{dv}) key_splits={ks}")
    got = _bwd(B, a, cfg, _cfgobj(B, cfg))
    want_b = orc.attn_bwd(a.q, a.k, a.v, a.seq_offsets, a.timestamps, a.rab_pos, a.rab_time,
                          a.d_out, a.num_candidates, 0, cfg.norm_len)
    for g, w, name in zip(got, want_b, ("dq", "dk", "dv", "drab_pos", "drab_time")):
        check_close(g, w, "bf16", f"{name} d=({dqk},{dv})")
