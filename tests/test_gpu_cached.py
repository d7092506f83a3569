"""GPU parity of ranking against a cached history: the cached attention
against the oracle (bf16 head sizes, fp32, windows, users without history
or candidates, key splits, strided history views); the cached layer stack
against the oracle's cached stack; and at the ranking workload's full size
the cached candidate rows against the GPU's own full target-aware pass plus
two users through the oracle."""
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


@pytest.fixture(scope="module")
def RK():
    from hstu_sequential_transduction_amd import ranking
    return ranking


def _attn_case(n_hist, n_cand, H, dqk, dv, dtype, seed, ld_pad=0):
    rng = np.random.default_rng(seed)
    rnd = synth.bf16_round if dtype == "bf16" else (lambda a: a.astype(np.float32))
    hist_off = np.concatenate([[0], np.cumsum(n_hist)]).astype(np.int64)
    cand_off = np.concatenate([[0], np.cumsum(n_cand)]).astype(np.int64)
    hts, cts = [], []
    for nh, nc in zip(n_hist, n_cand):
        t0 = int(rng.integers(1_600_000_000, 1_700_000_000))
        t = t0 + np.floor(np.cumsum(rng.exponential(60.0, size=nh))).astype(np.int64)
        last = int(t[-1]) if nh else t0
        hts.append(t)
        cts.append(last + rng.integers(0, 3600, size=nc))
    hist_ts = np.concatenate(hts).astype(np.int64)
    cand_ts = np.concatenate(cts).astype(np.int64)
    Th, Tc = int(hist_off[-1]), int(cand_off[-1])
    s = dqk ** -0.25
    q = rnd(rng.standard_normal((Tc, H, dqk)) * s)
    k = rnd(rng.standard_normal((Tc, H, dqk)) * s)
    v = rnd(rng.standard_normal((Tc, H, dv)))
    kh = rnd(rng.standard_normal((Th, H, dqk)) * s)
    vh = rnd(rng.standard_normal((Th, H, dv)))
    rp = rng.standard_normal((H, 128)).astype(np.float32)
    rt = rng.standard_normal((H, 128)).astype(np.float32)
    return dict(hist_off=hist_off, cand_off=cand_off, hist_ts=hist_ts, cand_ts=cand_ts, q=q, k=k,
                v=v, kh=kh, vh=vh, rp=rp, rt=rt)


ATTN_CASES = [
    # (n_hist, n_cand, H, d_qk, d_v, dtype, W_l, W_g)
    ([300, 0, 1500, 64], [40, 7, 300, 0], 4, 64, 64, "bf16", 0, 0),
    ([4096, 2000], [512, 33], 4, 64, 64, "bf16", 0, 0),          # key splits
    ([700, 129, 3000], [129, 64, 1], 4, 128, 128, "bf16", 0, 0),
    ([1000, 60, 2500], [70, 5, 200], 2, 32, 32, "bf16", 0, 0),
    ([900, 2000, 50], [100, 64, 10], 4, 64, 64, "bf16", 300, 70),
    ([3000, 130], [64, 33], 4, 128, 128, "bf16", 1, 0),          # own key only past W_g = 0
    ([300, 0, 1500], [40, 7, 100], 2, 32, 32, "f32", 0, 0),
    ([2000, 90], [30, 12], 2, 64, 64, "f32", 200, 16),
]


@pytest.mark.parametrize("n_hist,n_cand,H,dqk,dv,dtype,wl,wg", ATTN_CASES)
def test_cached_attention(B, n_hist, n_cand, H, dqk, dv, dtype, wl, wg):
    import torch
    say(f"cached attn hist={n_hist} cand={n_cand} H={H} d={dqk}/{dv} {dtype} W=({wl},{wg})")
    c = _attn_case(n_hist, n_cand, H, dqk, dv, dtype, seed=sum(n_hist) + dqk)
    td = torch_dtype(dtype)
    norm_len = 5000
    Th = c["kh"].shape[0]
    # history K and V as strided column views of one wider matrix
    wide = torch.zeros((Th, H * (dqk + dv) + 16), dtype=td, device="cuda")
    wide[:, :H * dqk] = dev(c["kh"].reshape(Th, -1), td)
    wide[:, H * dqk + 8:H * dqk + 8 + H * dv] = dev(c["vh"].reshape(Th, -1), td)
    hist = B.History(wide[:, :H * dqk], wide[:, H * dqk + 8:H * dqk + 8 + H * dv],
                     dev(c["hist_off"].astype(np.int32)), dev(c["hist_ts"]))
    cfg = B.AttnConfig(H=H, d_qk=dqk, d_v=dv, norm_len=norm_len, win_local=wl, win_global=wg)
    Tc = c["q"].shape[0]
    out = B.hstu_attn_cached_fwd(dev(c["q"].reshape(Tc, -1), td), dev(c["k"].reshape(Tc, -1), td),
                                 dev(c["v"].reshape(Tc, -1), td),
                                 dev(c["cand_off"].astype(np.int32)), dev(c["cand_ts"]), hist,
                                 dev(c["rp"]), dev(c["rt"]), cfg)
    want = orc.attn_fwd_cached(c["q"], c["k"], c["v"], c["cand_off"], c["cand_ts"], c["kh"],
                               c["vh"], c["hist_off"], c["hist_ts"], c["rp"], c["rt"], norm_len,
                               wl, wg)
    check_close(host(out), want.reshape(Tc, -1), dtype, "O cached")


def _split_users(inp):
    """History and candidate parts of a batch laid out as [history; candidates]."""
    offs, nc = inp.seq_offsets, inp.num_candidates
    rows_h, rows_c = [], []
    for b in range(len(offs) - 1):
        n_h = int(offs[b + 1] - offs[b] - nc[b])
        rows_h.append(np.arange(offs[b], offs[b] + n_h))
        rows_c.append(np.arange(offs[b] + n_h, offs[b + 1]))
    rh, rc = np.concatenate(rows_h), np.concatenate(rows_c)
    hist_off = np.concatenate([[0], np.cumsum([len(r) for r in rows_h])]).astype(np.int64)
    cand_off = np.concatenate([[0], np.cumsum([len(r) for r in rows_c])]).astype(np.int64)
    return rh, rc, hist_off, cand_off


def _lcfg(B, cfg, wl=0, wg=0):
    ac = B.AttnConfig(H=cfg.H, d_qk=cfg.d_qk, d_v=cfg.d_v, norm_len=cfg.norm_len,
                      win_local=wl, win_global=wg)
    return B.LayerConfig(D=cfg.D, attn=ac, ln_eps=1e-6)


STACK_CASES = [
    # (config, history lengths, candidates, layers, W_l, W_g)
    (5, [100, 300, 0, 64], 40, 2, 0, 0),
    (4, [300, 1100, 129], 64, 2, 0, 0),
    (5, [700, 90], 130, 2, 200, 32),
]


@pytest.mark.parametrize("ci,hist,c,nl,wl,wg", STACK_CASES)
def test_cached_stack_small(B, RK, ci, hist, c, nl, wl, wg):
    cfg = synth.get_config(ci).shrunk(B=len(hist), lengths=("list", hist), num_candidates=c,
                                      n_layers=nl).unit_scale()
    cfg = dataclasses.replace(cfg, norm_len=max(hist) + c)
    say(f"cached stack cfg{ci} hist={hist} c={c} layers={nl} W=({wl},{wg})")
    inp = synth.make_inputs(cfg, seed=1300 + ci)
    rh, rc, hist_off, cand_off = _split_users(inp)
    td = torch_dtype(cfg.dtype)
    lay = [(dev(w.W1, td), dev(w.W2, td), dev(w.rab_pos), dev(w.rab_time)) for w in inp.layers]
    lc = _lcfg(B, cfg, wl, wg)
    h_off, h_ts = dev(hist_off.astype(np.int32)), dev(inp.timestamps[rh])
    cache = RK.build_history_cache(dev(inp.X[rh], td), lay, h_off, h_ts, lc)
    y = RK.cached_stack_fwd(dev(inp.X[rc], td), lay, cache, dev(cand_off.astype(np.int32)),
                            dev(inp.timestamps[rc]), lc)
    f = orc.LayerFlags(H=cfg.H, d_qk=cfg.d_qk, d_v=cfg.d_v, norm_mode=0, norm_len=cfg.norm_len,
                       eps=1e-6, win_local=wl, win_global=wg)
    caches = orc.history_cache(inp.X[rh], inp.layers, hist_off, inp.timestamps[rh], f)
    want = orc.cached_stack_fwd(inp.X[rc], inp.layers, caches, hist_off, inp.timestamps[rh],
                                cand_off, inp.timestamps[rc], f)
    check_close(host(y), want, cfg.dtype, "Y candidates (cached)")


def test_cached_ranking_full_size(B, RK):
    """The ranking workload (16 x (4096 history + 512 candidates), 4 layers):
    cached candidate rows equal the candidate rows of the GPU's own full
    target-aware stack, and two users match the oracle."""
    cfg = synth.get_config(5).unit_scale()
    say("cached ranking full size cfg5")
    inp = synth.make_inputs(cfg)
    rh, rc, hist_off, cand_off = _split_users(inp)
    td = torch_dtype(cfg.dtype)
    lay = [(dev(w.W1, td), dev(w.W2, td), dev(w.rab_pos), dev(w.rab_time)) for w in inp.layers]
    lc = _lcfg(B, cfg)
    # full target-aware pass
    x = dev(inp.X, td)
    offs, ts = dev(inp.seq_offsets.astype(np.int32)), dev(inp.timestamps)
    nc = dev(inp.num_candidates.astype(np.int32))
    for (W1, W2, rp, rt) in lay:
        x = B.hstu_layer_fwd(x, W1, W2, rp, rt, offs, ts, lc, num_candidates=nc)
    full = host(x)[rc]
    cache = RK.build_history_cache(dev(inp.X[rh], td), lay, dev(hist_off.astype(np.int32)),
                                   dev(inp.timestamps[rh]), lc)
    y = host(RK.cached_stack_fwd(dev(inp.X[rc], td), lay, cache, dev(cand_off.astype(np.int32)),
                                 dev(inp.timestamps[rc]), lc))
    check_close(y, full, "bf16", "cached vs full target-aware (GPU)")
    f = orc.LayerFlags(H=cfg.H, d_qk=cfg.d_qk, d_v=cfg.d_v, norm_mode=0, norm_len=cfg.norm_len,
                       eps=1e-6)
    for b in (0, cfg.B - 1):
        sub = synth.sub_batch(inp, [b])
        srh, src, shoff, scoff = _split_users(sub)
        caches = orc.history_cache(sub.X[srh], sub.layers, shoff, sub.timestamps[srh], f)
        want = orc.cached_stack_fwd(sub.X[src], sub.layers, caches, shoff, sub.timestamps[srh],
                                    scoff, sub.timestamps[src], f)
        check_close(y[cand_off[b]:cand_off[b + 1]], want, "bf16", f"user {b} vs oracle")
