"""GPU parity of semi-local attention (local window W_l + global window W_g,
"Bending the Scaling Law Curve in Large-Scale Recommendation Systems", item
Semi-Local Attention) against the fp64 oracle, forward and backward.

Cases mix windows narrower and wider than the position table (128 buckets),
windows crossing tile boundaries, W_g = 0, self-only (W_l = 1), candidates,
both head sizes of the bf16 kernels and the fp32 kernel.
"""
import dataclasses

import numpy as np
import pytest

import synth
from oracle import hstu as orc
from tests.gpu_util import check_close, say
from tests.test_gpu_attn import _bwd, _cfgobj, _fwd

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from hstu_sequential_transduction_amd import binding
    return binding


FWD_CASES = [
    # (config, lengths, candidates, W_l, W_g)
    (2, [1, 64, 130, 257, 0, 700], 0, 64, 0),
    (2, [300, 700], 0, 100, 33),
    (3, [32, 2048, 95], 0, 300, 64),
    (4, [300, 1100, 129], 0, 200, 128),
    (4, [600, 1100], 0, 1, 0),
    (5, [100, 300, 0, 64], 40, 50, 16),
    (5, [400, 200], 60, 150, 0),
    (1, [16, 65, 128, 37], 0, 20, 8),
]


@pytest.mark.parametrize("ci,hist,c,wl,wg", FWD_CASES)
def test_semilocal_fwd(B, ci, hist, c, wl, wg):
    cfg = synth.get_config(ci).shrunk(B=len(hist), lengths=("list", hist), num_candidates=c)
    say(f"semilocal fwd cfg{ci} lengths={hist} c={c} W_l={wl} W_g={wg}")
    a = synth.make_attn_inputs(cfg, seed=500 + ci)
    ac = dataclasses.replace(_cfgobj(B, cfg), win_local=wl, win_global=wg)
    got = _fwd(B, a, cfg, ac)
    want = orc.attn_fwd(a.q, a.k, a.v, a.seq_offsets, a.timestamps, a.rab_pos, a.rab_time,
                        a.num_candidates, 0, cfg.norm_len, win_local=wl, win_global=wg)
    check_close(got, want, cfg.dtype, f"O cfg{ci} W=({wl},{wg})")


BWD_CASES = [
    (4, [300, 1100, 129], 0, 200, 128),
    (4, [700, 900], 0, 90, 0),
    (4, [1200], 0, 300, 40),
    (2, [1, 64, 130, 257, 0, 700], 0, 64, 16),
    (5, [100, 300, 0, 64], 40, 50, 16),
    (5, [260], 30, 300, 0),
]


@pytest.mark.parametrize("ci,hist,c,wl,wg", BWD_CASES)
def test_semilocal_bwd(B, ci, hist, c, wl, wg):
    cfg = synth.get_config(ci).shrunk(B=len(hist), lengths=("list", hist), num_candidates=c)
    say(f"semilocal bwd cfg{ci} lengths={hist} c={c} W_l={wl} W_g={wg}")
    a = synth.make_attn_inputs(cfg, seed=600 + ci)
    ac = dataclasses.replace(_cfgobj(B, cfg), win_local=wl, win_global=wg)
    got = _bwd(B, a, cfg, ac)
    want = orc.attn_bwd(a.q, a.k, a.v, a.seq_offsets, a.timestamps, a.rab_pos, a.rab_time,
                        a.d_out, a.num_candidates, 0, cfg.norm_len, win_local=wl,
                        win_global=wg)
    for name, g, w in zip(("dq", "dk", "dv", "drab_pos", "drab_time"), got, want):
        check_close(g, w, "bf16", f"{name} cfg{ci} W=({wl},{wg})")


def test_semilocal_wide_window_equals_full(B):
    """A window covering every sequence gives the full causal result bit for
    bit when both run 128-row work items (key_splits 1); the full pass's
    default for this small batch, 64-row items whose two key halves are
    added at the end, sums in another order and agrees to the tolerance."""
    cfg = synth.get_config(4).shrunk(B=2, lengths=("list", [500, 900]))
    a = synth.make_attn_inputs(cfg, seed=700)
    ac = dataclasses.replace(_cfgobj(B, cfg), key_splits=1)
    full = _fwd(B, a, cfg, ac)
    wide = _fwd(B, a, cfg, dataclasses.replace(ac, win_local=4096, win_global=7))
    assert np.array_equal(full, wide)
    halves = _fwd(B, a, cfg, dataclasses.replace(ac, key_splits=0))
    check_close(halves, full, "bf16", "key-half items vs 128-row items")
