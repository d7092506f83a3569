"""GPU parity of the backward that keeps dS (the scores' gradient) in its
workspace and forms dQ from it (d_qk = d_v = 128, bf16, max_len given):
attention and layer backward against the oracle, with candidates, the
fallback to recomputation when the batch does not fit max_len, and the full
training workload with both paths."""
import dataclasses

import numpy as np
import pytest

import synth
from oracle import hstu as orc
from tests.gpu_util import check_close, dev, host, say
from tests.test_gpu_attn import _bwd, _cfgobj
from tests.test_gpu_layer import Dev, _flags, _lcfg, _train_step

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from hstu_sequential_transduction_amd import binding
    return binding


ATTN_CASES = [
    # (history lengths, candidates, max_len) -- max_len below the longest
    # sequence forces the recomputing fallback
    ([300, 1100, 129], 0, 1100),
    ([300, 1100, 129], 0, 4096),
    ([64, 700, 0, 257], 40, 740),
    ([1, 128, 129, 255, 256, 257], 0, 257),
    ([300, 1100, 129], 0, 200),
]


@pytest.mark.parametrize("hist,c,max_len", ATTN_CASES)
def test_attn_bwd_keep_ds(B, hist, c, max_len):
    cfg = synth.get_config(4).shrunk(B=len(hist), lengths=("list", hist), num_candidates=c)
    say(f"attn bwd keep-dS lengths={hist} c={c} max_len={max_len}")
    a = synth.make_attn_inputs(cfg, seed=2100 + len(hist) + c)
    ac = dataclasses.replace(_cfgobj(B, cfg), max_len=max_len)
    got = _bwd(B, a, cfg, ac)
    want = orc.attn_bwd(a.q, a.k, a.v, a.seq_offsets, a.timestamps, a.rab_pos, a.rab_time,
                        a.d_out, a.num_candidates, 0, cfg.norm_len)
    for g_, w_, name in zip(got, want, ("dq", "dk", "dv", "drab_pos", "drab_time")):
        check_close(g_, w_, "bf16", f"{name} (max_len={max_len})")


@pytest.mark.parametrize("hist,c", [([300, 1100, 129], 0), ([100, 700, 0, 64], 64)])
def test_layer_bwd_keep_ds(B, hist, c):
    cfg = synth.get_config(4).shrunk(B=len(hist), lengths=("list", hist),
                                     num_candidates=c).unit_scale()
    say(f"layer bwd keep-dS lengths={hist} c={c}")
    inp = synth.make_inputs(cfg, seed=2200 + c, with_dy=True)
    d = Dev(inp, cfg)
    lc = _lcfg(B, cfg)
    lc = dataclasses.replace(lc, attn=dataclasses.replace(lc.attn, max_len=max(hist) + c))
    dx, g = _train_step(B, d, lc, inp.T)
    w = inp.layers[0]
    f = _flags(cfg)
    Y, sv = orc.layer_fwd(inp.X, w.W1, w.W2, w.rab_pos, w.rab_time, inp.seq_offsets,
                          inp.timestamps, inp.num_candidates, f)
    want = orc.layer_bwd(inp.dY, inp.X, w.W1, w.W2, w.rab_pos, w.rab_time, inp.seq_offsets,
                         inp.timestamps, inp.num_candidates, f, sv)
    check_close(host(dx) - inp.dY, want["dX"] - inp.dY, "bf16", "dX - dY")
    for k in ("dW1", "dW2", "drab_pos", "drab_time"):
        check_close(host(getattr(g, k)), want[k], "bf16", k)


def test_train_full_size_keep_ds_matches_recompute(B):
    """Training workload (8 x U[4096, 8192], 4 x 128): the kept-dS backward
    against the recomputing one (same GPU inputs) and one sequence's input
    gradient against the oracle."""
    cfg = synth.get_config(4)
    say("layer train full cfg4 keep-dS vs recompute")
    inp = synth.make_inputs(cfg)
    d = Dev(inp, cfg)
    lc0 = _lcfg(B, cfg)
    lc1 = dataclasses.replace(lc0, attn=dataclasses.replace(lc0.attn, max_len=8192))
    dx0, g0 = _train_step(B, d, lc0, inp.T)
    dx1, g1 = _train_step(B, d, lc1, inp.T)
    check_close(host(dx1) - inp.dY, host(dx0) - inp.dY, "bf16", "dX - dY (kept vs recomputed)")
    for k in ("dW1", "dW2", "drab_pos", "drab_time"):
        check_close(host(getattr(g1, k)), host(getattr(g0, k)), "bf16", f"{k} (kept vs recomputed)")
    b = int(np.argmin(inp.lengths))
    sub = synth.sub_batch(inp, [b])
    w = inp.layers[0]
    f = _flags(cfg)
    Y, sv = orc.layer_fwd(sub.X, w.W1, w.W2, w.rab_pos, w.rab_time, sub.seq_offsets,
                          sub.timestamps, None, f)
    want = orc.layer_bwd(sub.dY, sub.X, w.W1, w.W2, w.rab_pos, w.rab_time, sub.seq_offsets,
                         sub.timestamps, None, f, sv)
    o0, o1 = inp.seq_offsets[b], inp.seq_offsets[b + 1]
    check_close(host(dx1)[o0:o1], want["dX"], "bf16", "dX seq (kept dS)")


def test_keep_ds_reads_no_unwritten_workspace(B):
    """dQ from the kept dS must not depend on what the workspace held before:
    the same call on a workspace filled with NaN bytes and on a zeroed one
    gives the same result (masked sub-blocks are written as zeros)."""
    import ctypes as C
    import torch
    from hstu_sequential_transduction_amd import _lib
    from tests.test_gpu_attn import _upload
    hist, c = [64, 700, 0, 257], 40
    cfg = synth.get_config(4).shrunk(B=len(hist), lengths=("list", hist), num_candidates=c)
    say("keep-dS workspace independence")
    a = synth.make_attn_inputs(cfg, seed=2300)
    u = _upload(a, cfg)
    T, W = a.q.shape[0], cfg.H * cfg.d_qk
    ac = dataclasses.replace(_cfgobj(B, cfg), max_len=740)
    d = B.attn_desc(ac, len(hist), T, torch.bfloat16, B._rab_stride(u["rp"], u["rt"]))
    L = _lib.lib()
    nb = L.hstu_attn_bwd_workspace_size(C.byref(d))
    outs = []
    for fill in (0x00, 0xFF):
        ws = torch.full((nb,), fill, dtype=torch.uint8, device="cuda")
        g = [torch.empty((T, W), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
        drp, drt = torch.empty_like(u["rp"]), torch.empty_like(u["rt"])
        st = L.hstu_attn_bwd(C.byref(d), B._ptr(u["q"]), B._ptr(u["k"]), W, B._ptr(u["v"]), W,
                             B._ptr(u["offs"]), B._ptr(u["ts"]), B._ptr(u["rp"]), B._ptr(u["rt"]),
                             B._ptr(u["nc"]), B._ptr(u["dO"]), W, B._ptr(g[0]), B._ptr(g[1]),
                             B._ptr(g[2]), B._ptr(drp), B._ptr(drt), B._ptr(ws), nb, None)
        assert st == 0
        outs.append(host(g[0]))
    assert np.all(np.isfinite(outs[1]))
    np.testing.assert_array_equal(outs[0], outs[1])
