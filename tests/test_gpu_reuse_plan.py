"""A stack of forward layers run with one workspace, where every layer after
the first reuses the plan (time pre-pass and work list) that the first
wrote: the outputs are bit-identical to planning in every layer, and the
library's timer shows one plan launch per stack instead of one per layer."""
import ctypes as C
import dataclasses

import numpy as np
import pytest

import synth
from tests.gpu_util import host, say
from tests.test_gpu_layer import Dev, _lcfg

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from hstu_sequential_transduction_amd import binding
    return binding


def _plan_launches(L, fn):
    """Runs fn with the library timer on; returns how many plan launches it made."""
    import torch
    torch.cuda.synchronize()
    assert L.hstu_timer_enable(4096) == 0
    try:
        fn()
        torch.cuda.synchronize()
        n, ms = C.c_int64(0), C.c_double(0.0)
        tag = [L.hstu_timer_tag_name(t) for t in range(L.hstu_timer_tag_count())].index(b"plan")
        assert L.hstu_timer_query(tag, C.byref(n), C.byref(ms)) == 0
        return n.value
    finally:
        L.hstu_timer_enable(0)


@pytest.mark.parametrize("mx", [False, True])
@pytest.mark.parametrize("ci,hist,c", [(3, [32, 33, 520, 300, 95], 0), (5, [100, 300, 0, 64], 40)])
def test_stack_reuse_plan_bit_identical(B, ci, hist, c, mx):
    from hstu_sequential_transduction_amd import _lib
    cfg = synth.get_config(ci).shrunk(B=len(hist), lengths=("list", hist), num_candidates=c,
                                      n_layers=3)
    say(f"stack reuse_plan cfg{ci} lengths={hist} c={c} mx={mx}")
    inp = synth.make_inputs(cfg, seed=2500 + ci)
    d = Dev(inp, cfg)
    lc = _lcfg(B, cfg)
    lc_r = dataclasses.replace(lc, attn=dataclasses.replace(lc.attn, reuse_plan=1))
    mxw = [B.MxLayerWeights.from_bf16(W1, W2) for (W1, W2, _, _) in d.layers] if mx else None

    def stack(reuse, outs):
        ws = B.LayerWorkspace()
        x = d.X
        for li, (W1, W2, rp, rt) in enumerate(d.layers):
            cf = lc_r if reuse and li else lc
            if mx:
                x = B.hstu_layer_fwd_mx(x, mxw[li], rp, rt, d.offs, d.ts, cf,
                                        num_candidates=d.nc, workspace=ws)
            else:
                x = B.hstu_layer_fwd(x, W1, W2, rp, rt, d.offs, d.ts, cf, num_candidates=d.nc,
                                     workspace=ws)
            outs.append(host(x))

    L = _lib.lib()
    got, want = [], []
    n_reuse = _plan_launches(L, lambda: stack(True, got))
    n_plain = _plan_launches(L, lambda: stack(False, want))
    assert (n_reuse, n_plain) == (1, len(d.layers)), (n_reuse, n_plain)
    for li, (a, b) in enumerate(zip(got, want)):
        np.testing.assert_array_equal(a, b, err_msg=f"layer {li}")


def test_reuse_plan_of_another_batch_is_rejected(B):
    """A plan recorded for one batch cannot be reused by a call naming other
    offsets, nor after another call planned into the workspace."""
    import torch

    from hstu_sequential_transduction_amd import _lib
    cfg = synth.get_config(3).shrunk(B=3, lengths=("list", [40, 300, 70]), n_layers=1)
    inp = synth.make_inputs(cfg, seed=2600)
    d = Dev(inp, cfg)
    lc = _lcfg(B, cfg)
    lc_r = dataclasses.replace(lc, attn=dataclasses.replace(lc.attn, reuse_plan=1))
    W1, W2, rp, rt = d.layers[0]
    ws = B.LayerWorkspace()
    B.hstu_layer_fwd(d.X, W1, W2, rp, rt, d.offs, d.ts, lc, workspace=ws)
    B.hstu_layer_fwd(d.X, W1, W2, rp, rt, d.offs, d.ts, lc_r, workspace=ws)  # accepted
    offs2 = d.offs.clone()
    with pytest.raises(_lib.HstuError):   # same contents, another buffer: not the plan's input
        B.hstu_layer_fwd(d.X, W1, W2, rp, rt, offs2, d.ts, lc_r, workspace=ws)
    # a planning call for offs2 through the same workspace replaces the plan
    B.hstu_layer_fwd(d.X, W1, W2, rp, rt, offs2, d.ts, lc, workspace=ws)
    with pytest.raises(_lib.HstuError):
        B.hstu_layer_fwd(d.X, W1, W2, rp, rt, d.offs, d.ts, lc_r, workspace=ws)
    B.hstu_layer_fwd(d.X, W1, W2, rp, rt, offs2, d.ts, lc_r, workspace=ws)
    torch.cuda.synchronize()
