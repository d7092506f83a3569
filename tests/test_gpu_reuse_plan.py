"""A stack of forward layers run with one workspace, where every layer after
the first reuses the plan (time pre-pass and work list) that the first
wrote: the outputs are bit-identical to planning in every layer."""
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


@pytest.mark.parametrize("ci,hist,c", [(3, [32, 33, 520, 300, 95], 0), (5, [100, 300, 0, 64], 40)])
def test_stack_reuse_plan_bit_identical(B, ci, hist, c):
    cfg = synth.get_config(ci).shrunk(B=len(hist), lengths=("list", hist), num_candidates=c,
                                      n_layers=3)
    say(f"stack reuse_plan cfg{ci} lengths={hist} c={c}")
    inp = synth.make_inputs(cfg, seed=2500 + ci)
    d = Dev(inp, cfg)
    lc = _lcfg(B, cfg)
    lc_r = dataclasses.replace(lc, attn=dataclasses.replace(lc.attn, reuse_plan=1))

    def stack(reuse):
        ws = B.LayerWorkspace()
        x, outs = d.X, []
        for li, (W1, W2, rp, rt) in enumerate(d.layers):
            x = B.hstu_layer_fwd(x, W1, W2, rp, rt, d.offs, d.ts, lc_r if reuse and li else lc,
                                 num_candidates=d.nc, workspace=ws)
            outs.append(host(x))
        return outs

    for li, (a, b) in enumerate(zip(stack(True), stack(False))):
        np.testing.assert_array_equal(a, b, err_msg=f"layer {li}")
