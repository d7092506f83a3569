"""The layer backward captured into a HIP graph (through torch): its side
stream joins the capture, and every replay, with eager calls of the same
backward and synchronisations between replays, reproduces the eager result
(bit for bit except the rab gradients, which are sums of float atomics in
no fixed order)."""
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


def test_layer_bwd_graph_replays_match_eager(B):
    import torch
    hist = [300, 1100, 129]
    say(f"layer bwd graph capture lengths={hist}")
    cfg = synth.get_config(4).shrunk(B=len(hist), lengths=("list", hist),
                                     num_candidates=0).unit_scale()
    inp = synth.make_inputs(cfg, seed=601, with_dy=True)
    d = Dev(inp, cfg)
    lc = _lcfg(B, cfg)
    W1, W2, rp, rt = d.layers[0]
    saved = B.Saved(inp.T, lc, d.td, "cuda")
    B.hstu_layer_fwd(d.X, W1, W2, rp, rt, d.offs, d.ts, lc, saved=saved)

    def run():
        return B.hstu_layer_bwd(d.X, W1, W2, rp, rt, d.offs, d.ts, lc, saved, d.dY)

    def outputs(dx, g):
        return [host(dx), host(g.dW1), host(g.dW2), host(g.drab_pos), host(g.drab_time)]

    ref = outputs(*run())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dxg, gg = run()
    for rep in range(3):
        run()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = outputs(dxg, gg)
        for name, a, b in zip(("dx", "dW1", "dW2"), got[:3], ref[:3]):
            np.testing.assert_array_equal(a, b, err_msg=f"replay {rep}: {name}")
        for name, a, b in zip(("drab_pos", "drab_time"), got[3:], ref[3:]):
            np.testing.assert_allclose(a, b, rtol=1e-5, atol=1e-6 * np.abs(b).max(),
                                       err_msg=f"replay {rep}: {name}")
