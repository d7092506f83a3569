"""GPU parity of the whole HSTU layer (forward, stacked forward, backward)."""
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


def _lcfg(binding, cfg, residual=True):
    ac = binding.AttnConfig(H=cfg.H, d_qk=cfg.d_qk, d_v=cfg.d_v, norm_len=cfg.norm_len,
                            n_pos_buckets=cfg.n_pos_buckets, n_time_buckets=cfg.n_time_buckets)
    return binding.LayerConfig(D=cfg.D, attn=ac, residual=residual, ln_eps=1e-6)


def _flags(cfg, residual=True):
    return orc.LayerFlags(H=cfg.H, d_qk=cfg.d_qk, d_v=cfg.d_v, norm_mode=0,
                          norm_len=cfg.norm_len, residual=residual, eps=1e-6)


class Dev:
    def __init__(self, inp, cfg):
        td = torch_dtype(cfg.dtype)
        self.td = td
        self.X = dev(inp.X, td)
        self.offs = dev(inp.seq_offsets.astype(np.int32))
        self.ts = dev(inp.timestamps.astype(np.int64))
        self.nc = None if inp.num_candidates is None else dev(inp.num_candidates.astype(np.int32))
        self.layers = [(dev(w.W1, td), dev(w.W2, td), dev(w.rab_pos), dev(w.rab_time))
                       for w in inp.layers]
        self.dY = None if inp.dY is None else dev(inp.dY, td)


def _stack_gpu(binding, d, lc, n_layers=None):
    x = d.X
    outs = []
    ws = binding.LayerWorkspace()
    for (W1, W2, rp, rt) in d.layers[:n_layers]:
        x = binding.hstu_layer_fwd(x, W1, W2, rp, rt, d.offs, d.ts, lc, num_candidates=d.nc,
                                   workspace=ws)
        outs.append(host(x))
    return outs


SMALL = {
    1: [1, 16, 65, 128, 0, 37],
    2: [1, 64, 130, 257, 0, 700],
    3: [32, 33, 520, 300, 95],
    4: [300, 1100, 129],
    5: [100, 300, 0, 64],
}


@pytest.mark.parametrize("ci", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("variant", ["literal", "unit", "noresid"])
def test_layer_stack_fwd_small(B, ci, variant):
    base = synth.get_config(ci)
    cfg = base.shrunk(B=len(SMALL[ci]), lengths=("list", SMALL[ci]))
    if variant == "unit":
        cfg = cfg.unit_scale()
    resid = variant != "noresid"
    n_layers = cfg.n_layers if variant != "noresid" else 1
    say(f"layer fwd cfg{ci} {variant} lengths={SMALL[ci]} layers={n_layers}")
    inp = synth.make_inputs(cfg, seed=500 + ci)
    d = Dev(inp, cfg)
    got = _stack_gpu(B, d, _lcfg(B, cfg, resid), n_layers)
    want = orc.stack_fwd(inp.X, inp.layers[:n_layers], inp.seq_offsets, inp.timestamps,
                         inp.num_candidates, _flags(cfg, resid))
    for li, (g, w) in enumerate(zip(got, want)):
        check_close(g, w, cfg.dtype, f"Y[{li}] cfg{ci} {variant}")


@pytest.mark.parametrize("ci,splits", [(3, 3), (5, 2), (4, 4)])
def test_layer_stack_fwd_key_splits(B, ci, splits):
    """The layer's attention (fp32 output) with long blocks' keys split."""
    hist = {3: [2048, 33, 1500], 5: [1900, 64], 4: [1300, 129]}[ci]
    cfg = synth.get_config(ci).shrunk(B=len(hist), lengths=("list", hist)).unit_scale()
    say(f"layer fwd cfg{ci} key_splits={splits} lengths={hist}")
    inp = synth.make_inputs(cfg, seed=520 + ci)
    d = Dev(inp, cfg)
    lc = _lcfg(B, cfg)
    lc.attn.key_splits = splits
    n_layers = min(cfg.n_layers, 2)
    got = _stack_gpu(B, d, lc, n_layers)
    want = orc.stack_fwd(inp.X, inp.layers[:n_layers], inp.seq_offsets, inp.timestamps,
                         inp.num_candidates, _flags(cfg))
    for li, (g, w) in enumerate(zip(got, want)):
        check_close(g, w, cfg.dtype, f"Y[{li}] cfg{ci} key_splits={splits}")


def test_layer_fwd_saved_intermediates(B):
    cfg = synth.get_config(4).shrunk(B=3, lengths=("list", [300, 1100, 129])).unit_scale()
    inp = synth.make_inputs(cfg, seed=41)
    d = Dev(inp, cfg)
    lc = _lcfg(B, cfg)
    saved = B.Saved(inp.T, lc, d.td, "cuda")
    W1, W2, rp, rt = d.layers[0]
    y = B.hstu_layer_fwd(d.X, W1, W2, rp, rt, d.offs, d.ts, lc, saved=saved)
    w = inp.layers[0]
    Y, sv = orc.layer_fwd(inp.X, w.W1, w.W2, w.rab_pos, w.rab_time, inp.seq_offsets,
                          inp.timestamps, None, _flags(cfg))
    check_close(host(y), Y, "bf16", "Y")
    check_close(host(saved.Z), sv["Z"], "bf16", "Z")
    check_close(host(saved.Zh), sv["Zh"], "bf16", "Zh")
    check_close(host(saved.O), sv["O"], "bf16", "O")
    check_close(host(saved.G), sv["G"], "bf16", "G")
    check_close(host(saved.mu), sv["mu"], "bf16", "mu")
    check_close(host(saved.rstd), sv["rstd"], "bf16", "rstd")


def _train_step(binding, d, lc, inp_T, extras=None):
    extras = extras or {}
    W1, W2, rp, rt = d.layers[0]
    saved = binding.Saved(inp_T, lc, d.td, "cuda")
    binding.hstu_layer_fwd(d.X, W1, W2, rp, rt, d.offs, d.ts, lc, num_candidates=d.nc,
                           saved=saved, **extras)
    dx, g = binding.hstu_layer_bwd(d.X, W1, W2, rp, rt, d.offs, d.ts, lc, saved, d.dY,
                                   num_candidates=d.nc, **extras)
    return dx, g


BWD = [
    (4, [300, 1100, 129], 0, "unit"),
    (4, [300, 1100, 129], 0, "literal"),
    (4, [300, 1100, 129], 0, "literal-noresid"),
    (2, [1, 64, 130, 257, 0, 700], 0, "unit"),
    (5, [100, 300, 0, 64], 40, "unit"),
    (1, [1, 16, 65, 128, 0, 37], 0, "bf16-unit"),
]


@pytest.mark.parametrize("ci,hist,c,variant", BWD)
def test_layer_bwd_small(B, ci, hist, c, variant):
    cfg = synth.get_config(ci).shrunk(B=len(hist), lengths=("list", hist), num_candidates=c)
    if variant.startswith("bf16"):
        cfg = dataclasses.replace(cfg, dtype="bf16")
    if variant.endswith("unit"):
        cfg = cfg.unit_scale()
    say(f"layer bwd cfg{ci} {variant} lengths={hist} c={c}")
    resid = not variant.endswith("noresid")
    inp = synth.make_inputs(cfg, seed=600 + ci, with_dy=True)
    d = Dev(inp, cfg)
    lc = _lcfg(B, cfg, resid)
    dx, g = _train_step(B, d, lc, inp.T)
    w = inp.layers[0]
    f = _flags(cfg, resid)
    Y, sv = orc.layer_fwd(inp.X, w.W1, w.W2, w.rab_pos, w.rab_time, inp.seq_offsets,
                          inp.timestamps, inp.num_candidates, f)
    want = orc.layer_bwd(inp.dY, inp.X, w.W1, w.W2, w.rab_pos, w.rab_time, inp.seq_offsets,
                         inp.timestamps, inp.num_candidates, f, sv)
    # with the residual, dX = dY + (layer part); at literal scale the layer part is far
    # below bf16 resolution of dY, so it is checked on its own by the noresid variant
    check_close(host(dx), want["dX"], "bf16", "dX")
    if resid and variant.endswith("unit"):
        check_close(host(dx) - inp.dY, want["dX"] - inp.dY, "bf16", "dX - dY")
    check_close(host(g.dW1), want["dW1"], "bf16", "dW1")
    check_close(host(g.dW2), want["dW2"], "bf16", "dW2")
    check_close(host(g.drab_pos), want["drab_pos"], "bf16", "drab_pos")
    check_close(host(g.drab_time), want["drab_time"], "bf16", "drab_time")


def test_layer_train_unaligned_width(B):
    """d_model = 72: the projection's k extent is not a multiple of the DMA
    GEMM's k-step, so the forward and input-gradient GEMMs take the
    register-staged GEMM kernel; the weight gradients (k-major operands) keep
    the DMA kernel.  Both paths against the oracle in one training step."""
    cfg = dataclasses.replace(synth.get_config(2), D=72, H=2, d_qk=32, d_v=32)
    cfg = cfg.shrunk(B=3, lengths=("list", [70, 257, 33])).unit_scale()
    say("layer train d_model=72")
    inp = synth.make_inputs(cfg, seed=72, with_dy=True)
    d = Dev(inp, cfg)
    lc = _lcfg(B, cfg)
    dx, g = _train_step(B, d, lc, inp.T)
    w = inp.layers[0]
    f = _flags(cfg)
    Y, sv = orc.layer_fwd(inp.X, w.W1, w.W2, w.rab_pos, w.rab_time, inp.seq_offsets,
                          inp.timestamps, None, f)
    want = orc.layer_bwd(inp.dY, inp.X, w.W1, w.W2, w.rab_pos, w.rab_time, inp.seq_offsets,
                         inp.timestamps, None, f, sv)
    check_close(host(dx), want["dX"], "bf16", "dX")
    check_close(host(dx) - inp.dY, want["dX"] - inp.dY, "bf16", "dX - dY")
    for k in ("dW1", "dW2", "drab_pos", "drab_time"):
        check_close(host(getattr(g, k)), want[k], "bf16", k)


def test_layer_bwd_affine_and_biases(B):
    cfg = synth.get_config(2).shrunk(B=3, lengths=("list", [64, 257, 31])).unit_scale()
    inp = synth.make_inputs(cfg, seed=77, with_dy=True)
    rng = np.random.default_rng(77)
    F1, W = cfg.f1_width, cfg.H * cfg.d_v
    ex_np = dict(b1=(0.1 * rng.standard_normal(F1)).astype(np.float32),
                 b2=(0.1 * rng.standard_normal(cfg.D)).astype(np.float32),
                 gamma=(1 + 0.2 * rng.standard_normal(W)).astype(np.float32),
                 beta=(0.1 * rng.standard_normal(W)).astype(np.float32))
    d = Dev(inp, cfg)
    lc = _lcfg(B, cfg)
    ex = {k: dev(v) for k, v in ex_np.items()}
    dx, g = _train_step(B, d, lc, inp.T, ex)
    w = inp.layers[0]
    f = _flags(cfg)
    Y, sv = orc.layer_fwd(inp.X, w.W1, w.W2, w.rab_pos, w.rab_time, inp.seq_offsets,
                          inp.timestamps, None, f, **ex_np)
    want = orc.layer_bwd(inp.dY, inp.X, w.W1, w.W2, w.rab_pos, w.rab_time, inp.seq_offsets,
                         inp.timestamps, None, f, sv, **ex_np)
    check_close(host(dx), want["dX"], "bf16", "dX")
    for k in ("dW1", "dW2", "db1", "db2", "dgamma", "dbeta", "drab_pos", "drab_time"):
        check_close(host(getattr(g, k)), want[k], "bf16", k)


@pytest.mark.parametrize("ci", [2, 3, 5])
def test_layer_stack_full_size_sampled_sequences(B, ci):
    """Full batch through the GPU stack; a few whole sequences through the oracle."""
    cfg = synth.get_config(ci).unit_scale()
    say(f"layer stack full cfg{ci} (unit scale)")
    inp = synth.make_inputs(cfg)
    d = Dev(inp, cfg)
    got = _stack_gpu(B, d, _lcfg(B, cfg))
    order = np.argsort(inp.lengths)
    pick = sorted({int(order[0]), int(order[len(order) // 2]), int(order[-1])})
    sub = synth.sub_batch(inp, pick)
    want = orc.stack_fwd(sub.X, sub.layers, sub.seq_offsets, sub.timestamps, sub.num_candidates,
                         _flags(cfg))
    rows = np.concatenate([np.arange(inp.seq_offsets[b], inp.seq_offsets[b + 1]) for b in pick])
    check_close(got[-1][rows], want[-1], cfg.dtype, f"Y[last] full cfg{ci} seqs {pick}")


def test_layer_stack_full_size_config3_literal_scale(B):
    """The 8-layer Zipf workload at its literal scales (inputs and weights
    N(0, 1/sqrt(d)), rab N(0, 0.02)): the full batch through the GPU stack,
    every layer's output compared with the oracle on three whole sequences
    (the shortest, the median and the 90th-percentile length)."""
    cfg = synth.get_config(3)
    say("layer stack full cfg3 (literal scale)")
    inp = synth.make_inputs(cfg)
    d = Dev(inp, cfg)
    got = _stack_gpu(B, d, _lcfg(B, cfg))
    order = np.argsort(inp.lengths)
    pick = sorted({int(order[0]), int(order[len(order) // 2]), int(order[(9 * len(order)) // 10])})
    sub = synth.sub_batch(inp, pick)
    want = orc.stack_fwd(sub.X, sub.layers, sub.seq_offsets, sub.timestamps, sub.num_candidates,
                         _flags(cfg))
    rows = np.concatenate([np.arange(inp.seq_offsets[b], inp.seq_offsets[b + 1]) for b in pick])
    for li in range(cfg.n_layers):
        check_close(got[li][rows], want[li], cfg.dtype, f"Y[{li}] literal cfg3 seqs {pick}")


def test_layer_train_full_size_config4(B):
    """Full config-4 training step on the GPU against the oracle on one sequence
    (dX rows) and on the whole batch for the weight gradients."""
    cfg = synth.get_config(4)
    say("layer train full cfg4")
    inp = synth.make_inputs(cfg)
    d = Dev(inp, cfg)
    lc = _lcfg(B, cfg)
    dx, g = _train_step(B, d, lc, inp.T)
    b = int(np.argmin(inp.lengths))
    sub = synth.sub_batch(inp, [b])
    w = inp.layers[0]
    f = _flags(cfg)
    Y, sv = orc.layer_fwd(sub.X, w.W1, w.W2, w.rab_pos, w.rab_time, sub.seq_offsets,
                          sub.timestamps, None, f)
    want = orc.layer_bwd(sub.dY, sub.X, w.W1, w.W2, w.rab_pos, w.rab_time, sub.seq_offsets,
                         sub.timestamps, None, f, sv)
    o0, o1 = inp.seq_offsets[b], inp.seq_offsets[b + 1]
    check_close(host(dx)[o0:o1], want["dX"], "bf16", "dX seq")
    # the layer's own input gradient, without the residual's dY
    dxn, _ = _train_step(B, d, _lcfg(B, cfg, residual=False), inp.T)
    check_close(host(dxn)[o0:o1], want["dX"] - sub.dY, "bf16", "dX (no residual) seq")
    # weight gradients are sums over sequences: the one-sequence GPU step must
    # match the oracle, and the full batch must equal the sum of per-sequence steps
    d1 = Dev(sub, cfg)
    dx1, g1 = _train_step(B, d1, lc, sub.T)
    check_close(host(g1.dW1), want["dW1"], "bf16", "dW1 seq")
    check_close(host(g1.dW2), want["dW2"], "bf16", "dW2 seq")
    check_close(host(g1.drab_time), want["drab_time"], "bf16", "drab_time seq")
    check_close(host(g1.drab_pos), want["drab_pos"], "bf16", "drab_pos seq")
    tot = {k: 0.0 for k in ("dW1", "dW2", "drab_pos", "drab_time")}
    for bb in range(cfg.B):
        s = synth.sub_batch(inp, [bb])
        _, gb = _train_step(B, Dev(s, cfg), lc, s.T)
        for k in tot:
            tot[k] = tot[k] + host(getattr(gb, k))
    for k in tot:
        check_close(host(getattr(g, k)), tot[k], "bf16", f"{k} additivity")


def test_check_mode_gives_the_same_results(B):
    """Check mode (wait + launch-error read after every launch) changes only
    the timing: a training step with it on is bit-identical to one without."""
    import torch
    cfg = synth.get_config(4).shrunk(B=3, lengths=("list", [300, 1100, 129])).unit_scale()
    inp = synth.make_inputs(cfg, seed=610)
    d = Dev(inp, cfg)
    lc = _lcfg(B, cfg)
    lc.attn.max_len = 1100
    dx0, g0 = _train_step(B, d, lc, inp.T)
    torch.cuda.synchronize()
    B.set_check_mode(True)
    try:
        assert B.check_mode()
        dx1, g1 = _train_step(B, d, lc, inp.T)
        torch.cuda.synchronize()
    finally:
        B.set_check_mode(False)
    assert not B.check_mode()
    assert torch.equal(dx0, dx1)
    for k in ("dW1", "dW2"):
        assert torch.equal(getattr(g0, k), getattr(g1, k)), k
    # the rab-table gradients are sums of float atomics: same values up to
    # the order of the additions
    for k in ("drab_pos", "drab_time"):
        a, b = getattr(g0, k), getattr(g1, k)
        assert torch.allclose(a, b, rtol=1e-5, atol=1e-6 * float(a.abs().max())), k
