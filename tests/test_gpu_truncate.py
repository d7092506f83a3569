"""GPU parity of attention truncation: segment offsets, row gather and
gradient scatter bit-exact against the oracle's segment rows; N full + M
truncated layers (forward, and a training step) against the oracle's
composition; the full-size ranking workload with sampled sequences."""
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
def TR():
    from hstu_sequential_transduction_amd import truncation
    return truncation


def _offsets(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)


SEG_CASES = [
    # (lengths, candidates or None, keep)
    ([9, 0, 4, 12, 6, 1], [2, 0, 4, 0, 1, 1], 3),
    ([9, 0, 4, 12, 6, 1], [2, 0, 4, 0, 1, 1], 0),
    ([9, 0, 4, 12, 6, 1], None, 100),
    ([0, 0, 0], None, 5),
    ([1], [1], 0),
    ("many", None, 37),       # 3000 sequences: several per scan thread
    ("many", "some", 5),
]


def _seg_case(spec):
    lengths, cands, keep = spec
    if lengths == "many":
        rng = np.random.default_rng(3000)
        lengths = rng.integers(0, 90, size=3000)
        if cands == "some":
            cands = np.minimum(rng.integers(0, 6, size=3000), lengths)
    return np.asarray(lengths, np.int64), (None if cands is None else np.asarray(cands)), keep


@pytest.mark.parametrize("spec", SEG_CASES)
def test_segment_offsets_bit_exact(B, spec):
    lengths, cands, keep = _seg_case(spec)
    say(f"truncate offsets B={len(lengths)} keep={keep} cands={cands is not None}")
    offs = _offsets(lengths)
    seg, T_seg = B.hstu_truncate_offsets(dev(offs.astype(np.int32)), keep,
                                         None if cands is None else dev(cands.astype(np.int32)))
    want, rows = orc.truncate_rows(offs, cands, keep)
    assert T_seg == len(rows)
    np.testing.assert_array_equal(host(seg).astype(np.int64), want)


@pytest.mark.parametrize("dtype,D", [("bf16", 256), ("f32", 512), ("f32", 64), ("bf16", 72)])
@pytest.mark.parametrize("spec", [SEG_CASES[0], SEG_CASES[2], SEG_CASES[6]])
def test_gather_and_scatter_bit_exact(B, dtype, D, spec):
    import torch
    lengths, cands, keep = _seg_case(spec)
    say(f"truncate gather/scatter {dtype} D={D} B={len(lengths)} keep={keep}")
    offs = _offsets(lengths)
    T = int(offs[-1])
    rng = np.random.default_rng(D)
    td = torch_dtype(dtype)
    X = dev(rng.standard_normal((T, D)).astype(np.float32), td)
    ts = dev(rng.integers(0, 1 << 40, size=T).astype(np.int64))
    d_offs = dev(offs.astype(np.int32))
    seg, T_seg = B.hstu_truncate_offsets(d_offs, keep,
                                         None if cands is None else dev(cands.astype(np.int32)))
    xs, tss = B.hstu_truncate_gather(X, d_offs, seg, T_seg, ts)
    _, rows = orc.truncate_rows(offs, cands, keep)
    Xh = X.float().cpu().numpy()
    np.testing.assert_array_equal(xs.float().cpu().numpy(), Xh[rows])
    np.testing.assert_array_equal(host(tss), host(ts)[rows])
    G = dev(rng.standard_normal((T_seg, D)).astype(np.float32), td)
    dx = B.hstu_truncate_scatter(G, d_offs, seg, T)
    want = np.zeros((T, D), np.float32)
    want[rows] = G.float().cpu().numpy()
    np.testing.assert_array_equal(dx.float().cpu().numpy(), want)
    torch.cuda.synchronize()


def _cfgs(B, cfg):
    """Layer configurations of the full and the truncated layers (the same
    length normaliser N for both: these workloads are unit-scale, N = 1)."""
    ac = B.AttnConfig(H=cfg.H, d_qk=cfg.d_qk, d_v=cfg.d_v, norm_len=cfg.norm_len)
    at = dataclasses.replace(ac)
    return (B.LayerConfig(D=cfg.D, attn=ac, ln_eps=1e-6),
            B.LayerConfig(D=cfg.D, attn=at, ln_eps=1e-6))


def _flags(cfg, norm_len):
    return orc.LayerFlags(H=cfg.H, d_qk=cfg.d_qk, d_v=cfg.d_v, norm_mode=0, norm_len=norm_len,
                          eps=1e-6)


def _dev_layers(ws, td):
    return [(dev(w.W1, td), dev(w.W2, td), dev(w.rab_pos), dev(w.rab_time)) for w in ws]


FWD_CASES = [
    # (config, history lengths, candidates, n_full, n_tail, keep)
    (5, [100, 300, 0, 64, 700], 40, 2, 2, 128),
    (3, [32, 33, 520, 300, 95], 0, 1, 3, 200),
    (1, [1, 16, 65, 128, 0, 37], 0, 1, 1, 20),
    (2, [64, 257, 1000], 0, 2, 1, 0),
]


@pytest.mark.parametrize("ci,hist,c,nf,nt,keep", FWD_CASES)
def test_truncated_stack_fwd_small(B, TR, ci, hist, c, nf, nt, keep):
    cfg = synth.get_config(ci).shrunk(B=len(hist), lengths=("list", hist), num_candidates=c,
                                      n_layers=nf + nt).unit_scale()
    say(f"truncated stack fwd cfg{ci} lengths={hist} c={c} {nf}+{nt} keep={keep}")
    inp = synth.make_inputs(cfg, seed=900 + ci)
    td = torch_dtype(cfg.dtype)
    lay = _dev_layers(inp.layers, td)
    cf, ct = _cfgs(B, cfg)
    nc = None if inp.num_candidates is None else dev(inp.num_candidates.astype(np.int32))
    y, seg, _ = TR.truncated_stack_fwd(dev(inp.X, td), lay[:nf], lay[nf:],
                                       dev(inp.seq_offsets.astype(np.int32)),
                                       dev(inp.timestamps), cf, ct, keep, num_candidates=nc)
    want, rec = orc.truncated_stack_fwd(inp.X, inp.layers[:nf], inp.layers[nf:],
                                        inp.seq_offsets, inp.timestamps, inp.num_candidates,
                                        _flags(cfg, cfg.norm_len), _flags(cfg, cfg.norm_len), keep)
    np.testing.assert_array_equal(host(seg).astype(np.int64), rec["seg_offsets"])
    check_close(host(y), want, cfg.dtype, f"Y_seg cfg{ci}")


@pytest.mark.parametrize("ci,hist,c,keep", [(4, [300, 1100, 129], 0, 256),
                                            (5, [100, 300, 0, 64], 40, 80)])
def test_truncated_stack_train_small(B, TR, ci, hist, c, keep):
    """One full and one truncated layer, forward and backward: the input
    gradient passes the scatter (zeros outside the segments) into the full
    layer's backward."""
    cfg = synth.get_config(ci).shrunk(B=len(hist), lengths=("list", hist), num_candidates=c,
                                      n_layers=2).unit_scale()
    say(f"truncated stack train cfg{ci} lengths={hist} c={c} keep={keep}")
    inp = synth.make_inputs(cfg, seed=950 + ci, with_dy=False)
    td = torch_dtype(cfg.dtype)
    lay = _dev_layers(inp.layers, td)
    cf, ct = _cfgs(B, cfg)
    nc = None if inp.num_candidates is None else dev(inp.num_candidates.astype(np.int32))
    offs, ts = dev(inp.seq_offsets.astype(np.int32)), dev(inp.timestamps)
    y, seg, rec_g = TR.truncated_stack_fwd(dev(inp.X, td), lay[:1], lay[1:], offs, ts, cf, ct,
                                           keep, num_candidates=nc, training=True)
    fF = fT = _flags(cfg, cfg.norm_len)
    want_y, rec = orc.truncated_stack_fwd(inp.X, inp.layers[:1], inp.layers[1:],
                                          inp.seq_offsets, inp.timestamps, inp.num_candidates,
                                          fF, fT, keep)
    check_close(host(y), want_y, cfg.dtype, "Y_seg")
    rng = np.random.default_rng(ci)
    dY = synth.bf16_round(rng.standard_normal(want_y.shape))
    dx, gF, gT = TR.truncated_stack_bwd(dev(dY, td), lay[:1], lay[1:], offs, ts, cf, ct, rec_g,
                                        num_candidates=nc)
    wdx, wF, wT = orc.truncated_stack_bwd(dY, inp.layers[:1], inp.layers[1:], inp.seq_offsets,
                                          inp.timestamps, inp.num_candidates, fF, fT, rec)
    check_close(host(dx), wdx, "bf16", "dX")
    for name, g, w in (("full", gF[0], wF[0]), ("tail", gT[0], wT[0])):
        for k in ("dW1", "dW2", "drab_pos", "drab_time"):
            check_close(host(getattr(g, k)), w[k], "bf16", f"{k} {name}")


def test_truncated_stack_full_size_ranking_sampled(B, TR):
    """The ranking workload's full batch (16 x (4096 history + 512
    candidates), D = 256, 4 x 64) through 3 full and 6 truncated layers
    (keep = 1024) on the GPU; two whole sequences through the oracle."""
    base = synth.get_config(5)
    cfg = dataclasses.replace(base, n_layers=9).unit_scale()
    keep = 1024
    say("truncated stack full-size ranking 3+6 keep=1024")
    inp = synth.make_inputs(cfg)
    td = torch_dtype(cfg.dtype)
    lay = _dev_layers(inp.layers, td)
    cf, ct = _cfgs(B, cfg)
    nc = dev(inp.num_candidates.astype(np.int32))
    y, seg, _ = TR.truncated_stack_fwd(dev(inp.X, td), lay[:3], lay[3:],
                                       dev(inp.seq_offsets.astype(np.int32)),
                                       dev(inp.timestamps), cf, ct, keep, num_candidates=nc)
    y = host(y)
    seg = host(seg).astype(np.int64)
    for b in (0, cfg.B - 1):
        sub = synth.sub_batch(inp, [b])
        want, _ = orc.truncated_stack_fwd(sub.X, sub.layers[:3], sub.layers[3:], sub.seq_offsets,
                                          sub.timestamps, sub.num_candidates,
                                          _flags(cfg, cfg.norm_len), _flags(cfg, cfg.norm_len), keep)
        check_close(y[seg[b]:seg[b + 1]], want, "bf16", f"Y_seg seq {b}")
