"""GPU parity of the MXFP8 matmuls ("Bending the Scaling Law Curve in
Large-Scale Recommendation Systems", Mixed precision; OCP MX formats):
quantization bit-exact against the oracle's codes and scales, the MX GEMM
against the exact product of the dequantized operands, and the layer with
MXFP8 projection and output products against the oracle's MX layer (and its
distance from the exact layer)."""
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


def _bf16_spread(rng, shape):
    """bf16 values whose 32-blocks span many binades, with zero blocks and
    single large outliers (the cases the block scale decides)."""
    x = rng.standard_normal(shape) * np.exp2(rng.integers(-24, 24, size=shape[:-1] + (1,)))
    x = x * np.exp2(rng.integers(-3, 4, size=shape))
    flat = x.reshape(-1, 32)
    flat[::7] = 0.0
    flat[3::11, 5] *= 1e4
    return synth.bf16_round(x)


@pytest.mark.parametrize("rows,K", [(1, 32), (77, 256), (300, 512), (1025, 128)])
def test_mx_quantize_bit_exact(B, rows, K):
    import torch
    say(f"mx quantize rows={rows} K={K}")
    rng = np.random.default_rng(rows + K)
    x = _bf16_spread(rng, (rows, K))
    codes, scales = B.hstu_mx_quantize(dev(x, torch.bfloat16))
    wc, ws = orc.mx_quantize(x, axis=1)
    np.testing.assert_array_equal(host(scales), ws)
    np.testing.assert_array_equal(host(codes), wc)


@pytest.mark.parametrize("K,N", [(256, 1024), (512, 96), (128, 40)])
def test_mx_quantize_weight_bit_exact(B, K, N):
    import torch
    say(f"mx quantize weight K={K} N={N}")
    rng = np.random.default_rng(K * N)
    w = _bf16_spread(rng, (N, K)).T.copy()          # blocks run down the columns
    codes, scales = B.hstu_mx_quantize_weight(dev(w, torch.bfloat16))
    wc, ws = orc.mx_quantize(w, axis=0)
    np.testing.assert_array_equal(host(scales), ws.T)
    np.testing.assert_array_equal(host(codes), wc.T)


@pytest.mark.parametrize("M,N,K", [(128, 128, 128), (300, 1024, 256), (1000, 200, 512),
                                   (57, 33, 384)])
def test_mx_gemm(B, M, N, K):
    import torch
    say(f"mx gemm M={M} N={N} K={K}")
    rng = np.random.default_rng(M + N + K)
    a = synth.bf16_round(rng.standard_normal((M, K)) * np.exp2(rng.integers(-6, 6, (M, 1))))
    b = synth.bf16_round(rng.standard_normal((N, K)) * np.exp2(rng.integers(-6, 6, (1, K))))
    qa, sa = B.hstu_mx_quantize(dev(a, torch.bfloat16))
    qb, sb = B.hstu_mx_quantize(dev(b, torch.bfloat16))
    c = B.hstu_mx_gemm(qa, sa, qb, sb)
    want = (orc.mx_dequantize(host(qa), host(sa), axis=1)
            @ orc.mx_dequantize(host(qb), host(sb), axis=1).T)
    check_close(host(c), want, "f32", "C")


def _lcfg(B, cfg):
    ac = B.AttnConfig(H=cfg.H, d_qk=cfg.d_qk, d_v=cfg.d_v, norm_len=cfg.norm_len)
    return B.LayerConfig(D=cfg.D, attn=ac, ln_eps=1e-6)


LAYER_CASES = [
    (5, [100, 300, 0, 64], 40, "unit"),
    (5, [100, 300, 0, 64], 40, "literal"),
    (3, [32, 33, 520, 300, 95], 0, "unit"),
    (4, [300, 1100, 129], 0, "unit"),
]


@pytest.mark.parametrize("ci,hist,c,variant", LAYER_CASES)
def test_mx_layer_fwd(B, ci, hist, c, variant):
    """Two stages.  (1) The quantized gated output G the GPU fed to the output
    product is, element by element, a valid E4M3 rounding of a value within
    the bf16 tolerance of the oracle's G (the GPU's G carries bf16 rounding,
    so codes next to a rounding midpoint may differ by one step).  (2) Y is
    the exact product of those codes with the MXFP8 W2, plus X, to the bf16
    tolerance.  End to end, the distance from the oracle's MX layer and
    from the exact layer is reported and bounded."""
    import torch
    cfg = synth.get_config(ci).shrunk(B=len(hist), lengths=("list", hist), num_candidates=c,
                                      n_layers=1)
    if variant == "unit":
        cfg = cfg.unit_scale()
    say(f"mx layer cfg{ci} {variant} lengths={hist} c={c}")
    inp = synth.make_inputs(cfg, seed=1700 + ci)
    w = inp.layers[0]
    td = torch.bfloat16
    T, W = inp.T, cfg.H * cfg.d_v
    wm = B.MxLayerWeights.from_bf16(dev(w.W1, td), dev(w.W2, td))
    nc = None if inp.num_candidates is None else dev(inp.num_candidates.astype(np.int32))
    gc = torch.empty((T, W), dtype=torch.uint8, device="cuda")
    gs = torch.empty((T, W // 32), dtype=torch.uint8, device="cuda")
    y = B.hstu_layer_fwd_mx(dev(inp.X, td), wm, dev(w.rab_pos), dev(w.rab_time),
                            dev(inp.seq_offsets.astype(np.int32)), dev(inp.timestamps),
                            _lcfg(B, cfg), num_candidates=nc, g_out=(gc, gs))
    f = orc.LayerFlags(H=cfg.H, d_qk=cfg.d_qk, d_v=cfg.d_v, norm_len=cfg.norm_len, eps=1e-6)
    want, G = orc.layer_fwd_mx(inp.X, w.W1, w.W2, w.rab_pos, w.rab_time, inp.seq_offsets,
                               inp.timestamps, inp.num_candidates, f, return_g=True)
    got = host(y)
    # (1) the GPU's quantized G
    codes, scales = host(gc), host(gs)
    deq = orc.mx_dequantize(codes, scales, axis=1)
    X = np.exp2(scales.astype(np.float64) - 127).repeat(32, axis=1)
    half_step = np.where(np.abs(deq) >= 448 * X, 64 * X,
                         np.maximum(np.abs(deq) * 2.0 ** -4, 2.0 ** -10 * X))
    slack = 2e-2 * np.abs(G) + 2e-2 * np.abs(G).max()
    assert np.all(np.abs(deq - G) <= half_step + slack), "G codes not a rounding of G"
    oc, osc = orc.mx_quantize(G, axis=1)
    flips = float(np.mean(orc.mx_dequantize(oc, osc, axis=1) != deq))
    say(f"  G codes differing from the oracle's rounding: {100 * flips:.2f} %")
    assert flips < 0.15
    # (2) Y from the GPU's own quantized G (at the literal scale the layer's
    # contribution is below bf16 resolution next to X, so Y itself is
    # compared; the unit-scale variants also compare Y - X)
    w2c, w2s = orc.mx_quantize(w.W2, axis=0)
    want2 = deq @ orc.mx_dequantize(w2c, w2s, axis=0) + inp.X
    check_close(got, want2, "bf16", "Y from the GPU's G")
    if variant != "unit":
        return
    check_close(got - inp.X, want2 - inp.X, "bf16", "Y - X from the GPU's G")
    # end to end
    rel_mx = np.linalg.norm((got - inp.X) - (want - inp.X)) / np.linalg.norm(want - inp.X)
    exact, _ = orc.layer_fwd(inp.X, w.W1, w.W2, w.rab_pos, w.rab_time, inp.seq_offsets,
                             inp.timestamps, inp.num_candidates, f)
    rel = np.linalg.norm((got - inp.X) - (exact - inp.X)) / np.linalg.norm(exact - inp.X)
    say(f"  relative L2 of Y - X: {rel_mx:.4f} vs the oracle's MX layer, {rel:.4f} vs exact")
    assert rel_mx < 2e-2
    # FP8's own rounding (3 mantissa bits, two chained products): an accuracy
    # figure of the format, not a parity bound
    assert rel < 0.15


def test_mx_layer_chain_hands_y_codes_to_the_next_layer(B):
    """The output product's epilogue writes Y in MXFP8 for the next layer:
    those codes equal the quantizer's on the stored bf16 Y, and a two-layer
    chain that passes them on is bit-identical to one quantizing X itself."""
    import torch
    cfg = synth.get_config(5).shrunk(B=4, lengths=("list", [100, 300, 0, 64]), num_candidates=40,
                                     n_layers=2).unit_scale()
    say("mx layer chain cfg5 2 layers")
    inp = synth.make_inputs(cfg, seed=1800)
    td = torch.bfloat16
    T, D = inp.T, cfg.D
    lc = _lcfg(B, cfg)
    offs, ts = dev(inp.seq_offsets.astype(np.int32)), dev(inp.timestamps)
    nc = dev(inp.num_candidates.astype(np.int32))
    ws = [(dev(w.rab_pos), dev(w.rab_time),
           B.MxLayerWeights.from_bf16(dev(w.W1, td), dev(w.W2, td))) for w in inp.layers]
    x0 = dev(inp.X, td)
    yc = torch.empty((T, D), dtype=torch.uint8, device="cuda")
    ys = torch.empty((T, D // 32), dtype=torch.uint8, device="cuda")
    y1 = B.hstu_layer_fwd_mx(x0, ws[0][2], ws[0][0], ws[0][1], offs, ts, lc, num_candidates=nc,
                             y_mx=(yc, ys))
    qc, qs = B.hstu_mx_quantize(y1)
    np.testing.assert_array_equal(host(ys), host(qs))
    np.testing.assert_array_equal(host(yc), host(qc))
    chained = B.hstu_layer_fwd_mx(y1, ws[1][2], ws[1][0], ws[1][1], offs, ts, lc,
                                  num_candidates=nc, x_mx=(yc, ys))
    plain = B.hstu_layer_fwd_mx(y1, ws[1][2], ws[1][0], ws[1][1], offs, ts, lc,
                                num_candidates=nc)
    np.testing.assert_array_equal(host(chained), host(plain))
