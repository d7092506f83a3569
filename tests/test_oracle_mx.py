"""Pins of the oracle's MXFP8 pieces (CPU only): the E4M3 element format and
E8M0 block scales of the OCP Microscaling spec, round-to-nearest-even with
saturation, the exact MX matmul, and the MX layer's reduction to the plain
layer when every operand is already representable."""
import numpy as np
import pytest

from oracle import hstu as orc


def _decode_by_fields(c):
    """E4M3 from its bit fields, written out: sign, exponent (bias 7), mantissa."""
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    if e == 15 and m == 7:
        return float("nan")
    mag = (m / 8.0) * 2.0 ** (1 - 7) if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


def test_e4m3_decode_table():
    got = orc.e4m3_decode(np.arange(256))
    for c in range(256):
        w = _decode_by_fields(c)
        if np.isnan(w):
            assert np.isnan(got[c]) and c in (0x7F, 0xFF)
        else:
            assert got[c] == w, hex(c)
    # landmarks of the format
    assert got[0x00] == 0.0 and got[0x01] == 2.0 ** -9 and got[0x07] == 7 * 2.0 ** -9
    assert got[0x08] == 2.0 ** -6 and got[0x38] == 1.0 and got[0x7E] == 448.0
    assert got[0x78] == 256.0 and got[0xB8] == -1.0
    assert np.all(np.diff(got[:0x7F]) > 0)                       # increasing, no duplicates


def test_e4m3_round_trip_ties_and_saturation():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    assert np.array_equal(orc.e4m3_encode(orc.e4m3_decode(codes)), codes.astype(np.uint8))
    pos = orc.e4m3_decode(np.arange(0x7F))
    mids = (pos[:-1] + pos[1:]) / 2
    got = orc.e4m3_encode(mids)
    for i, c in enumerate(got):
        assert c in (i, i + 1) and c % 2 == 0, (i, c)        # ties go to the even code
    assert np.array_equal(orc.e4m3_encode(np.nextafter(mids, 0)), np.arange(0x7E))
    assert np.array_equal(orc.e4m3_encode(np.nextafter(mids, 1e9)), np.arange(1, 0x7F))
    assert orc.e4m3_encode(449.0) == 0x7E and orc.e4m3_encode(1e6) == 0x7E
    assert orc.e4m3_encode(-1e6) == 0xFE and orc.e4m3_encode(-0.0) == 0x80
    # the smallest step is 2^-9: a quarter step rounds down, half a step and
    # one and a half steps are ties that go to the even codes 0 and 2
    assert orc.e4m3_encode(2.0 ** -11) == 0x00
    assert orc.e4m3_encode(3 * 2.0 ** -11) == 0x01
    assert orc.e4m3_encode(2.0 ** -10) == 0x00
    assert orc.e4m3_encode(3 * 2.0 ** -10) == 0x02


def test_mx_block_scales_and_error_bound():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((16, 128)) * np.exp2(rng.integers(-20, 20, size=(16, 1)))
    x[3, 32:64] = 0.0
    codes, scales = orc.mx_quantize(x, axis=1)
    assert scales.shape == (16, 4) and codes.shape == x.shape
    blk = x.reshape(16, 4, 32)
    amax = np.abs(blk).max(-1)
    for i in range(16):
        for j in range(4):
            if amax[i, j] == 0:
                assert scales[i, j] == 0 and np.all(codes[i, 32 * j:32 * j + 32] == 0)
                continue
            e = int(np.floor(np.log2(amax[i, j])))
            assert int(scales[i, j]) == e - 8 + 127
            v = np.abs(orc.e4m3_decode(codes[i, 32 * j:32 * j + 32]))
            assert 256 <= v.max() <= 448                       # the block's largest element
    deq = orc.mx_dequantize(codes, scales, axis=1)
    X = np.exp2(scales.astype(np.float64) - 127).repeat(32, axis=1)
    err = np.abs(deq - x)
    # half a step of the element grid (2^-4 relative for normals), the
    # subnormal step 2^-9 X, and the saturated range [448, 512) X
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * X)
    bound = np.where(np.abs(x) >= 448 * X, 64 * X, bound)
    assert np.all(err <= bound + 1e-300)


def test_mx_power_of_two_invariance():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, 64))
    c0, s0 = orc.mx_quantize(x, axis=1)
    c1, s1 = orc.mx_quantize(x * 2.0 ** 13, axis=1)
    assert np.array_equal(c0, c1) and np.array_equal(s1.astype(int), s0.astype(int) + 13)
    c2, s2 = orc.mx_quantize(x.T, axis=0)
    assert np.array_equal(c2, c0.T) and np.array_equal(s2, s0.T)


def test_mx_matmul_matches_a_block_loop():
    rng = np.random.default_rng(5)
    a, b = rng.standard_normal((3, 64)), rng.standard_normal((64, 2)) * 7.0
    got = orc.mx_matmul(a, b)
    qa, sa = orc.mx_quantize(a, axis=1)
    qb, sb = orc.mx_quantize(b, axis=0)
    want = np.zeros((3, 2))
    for i in range(3):
        for j in range(2):
            acc = 0.0
            for k in range(64):
                blk = k // 32
                acc += (_decode_by_fields(int(qa[i, k])) * 2.0 ** (int(sa[i, blk]) - 127)
                        * _decode_by_fields(int(qb[k, j])) * 2.0 ** (int(sb[blk, j]) - 127))
            want[i, j] = acc
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=1e-14)
    # and over a larger product it stays within a few percent of the exact
    # one (E4M3 keeps 3 mantissa bits: about 3 % RMS rounding per element)
    a, b = rng.standard_normal((16, 256)), rng.standard_normal((256, 16))
    ex = a @ b
    assert np.linalg.norm(orc.mx_matmul(a, b) - ex) <= 0.06 * np.linalg.norm(ex)


def _representable(rng, shape, axis):
    """Values MXFP8 holds exactly: E4M3 grid values, each block with one
    element of magnitude in [256, 448] times the block's power of two."""
    grid = orc.e4m3_decode(np.arange(0x7F))
    v = rng.choice(np.concatenate([grid, -grid]), size=shape)
    vm = np.moveaxis(v, axis, -1)
    blocks = vm.reshape(vm.shape[:-1] + (vm.shape[-1] // 32, 32))
    blocks[..., 0] = rng.choice(grid[(grid >= 256) & (grid <= 448)], size=blocks.shape[:-1])
    sc = np.exp2(rng.integers(-14, -6, size=blocks.shape[:-1]))[..., None]
    return np.moveaxis((blocks * sc).reshape(vm.shape), -1, axis)


def test_mx_layer_equals_the_plain_layer_on_representable_operands():
    rng = np.random.default_rng(6)
    H, dqk, dv, D = 2, 32, 32, 64
    lengths = [5, 9]
    offs = np.array([0, 5, 14])
    ts = np.concatenate([1_600_000_000 + np.arange(n) * 40 for n in lengths]).astype(np.int64)
    X = _representable(rng, (14, D), axis=1)
    W1 = _representable(rng, (D, H * (2 * dv + 2 * dqk)), axis=0)
    W2 = rng.standard_normal((H * dv, D)) / 8
    rp, rt = rng.standard_normal((H, 128)), rng.standard_normal((H, 128))
    f = orc.LayerFlags(H=H, d_qk=dqk, d_v=dv, norm_len=16, eps=1e-3)
    # the output matmul's left operand (the gated LayerNorm) is not on the
    # grid, so compare the projection step alone and then the whole layer
    # with an MX-exact W2 against the plain layer with G rounded the same way
    np.testing.assert_allclose(orc.mx_matmul(X, W1), X @ W1, rtol=1e-13, atol=1e-15)
    Y = orc.layer_fwd_mx(X, W1, W2, rp, rt, offs, ts, None, f)
    Yp, sv = orc.layer_fwd(X, W1, W2, rp, rt, offs, ts, None, f)
    Gq, Gs = orc.mx_quantize(sv["G"], axis=1)
    W2q, W2s = orc.mx_quantize(W2, axis=0)
    want = (orc.mx_dequantize(Gq, Gs, axis=1) @ orc.mx_dequantize(W2q, W2s, axis=0)) + X
    np.testing.assert_allclose(Y, want, rtol=1e-12, atol=1e-13)
    # and the MX layer stays within a few percent of the plain one
    assert np.linalg.norm((Y - X) - (Yp - X)) <= 0.08 * np.linalg.norm(Yp - X)


def _mx_err_bound(x, axis):
    """Largest rounding error MXFP8 can make on each element of x (blocks of
    32 along `axis`): half a spacing of the E4M3 grid scaled by the block's
    power of two X = 2^(floor(log2 amax) - 8) -- 2^-4 |x| for normal values,
    2^-10 X below E4M3's normal range -- or the clamp to 448 X above it."""
    x = np.asarray(x, np.float64)
    xm = np.moveaxis(x, axis, -1)
    blocks = np.abs(xm).reshape(xm.shape[:-1] + (xm.shape[-1] // 32, 32))
    amax = blocks.max(axis=-1, keepdims=True)
    X = np.where(amax > 0, np.exp2(np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8), 0.0)
    e = np.maximum(np.maximum(2.0 ** -4 * blocks, 2.0 ** -10 * X), blocks - 448 * X)
    return np.moveaxis(e.reshape(xm.shape), -1, axis)


def _mx_case(seed, representable=False):
    rng = np.random.default_rng(seed)
    H, dqk, dv, D = 2, 32, 32, 64
    lengths = [7, 12, 3]
    offs = np.concatenate([[0], np.cumsum(lengths)])
    T = int(offs[-1])
    ts = np.concatenate([1_600_000_000 + np.arange(n) * 50 for n in lengths]).astype(np.int64)
    F1 = H * (2 * dv + 2 * dqk)
    if representable:
        X = _representable(rng, (T, D), axis=1)
        W1 = _representable(rng, (D, F1), axis=1)   # rows along F1: dX's operand
        W2 = _representable(rng, (H * dv, D), axis=1)  # rows along D: dG's operand
        dY = _representable(rng, (T, D), axis=1)
    else:
        X = rng.standard_normal((T, D))
        W1 = rng.standard_normal((D, F1)) / 8
        W2 = rng.standard_normal((H * dv, D)) / 8
        dY = rng.standard_normal((T, D))
    rp, rt = rng.standard_normal((H, 128)) * 0.1, rng.standard_normal((H, 128)) * 0.1
    f = orc.LayerFlags(H=H, d_qk=dqk, d_v=dv, norm_len=16, eps=1e-3)
    return X, W1, W2, dY, rp, rt, offs, ts, f


def _pad_k(a, b):
    """a [M, K], b [K, N] with K zero-padded to a multiple of 32."""
    k = a.shape[1]
    kp = -(-k // 32) * 32
    return np.pad(a, ((0, 0), (0, kp - k))), np.pad(b, ((0, kp - k), (0, 0)))


def test_mx_backward_products_within_the_rounding_bound():
    """All four products of the MX backward differ from the exact products of
    the same operands by at most the bound the per-element rounding allows:
    |MX(a) MX(b) - a b| <= sum_k e_a |b| + |a| e_b + e_a e_b, each operand
    rounded along the contraction (for the weight gradients the 22 tokens,
    one short block)."""
    X, W1, W2, dY, rp, rt, offs, ts, f = _mx_case(21)
    _, sv = orc.layer_fwd_mx(X, W1, W2, rp, rt, offs, ts, None, f, return_saved=True)
    g = orc.layer_bwd_mx(dY, X, W1, W2, rp, rt, offs, ts, None, f, sv)

    def check(a, b, got):
        a, b = _pad_k(np.asarray(a, np.float64), np.asarray(b, np.float64))
        ea, eb = _mx_err_bound(a, axis=1), _mx_err_bound(b, axis=0)
        bound = ea @ np.abs(b) + np.abs(a) @ eb + ea @ eb
        assert np.all(np.abs(got - a @ b) <= bound * (1 + 1e-9) + 1e-300)
        # and the bound is not vacuous: the rounding changed the product
        assert np.abs(got - a @ b).max() > 0

    check(dY, W2.T, g["dG"])
    check(g["dZ"], W1.T, g["dX"] - dY)
    check(sv["G"].T, dY, g["dW2"])
    check(X.T, g["dZ"], g["dW1"])


def test_mx_matmul_short_last_block():
    """A contraction of 40: the second block holds 8 values.  It equals the
    product of the operands zero-padded to 64 (the reading), is exact when
    both operands lie on the MXFP8 grid of their padded blocks, and is not
    the product with the short block dropped."""
    rng = np.random.default_rng(31)
    a = rng.standard_normal((5, 40))
    b = rng.standard_normal((40, 6))
    ap, bp = _pad_k(a, b)
    qa, sa = orc.mx_quantize(ap, axis=1)
    qb, sb = orc.mx_quantize(bp, axis=0)
    want = orc.mx_dequantize(qa, sa, axis=1) @ orc.mx_dequantize(qb, sb, axis=0)
    got = orc.mx_matmul(a, b)
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=1e-300)
    assert np.abs(got - orc.mx_matmul(a[:, :32], b[:32])).max() > 1e-3
    ar = orc.mx_dequantize(qa, sa, axis=1)[:, :40]
    br = orc.mx_dequantize(qb, sb, axis=0)[:40]
    np.testing.assert_allclose(orc.mx_matmul(ar, br), ar @ br, rtol=1e-13, atol=1e-300)


def test_mx_backward_exact_on_representable_operands():
    """With dY and W2 on the MXFP8 grid along D (the contraction of dG), dG is
    the exact product; with X and dY on the grid along the tokens as well,
    the only rounding left in dW1 and dW2 is that of dZ and G."""
    X, W1, W2, dY, rp, rt, offs, ts, f = _mx_case(22, representable=True)
    rng = np.random.default_rng(22)
    _, sv = orc.layer_fwd_mx(X, W1, W2, rp, rt, offs, ts, None, f, return_saved=True)
    g = orc.layer_bwd_mx(dY, X, W1, W2, rp, rt, offs, ts, None, f, sv)
    np.testing.assert_allclose(g["dG"], dY @ W2.T, rtol=1e-13, atol=1e-300)
    # tokens-axis grid: operands whose MXFP8 along the (padded) tokens is exact
    Xt = _representable(rng, (32, X.shape[1]), axis=0)[:X.shape[0]]
    dYt = _representable(rng, (32, dY.shape[1]), axis=0)[:dY.shape[0]]
    Gq = orc.mx_quantize(np.pad(sv["G"], ((0, 32 - sv["G"].shape[0]), (0, 0))), axis=0)
    Gr = orc.mx_dequantize(*Gq, axis=0)[:sv["G"].shape[0]]
    np.testing.assert_allclose(orc.mx_matmul(Gr.T, dYt), Gr.T @ dYt, rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(orc.mx_matmul(Xt.T, dYt), Xt.T @ dYt, rtol=1e-13, atol=1e-300)
    # quantizing along the other axis would not be exact here
    q, s = orc.mx_quantize(W2.T, axis=1)
    assert np.abs(orc.mx_dequantize(q, s, axis=1) - W2.T).max() > 0


def test_mx_backward_close_to_the_exact_backward():
    """The FP8 error of the backward on ordinary operands: a few percent of
    the exact gradients (accuracy of the format, not a parity bound)."""
    X, W1, W2, dY, rp, rt, offs, ts, f = _mx_case(23)
    _, sv = orc.layer_fwd_mx(X, W1, W2, rp, rt, offs, ts, None, f, return_saved=True)
    g = orc.layer_bwd_mx(dY, X, W1, W2, rp, rt, offs, ts, None, f, sv)
    ex = orc.layer_bwd(dY, X, W1, W2, rp, rt, offs, ts, None, f, sv)
    for k in ("dX", "dW1", "dW2", "drab_pos", "drab_time"):
        rel = np.linalg.norm(g[k] - ex[k]) / np.linalg.norm(ex[k])
        assert rel < 0.1, (k, rel)
    # the output product's weight gradient: the same operands (G, dY) in both,
    # so its difference is the MXFP8 rounding alone, within its bound
    G, dYp = _pad_k(sv["G"].T, dY)
    bound = _mx_err_bound(G, 1) @ np.abs(dYp) + np.abs(G) @ _mx_err_bound(dYp, 0) + \
        _mx_err_bound(G, 1) @ _mx_err_bound(dYp, 0)
    assert np.all(np.abs(g["dW2"] - ex["dW2"]) <= bound * (1 + 1e-9))


# ---- the attention's score product in MXFP8 (attn_fwd_mx) -------------------

def _attn_mx_case(seed, representable=False, d=64):
    rng = np.random.default_rng(seed)
    H = 2
    lengths, cands = [9, 1, 14, 6], [0, 0, 3, 6]
    offs = np.concatenate([[0], np.cumsum(lengths)])
    T = int(offs[-1])
    ts = np.concatenate([1_600_000_000 + np.cumsum(rng.integers(0, 400, n)) for n in lengths])
    if representable:
        q = _representable(rng, (T, H, d), axis=2)
        k = _representable(rng, (T, H, d), axis=2)
    else:
        # channels spread over binades so that blocks saturate and go subnormal
        q = rng.standard_normal((T, H, d)) * np.exp2(rng.integers(-3, 3, (T, H, d))) / 4
        k = rng.standard_normal((T, H, d)) * np.exp2(rng.integers(-3, 3, (T, H, d))) / 4
    v = rng.standard_normal((T, H, d))
    rp, rt = rng.standard_normal((H, 128)) * 0.1, rng.standard_normal((H, 128)) * 0.1
    return q, k, v, offs, ts.astype(np.int64), rp, rt, np.array(cands, np.int32)


def test_attn_mx_exact_on_representable_qk():
    """Q and K already on the MXFP8 grid with their blocks along each head's
    channels: the MX score product is the exact one, so attn_fwd_mx equals
    attn_fwd (blocks taken along the tokens or across heads would round)."""
    q, k, v, offs, ts, rp, rt, nc = _attn_mx_case(11, representable=True)
    got = orc.attn_fwd_mx(q, k, v, offs, ts, rp, rt, nc, norm_len=16)
    want = orc.attn_fwd(q, k, v, offs, ts, rp, rt, nc, norm_len=16)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


@pytest.mark.parametrize("d", [32, 64, 128])
def test_attn_mx_within_the_rounding_bound(d):
    """|O_mx - O| per element stays within what the per-element MXFP8
    rounding of q and k (blocks of 32 along each head's channels) allows,
    written out pair by pair: |dS_ij| <= sum_c (eq|k| + |q|ek + eq ek), and
    SiLU is Lipschitz with constant max|SiLU'| < 1.1, so
    |dO_i| <= (1/N) sum_{j allowed} 1.1 |dS_ij| |v_j|.  The bound is not
    vacuous: the rounding changes the output."""
    q, k, v, offs, ts, rp, rt, nc = _attn_mx_case(12 + d, d=d)
    N = 16
    got = orc.attn_fwd_mx(q, k, v, offs, ts, rp, rt, nc, norm_len=N)
    ex = orc.attn_fwd(q, k, v, offs, ts, rp, rt, nc, norm_len=N)
    eq, ek = _mx_err_bound(q, axis=2), _mx_err_bound(k, axis=2)
    T, H, _ = q.shape
    bound = np.zeros_like(ex)
    for b in range(len(offs) - 1):
        o0, o1, c = int(offs[b]), int(offs[b + 1]), int(nc[b])
        n, nh = o1 - o0, o1 - o0 - c
        for i in range(n):
            for j in range(n):
                ok = j <= i if i < nh else (j < nh or j == i)
                if not ok:
                    continue
                for h in range(H):
                    qi, kj = q[o0 + i, h], k[o0 + j, h]
                    ei, ej = eq[o0 + i, h], ek[o0 + j, h]
                    ds = np.sum(ei * np.abs(kj) + np.abs(qi) * ej + ei * ej)
                    bound[o0 + i, h] += 1.1 * ds * np.abs(v[o0 + j, h]) / N
    assert np.all(np.abs(got - ex) <= bound * (1 + 1e-9) + 1e-300)
    assert np.abs(got - ex).max() > 0.0


def _round_block_by_search(vals):
    """One 32-value block rounded to MXFP8 by a search over all 254 finite
    E4M3 values (decoded from their fields): scale 2^(floor(log2 amax) - 8)
    from math.frexp, each value clamped to +-448 scaled units and sent to the
    nearest grid value, ties to the even code."""
    import math
    amax = max(abs(x) for x in vals)
    if amax == 0.0:
        return [0.0] * len(vals)
    X = 2.0 ** (math.frexp(amax)[1] - 1 - 8)
    grid = [(c, _decode_by_fields(c)) for c in range(256) if not math.isnan(_decode_by_fields(c))]
    out = []
    for x in vals:
        y = min(max(x / X, -448.0), 448.0)
        best = min(grid, key=lambda cv: (abs(cv[1] - y), cv[0] & 1))
        out.append(best[1] * X)
    return out


def test_attn_mx_matches_brute_force_on_searched_roundings():
    """attn_fwd_mx against the per-pair brute-force attention run on q and k
    rounded block by block (32 channels of one head) by a grid search."""
    from tests.brute import brute_attn_fwd
    q, k, v, offs, ts, rp, rt, nc = _attn_mx_case(21, d=64)
    T, H, d = q.shape
    qr, kr = np.empty_like(q), np.empty_like(k)
    for t in range(T):
        for h in range(H):
            for b0 in range(0, d, 32):
                qr[t, h, b0:b0 + 32] = _round_block_by_search(list(q[t, h, b0:b0 + 32]))
                kr[t, h, b0:b0 + 32] = _round_block_by_search(list(k[t, h, b0:b0 + 32]))
    want = brute_attn_fwd(qr, kr, v, offs, ts, rp, rt, nc, 0, 16)
    got = orc.attn_fwd_mx(q, k, v, offs, ts, rp, rt, nc, norm_len=16)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)
    # the rounding is not a no-op here
    assert np.abs(got - orc.attn_fwd(q, k, v, offs, ts, rp, rt, nc, norm_len=16)).max() > 1e-6


def test_bf16_round_against_torch_and_ties():
    """The oracle's bf16 rounding equals torch's float32 -> bfloat16
    conversion (round to nearest even) on spread values, and sends exact
    midpoints to the even neighbour."""
    import torch
    rng = np.random.default_rng(31)
    x = (rng.standard_normal(20000) * np.exp2(rng.integers(-30, 30, 20000))).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(orc.bf16_round(x), want)
    k = np.arange(128, 256, dtype=np.float64)
    mid = (k + 0.5) / 128.0                       # halfway between bf16 neighbours in [1, 2)
    even = np.where(k % 2 == 0, k, k + 1) / 128.0
    np.testing.assert_array_equal(orc.bf16_round(mid), even)
    assert orc.bf16_round(0.0) == 0.0 and orc.bf16_round(-3.0) == -3.0


def test_mx_layer_scores_quantize_the_bf16_activations():
    """layer_fwd_mx with mx_scores equals its composition written out: the
    MX projection, SiLU, the attention with q and k rounded to bf16 and then
    to MXFP8, and the plain LayerNorm-gate and MX output product."""
    X, W1, W2, dY, rp, rt, offs, ts, f = _mx_case(41)
    f = orc.LayerFlags(H=f.H, d_qk=32, d_v=32, norm_len=16, eps=1e-3)
    Y = orc.layer_fwd_mx(X, W1, W2, rp, rt, offs, ts, None, f, mx_scores=True)
    Zh = orc.silu(orc.mx_matmul(X, W1))
    T, H, d = X.shape[0], f.H, 32
    U, V, Q, K = (Zh[:, i * H * d:(i + 1) * H * d].reshape(T, H, d) for i in range(4))
    qc, qs = orc.mx_quantize(orc.bf16_round(Q), axis=2)
    kc, ks = orc.mx_quantize(orc.bf16_round(K), axis=2)
    O = orc.attn_fwd(orc.mx_dequantize(qc, qs, axis=2), orc.mx_dequantize(kc, ks, axis=2), V,
                     offs, ts, rp, rt, None, 0, 16).reshape(T, H * d)
    mu = O.mean(axis=1, keepdims=True)
    var = ((O - mu) ** 2).mean(axis=1, keepdims=True)
    G = (O - mu) / np.sqrt(var + 1e-3) * U.reshape(T, H * d)
    want = orc.mx_matmul(G, W2) + X
    np.testing.assert_allclose(Y, want, rtol=1e-10, atol=1e-12)
    # and the score rounding changes the layer
    assert np.abs(Y - orc.layer_fwd_mx(X, W1, W2, rp, rt, offs, ts, None, f)).max() > 0


def test_mx_layer_scores_training_saves_the_mx_values():
    """With mx_scores and return_saved, the saved U|V|Q|K holds q and k as
    their MXFP8 values (U and V unchanged), the forward output is the one
    without return_saved, and the backward on those values equals the MX
    backward of the plain MX layer when q and k are replaced by them: the
    gradients reach Z through the quantizer as through the identity."""
    X, W1, W2, dY, rp, rt, offs, ts, f = _mx_case(43)
    f = orc.LayerFlags(H=f.H, d_qk=32, d_v=32, norm_len=16, eps=1e-3)
    Y, sv = orc.layer_fwd_mx(X, W1, W2, rp, rt, offs, ts, None, f, mx_scores=True,
                             return_saved=True)
    np.testing.assert_array_equal(Y, orc.layer_fwd_mx(X, W1, W2, rp, rt, offs, ts, None, f,
                                                      mx_scores=True))
    Zh = orc.silu(orc.mx_matmul(X, W1))
    T, H, d = X.shape[0], f.H, 32
    U, V, Q, K = (Zh[:, i * H * d:(i + 1) * H * d].reshape(T, H, d) for i in range(4))
    qc, qs = orc.mx_quantize(orc.bf16_round(Q), axis=2)
    kc, ks = orc.mx_quantize(orc.bf16_round(K), axis=2)
    Qm = orc.mx_dequantize(qc, qs, axis=2).reshape(T, -1)
    Km = orc.mx_dequantize(kc, ks, axis=2).reshape(T, -1)
    np.testing.assert_array_equal(sv["Zh"][:, :2 * H * d], Zh[:, :2 * H * d])
    np.testing.assert_array_equal(sv["Zh"][:, 2 * H * d:3 * H * d], Qm)
    np.testing.assert_array_equal(sv["Zh"][:, 3 * H * d:], Km)
    # the backward: dQ and dK of the attention on (Qm, Km), straight through
    g = orc.layer_bwd_mx(dY, X, W1, W2, rp, rt, offs, ts, None, f, sv)
    dO = g["dO"].reshape(T, H, d)
    dQ, dK, dV, _, _ = orc.attn_bwd(Qm.reshape(T, H, d), Km.reshape(T, H, d), V, offs, ts, rp,
                                    rt, dO, None, 0, 16)
    sg = orc.silu_grad(sv["Z"])
    np.testing.assert_allclose(g["dZ"][:, 2 * H * d:3 * H * d], dQ.reshape(T, -1) *
                               sg[:, 2 * H * d:3 * H * d], rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(g["dZ"][:, 3 * H * d:], dK.reshape(T, -1) * sg[:, 3 * H * d:],
                               rtol=1e-10, atol=1e-13)
