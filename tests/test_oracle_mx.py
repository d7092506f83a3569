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
