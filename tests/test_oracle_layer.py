"""Pins of the oracle's LayerNorm/gating, whole layer and backward (CPU only)."""
import numpy as np
import pytest

from oracle import hstu as orc
from tests.brute import (brute_attn_bwd, brute_attn_fwd, brute_layernorm,
                         brute_matmul)


def _layer_case(rng, lengths, cands=None, D=6, H=2, dqk=3, dv=3, affine=True, biases=True):
    lengths = np.asarray(lengths)
    offs = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(offs[-1])
    X = rng.standard_normal((T, D))
    W1 = rng.standard_normal((D, H * (2 * dv + 2 * dqk))) / np.sqrt(D)
    W2 = rng.standard_normal((H * dv, D)) / np.sqrt(H * dv)
    rp = rng.standard_normal((H, 128))
    rt = rng.standard_normal((H, 128))
    ts = []
    for b, n in enumerate(lengths):
        c = 0 if cands is None else cands[b]
        t = 1_600_000_000 + np.floor(np.cumsum(rng.exponential(5.0, size=n - c))).astype(np.int64)
        if c:
            t = np.concatenate([t, np.full(c, t[-1])])
        ts.append(t)
    ts = np.concatenate(ts).astype(np.int64)
    extra = {}
    if affine:
        extra["gamma"] = 1.0 + 0.3 * rng.standard_normal(H * dv)
        extra["beta"] = 0.2 * rng.standard_normal(H * dv)
    if biases:
        extra["b1"] = 0.1 * rng.standard_normal(W1.shape[1])
        extra["b2"] = 0.1 * rng.standard_normal(D)
    f = orc.LayerFlags(H=H, d_qk=dqk, d_v=dv, norm_mode=0, norm_len=max(lengths.max(), 1),
                       eps=1e-3)
    return X, W1, W2, rp, rt, offs, ts, f, extra


def test_layernorm_matches_loops_and_invariants():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 12)) * 3 + 1
    eps = 1e-2
    y, mu, rstd, xhat = orc.layernorm_fwd(x, eps)
    np.testing.assert_allclose(y, brute_layernorm(x, eps), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(y.mean(axis=1), 0, atol=1e-14)
    var = x.var(axis=1)
    np.testing.assert_allclose((y ** 2).mean(axis=1), var / (var + eps), rtol=1e-13)


def test_matmul_pin():
    rng = np.random.default_rng(2)
    a, b = rng.standard_normal((5, 7)), rng.standard_normal((7, 4))
    np.testing.assert_allclose(a @ b, brute_matmul(a, b), rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("cands", [None, [2, 0, 3]])
def test_layer_fwd_matches_loops(cands):
    rng = np.random.default_rng(3)
    X, W1, W2, rp, rt, offs, ts, f, ex = _layer_case(rng, [4, 6, 5], cands)
    Y, saved = orc.layer_fwd(X, W1, W2, rp, rt, offs, ts, cands, f, **ex)
    Z = brute_matmul(X, W1) + ex["b1"]
    Zh = np.array([[z / (1 + np.exp(-z)) for z in row] for row in Z])
    T, H, dv, dqk = X.shape[0], f.H, f.d_v, f.d_qk
    U = Zh[:, :H * dv]
    V = Zh[:, H * dv:2 * H * dv].reshape(T, H, dv)
    Q = Zh[:, 2 * H * dv:2 * H * dv + H * dqk].reshape(T, H, dqk)
    K = Zh[:, 2 * H * dv + H * dqk:].reshape(T, H, dqk)
    O = brute_attn_fwd(Q, K, V, offs, ts, rp, rt, cands, 0, f.norm_len).reshape(T, H * dv)
    G = (brute_layernorm(O, f.eps) * ex["gamma"] + ex["beta"]) * U
    Yb = brute_matmul(G, W2) + ex["b2"] + X
    np.testing.assert_allclose(Y, Yb, rtol=1e-11, atol=1e-13)


def test_attn_bwd_matches_pairwise_loops():
    rng = np.random.default_rng(4)
    lengths = [5, 4]
    cands = [2, 0]
    offs = np.array([0, 5, 9])
    q = rng.standard_normal((9, 2, 3)); k = rng.standard_normal((9, 2, 3))
    v = rng.standard_normal((9, 2, 2)); dO = rng.standard_normal((9, 2, 2))
    ts = np.array([0, 3, 9, 9, 9, 100, 250, 1000, 1000], dtype=np.int64)
    rp = rng.standard_normal((2, 128)); rt = rng.standard_normal((2, 128))
    got = orc.attn_bwd(q, k, v, offs, ts, rp, rt, dO, cands, 0, 6)
    want = brute_attn_bwd(q, k, v, offs, ts, rp, rt, dO, cands, 0, 6)
    for g, w in zip(got, want):
        np.testing.assert_allclose(g, w, rtol=1e-11, atol=1e-13)


def test_bias_gradients_have_equal_totals_and_dv_is_a_transpose_product():
    rng = np.random.default_rng(5)
    n = 10
    offs = np.array([0, n])
    q = rng.standard_normal((n, 2, 4)); k = rng.standard_normal((n, 2, 4))
    v = rng.standard_normal((n, 2, 3)); dO = rng.standard_normal((n, 2, 3))
    ts = np.cumsum(rng.integers(0, 50, size=n)).astype(np.int64)
    rp = np.zeros((2, 128)); rt = np.zeros((2, 128))
    dq, dk, dv, drp, drt = orc.attn_bwd(q, k, v, offs, ts, rp, rt, dO, None, 0, 12)
    np.testing.assert_allclose(drp.sum(axis=1), drt.sum(axis=1), rtol=1e-12)
    for h in range(2):
        S = q[:, h] @ k[:, h].T
        A = np.tril(S / (1 + np.exp(-S))) / 12
        np.testing.assert_allclose(dv[:, h], A.T @ dO[:, h], rtol=1e-12, atol=1e-14)


def _loss(params, names, base_args, f, dY):
    X, W1, W2, rp, rt, offs, ts, cands = base_args
    kw = {k: params[k] for k in ("gamma", "beta", "b1", "b2") if k in params}
    Y, _ = orc.layer_fwd(params["X"], params["W1"], params["W2"], params["rab_pos"],
                         params["rab_time"], offs, ts, cands, f, **kw)
    return float((Y * dY).sum())


@pytest.mark.parametrize("cands,residual,proj_silu", [(None, True, True), ([1, 3], True, True),
                                                      ([0, 2], False, False)])
def test_layer_bwd_finite_differences(cands, residual, proj_silu):
    rng = np.random.default_rng(6)
    X, W1, W2, rp, rt, offs, ts, f, ex = _layer_case(rng, [5, 6], cands, D=5, H=2, dqk=2, dv=3)
    f.residual = residual
    f.proj_silu = proj_silu
    dY = rng.standard_normal((X.shape[0], X.shape[1]))
    Y, saved = orc.layer_fwd(X, W1, W2, rp, rt, offs, ts, cands, f, **ex)
    g = orc.layer_bwd(dY, X, W1, W2, rp, rt, offs, ts, cands, f, saved, **ex)
    params = dict(X=X, W1=W1, W2=W2, rab_pos=rp, rab_time=rt, **ex)
    grads = dict(X=g["dX"], W1=g["dW1"], W2=g["dW2"], rab_pos=g["drab_pos"],
                 rab_time=g["drab_time"], gamma=g["dgamma"], beta=g["dbeta"], b1=g["db1"],
                 b2=g["db2"])
    base_args = (X, W1, W2, rp, rt, offs, ts, cands)
    h = 1e-6
    for name, arr in params.items():
        num = np.zeros_like(arr)
        flat = arr.reshape(-1)
        idxs = range(flat.size)
        if name in ("rab_pos", "rab_time"):
            idxs = list(range(0, 20)) + [127, 128, 255]
        for i in idxs:
            old = flat[i]
            flat[i] = old + h
            lp = _loss(params, None, base_args, f, dY)
            flat[i] = old - h
            lm = _loss(params, None, base_args, f, dY)
            flat[i] = old
            num.reshape(-1)[i] = (lp - lm) / (2 * h)
        an = grads[name].reshape(-1)[list(idxs)]
        nu = num.reshape(-1)[list(idxs)]
        scale = max(np.abs(nu).max(), 1e-3)
        assert np.abs(an - nu).max() <= 1e-6 * scale + 1e-9, name


def test_stack_feeds_outputs_forward():
    rng = np.random.default_rng(7)
    X, W1, W2, rp, rt, offs, ts, f, _ = _layer_case(rng, [4, 3], None, affine=False,
                                                    biases=False)

    class L:
        pass
    l1, l2 = L(), L()
    l1.W1, l1.W2, l1.rab_pos, l1.rab_time = W1, W2, rp, rt
    l2.W1, l2.W2, l2.rab_pos, l2.rab_time = W1 * 0.5, W2 * 2, rt, rp
    outs = orc.stack_fwd(X, [l1, l2], offs, ts, None, f)
    y1, _ = orc.layer_fwd(X, W1, W2, rp, rt, offs, ts, None, f)
    y2, _ = orc.layer_fwd(y1, W1 * 0.5, W2 * 2, rt, rp, offs, ts, None, f)
    np.testing.assert_array_equal(outs[0], y1)
    np.testing.assert_array_equal(outs[1], y2)


@pytest.mark.parametrize("wl,wg", [(2, 0), (3, 2)])
def test_semilocal_attn_bwd_matches_pairwise_loops(wl, wg):
    rng = np.random.default_rng(14)
    offs = np.array([0, 6, 11])
    cands = [2, 0]
    q = rng.standard_normal((11, 2, 3)); k = rng.standard_normal((11, 2, 3))
    v = rng.standard_normal((11, 2, 2)); dO = rng.standard_normal((11, 2, 2))
    ts = np.array([0, 3, 9, 20, 20, 20, 100, 250, 1000, 1100, 4000], dtype=np.int64)
    rp = rng.standard_normal((2, 128)); rt = rng.standard_normal((2, 128))
    got = orc.attn_bwd(q, k, v, offs, ts, rp, rt, dO, cands, 0, 6, win_local=wl,
                       win_global=wg)
    want = brute_attn_bwd(q, k, v, offs, ts, rp, rt, dO, cands, 0, 6, win_local=wl,
                          win_global=wg)
    for g, w in zip(got, want):
        np.testing.assert_allclose(g, w, rtol=1e-11, atol=1e-13)
