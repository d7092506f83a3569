"""GPU parity of the attention with its score product in MXFP8 ("Bending the
Scaling Law Curve in Large-Scale Recommendation Systems", Mixed precision;
OCP MX formats): q and k quantized by hstu_mx_quantize_heads bit-exactly
against the oracle's codes and scales, then hstu_attn_fwd_mx against the
oracle's attn_fwd_mx (the same codes, products summed exactly, the rest of the
attention in fp64) at the bf16 tolerance -- the GPU's remaining differences
are fp32 accumulation and the bf16 rounding of P, as in the bf16 attention."""
import numpy as np
import pytest

import synth
from oracle import hstu as orc
from tests.gpu_util import check_close, dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from hstu_sequential_transduction_amd import binding
    return binding


def _ac(binding, cfg, ks=0):
    ac = binding.AttnConfig(H=cfg.H, d_qk=cfg.d_qk, d_v=cfg.d_v, norm_len=cfg.norm_len,
                            n_pos_buckets=cfg.n_pos_buckets, n_time_buckets=cfg.n_time_buckets)
    ac.key_splits = ks
    return ac


def _quantize_checked(binding, x, H, d):
    """GPU codes and scale words of x [T, H, d], checked bit for bit against
    the oracle's MXFP8 along each head's channels."""
    import torch
    T = x.shape[0]
    codes, words = binding.hstu_mx_quantize_heads(dev(x.reshape(T, H * d), torch.bfloat16), H, d)
    wc, ws = orc.mx_quantize(x, axis=2)                 # [T, H, d], [T, H, d/32]
    np.testing.assert_array_equal(host(codes).astype(np.uint8), wc.reshape(T, H * d))
    w = host(words).astype(np.int64) & 0xFFFFFFFF       # [H, T]
    nb = d // 32
    got_s = np.stack([(w >> (8 * b)) & 0xFF for b in range(nb)], axis=-1)  # [H, T, nb]
    np.testing.assert_array_equal(got_s, np.transpose(ws, (1, 0, 2)).astype(np.int64))
    if nb < 4:
        assert not np.any(w >> (8 * nb)), "unused scale bytes must be zero"
    return codes, words


def _run(binding, a, cfg, ks=0):
    import torch
    T = a.q.shape[0]
    qc, qs = _quantize_checked(binding, a.q, cfg.H, cfg.d_qk)
    kc, ksw = _quantize_checked(binding, a.k, cfg.H, cfg.d_qk)
    nc = None if a.num_candidates is None else dev(a.num_candidates.astype(np.int32))
    out = binding.hstu_attn_fwd_mx(qc, qs, kc, ksw,
                                   dev(a.v.reshape(T, cfg.H * cfg.d_v), torch.bfloat16),
                                   dev(a.seq_offsets.astype(np.int32)),
                                   dev(a.timestamps.astype(np.int64)), dev(a.rab_pos),
                                   dev(a.rab_time), _ac(binding, cfg, ks), num_candidates=nc)
    return host(out).reshape(a.v.shape)


SMALL = {
    2: [1, 64, 130, 257, 0, 700],
    3: [32, 33, 520, 2048, 95],
    4: [300, 1100, 129],
    5: [100, 300, 0, 64],
}


# key_splits 0: 64-row items sharing each key tile between two waves (the
# default for these small batches); 1: 128-row items
@pytest.mark.parametrize("ks", [0, 1])
@pytest.mark.parametrize("ci", [2, 3, 4, 5])
def test_attn_fwd_mx_small(B, ci, ks):
    cfg = synth.get_config(ci).shrunk(B=len(SMALL[ci]), lengths=("list", SMALL[ci]))
    say(f"attn fwd mx small cfg{ci} key_splits={ks} lengths={SMALL[ci]} d={cfg.d_qk}")
    a = synth.make_attn_inputs(cfg, seed=300 + ci)
    got = _run(B, a, cfg, ks)
    want = orc.attn_fwd_mx(a.q, a.k, a.v, a.seq_offsets, a.timestamps, a.rab_pos, a.rab_time,
                           a.num_candidates, 0, cfg.norm_len)
    check_close(got, want, "bf16", f"O mx cfg{ci}")
    # the FP8 scores stay near the exact attention (format accuracy, not parity)
    ex = orc.attn_fwd(a.q, a.k, a.v, a.seq_offsets, a.timestamps, a.rab_pos, a.rab_time,
                      a.num_candidates, 0, cfg.norm_len)
    rel = np.linalg.norm(got - ex) / np.linalg.norm(ex)
    say(f"  O mx vs exact attention: rel_l2={rel:.3e}")
    assert rel < 0.1


@pytest.mark.parametrize("ci", [2, 5])
def test_attn_fwd_mx_literal_scale(B, ci):
    """q, k of std 0.15 and bias tables of std 0.02 (the workloads' literal scales)."""
    cfg = synth.get_config(ci).shrunk(B=len(SMALL[ci]), lengths=("list", SMALL[ci]))
    a = synth.make_attn_inputs(cfg, seed=400 + ci, qk_std=0.15, rab_std=0.02)
    got = _run(B, a, cfg)
    want = orc.attn_fwd_mx(a.q, a.k, a.v, a.seq_offsets, a.timestamps, a.rab_pos, a.rab_time,
                           a.num_candidates, 0, cfg.norm_len)
    check_close(got, want, "bf16", f"O mx literal cfg{ci}")


@pytest.mark.parametrize("ks", [0, 1])
def test_attn_fwd_mx_edge_sequences(B, ks):
    """Empty, one-row, all-candidate and tile-edge sequences."""
    cfg = synth.get_config(5).shrunk(B=4, lengths=("list", [0, 1, 127, 128]), num_candidates=3)
    a = synth.make_attn_inputs(cfg, seed=9)
    got = _run(B, a, cfg, ks)
    want = orc.attn_fwd_mx(a.q, a.k, a.v, a.seq_offsets, a.timestamps, a.rab_pos, a.rab_time,
                           a.num_candidates, 0, cfg.norm_len)
    check_close(got, want, "bf16", "O mx edge")


@pytest.mark.parametrize("ks", [0, 1])
def test_attn_fwd_mx_unsorted_and_wide_timestamps(B, ks):
    """The MX kernels share the bias paths: negative time distances (bucket 0)
    and a span beyond 2^31 s (the 64-bit path)."""
    import dataclasses
    cfg = synth.get_config(2).shrunk(B=3, lengths=("list", [150, 90, 200]))
    a = synth.make_attn_inputs(cfg, seed=19)
    rng = np.random.default_rng(19)
    ts = a.timestamps.copy()
    o = a.seq_offsets
    ts[o[0]:o[1]] = ts[o[0]] + rng.integers(-5000, 5000, size=150)          # unsorted
    ts[o[1]:o[2]] = np.sort(rng.integers(0, 1 << 40, size=90))               # wide span
    a = dataclasses.replace(a, timestamps=ts)
    got = _run(B, a, cfg, ks)
    want = orc.attn_fwd_mx(a.q, a.k, a.v, a.seq_offsets, a.timestamps, a.rab_pos, a.rab_time,
                           None, 0, cfg.norm_len)
    check_close(got, want, "bf16", f"O mx unsorted/wide key_splits={ks}")


def test_attn_fwd_mx_reused_plan_across_calls(B):
    """reuse_plan with the MX entry point: a second call on the same batch and
    workspace skips the plan and gives the same output bit for bit."""
    import dataclasses
    import torch
    cfg = synth.get_config(5).shrunk(B=3, lengths=("list", [300, 100, 64]), num_candidates=20)
    a = synth.make_attn_inputs(cfg, seed=23)
    T = a.q.shape[0]
    qc, qs = _quantize_checked(B, a.q, cfg.H, cfg.d_qk)
    kc, ksw = _quantize_checked(B, a.k, cfg.H, cfg.d_qk)
    v = dev(a.v.reshape(T, -1), torch.bfloat16)
    offs, ts = dev(a.seq_offsets.astype(np.int32)), dev(a.timestamps.astype(np.int64))
    rp, rt = dev(a.rab_pos), dev(a.rab_time)
    nc = dev(a.num_candidates.astype(np.int32))
    ws = B.LayerWorkspace()
    ac = _ac(B, cfg)
    first = B.hstu_attn_fwd_mx(qc, qs, kc, ksw, v, offs, ts, rp, rt, ac, num_candidates=nc,
                               workspace=ws)
    again = B.hstu_attn_fwd_mx(qc, qs, kc, ksw, v, offs, ts, rp, rt,
                               dataclasses.replace(ac, reuse_plan=1), num_candidates=nc,
                               workspace=ws)
    assert torch.equal(first, again)
    want = orc.attn_fwd_mx(a.q, a.k, a.v, a.seq_offsets, a.timestamps, a.rab_pos, a.rab_time,
                           a.num_candidates, 0, cfg.norm_len)
    check_close(host(again).reshape(a.v.shape), want, "bf16", "O mx reused plan")


@pytest.mark.parametrize("ci", [4, 5])
def test_attn_fwd_mx_full_size_sampled_rows(B, ci):
    """The training (d 128) and ranking (d 64) batches at full size, checked
    on sampled rows of every sequence."""
    cfg = synth.get_config(ci)
    say(f"attn fwd mx full cfg{ci}")
    a = synth.make_attn_inputs(cfg)
    got = _run(B, a, cfg)
    rng = np.random.default_rng(50 + ci)
    rows = []
    for b in range(cfg.B):
        n = int(a.lengths[b])
        r = {0, n - 1, n // 2} | set(rng.integers(0, n, size=5).tolist())
        if cfg.num_candidates:
            r |= {n - cfg.num_candidates - 1, n - cfg.num_candidates, n - 2}
        rows.append(sorted(x for x in r if 0 <= x < n))
    want = orc.attn_fwd_mx(a.q, a.k, a.v, a.seq_offsets, a.timestamps, a.rab_pos, a.rab_time,
                           a.num_candidates, 0, cfg.norm_len, return_rows=rows)
    sel = np.concatenate([a.seq_offsets[b] + np.asarray(rows[b], dtype=np.int64)
                          for b in range(cfg.B)])
    check_close(got[sel], want[sel], "bf16", f"O mx full cfg{ci} sampled", scale_ref=want[sel])


def test_attn_fwd_mx_empty_batch(B):
    """A batch of empty sequences: nothing to quantize or attend, no error."""
    cfg = synth.get_config(5).shrunk(B=2, lengths=("list", [0, 0]), num_candidates=0)
    a = synth.make_attn_inputs(cfg, seed=5)
    assert a.q.shape[0] == 0
    got = _run(B, a, cfg)
    assert got.shape == a.v.shape


def test_attn_fwd_mx_unsupported(B):
    """Descriptors outside the MX kernels (d_qk != d_v, windows) are refused
    before launch with HSTU_ERR_UNSUPPORTED."""
    import torch
    cfg = synth.get_config(2).shrunk(B=2, lengths=("list", [10, 20]))
    a = synth.make_attn_inputs(cfg, seed=3)
    T = a.q.shape[0]
    qc, qs = B.hstu_mx_quantize_heads(dev(a.q.reshape(T, -1), torch.bfloat16), cfg.H, cfg.d_qk)
    ac = _ac(B, cfg)
    ac.win_local, ac.win_global = 8, 2
    with pytest.raises(RuntimeError, match="UNSUPPORTED"):
        B.hstu_attn_fwd_mx(qc, qs, qc, qs, dev(a.v.reshape(T, -1), torch.bfloat16),
                           dev(a.seq_offsets.astype(np.int32)), dev(a.timestamps.astype(np.int64)),
                           dev(a.rab_pos), dev(a.rab_time), ac)
