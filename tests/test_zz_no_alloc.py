"""The no-allocation forward (hstu_attn_fwd_noalloc, plan in the library's
per-GPU scratch) against hstu_attn_fwd with a caller workspace: two calls in
a row, the second on a smaller batch, each bit-identical to the workspace
entry point (same kernels, deterministic forward), with and without a key
split; a split whose partial sums do not fit the scratch is refused."""
import dataclasses

import numpy as np
import pytest

import synth
from hstu_sequential_transduction_amd import _lib
from tests.gpu_util import host, say
from tests.test_gpu_layer import Dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from hstu_sequential_transduction_amd import binding
    return binding


def _case(B, ci, lengths, c, seed):
    cfg = synth.get_config(ci).shrunk(B=len(lengths), lengths=("list", lengths),
                                      num_candidates=c).unit_scale()
    inp = synth.make_inputs(cfg, seed=seed)
    d = Dev(inp, cfg)
    import torch
    td = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    g = torch.Generator(device="cpu").manual_seed(seed)
    HQ, HV = cfg.H * cfg.d_qk, cfg.H * cfg.d_v
    q = torch.randn(inp.T, HQ, generator=g).to(td).cuda()
    k = torch.randn(inp.T, HQ, generator=g).to(td).cuda()
    v = torch.randn(inp.T, HV, generator=g).to(td).cuda()
    W1, W2, rp, rt = d.layers[0]
    ac = B.AttnConfig(H=cfg.H, d_qk=cfg.d_qk, d_v=cfg.d_v, norm_len=cfg.norm_len)
    return ac, (q, k, v, d.offs, d.ts, rp, rt), d.nc


def _ws_bytes(B, ac, args):
    import ctypes as C
    q, offs = args[0], args[3]
    d = B.attn_desc(ac, offs.shape[0] - 1, q.shape[0], q.dtype, 0)
    return _lib.lib().hstu_attn_fwd_workspace_size(C.byref(d))


@pytest.mark.parametrize("ci,big_len,small_len,c", [
    (2, [700, 129, 1, 0, 333], [64, 17, 200], 0),
    (4, [700, 129, 1, 0, 333], [64, 17, 200], 0),
    (1, [120, 16, 1, 0, 77], [64, 17], 0),
    (5, [600, 90, 300], [100, 45], 40),
])
@pytest.mark.parametrize("splits", [0, 3])
def test_noalloc_matches_workspace_entry_point(B, ci, big_len, small_len, c, splits):
    import torch
    big = _case(B, ci, big_len, c, 4100 + ci)
    small = _case(B, ci, small_len, c, 4200 + ci)
    for name, (ac, args, nc) in (("first, larger", big), ("second, smaller", small)):
        say(f"noalloc cfg{ci} key_splits={splits} {name}: T={args[0].shape[0]}")
        ac = dataclasses.replace(ac, key_splits=splits)
        want = B.hstu_attn_fwd(*args, ac, num_candidates=nc)
        if splits and _ws_bytes(B, ac, args) > (8 << 20):
            # the partial sums of a forced split count against the scratch
            with pytest.raises(_lib.HstuError):
                B.hstu_attn_fwd_noalloc(*args, ac, num_candidates=nc)
            continue
        got = B.hstu_attn_fwd_noalloc(*args, ac, num_candidates=nc)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(got), host(want), err_msg=name)


def test_noalloc_rejects_problems_beyond_its_scratch(B):
    import torch
    from hstu_sequential_transduction_amd import _lib
    # a plan larger than HSTU_NOALLOC_SCRATCH_BYTES: refused before any launch
    T = 4_000_000
    ac = B.AttnConfig(H=1, d_qk=32, d_v=32, norm_len=128)
    d = B.attn_desc(ac, 1, T, torch.bfloat16, 0)
    L = _lib.lib()
    assert L.hstu_attn_fwd_workspace_size(d) > (8 << 20)
    p = 1 << 20
    st = L.hstu_attn_fwd_noalloc(d, p, p, 32, p, 32, p, p, p, p, None, p, 32, None)
    assert st == -3   # HSTU_ERR_WORKSPACE
