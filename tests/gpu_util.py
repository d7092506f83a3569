"""Helpers of the GPU parity tests: uploads through torch and the tolerance check.

Tolerance: the workloads state rel 1e-4 for fp32 and rel/abs 2e-2 for bf16.
A tensor passes iff both hold:
  * elementwise  |gpu - oracle| <= rtol*|oracle| + atol*max|oracle|
    (the absolute part is measured in units of the tensor's own range, so it
    is meaningful for outputs of magnitude 1e-5 as well as 1e+2), and
  * norm-wise    ||gpu - oracle||_2 <= rtol * ||oracle||_2,
with (rtol, atol) = (1e-4, 1e-4) for fp32 and (2e-2, 2e-2) for bf16.
The oracle is exact (fp64, no intermediate rounding); the bf16 path stores
U|V|Q|K, P, G and the outputs in bf16, which gives a relative RMS error of
about 2-5e-3 per layer and tails near 2e-2 of the RMS over 10^5-10^6 elements.
"""
import sys

import numpy as np

TOL = {"f32": (1e-4, 1e-4), "bf16": (2e-2, 2e-2)}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def torch_dtype(name):
    import torch
    return torch.bfloat16 if name == "bf16" else torch.float32


def dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to("cuda")


def host(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy() if t.dtype in (torch.bfloat16, torch.float16) \
        else t.detach().cpu().numpy().astype(np.float64)


def check_close(got, want, dtype: str, name: str, scale_ref=None):
    """Raise AssertionError with a summary unless got matches want within TOL[dtype]."""
    rtol, atol = TOL[dtype]
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    if want.size == 0:
        return
    ref = want if scale_ref is None else np.asarray(scale_ref, np.float64)
    amax = float(np.max(np.abs(ref)))
    err = np.abs(got - want)
    bound = rtol * np.abs(want) + atol * amax
    bad = ~(err <= bound)
    nw = float(np.linalg.norm(want))
    rel_l2 = float(np.linalg.norm(got - want) / nw) if nw > 0 else float(np.linalg.norm(got))
    ratio = float(np.max(err / np.maximum(bound, 1e-300)))
    rms = float(np.sqrt(np.mean(want ** 2)))
    say(f"  {name}: rel_l2={rel_l2:.3e} max_err/bound={ratio:.3f} rms={rms:.3e} max={amax:.3e}")
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(
            f"{name}: {int(bad.sum())}/{bad.size} elements out of tolerance "
            f"(rel_l2={rel_l2:.3e}, worst err/bound={ratio:.2f}); first at {idx.tolist()}: "
            f"got={got[tuple(idx[0])]!r} want={want[tuple(idx[0])]!r}")
    if nw > 0 and not rel_l2 <= rtol:
        raise AssertionError(f"{name}: relative L2 error {rel_l2:.3e} exceeds {rtol}")
