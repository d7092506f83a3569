"""The C-ABI library loads and exports what include/hstu.h declares (CPU only).

Calls made here return before any device work: workspace sizing and host-side
argument validation.
"""
import ctypes as C
import os
import re

import pytest

from hstu_sequential_transduction_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hstu.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(hstu_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libhstu.so is not built (run __graft_entry__.build())")
    return _lib.lib()


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib.EXPORTED)


def test_version_and_status_strings(L):
    assert b"gfx950" in L.hstu_version()
    assert L.hstu_status_string(0) == b"ok"
    assert L.hstu_status_string(-3) == b"workspace too small"


def _desc(**kw):
    base = dict(B=4, T=300, H=2, d_qk=32, d_v=32, n_pos_buckets=128, n_time_buckets=128,
                norm_mode=0, norm_len=128, dtype=1, rab_head_stride=128, win_local=0,
                win_global=0, max_len=0, reuse_plan=0, key_splits=0)
    base.update(kw)
    return _lib.AttnDesc(*[base[f] for f, _ in _lib.AttnDesc._fields_])


def test_workspace_sizes_grow_with_T(L):
    a = L.hstu_attn_fwd_workspace_size(C.byref(_desc(T=1000, key_splits=1)))
    b = L.hstu_attn_fwd_workspace_size(C.byref(_desc(T=100000, key_splits=1)))
    assert 0 < a < b
    # the default (key_splits 0) plans 64-row work items (twice the list) when
    # even T/128 + B items per head fit the GPU at once, 128-row ones otherwise
    assert L.hstu_attn_fwd_workspace_size(C.byref(_desc(T=1000))) > a
    assert L.hstu_attn_fwd_workspace_size(C.byref(_desc(T=100000))) == b
    assert L.hstu_attn_fwd_workspace_size(C.byref(_desc(T=1000, win_local=64))) == a
    assert L.hstu_attn_fwd_workspace_size(C.byref(_desc(T=1000, dtype=0))) == \
        L.hstu_attn_fwd_workspace_size(C.byref(_desc(T=1000, key_splits=1, dtype=0)))
    # the workloads: 32 x U[64,1024] with 4 heads of 64 takes the 64-row items,
    # the 8-layer Zipf batch (64 sequences, 8 heads) does not
    c2 = dict(B=32, T=17016, H=4, d_qk=64, d_v=64)
    c3 = dict(B=64, T=34485, H=8, d_qk=64, d_v=64)
    assert L.hstu_attn_fwd_workspace_size(C.byref(_desc(**c2))) > \
        L.hstu_attn_fwd_workspace_size(C.byref(_desc(key_splits=1, **c2)))
    assert L.hstu_attn_fwd_workspace_size(C.byref(_desc(**c3))) == \
        L.hstu_attn_fwd_workspace_size(C.byref(_desc(key_splits=1, **c3)))
    # split keys keep partial sums of [block rows x d_v] per part and work item
    s4 = L.hstu_attn_fwd_workspace_size(C.byref(_desc(T=1000, key_splits=4)))
    s2 = L.hstu_attn_fwd_workspace_size(C.byref(_desc(T=1000, key_splits=2)))
    assert a < s2 < s4
    # fp32 and windowed attention never split
    assert L.hstu_attn_fwd_workspace_size(C.byref(_desc(T=1000, key_splits=4, dtype=0))) == \
        L.hstu_attn_fwd_workspace_size(C.byref(_desc(T=1000, key_splits=1, dtype=0)))
    assert L.hstu_attn_fwd_workspace_size(C.byref(_desc(T=1000, key_splits=4, win_local=64))) == a
    assert L.hstu_attn_bwd_workspace_size(C.byref(_desc(T=1000))) > 0
    ld = _lib.LayerDesc(_desc(T=1000), 64, 1, 1, 1e-6)
    assert L.hstu_layer_fwd_workspace_size(C.byref(ld), 0) > \
        L.hstu_layer_fwd_workspace_size(C.byref(ld), 1)
    assert L.hstu_layer_bwd_workspace_size(C.byref(ld)) > 0


@pytest.mark.parametrize("bad,code", [
    (dict(d_qk=48), -2), (dict(d_v=256), -2), (dict(H=0), -2), (dict(H=65), -2),
    (dict(n_pos_buckets=0), -2), (dict(n_time_buckets=2000), -2), (dict(norm_mode=2), -1),
    (dict(norm_len=0), -1), (dict(dtype=7), -2), (dict(T=1 << 31), -1), (dict(B=-1), -1),
    (dict(rab_head_stride=64), -1), (dict(max_len=-1), -1), (dict(reuse_plan=2), -1),
    (dict(key_splits=-1), -1), (dict(key_splits=9), -1),
])
def test_host_side_argument_errors(L, bad, code):
    d = _desc(**bad)
    assert L.hstu_attn_fwd_workspace_size(C.byref(d)) == 0
    buf = C.create_string_buffer(1 << 16)
    ws = C.c_void_p((C.addressof(buf) + 255) & ~255)
    fake = C.c_void_p(1 << 20)  # never dereferenced: validation fails first
    st = L.hstu_attn_fwd(C.byref(d), fake, fake, 64, fake, 64, fake, fake, fake, fake, None, fake,
                         64, ws, 1 << 15, None)
    assert st == code


def test_workspace_too_small_is_reported(L):
    d = _desc()
    buf = C.create_string_buffer(1024)
    ws = C.c_void_p((C.addressof(buf) + 255) & ~255)
    p = C.c_void_p(1 << 20)
    st = L.hstu_attn_fwd(C.byref(d), p, p, 64, p, 64, p, p, p, p, None, p, 64, ws, 16, None)
    assert st == -3


def test_misaligned_stride_rejected(L):
    d = _desc()
    buf = C.create_string_buffer(1 << 16)
    ws = C.c_void_p((C.addressof(buf) + 255) & ~255)
    p = C.c_void_p(1 << 20)
    # bf16 rows must be multiples of 8 elements
    st = L.hstu_attn_fwd(C.byref(d), p, p, 65, p, 64, p, p, p, p, None, p, 64, ws, 1 << 15, None)
    assert st == -1


def test_fp32_backward_is_reported_unsupported(L):
    d = _desc(dtype=0)
    buf = C.create_string_buffer(1 << 16)
    ws = C.c_void_p((C.addressof(buf) + 255) & ~255)
    p = C.c_void_p(1 << 20)
    st = L.hstu_attn_bwd(C.byref(d), p, p, 64, p, 64, p, p, p, p, None, p, 64, p, p, p, p, p, ws,
                         1 << 15, None)
    assert st == -2


def test_schedule_capacity_bound(L):
    # sum_b ceil(n_b / BM) <= (T + B*(BM-1)) / BM
    assert L.hstu_schedule_capacity(1000, 10, 128) >= (1000 + 10 * 127) // 128


def test_descriptor_layouts_match_the_header(tmp_path):
    """The ctypes mirrors have the sizes and field offsets the C compiler gives
    the structs of include/hstu.h (a C program built here prints them)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc") or shutil.which("cc")
    if gcc is None:
        pytest.skip("no C compiler")
    structs = {"hstu_attn_desc": _lib.AttnDesc, "hstu_layer_desc": _lib.LayerDesc,
               "hstu_layer_weights": _lib.LayerWeights, "hstu_layer_saved": _lib.LayerSaved,
               "hstu_layer_grads": _lib.LayerGrads, "hstu_history_kv": _lib.HistoryKV,
               "hstu_mx_weights": _lib.MxWeights, "hstu_mx_io": _lib.MxIO,
               "hstu_attn_mx_qk": _lib.AttnMxQK}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "hstu.h"', "int main(void) {"]
    for cname, ct in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for fname, _ in ct._fields_:
            lines.append(f'  printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines.append("  return 0;\n}")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run([gcc, "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {}
    for line in out:
        if line.strip():
            a, b, c = line.split()
            got[(a, b)] = int(c)
    for cname, ct in structs.items():
        assert got[(cname, "size")] == C.sizeof(ct), cname
        for fname, _ in ct._fields_:
            assert got[(cname, fname)] == getattr(ct, fname).offset, (cname, fname)


def test_negative_windows_rejected(L):
    buf = C.create_string_buffer(1 << 16)
    ws = C.c_void_p((C.addressof(buf) + 255) & ~255)
    p = C.c_void_p(1 << 20)
    for wl, wg in ((-1, 0), (4, -2)):
        d = _desc(win_local=wl, win_global=wg)
        st = L.hstu_attn_fwd(C.byref(d), p, p, 64, p, 64, p, p, p, p, None, p, 64, ws, 1 << 15,
                             None)
        assert st == -1


def test_truncation_argument_errors(L):
    """Host-side checks of the truncation entry points (nothing is launched)."""
    p = C.c_void_p(1 << 20)            # 16-byte aligned, never dereferenced
    odd = C.c_void_p((1 << 20) + 8)    # not 16-byte aligned
    assert L.hstu_truncate_offsets(-1, p, None, 4, p, None) == -1
    assert L.hstu_truncate_offsets(2, p, None, -1, p, None) == -1
    assert L.hstu_truncate_offsets(2, None, None, 4, p, None) == -1
    g = L.hstu_truncate_gather
    # dtype, D not a multiple of 16 bytes, misaligned rows, NULL seg_offsets
    assert g(2, 10, 4, 64, 9, p, p, p, None, p, None, None) == -2
    assert g(2, 10, 4, 4, 1, p, p, p, None, p, None, None) == -1
    assert g(2, 10, 4, 64, 1, odd, p, p, None, p, None, None) == -1
    assert g(2, 10, 4, 64, 1, p, p, None, None, p, None, None) == -1
    # timestamps without their output (or the reverse)
    assert g(2, 10, 4, 64, 1, p, p, p, p, p, None, None) == -1
    assert g(2, 10, 1 << 31, 64, 1, p, p, p, None, p, None, None) == -1
    s = L.hstu_truncate_scatter
    assert s(2, 10, 4, 64, 1, odd, p, p, p, None) == -1
    assert s(2, -1, 4, 64, 1, p, p, p, p, None) == -1
    assert s(2, 10, 4, 6, 0, p, p, p, p, None) == -1    # fp32 rows of 24 bytes
    assert s(2, 10, 4, 64, 1, p, p, p, None, None) == -1  # NULL dx


def test_cached_ranking_argument_errors(L):
    """Host-side checks of the cached-history entry points (nothing is launched)."""
    buf = C.create_string_buffer(1 << 20)
    ws = C.c_void_p((C.addressof(buf) + 255) & ~255)
    p = C.c_void_p(1 << 20)
    hist = _lib.HistoryKV(p, p, 64, 64, p, p, 100)
    d = _desc()
    assert L.hstu_attn_cached_workspace_size(C.byref(d), 100) > 0
    assert L.hstu_attn_cached_workspace_size(C.byref(d), -1) == 0
    call = lambda d_, h_: L.hstu_attn_cached_fwd(C.byref(d_), p, p, 64, p, 64, p, p,
                                                 None if h_ is None else C.byref(h_), p, p, p,
                                                 64, ws, 1 << 19, None)
    assert call(d, None) == -1                                   # no history
    assert call(_desc(norm_mode=1), hist) == -2                  # N must be fixed
    assert call(d, _lib.HistoryKV(p, p, 60, 64, p, p, 100)) == -1  # bf16 row stride
    assert call(d, _lib.HistoryKV(None, p, 64, 64, p, p, 100)) == -1
    assert call(d, _lib.HistoryKV(p, p, 64, 64, None, p, 100)) == -1
    small = L.hstu_attn_cached_fwd(C.byref(d), p, p, 64, p, 64, p, p, C.byref(hist), p, p, p, 64,
                                   ws, 16, None)
    assert small == -3


def test_reuse_plan_without_a_recorded_plan_is_rejected(L):
    """reuse_plan = 1 is checked against the plans the library recorded; a
    workspace no forward call planned into is refused before any launch."""
    buf = C.create_string_buffer(1 << 22)
    ws = C.c_void_p((C.addressof(buf) + 255) & ~255)
    p = C.c_void_p(1 << 20)
    d = _desc(reuse_plan=1)
    st = L.hstu_attn_fwd(C.byref(d), p, p, 64, p, 64, p, p, p, p, None, p, 64, ws, 1 << 21, None)
    assert st == -1
    ld = _lib.LayerDesc(_desc(reuse_plan=1, d_qk=32, d_v=32, H=2), 64, 1, 1, 1e-6)
    w = _lib.LayerWeights(p, p, None, None, None, None, p, p)
    st = L.hstu_layer_fwd(C.byref(ld), p, C.byref(w), p, p, None, C.c_void_p((1 << 20) + 4096),
                          None, ws, 1 << 21, None)
    assert st == -1


def test_binding_refuses_reuse_plan_without_its_workspace():
    import torch

    from hstu_sequential_transduction_amd import binding as B
    with pytest.raises(ValueError):
        B._layer_ws(None, 1024, torch.device("cpu"), 1)
    lw = B.LayerWorkspace()
    with pytest.raises(ValueError):   # nothing planned into it yet: it would be allocated now
        lw.get(1024, torch.device("cpu"), 1)
    buf = lw.get(1024, torch.device("cpu"))
    assert lw.get(512, torch.device("cpu"), 1) is buf
    with pytest.raises(ValueError):   # too small: would be reallocated
        lw.get(4096, torch.device("cpu"), 1)


def test_check_mode_switch(L):
    """Check mode (sync + launch-error read after every launch) is a
    process-wide switch; HSTU_CHECK in the environment turns it on at load."""
    import subprocess
    import sys
    assert L.hstu_check_mode() == 0
    assert L.hstu_set_check_mode(1) == 0 and L.hstu_check_mode() == 1
    assert L.hstu_set_check_mode(0) == 0 and L.hstu_check_mode() == 0
    assert L.hstu_set_check_mode(2) == -1 and L.hstu_check_mode() == 0
    assert L.hstu_last_error_site() == b""
    code = ("from hstu_sequential_transduction_amd import _lib; "
            "print(_lib.lib().hstu_check_mode())")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for val, want in (("1", "1"), ("0", "0")):
        env = dict(os.environ, HSTU_CHECK=val)
        out = subprocess.run([sys.executable, "-c", code], cwd=root, env=env,
                             capture_output=True, text=True, timeout=120)
        assert out.stdout.strip().splitlines()[-1] == want, out.stderr[-2000:]


def test_mx_attention_argument_errors(L):
    """Host-side checks of the MXFP8-score attention and its quantizer
    (nothing is launched): unsupported descriptors, missing operands,
    misaligned codes or strides."""
    buf = C.create_string_buffer(1 << 20)
    ws = C.c_void_p((C.addressof(buf) + 255) & ~255)
    p = C.c_void_p(1 << 20)
    odd = C.c_void_p((1 << 20) + 8)
    qk = _lib.AttnMxQK(p, p, 256, p, p)

    def call(d_, qk_=qk, nbytes=1 << 19):
        return L.hstu_attn_fwd_mx(C.byref(d_), None if qk_ is None else C.byref(qk_), p, 256,
                                  p, p, p, p, None, p, 256, ws, nbytes, None)
    bf = dict(dtype=1, H=2, d_qk=64, d_v=64)
    assert call(_desc(**bf), None) == -1                         # no q/k
    assert call(_desc(**{**bf, "dtype": 0})) == -2                # fp32
    assert call(_desc(**{**bf, "d_qk": 32, "d_v": 32})) == -2     # d_qk below one FP8 k-step
    assert call(_desc(**{**bf, "d_v": 128})) == -2                # d_qk != d_v
    assert call(_desc(**bf, win_local=8)) == -2                   # windows
    assert call(_desc(**bf, key_splits=2)) == -2                  # key split
    assert call(_desc(**bf), _lib.AttnMxQK(odd, p, 256, p, p)) == -1   # misaligned codes
    assert call(_desc(**bf), _lib.AttnMxQK(p, p, 120, p, p)) == -1     # ld below H*d_qk
    assert call(_desc(**bf), _lib.AttnMxQK(p, p, 136, p, p)) == -1     # ld not 16-byte
    assert call(_desc(**bf), _lib.AttnMxQK(p, p, 256, None, p)) == -1  # no scales
    assert call(_desc(**bf), nbytes=16) == -3                          # workspace
    q = L.hstu_mx_quantize_heads
    assert q(10, 2, 48, p, 128, p, 128, p, None) == -1       # d not a multiple of 32
    assert q(10, 2, 160, p, 512, p, 512, p, None) == -1      # d above 128
    assert q(10, 65, 32, p, 2080, p, 2080, p, None) == -1    # more than 64 heads
    assert q(10, 2, 64, p, 100, p, 128, p, None) == -1       # ld below H*d
    assert q(10, 2, 64, p, 128, p, 136, p, None) == -1       # codes stride not 16-byte
    assert q(10, 2, 64, odd, 128, p, 128, p, None) == -1     # misaligned input
    assert q(10, 2, 64, p, 128, p, 128, C.c_void_p((1 << 20) + 2), None) == -1


def test_mx_layer_scores_argument_errors(L):
    """hstu_layer_fwd_mx with mx_scores: descriptors the MX-score attention
    does not take, training (saved) without the projection SiLU and flag
    values other than 0/1 are refused before launch."""
    buf = C.create_string_buffer(1 << 22)
    ws = C.c_void_p((C.addressof(buf) + 255) & ~255)
    p = C.c_void_p(1 << 20)
    w = _lib.LayerWeights(p, p, None, None, None, None, p, p)
    m = _lib.MxWeights(p, p, p, p)
    sv = _lib.LayerSaved(p, p, p, p, p, p)

    def call(ad, flag, saved=None, proj_silu=1):
        ld = _lib.LayerDesc(ad, 128, proj_silu, 1, 1e-6)
        nb = L.hstu_layer_fwd_mx_workspace_size(C.byref(ld))
        io = _lib.MxIO(None, None, None, None, None, None, flag)
        return L.hstu_layer_fwd_mx(C.byref(ld), p, C.byref(w), C.byref(m), p, p, None,
                                   C.c_void_p((1 << 20) + 4096), C.byref(io),
                                   None if saved is None else C.byref(saved), ws,
                                   max(nb, 1 << 21), None)
    ok = dict(T=300, H=2, d_qk=64, d_v=64)
    assert call(_desc(**ok), 2) == -1                                # flag not 0/1
    assert call(_desc(**ok, win_local=16), 1) == -2                  # windows
    assert call(_desc(T=300, H=4, d_qk=32, d_v=32), 1) == -2         # d_qk 32
    assert call(_desc(**ok, key_splits=3), 1) == -2                  # key split
    assert call(_desc(**ok), 1, saved=sv, proj_silu=0) == -2         # training without SiLU
