"""ctypes declarations of libhstu.so's C ABI (include/hstu.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation anywhere in this package.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhstu.so")

HSTU_OK = 0
STATUS_NAMES = {0: "HSTU_OK", -1: "HSTU_ERR_INVALID_ARG", -2: "HSTU_ERR_UNSUPPORTED",
                -3: "HSTU_ERR_WORKSPACE", -4: "HSTU_ERR_HIP", -5: "HSTU_ERR_VALIDATION"}
HSTU_F32, HSTU_BF16 = 0, 1

EXPORTED = [
    "hstu_status_string", "hstu_version", "hstu_last_hip_error", "hstu_last_error_site",
    "hstu_set_check_mode", "hstu_check_mode",
    "hstu_attn_fwd_workspace_size", "hstu_attn_bwd_workspace_size",
    "hstu_attn_fwd", "hstu_attn_bwd", "hstu_attn_fwd_noalloc", "hstu_diag_mfma_loop",
    "hstu_layer_fwd_workspace_size", "hstu_layer_bwd_workspace_size",
    "hstu_layer_fwd", "hstu_layer_bwd",
    "hstu_bias_buckets", "hstu_schedule_capacity", "hstu_schedule",
    "hstu_schedule_workspace_size", "hstu_validate_inputs",
    "hstu_truncate_offsets", "hstu_truncate_gather", "hstu_truncate_scatter",
    "hstu_attn_cached_workspace_size", "hstu_attn_cached_fwd",
    "hstu_mx_quantize", "hstu_mx_quantize_weight", "hstu_mx_gemm",
    "hstu_mx_quantize_heads", "hstu_attn_fwd_mx",
    "hstu_layer_fwd_mx_workspace_size", "hstu_layer_fwd_mx",
    "hstu_layer_bwd_mx_workspace_size", "hstu_layer_bwd_mx",
    "hstu_layer_cached_workspace_size", "hstu_layer_fwd_cached",
    "hstu_timer_enable", "hstu_timer_reset", "hstu_timer_tag_count", "hstu_timer_tag_name",
    "hstu_timer_query",
]


class AttnDesc(C.Structure):
    _fields_ = [("B", C.c_int32), ("T", C.c_int64), ("H", C.c_int32), ("d_qk", C.c_int32),
                ("d_v", C.c_int32), ("n_pos_buckets", C.c_int32),
                ("n_time_buckets", C.c_int32), ("norm_mode", C.c_int32),
                ("norm_len", C.c_int32), ("dtype", C.c_int32),
                ("rab_head_stride", C.c_int64), ("win_local", C.c_int32),
                ("win_global", C.c_int32), ("max_len", C.c_int32), ("reuse_plan", C.c_int32),
                ("key_splits", C.c_int32)]


class LayerDesc(C.Structure):
    _fields_ = [("attn", AttnDesc), ("D", C.c_int32), ("proj_silu", C.c_int32),
                ("residual", C.c_int32), ("ln_eps", C.c_float)]


class LayerWeights(C.Structure):
    _fields_ = [("W1", C.c_void_p), ("W2", C.c_void_p), ("b1", C.c_void_p), ("b2", C.c_void_p),
                ("ln_gamma", C.c_void_p), ("ln_beta", C.c_void_p), ("rab_pos", C.c_void_p),
                ("rab_time", C.c_void_p)]


class LayerSaved(C.Structure):
    _fields_ = [("Z", C.c_void_p), ("Zh", C.c_void_p), ("O", C.c_void_p), ("G", C.c_void_p),
                ("mu", C.c_void_p), ("rstd", C.c_void_p)]


class LayerGrads(C.Structure):
    _fields_ = [("dW1", C.c_void_p), ("dW2", C.c_void_p), ("db1", C.c_void_p),
                ("db2", C.c_void_p), ("dgamma", C.c_void_p), ("dbeta", C.c_void_p),
                ("drab_pos", C.c_void_p), ("drab_time", C.c_void_p)]


class MxWeights(C.Structure):
    _fields_ = [("W1", C.c_void_p), ("W1_scales", C.c_void_p), ("W2", C.c_void_p),
                ("W2_scales", C.c_void_p)]


class MxIO(C.Structure):
    _fields_ = [("x_codes", C.c_void_p), ("x_scales", C.c_void_p), ("y_codes", C.c_void_p),
                ("y_scales", C.c_void_p), ("g_codes", C.c_void_p), ("g_scales", C.c_void_p),
                ("mx_scores", C.c_int32)]


class AttnMxQK(C.Structure):
    _fields_ = [("q_codes", C.c_void_p), ("k_codes", C.c_void_p), ("ld_codes", C.c_int64),
                ("q_scales", C.c_void_p), ("k_scales", C.c_void_p)]


class HistoryKV(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("ld_k", C.c_int64), ("ld_v", C.c_int64),
                ("offsets", C.c_void_p), ("timestamps", C.c_void_p), ("T", C.c_int64)]


_lib = None


def lib() -> C.CDLL:
    """The loaded library (raises if libhstu.so is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it first "
            "(python -c 'import __graft_entry__ as g; g.build()' or "
            "python hstu_sequential_transduction_amd/build.py)")
    # torch ships its own HIP runtime (torch/lib/libamdhip64.so, soname
    # libamdhip64.so.7).  Loaded first, it satisfies this library's
    # libamdhip64.so.7 dependency, so both share one runtime (and so one view
    # of device memory and streams).  Loaded the other way round, the process
    # would hold two HIP runtimes and the second would find no device.
    import torch  # noqa: F401
    L = C.CDLL(LIB_PATH)
    vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    P = C.POINTER
    L.hstu_status_string.restype = C.c_char_p
    L.hstu_status_string.argtypes = [C.c_int]
    L.hstu_last_hip_error.restype = C.c_char_p
    L.hstu_last_hip_error.argtypes = []
    L.hstu_last_error_site.restype = C.c_char_p
    L.hstu_last_error_site.argtypes = []
    L.hstu_set_check_mode.restype = C.c_int
    L.hstu_set_check_mode.argtypes = [C.c_int32]
    L.hstu_check_mode.restype = C.c_int32
    L.hstu_check_mode.argtypes = []
    L.hstu_version.restype = C.c_char_p
    L.hstu_version.argtypes = []
    for f in ("hstu_attn_fwd_workspace_size", "hstu_attn_bwd_workspace_size"):
        getattr(L, f).restype = sz
        getattr(L, f).argtypes = [P(AttnDesc)]
    L.hstu_layer_fwd_workspace_size.restype = sz
    L.hstu_layer_fwd_workspace_size.argtypes = [P(LayerDesc), C.c_int]
    L.hstu_layer_bwd_workspace_size.restype = sz
    L.hstu_layer_bwd_workspace_size.argtypes = [P(LayerDesc)]
    L.hstu_attn_fwd.restype = C.c_int
    L.hstu_attn_fwd.argtypes = [P(AttnDesc), vp, vp, i64, vp, i64, vp, vp, vp, vp, vp, vp, i64,
                                vp, sz, vp]
    L.hstu_diag_mfma_loop.restype = C.c_int
    L.hstu_diag_mfma_loop.argtypes = [i32, i32, vp, vp]
    L.hstu_attn_fwd_noalloc.restype = C.c_int
    L.hstu_attn_fwd_noalloc.argtypes = [P(AttnDesc), vp, vp, i64, vp, i64, vp, vp, vp, vp, vp,
                                        vp, i64, vp]
    L.hstu_attn_bwd.restype = C.c_int
    L.hstu_attn_bwd.argtypes = [P(AttnDesc), vp, vp, i64, vp, i64, vp, vp, vp, vp, vp, vp, i64,
                                vp, vp, vp, vp, vp, vp, sz, vp]
    L.hstu_layer_fwd.restype = C.c_int
    L.hstu_layer_fwd.argtypes = [P(LayerDesc), vp, P(LayerWeights), vp, vp, vp, vp,
                                 P(LayerSaved), vp, sz, vp]
    L.hstu_layer_bwd.restype = C.c_int
    L.hstu_layer_bwd.argtypes = [P(LayerDesc), vp, P(LayerWeights), vp, vp, vp, P(LayerSaved),
                                 vp, vp, P(LayerGrads), vp, sz, vp]
    L.hstu_bias_buckets.restype = C.c_int
    L.hstu_bias_buckets.argtypes = [P(AttnDesc), vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, sz, vp]
    L.hstu_schedule_capacity.restype = i64
    L.hstu_schedule_capacity.argtypes = [i64, i32, i32]
    L.hstu_schedule_workspace_size.restype = sz
    L.hstu_schedule_workspace_size.argtypes = [i32, i64, i32]
    L.hstu_schedule.restype = C.c_int
    L.hstu_schedule.argtypes = [i32, i64, vp, i32, i32, vp, vp, vp, sz, vp]
    L.hstu_validate_inputs.restype = C.c_int
    L.hstu_validate_inputs.argtypes = [i32, i64, vp, vp, vp, vp]
    L.hstu_mx_quantize.restype = C.c_int
    L.hstu_mx_quantize_heads.restype = C.c_int
    L.hstu_mx_quantize_heads.argtypes = [i64, i32, i32, vp, i64, vp, i64, vp, vp]
    L.hstu_attn_fwd_mx.restype = C.c_int
    L.hstu_attn_fwd_mx.argtypes = [P(AttnDesc), P(AttnMxQK), vp, i64, vp, vp, vp, vp, vp, vp,
                                   i64, vp, sz, vp]
    L.hstu_mx_quantize.argtypes = [i64, i64, vp, i64, vp, vp, vp]
    L.hstu_mx_quantize_weight.restype = C.c_int
    L.hstu_mx_quantize_weight.argtypes = [i64, i64, vp, vp, vp, vp]
    L.hstu_mx_gemm.restype = C.c_int
    L.hstu_mx_gemm.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp, i64, vp]
    L.hstu_layer_fwd_mx_workspace_size.restype = sz
    L.hstu_layer_fwd_mx_workspace_size.argtypes = [P(LayerDesc)]
    L.hstu_layer_fwd_mx.restype = C.c_int
    L.hstu_layer_fwd_mx.argtypes = [P(LayerDesc), vp, P(LayerWeights), P(MxWeights), vp, vp, vp,
                                    vp, P(MxIO), P(LayerSaved), vp, sz, vp]
    L.hstu_layer_bwd_mx_workspace_size.restype = sz
    L.hstu_layer_bwd_mx_workspace_size.argtypes = [P(LayerDesc)]
    L.hstu_layer_bwd_mx.restype = C.c_int
    L.hstu_layer_bwd_mx.argtypes = [P(LayerDesc), vp, P(LayerWeights), vp, vp, vp, P(LayerSaved),
                                    vp, vp, P(LayerGrads), vp, sz, vp]
    L.hstu_attn_cached_workspace_size.restype = sz
    L.hstu_attn_cached_workspace_size.argtypes = [P(AttnDesc), i64]
    L.hstu_attn_cached_fwd.restype = C.c_int
    L.hstu_attn_cached_fwd.argtypes = [P(AttnDesc), vp, vp, i64, vp, i64, vp, vp, P(HistoryKV),
                                       vp, vp, vp, i64, vp, sz, vp]
    L.hstu_layer_cached_workspace_size.restype = sz
    L.hstu_layer_cached_workspace_size.argtypes = [P(LayerDesc), i64]
    L.hstu_layer_fwd_cached.restype = C.c_int
    L.hstu_layer_fwd_cached.argtypes = [P(LayerDesc), vp, P(LayerWeights), vp, vp,
                                        P(HistoryKV), vp, vp, sz, vp]
    L.hstu_truncate_offsets.restype = C.c_int
    L.hstu_truncate_offsets.argtypes = [i32, vp, vp, i32, vp, vp]
    L.hstu_truncate_gather.restype = C.c_int
    L.hstu_truncate_gather.argtypes = [i32, i64, i64, i32, i32, vp, vp, vp, vp, vp, vp, vp]
    L.hstu_truncate_scatter.restype = C.c_int
    L.hstu_truncate_scatter.argtypes = [i32, i64, i64, i32, i32, vp, vp, vp, vp, vp]
    L.hstu_timer_enable.restype = C.c_int
    L.hstu_timer_enable.argtypes = [i32]
    L.hstu_timer_reset.restype = C.c_int
    L.hstu_timer_reset.argtypes = []
    L.hstu_timer_tag_count.restype = i32
    L.hstu_timer_tag_count.argtypes = []
    L.hstu_timer_tag_name.restype = C.c_char_p
    L.hstu_timer_tag_name.argtypes = [i32]
    L.hstu_timer_query.restype = C.c_int
    L.hstu_timer_query.argtypes = [i32, P(i64), P(C.c_double)]
    _lib = L
    return L


class HstuError(RuntimeError):
    def __init__(self, fn: str, status: int):
        name = STATUS_NAMES.get(status, str(status))
        try:
            msg = lib().hstu_status_string(status).decode()
            if status == -4:
                msg += ": " + lib().hstu_last_hip_error().decode()
                site = lib().hstu_last_error_site().decode()
                if site:
                    msg += " at " + site
        except Exception:  # pragma: no cover
            msg = ""
        super().__init__(f"{fn} failed: {name} ({msg})")
        self.status = status


def check(fn: str, status: int) -> None:
    if status != HSTU_OK:
        raise HstuError(fn, status)
