#!/usr/bin/env python3
"""Benchmark of the HSTU layer on one MI355X.

One step = one full training step of one HSTU layer (forward with saved
intermediates + backward, every kernel of the path) on the long-sequence
training workload: 8 jagged sequences of uniform length in [4096, 8192],
d_model 512, 4 heads x 128, causal, bf16 with fp32 accumulation, synthetic
seeded inputs resident in HBM before timing starts.

Prints one JSON line.  `value` is whole-step algorithmic TFLOP/s (the DLRMv4
page's Table 7 convention: weight GEMMs x3, attention x3.5 for fwd+bwd, S^2/2
pairs per sequence); tokens/s and the fraction of the 2.5 PFLOP/s bf16 peak
are reported alongside, with a per-kernel breakdown taken with HIP events
inside the timed region, the roofline of the dominant kernel, forward-only
figures for the other workloads, and the fp64 CPU oracle timed on a bounded
sample (one sequence) of the same workload.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "HSTU layer fwd+bwd TFLOP/s and tokens/s on 1 MI355X; % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash(kernel: str) -> str:
    from hstu_sequential_transduction_amd.traffic import source_hash as sh
    return sh(kernel)


def kernel_work(cfg, lengths, T, cand=None, keep_ds=True):
    """Algorithmic work per launch of each kernel tag: (kind, amount).  With
    dS kept by the dK/dV kernel, dQ is the single product dS K (and the dK/dV
    kernel also writes dS: 2 bytes per pair and head of the causal blocks)."""
    from hstu_sequential_transduction_amd import flops
    H, dq, dv, D = cfg.H, cfg.d_qk, cfg.d_v, cfg.D
    W, F1 = H * dv, cfg.f1_width
    P = flops.attn_pairs(lengths, cand)
    return {
        "attn_fwd": ("mfma", 2 * P * H * (dq + dv)),
        # the products each backward kernel's outputs need: S, dA, dV, dK / S, dA, dQ
        "attn_bwd_dkdv": ("mfma", 2 * P * H * (2 * dq + 2 * dv)),
        "attn_bwd_dq": ("mfma", 2 * P * H * (dq if keep_ds else (2 * dq + dv))),
        "gemm_uvqk": ("mfma", 2.0 * T * D * F1),
        "gemm_out": ("mfma", 2.0 * T * W * D),
        "gemm_dG": ("mfma", 2.0 * T * D * W),
        "gemm_dW2": ("mfma", 2.0 * W * D * T),
        "gemm_dW1": ("mfma", 2.0 * D * F1 * T),
        "gemm_dX": ("mfma", 2.0 * T * F1 * D),
        # O (fp32) + U read, G written, mu/rstd written
        "ln_gate_fwd": ("hbm", T * (4.0 * W + 2 * W + 2 * W + 8)),
        # O (fp32), U, dG, Z_U read; dU, dO written; mu/rstd read
        "ln_gate_bwd": ("hbm", T * (4.0 * W + 2 * W * 5 + 8)),
    }


class Timer:
    def __init__(self, L):
        self.L = L

    def enable(self, n):
        from hstu_sequential_transduction_amd._lib import check
        check("hstu_timer_enable", self.L.hstu_timer_enable(n))

    def reset(self):
        self.L.hstu_timer_reset()

    def read(self):
        import ctypes as C
        out = {}
        for t in range(self.L.hstu_timer_tag_count()):
            n, ms = C.c_int64(0), C.c_double(0.0)
            self.L.hstu_timer_query(t, C.byref(n), C.byref(ms))
            if n.value:
                out[self.L.hstu_timer_tag_name(t).decode()] = (n.value, ms.value)
        return out


def upload_layer(inp, cfg, li=0):
    import numpy as np
    import torch
    td = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    w = inp.layers[li]
    return dict(
        W1=torch.from_numpy(w.W1).to(td).cuda(), W2=torch.from_numpy(w.W2).to(td).cuda(),
        rp=torch.from_numpy(w.rab_pos).cuda(), rt=torch.from_numpy(w.rab_time).cuda())


def bench_train(args, timer, window=(0, 0)):
    import numpy as np
    import torch

    import synth
    from hstu_sequential_transduction_amd import binding as B
    from hstu_sequential_transduction_amd import flops

    cfg = synth.get_config(4)
    inp = synth.make_inputs(cfg)
    T = inp.T
    td = torch.bfloat16
    X = torch.from_numpy(inp.X).to(td).cuda()
    dY = torch.from_numpy(inp.dY).to(td).cuda()
    offs = torch.from_numpy(inp.seq_offsets.astype(np.int32)).cuda()
    ts = torch.from_numpy(inp.timestamps).cuda()
    w = upload_layer(inp, cfg)
    # max_len: the workload's longest sequence, which lets the backward keep dS
    ac = B.AttnConfig(H=cfg.H, d_qk=cfg.d_qk, d_v=cfg.d_v, norm_len=cfg.norm_len,
                      win_local=window[0], win_global=window[1],
                      max_len=int(inp.lengths.max()))
    lc = B.LayerConfig(D=cfg.D, attn=ac)
    saved = B.Saved(T, lc, td, "cuda")
    y = torch.empty_like(X)
    dx = torch.empty_like(X)
    f32 = dict(dtype=torch.float32, device="cuda")
    grads = B.Grads(torch.empty(w["W1"].shape, **f32), torch.empty(w["W2"].shape, **f32),
                    torch.empty(w["rp"].shape, **f32), torch.empty(w["rt"].shape, **f32))
    wsf, wsb = B.LayerWorkspace(), B.LayerWorkspace()

    def step():
        B.hstu_layer_fwd(X, w["W1"], w["W2"], w["rp"], w["rt"], offs, ts, lc, saved=saved, y=y,
                         workspace=wsf)
        B.hstu_layer_bwd(X, w["W1"], w["W2"], w["rp"], w["rt"], offs, ts, lc, saved, dY, dx=dx,
                         grads=grads, workspace=wsb)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed region: K steps between two events on the stream the library launches on
    timer.enable(64 * max(args.steps, 1))
    timer.reset()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / max(args.steps, 1)
    kern = timer.read()
    timer.enable(0)
    lf = flops.layer_flops(inp.lengths, None, cfg.D, cfg.H, cfg.d_qk, cfg.d_v, backward=True,
                           window=window if window[0] > 0 else None)
    return cfg, inp, ms, kern, lf


# Semi-local attention windows of the extra training-step measurement: the
# pages give no sizes, so these are chosen parameters (a local window of 1024
# positions and the first 128 tokens), stated with the result.
SEMILOCAL_WINDOW = (1024, 128)


def bench_semilocal(args, timer, full_ms):
    """The same training step with semi-local attention; TFLOP/s on the
    windowed work (exact pair count), and the speedup over full causal."""
    from hstu_sequential_transduction_amd import flops
    cfg, inp, ms, kern, lf = bench_train(args, timer, window=SEMILOCAL_WINDOW)
    full_pairs = flops.attn_pairs_window(inp.lengths, None, 0, 0)
    win_pairs = flops.attn_pairs_window(inp.lengths, None, *SEMILOCAL_WINDOW)
    out = {"win_local": SEMILOCAL_WINDOW[0], "win_global": SEMILOCAL_WINDOW[1],
           "ms_per_step": round(ms, 4), "tflops": round(lf["total"] / (ms * 1e-3) / 1e12, 2),
           "tokens_per_s": round(inp.T / (ms * 1e-3), 1),
           "attn_pairs_frac": round(win_pairs / full_pairs, 4),
           "speedup_vs_full_causal": round(full_ms / ms, 3),
           "kernel_ms_per_launch": {k: round(v[1] / v[0], 4) for k, v in kern.items()}}
    log(f"semi-local step (W_l={SEMILOCAL_WINDOW[0]}, W_g={SEMILOCAL_WINDOW[1]}): "
        f"{ms:.3f} ms, x{full_ms / ms:.2f} vs full causal")
    return out


# Attention truncation on the ranking workload (16 x (4096 history + 512
# candidates), d_model 256, 4 heads x 64), in the pages' 3 + 6 layer scheme
# against 6 full layers.  The segment length L' is not on the pages: 1024
# history events (plus the candidates) is a chosen parameter.
TRUNC_KEEP = 1024
TRUNC_SCHEME = (3, 6)


def bench_truncation(timer, reps=3):
    """Inference forward of (a) 6 full layers, (b) 3 full + 6 truncated
    layers, (c) as (b) with semi-local windows in the full layers."""
    import dataclasses

    import numpy as np
    import torch

    import synth
    from hstu_sequential_transduction_amd import binding as B
    from hstu_sequential_transduction_amd import flops
    from hstu_sequential_transduction_amd import truncation as TR
    nf, nt = TRUNC_SCHEME
    cfg = dataclasses.replace(synth.get_config(5), n_layers=max(nf + nt, 6))
    inp = synth.make_inputs(cfg)
    td = torch.bfloat16
    X = torch.from_numpy(inp.X).to(td).cuda()
    offs = torch.from_numpy(inp.seq_offsets.astype(np.int32)).cuda()
    ts = torch.from_numpy(inp.timestamps).cuda()
    nc = torch.from_numpy(inp.num_candidates.astype(np.int32)).cuda()
    lay = [tuple(upload_layer(inp, cfg, li).values()) for li in range(cfg.n_layers)]
    c = int(inp.num_candidates[0])
    seg_len = np.minimum(inp.lengths - inp.num_candidates, TRUNC_KEEP) + inp.num_candidates
    T_seg = int(seg_len.sum())     # known on the host from the batch's lengths, like T
    ac = B.AttnConfig(H=cfg.H, d_qk=cfg.d_qk, d_v=cfg.d_v, norm_len=cfg.norm_len)
    lc_full = B.LayerConfig(D=cfg.D, attn=ac)
    lc_semi = B.LayerConfig(D=cfg.D, attn=dataclasses.replace(
        ac, win_local=SEMILOCAL_WINDOW[0], win_global=SEMILOCAL_WINDOW[1]))
    # the truncated batch's length normaliser: its own maximum length
    lc_tail = B.LayerConfig(D=cfg.D, attn=dataclasses.replace(ac, norm_len=TRUNC_KEEP + c))
    ws = B.LayerWorkspace()
    bufs = [torch.empty_like(X), torch.empty_like(X)]

    def full6():
        x = X
        for li in range(6):
            W1, W2, rp, rt = lay[li]
            x = B.hstu_layer_fwd(x, W1, W2, rp, rt, offs, ts, lc_full, num_candidates=nc,
                                 y=bufs[li % 2], workspace=ws)

    def trunc(lc_first):
        return lambda: TR.truncated_stack_fwd(X, lay[:nf], lay[nf:nf + nt], offs, ts, lc_first,
                                              lc_tail, TRUNC_KEEP, num_candidates=nc,
                                              T_seg=T_seg, workspace=ws)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        timer.enable(64 * reps * 10)
        timer.reset()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        kern = timer.read()
        timer.enable(0)
        return e0.elapsed_time(e1) / reps, kern

    def lf(lengths, window=None):
        return flops.layer_flops(lengths, inp.num_candidates, cfg.D, cfg.H, cfg.d_qk, cfg.d_v,
                                 backward=False, window=window)["total"]

    f_full, f_tail = lf(inp.lengths), lf(seg_len)
    f_semi = lf(inp.lengths, SEMILOCAL_WINDOW)
    work = {"6_full": 6 * f_full, "3_full_6_trunc": nf * f_full + nt * f_tail,
            "3_semilocal_6_trunc": nf * f_semi + nt * f_tail}
    out = {"workload": "ranking batch 16 x (4096 history + 512 candidates), d_model 256, "
                       "4 heads x 64, bf16, inference forward",
           "keep": TRUNC_KEEP, "scheme": f"{nf} full + {nt} truncated vs 6 full",
           "semilocal_window": list(SEMILOCAL_WINDOW), "tokens": inp.T, "tokens_truncated": T_seg}
    for name, fn in (("6_full", full6), ("3_full_6_trunc", trunc(lc_full)),
                     ("3_semilocal_6_trunc", trunc(lc_semi))):
        ms, kern = timed(fn)
        out[name] = {"ms": round(ms, 4), "tflops": round(work[name] / (ms * 1e-3) / 1e12, 2),
                     "truncate_ms": round(kern.get("truncate", (0, 0.0))[1] / reps, 4)}
    base = out["6_full"]["ms"]
    for name in ("3_full_6_trunc", "3_semilocal_6_trunc"):
        out[name]["speedup_vs_6_full"] = round(base / out[name]["ms"], 3)
        out[name]["flop_ratio_vs_6_full"] = round(work["6_full"] / work[name], 3)
    log(f"truncation: {out}")
    return out


def bench_cached(timer, reps=5):
    """Ranking workload (16 users x (4096 history + 512 candidates), 4 layers,
    inference): the full target-aware pass against the cached path, which
    runs the histories once (cache build) and then only the candidates."""
    import numpy as np
    import torch

    import synth
    from hstu_sequential_transduction_amd import binding as B
    from hstu_sequential_transduction_amd import ranking as RK
    cfg = synth.get_config(5)
    inp = synth.make_inputs(cfg)
    nc_h = inp.num_candidates
    rows_h = np.concatenate([np.arange(inp.seq_offsets[b], inp.seq_offsets[b + 1] - nc_h[b])
                             for b in range(cfg.B)])
    rows_c = np.concatenate([np.arange(inp.seq_offsets[b + 1] - nc_h[b], inp.seq_offsets[b + 1])
                             for b in range(cfg.B)])
    n_hist = inp.lengths - nc_h
    hist_off = np.concatenate([[0], np.cumsum(n_hist)]).astype(np.int32)
    cand_off = np.concatenate([[0], np.cumsum(nc_h)]).astype(np.int32)
    td = torch.bfloat16
    cu = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    X = cu(inp.X).to(td)
    Xh, Xc = cu(inp.X[rows_h]).to(td), cu(inp.X[rows_c]).to(td)
    offs, ts = cu(inp.seq_offsets.astype(np.int32)), cu(inp.timestamps)
    nc = cu(nc_h.astype(np.int32))
    h_off, h_ts = cu(hist_off), cu(inp.timestamps[rows_h])
    c_off, c_ts = cu(cand_off), cu(inp.timestamps[rows_c])
    lay = [tuple(upload_layer(inp, cfg, li).values()) for li in range(cfg.n_layers)]
    ac = B.AttnConfig(H=cfg.H, d_qk=cfg.d_qk, d_v=cfg.d_v, norm_len=cfg.norm_len)
    lc = B.LayerConfig(D=cfg.D, attn=ac)
    ws = B.LayerWorkspace()
    bufs = [torch.empty_like(X), torch.empty_like(X)]
    cbufs = [torch.empty_like(Xc), torch.empty_like(Xc)]

    def full():
        x = X
        for li, (W1, W2, rp, rt) in enumerate(lay):
            x = B.hstu_layer_fwd(x, W1, W2, rp, rt, offs, ts, lc, num_candidates=nc,
                                 y=bufs[li % 2], workspace=ws)

    cache = RK.build_history_cache(Xh, lay, h_off, h_ts, lc, workspace=ws)

    def build():
        RK.build_history_cache(Xh, lay, h_off, h_ts, lc, workspace=ws)

    def cand():
        RK.cached_stack_fwd(Xc, lay, cache, c_off, c_ts, lc, workspace=ws, out_bufs=cbufs)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        timer.enable(64 * reps * cfg.n_layers)
        timer.reset()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        kern = timer.read()
        timer.enable(0)
        return e0.elapsed_time(e1) / reps, kern

    ms_full, _ = timed(full)
    ms_build, _ = timed(build)
    ms_cand, kern = timed(cand)
    # algorithmic work of the cached attention: every candidate x its history
    # keys, plus its own key, 2 (d_qk + d_v) flops per pair and head
    pairs = float(np.sum(nc_h * n_hist) + np.sum(nc_h))
    attn_flops = 2.0 * pairs * cfg.H * (cfg.d_qk + cfg.d_v)
    n_a, ms_a = kern.get("attn_cached", (0, 0.0))
    a_ms = ms_a / max(n_a, 1)
    a_tf = attn_flops / (a_ms * 1e-3) / 1e12 if n_a else None
    Tc = int(cand_off[-1])
    gemm = 2.0 * Tc * cfg.D * cfg.f1_width + 2.0 * Tc * cfg.H * cfg.d_v * cfg.D
    tot = cfg.n_layers * (attn_flops + gemm)
    out = {"workload": "ranking batch 16 x (4096 history + 512 candidates), d_model 256, "
                       "4 heads x 64, 4 layers, bf16, inference",
           "full_target_aware_ms": round(ms_full, 4),
           "history_cache_build_ms": round(ms_build, 4),
           "cached_candidates_ms": round(ms_cand, 4),
           "speedup_vs_full": round(ms_full / ms_cand, 2),
           "candidates_per_s": round(Tc / (ms_cand * 1e-3), 1),
           "cached_tflops": round(tot / (ms_cand * 1e-3) / 1e12, 2),
           "attn_cached_ms_per_launch": round(a_ms, 4),
           "attn_cached_tflops": None if a_tf is None else round(a_tf, 2),
           "attn_cached_frac_bf16_peak": None if a_tf is None else round(a_tf / PEAK_BF16_TFLOPS, 4),
           "kernel_ms": {k: round(v[1] / reps, 4) for k, v in kern.items()}}
    log(f"cached ranking: {out}")
    return out


def bench_mx(timer, reps=5):
    """Inference forward of the ranking workload (4 layers) with bf16 products
    against MXFP8 projection and output products (attention bf16 in both)."""
    import numpy as np
    import torch

    import synth
    from hstu_sequential_transduction_amd import binding as B
    from hstu_sequential_transduction_amd import flops
    cfg = synth.get_config(5)
    inp = synth.make_inputs(cfg)
    td = torch.bfloat16
    X = torch.from_numpy(inp.X).to(td).cuda()
    offs = torch.from_numpy(inp.seq_offsets.astype(np.int32)).cuda()
    ts = torch.from_numpy(inp.timestamps).cuda()
    nc = torch.from_numpy(inp.num_candidates.astype(np.int32)).cuda()
    lay = [upload_layer(inp, cfg, li) for li in range(cfg.n_layers)]
    mxw = [B.MxLayerWeights.from_bf16(w["W1"], w["W2"]) for w in lay]
    ac = B.AttnConfig(H=cfg.H, d_qk=cfg.d_qk, d_v=cfg.d_v, norm_len=cfg.norm_len)
    lc = B.LayerConfig(D=cfg.D, attn=ac)
    ws = B.LayerWorkspace()
    bufs = [torch.empty_like(X), torch.empty_like(X)]

    def run_bf16():
        x = X
        for li, w in enumerate(lay):
            x = B.hstu_layer_fwd(x, w["W1"], w["W2"], w["rp"], w["rt"], offs, ts, lc,
                                 num_candidates=nc, y=bufs[li % 2], workspace=ws)

    # each layer's output product also writes its Y in MXFP8 for the next
    # layer, so only the first layer quantizes its input
    T, D = inp.T, cfg.D
    mxb = [(torch.empty((T, D), dtype=torch.uint8, device="cuda"),
            torch.empty((T, D // 32), dtype=torch.uint8, device="cuda")) for _ in range(2)]

    def run_mx():
        x, x_mx = X, None
        for li, (w, m) in enumerate(zip(lay, mxw)):
            y_mx = mxb[li % 2] if li + 1 < len(lay) else None
            x = B.hstu_layer_fwd_mx(x, m, w["rp"], w["rt"], offs, ts, lc, num_candidates=nc,
                                    y=bufs[li % 2], workspace=ws, x_mx=x_mx, y_mx=y_mx)
            x_mx = y_mx

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        timer.enable(64 * reps * cfg.n_layers)
        timer.reset()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        kern = timer.read()
        timer.enable(0)
        return e0.elapsed_time(e1) / reps, {k: round(v[1] / reps, 4) for k, v in kern.items()}

    ms_b, kb = timed(run_bf16)
    ms_m, km = timed(run_mx)
    proj = 2.0 * T * cfg.D * cfg.f1_width * cfg.n_layers
    outp = 2.0 * T * cfg.H * cfg.d_v * cfg.D * cfg.n_layers
    tf = lambda fl, ms: round(fl / (ms * 1e-3) / 1e12, 2) if ms else None
    lf = flops.layer_flops(inp.lengths, inp.num_candidates, cfg.D, cfg.H, cfg.d_qk, cfg.d_v,
                           backward=False)["total"] * cfg.n_layers
    out = {"workload": "ranking batch 16 x (4096 history + 512 candidates), d_model 256, "
                       "4 heads x 64, 4 layers, inference",
           "format": "MXFP8 (E4M3, E8M0 scale per 32 along the contraction) for the "
                     "projection and output products; attention bf16",
           "bf16_ms": round(ms_b, 4), "mx_ms": round(ms_m, 4),
           "speedup": round(ms_b / ms_m, 3),
           "tflops_bf16": tf(lf, ms_b), "tflops_mx": tf(lf, ms_m),
           "proj_gemm_tflops_bf16": tf(proj, kb.get("gemm_uvqk")),
           "proj_gemm_tflops_mx": tf(proj, km.get("gemm_uvqk")),
           "out_gemm_tflops_bf16": tf(outp, kb.get("gemm_out")),
           "out_gemm_tflops_mx": tf(outp, km.get("gemm_out")),
           "kernel_ms_bf16": kb, "kernel_ms_mx": km}
    log(f"mxfp8: {out}")
    return out


def roofline(cfg, inp, kern, steps, traffic_dir):
    work = kernel_work(cfg, inp.lengths, inp.T)
    best = max(((ms, name, n) for name, (n, ms) in kern.items() if name in work), default=None)
    if best is None:
        return None, {}
    table = {}
    for name, (n, ms) in kern.items():
        per = ms / max(n, 1)
        entry = {"launches_per_step": n / max(steps, 1), "ms_per_launch": round(per, 5)}
        if name in work:
            kind, amt = work[name]
            if kind == "mfma":
                entry["tflops"] = round(amt / (per * 1e-3) / 1e12, 2)
            else:
                entry["gbs"] = round(amt / (per * 1e-3) / 1e9, 1)
        table[name] = entry
    ms, name, n = best
    kind, amt = work[name]
    per_s = ms / n * 1e-3
    if kind == "mfma":
        achieved, peak, unit = amt / per_s / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = amt / per_s / 1e9, PEAK_HBM_GBS, "GB/s"
    traffic = None
    tf = os.path.join(traffic_dir, f"{name}_traffic.json")
    if os.path.exists(tf):
        with open(tf) as fh:
            rec = json.load(fh)
        if rec.get("source_hash") == source_hash(name) and rec.get("workload") == cfg.name:
            traffic = rec.get("bytes_per_launch")
    roof = {"kernel": name, "bound": "mfma" if kind == "mfma" else "hbm",
            "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic,
            "work_per_launch": amt, "ms_per_launch": round(ms / n, 5),
            "source_hash": source_hash(name)}
    return roof, table


def bench_fwd_configs(timer, reps=3):
    """Forward-only figures of the inference workloads (context for the forward kernel)."""
    import numpy as np
    import torch

    import synth
    from hstu_sequential_transduction_amd import binding as B
    from hstu_sequential_transduction_amd import flops
    out = {}
    for ci in (2, 3, 5):
        cfg = synth.get_config(ci)
        inp = synth.make_inputs(cfg)
        td = torch.bfloat16
        X = torch.from_numpy(inp.X).to(td).cuda()
        offs = torch.from_numpy(inp.seq_offsets.astype(np.int32)).cuda()
        ts = torch.from_numpy(inp.timestamps).cuda()
        nc = None if inp.num_candidates is None else \
            torch.from_numpy(inp.num_candidates.astype(np.int32)).cuda()
        layers = [upload_layer(inp, cfg, li) for li in range(cfg.n_layers)]
        ac = B.AttnConfig(H=cfg.H, d_qk=cfg.d_qk, d_v=cfg.d_v, norm_len=cfg.norm_len)
        lc = B.LayerConfig(D=cfg.D, attn=ac)
        ws = B.LayerWorkspace()
        bufs = [torch.empty_like(X), torch.empty_like(X)]

        # layers after the first reuse the plan the first wrote into the
        # shared workspace (same offsets, timestamps and candidates)
        lc_r = dataclasses.replace(lc, attn=dataclasses.replace(ac, reuse_plan=1))

        def run():
            x = X
            for li, w in enumerate(layers):
                x = B.hstu_layer_fwd(x, w["W1"], w["W2"], w["rp"], w["rt"], offs, ts,
                                     lc if li == 0 else lc_r, num_candidates=nc,
                                     y=bufs[li % 2], workspace=ws)

        run()
        torch.cuda.synchronize()
        timer.enable(64 * reps * cfg.n_layers)
        timer.reset()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        kern = timer.read()
        timer.enable(0)
        lf = flops.layer_flops(inp.lengths, inp.num_candidates, cfg.D, cfg.H, cfg.d_qk, cfg.d_v,
                               backward=False)
        tot = lf["total"] * cfg.n_layers
        af = lf["attn_fwd"]
        n_a, ms_a = kern.get("attn_fwd", (0, 0.0))
        a_tf = af / (ms_a / max(n_a, 1) * 1e-3) / 1e12 if n_a else None
        out[cfg.name] = {
            "ms": round(ms, 4), "tokens": inp.T, "layers": cfg.n_layers,
            "tflops": round(tot / (ms * 1e-3) / 1e12, 2),
            "tokens_per_s": round(inp.T / (ms * 1e-3), 1),
            "attn_fwd_tflops": None if a_tf is None else round(a_tf, 2),
            "attn_fwd_frac_bf16_peak": None if a_tf is None else round(a_tf / PEAK_BF16_TFLOPS, 4),
            "kernel_ms": {k: round(v[1] / reps, 4) for k, v in kern.items()},
        }
        log(f"fwd {cfg.name}: {out[cfg.name]}")
    return out


CPU_SAMPLE_SEQS = 3


def cpu_baseline(cfg, inp):
    """The fp64 oracle on the CPU_SAMPLE_SEQS shortest sequences of the training
    batch (about 10 s of CPU work on 16 cores for the training workload)."""
    import numpy as np

    import synth
    from hstu_sequential_transduction_amd import flops
    from oracle import hstu as orc
    try:
        from threadpoolctl import threadpool_info
        cores = max((p.get("num_threads", 1) for p in threadpool_info()), default=os.cpu_count())
    except Exception:
        cores = os.cpu_count()
    idx = sorted(int(i) for i in np.argsort(inp.lengths, kind="stable")[:CPU_SAMPLE_SEQS])
    sub = synth.sub_batch(inp, idx)
    w = sub.layers[0]
    f = orc.LayerFlags(H=cfg.H, d_qk=cfg.d_qk, d_v=cfg.d_v, norm_len=cfg.norm_len, eps=1e-6)
    t0 = time.perf_counter()
    Y, sv = orc.layer_fwd(sub.X, w.W1, w.W2, w.rab_pos, w.rab_time, sub.seq_offsets,
                          sub.timestamps, None, f)
    orc.layer_bwd(sub.dY, sub.X, w.W1, w.W2, w.rab_pos, w.rab_time, sub.seq_offsets,
                  sub.timestamps, None, f, sv)
    dt = time.perf_counter() - t0
    lf = flops.layer_flops(sub.lengths, None, cfg.D, cfg.H, cfg.d_qk, cfg.d_v, backward=True)
    return {"value": round(lf["total"] / dt / 1e12, 5), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle", "seconds": round(dt, 2),
            "tokens_per_s": round(sub.T / dt, 1),
            "sample": f"the {len(idx)} shortest sequences ({sub.T} tokens) of the training "
                      f"batch, fwd+bwd of one layer, fp64 numpy"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the forward-only workloads, the semi-local training step, "
                         "the attention-truncation forward, the cached ranking and the MXFP8 forward")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the data-parallel "
              "sharding over GPUs is a design note, not built).", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    from hstu_sequential_transduction_amd import _lib
    timer = Timer(_lib.lib())

    cfg, inp, ms, kern, lf = bench_train(args, timer)
    tflops = lf["total"] / (ms * 1e-3) / 1e12
    log(f"train step: {ms:.3f} ms, {tflops:.1f} TFLOP/s")
    roof, table = roofline(cfg, inp, kern, args.steps, os.path.join(ROOT, "profiles"))
    extra = None if args.no_extra else bench_fwd_configs(timer)
    semi = None if args.no_extra else bench_semilocal(args, timer, ms)
    trunc = None if args.no_extra else bench_truncation(timer)
    cached = None if args.no_extra else bench_cached(timer)
    mx = None if args.no_extra else bench_mx(timer)
    cpu = None if args.no_cpu_baseline else cpu_baseline(cfg, inp)
    line = {
        "metric": METRIC, "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; inputs resident in HBM)",
        "config": {"workload": "1 HSTU layer fwd+bwd (training), bf16: batch 8, lengths U[4096,8192],"
                               " d_model 512, 4 heads x 128, causal",
                   "global_batch": cfg.B, "tokens": inp.T, "seq_len": "U[4096,8192]",
                   "parallelism": "single GPU"},
        "tokens_per_s": round(inp.T / (ms * 1e-3), 1),
        "frac_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "flops_per_step": {k: v for k, v in lf.items()},
        "kernels": table,
        "roofline": roof,
        "cpu_baseline": cpu,
        "forward_workloads": extra,
        "semilocal": semi,
        "truncation": trunc,
        "cached_ranking": cached,
        "mxfp8": mx,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
