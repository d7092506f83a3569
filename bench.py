#!/usr/bin/env python3
"""Benchmark of the HSTU layer on one MI355X.

One step = one full training step of one HSTU layer (forward with saved
intermediates + backward, every kernel of the path) on the long-sequence
training workload: 8 jagged sequences of uniform length in [4096, 8192],
d_model 512, 4 heads x 128, causal, bf16 with fp32 accumulation, synthetic
seeded inputs resident in HBM before timing starts.

Prints one JSON line.  `value` is whole-step algorithmic TFLOP/s (the DLRMv4
page's Table 7 convention: weight GEMMs x3, attention x3.5 for fwd+bwd, S^2/2
pairs per sequence) over exactly --steps steps timed between two events with
no instrumentation in the region; per-step events give the median and
p10/p90.  A separate instrumented pass of the same steps (the library's HIP
event pairs around every launch) gives the per-kernel table and the roofline
of the dominant kernel.  Alongside: the step with dQ recomputed instead of
formed from the kept score gradient, forward-only figures of the other
workloads, the LayerNorm-gate epilogue's bandwidth warm, after a cache flush
and with a working set larger than the last-level cache, a measured MFMA
rate and copy bandwidth beside the nominal peaks, and the fp64 CPU oracle
timed on bounded samples of every workload.
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
    """The library's diagnostic per-kernel timer (HIP event pairs around each
    launch site, on the stream the launch uses)."""

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


def time_region(fn, steps, warmup, between=None):
    """Runs `warmup` untimed calls, then `steps` calls between events on the
    current stream (one event per call boundary; nothing else in the region
    unless `between` is given, which runs before each call and is excluded
    from the per-call times but not from the total).  Returns mean (total /
    steps), median, p10, p90 in ms."""
    import numpy as np
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    steps = max(int(steps), 1)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        if between is not None:
            between()
        ev[2 * i].record()
        fn()
        ev[2 * i + 1].record()
    torch.cuda.synchronize()
    per = np.array([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(steps)])
    total = ev[0].elapsed_time(ev[-1])
    return {"ms_mean": round(float(total / steps) if between is None else float(per.mean()), 4),
            "ms_median": round(float(np.median(per)), 4),
            "ms_p10": round(float(np.percentile(per, 10)), 4),
            "ms_p90": round(float(np.percentile(per, 90)), 4), "reps": steps}


def instrumented(fn, timer, steps, per_call_launches=64):
    """Per-kernel times of `steps` calls of fn with the library timer on."""
    import torch
    torch.cuda.synchronize()
    timer.enable(per_call_launches * max(steps, 1))
    timer.reset()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    kern = timer.read()
    timer.enable(0)
    return kern, e0.elapsed_time(e1) / max(steps, 1)


def timed_pair(fn, timer, reps, per_call_launches):
    """Mean ms of `reps` uninstrumented calls, then the per-kernel times of
    `reps` instrumented calls (summed: {tag: (launches, ms)})."""
    st = time_region(fn, reps, 1)
    kern, _ = instrumented(fn, timer, reps, per_call_launches)
    return st["ms_mean"], kern


def upload_layer(inp, cfg, li=0):
    import numpy as np
    import torch
    td = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    w = inp.layers[li]
    return dict(
        W1=torch.from_numpy(w.W1).to(td).cuda(), W2=torch.from_numpy(w.W2).to(td).cuda(),
        rp=torch.from_numpy(w.rab_pos).cuda(), rt=torch.from_numpy(w.rab_time).cuda())


def train_setup(window=(0, 0), keep_ds=True, mx=False, mx_scores=False):
    """The training workload on the device and one step (layer fwd + bwd) as a
    closure.  keep_ds: pass the longest sequence as max_len, which lets the
    backward keep the score gradient dS and form dQ from it.  mx: the MXFP8
    step (hstu_layer_fwd_mx + hstu_layer_bwd_mx; the weights are quantized
    inside the step, as they change every step)."""
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
    ac = B.AttnConfig(H=cfg.H, d_qk=cfg.d_qk, d_v=cfg.d_v, norm_len=cfg.norm_len,
                      win_local=window[0], win_global=window[1],
                      max_len=int(inp.lengths.max()) if keep_ds else 0)
    lc = B.LayerConfig(D=cfg.D, attn=ac)
    saved = B.Saved(T, lc, td, "cuda")
    y = torch.empty_like(X)
    dx = torch.empty_like(X)
    f32 = dict(dtype=torch.float32, device="cuda")
    grads = B.Grads(torch.empty(w["W1"].shape, **f32), torch.empty(w["W2"].shape, **f32),
                    torch.empty(w["rp"].shape, **f32), torch.empty(w["rt"].shape, **f32))
    wsf, wsb = B.LayerWorkspace(), B.LayerWorkspace()

    def step():
        if mx:
            wm = B.MxLayerWeights.from_bf16(w["W1"], w["W2"])
            B.hstu_layer_fwd_mx(X, wm, w["rp"], w["rt"], offs, ts, lc, saved=saved, y=y,
                                workspace=wsf, mx_scores=mx_scores)
        else:
            B.hstu_layer_fwd(X, w["W1"], w["W2"], w["rp"], w["rt"], offs, ts, lc, saved=saved,
                             y=y, workspace=wsf)
        B.hstu_layer_bwd(X, w["W1"], w["W2"], w["rp"], w["rt"], offs, ts, lc, saved, dY, dx=dx,
                         grads=grads, workspace=wsb, mx=mx)

    lf = flops.layer_flops(inp.lengths, None, cfg.D, cfg.H, cfg.d_qk, cfg.d_v, backward=True,
                           window=window if window[0] > 0 else None)
    return cfg, inp, step, lf


def bench_train(args, timer, window=(0, 0), keep_ds=True, mx=False, mx_scores=False):
    """Uninstrumented timed region of --steps steps, then an instrumented pass
    of the same number of steps (at most 20) for the per-kernel table."""
    cfg, inp, step, lf = train_setup(window, keep_ds, mx, mx_scores)
    stats = time_region(step, args.steps, args.warmup)
    kern, ms_instr = instrumented(step, timer, min(args.steps, 20))
    stats["ms_instrumented"] = round(ms_instr, 4)
    stats["instrumented_steps"] = min(args.steps, 20)
    return cfg, inp, stats, kern, lf


def bench_recompute(args, timer, kept_ms):
    """The same training step without max_len: dQ recomputes S and dA instead
    of reading the kept score gradient (no O(sum n^2) buffer)."""
    cfg, inp, stats, kern, lf = bench_train(args, timer, keep_ds=False)
    ms = stats["ms_mean"]
    work = kernel_work(cfg, inp.lengths, inp.T, keep_ds=False)
    kt = {}
    for name in ("attn_bwd_dkdv", "attn_bwd_dq"):
        if name in kern:
            n, t = kern[name]
            kt[name] = {"ms_per_launch": round(t / n, 5),
                        "tflops": round(work[name][1] / (t / n * 1e-3) / 1e12, 2)}
    out = {"ms_per_step": ms, **{k: v for k, v in stats.items() if k != "ms_mean"},
           "tflops": round(lf["total"] / (ms * 1e-3) / 1e12, 2),
           "tokens_per_s": round(inp.T / (ms * 1e-3), 1),
           "slowdown_vs_kept_ds": round(ms / kept_ms, 3), "kernels": kt}
    log(f"train step, dQ recomputed: {ms:.3f} ms ({out['tflops']} TFLOP/s)")
    return out


def bench_train_mx(args, timer, bf16_ms):
    """The training step with MXFP8 products: forward projection and output
    products, backward dG, dX, dW2 and dW1 (attention and LayerNorm in
    bf16 / fp32; the quantization passes are inside the timed step).
    TFLOP/s on the same work as the bf16 step."""
    cfg, inp, stats, kern, lf = bench_train(args, timer, mx=True)
    ms = stats["ms_mean"]
    out = {"ms_per_step": ms, **{k: v for k, v in stats.items() if k != "ms_mean"},
           "tflops": round(lf["total"] / (ms * 1e-3) / 1e12, 2),
           "tokens_per_s": round(inp.T / (ms * 1e-3), 1),
           "speedup_vs_bf16": round(bf16_ms / ms, 3),
           "kernel_ms_per_launch": {k: round(v[1] / v[0], 4) for k, v in kern.items()},
           "kernel_launches_per_step": {k: round(v[0] / max(stats["instrumented_steps"], 1), 2)
                                        for k, v in kern.items()}}
    log(f"train step, MXFP8 products: {ms:.3f} ms ({out['tflops']} TFLOP/s, "
        f"{out['speedup_vs_bf16']}x the bf16 step)")
    # and with the attention's score product in MXFP8 too
    _, _, st2, kern2, _ = bench_train(args, timer, mx=True, mx_scores=True)
    ms2 = st2["ms_mean"]
    out["with_mx_scores"] = {
        "ms_per_step": ms2, "ms_median": st2["ms_median"],
        "tflops": round(lf["total"] / (ms2 * 1e-3) / 1e12, 2),
        "speedup_vs_bf16": round(bf16_ms / ms2, 3),
        "kernel_ms_per_launch": {k: round(v[1] / v[0], 4) for k, v in kern2.items()}}
    log(f"train step, MXFP8 products and scores: {ms2:.3f} ms "
        f"({out['with_mx_scores']['speedup_vs_bf16']}x the bf16 step)")
    return out


# Semi-local attention windows of the extra training-step measurement: the
# pages give no sizes, so these are chosen parameters (a local window of 1024
# positions and the first 128 tokens), stated with the result.
SEMILOCAL_WINDOW = (1024, 128)


def bench_semilocal(args, timer, full_ms):
    """The same training step with semi-local attention; TFLOP/s on the
    windowed work (exact pair count), and the speedup over full causal."""
    from hstu_sequential_transduction_amd import flops
    cfg, inp, stats, kern, lf = bench_train(args, timer, window=SEMILOCAL_WINDOW)
    ms = stats["ms_mean"]
    full_pairs = flops.attn_pairs_window(inp.lengths, None, 0, 0)
    win_pairs = flops.attn_pairs_window(inp.lengths, None, *SEMILOCAL_WINDOW)
    out = {"win_local": SEMILOCAL_WINDOW[0], "win_global": SEMILOCAL_WINDOW[1],
           "ms_per_step": ms, "ms_median": stats["ms_median"],
           "tflops": round(lf["total"] / (ms * 1e-3) / 1e12, 2),
           "tokens_per_s": round(inp.T / (ms * 1e-3), 1),
           "attn_pairs_frac": round(win_pairs / full_pairs, 4),
           "speedup_vs_full_causal": round(full_ms / ms, 3),
           "kernel_ms_per_launch": {k: round(v[1] / v[0], 4) for k, v in kern.items()},
           "kernel_launches_per_step": {k: round(v[0] / max(stats["instrumented_steps"], 1), 2)
                                        for k, v in kern.items()}}
    log(f"semi-local step (W_l={SEMILOCAL_WINDOW[0]}, W_g={SEMILOCAL_WINDOW[1]}): "
        f"{ms:.3f} ms, x{full_ms / ms:.2f} vs full causal")
    return out


# Attention truncation on the ranking workload (16 x (4096 history + 512
# candidates), d_model 256, 4 heads x 64), in the pages' 3 + 6 layer scheme
# against 6 full layers.  The segment length L' is not on the pages: 1024
# history events (plus the candidates) is a chosen parameter.
TRUNC_KEEP = 1024
TRUNC_SCHEME = (3, 6)


def bench_truncation(timer, reps=5):
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
        return timed_pair(fn, timer, reps, 64 * 10)

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


def bench_cached(timer, reps=10):
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
        return timed_pair(fn, timer, reps, 64 * cfg.n_layers)

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


def bench_mx(timer, reps=10):
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

    def run_mx_scores():
        x, x_mx = X, None
        for li, (w, m) in enumerate(zip(lay, mxw)):
            y_mx = mxb[li % 2] if li + 1 < len(lay) else None
            x = B.hstu_layer_fwd_mx(x, m, w["rp"], w["rt"], offs, ts, lc, num_candidates=nc,
                                    y=bufs[li % 2], workspace=ws, x_mx=x_mx, y_mx=y_mx,
                                    mx_scores=True)
            x_mx = y_mx

    def timed(fn):
        ms, kern = timed_pair(fn, timer, reps, 64 * cfg.n_layers)
        return ms, {k: round(v[1] / reps, 4) for k, v in kern.items()}

    ms_b, kb = timed(run_bf16)
    ms_m, km = timed(run_mx)
    ms_s, ks = timed(run_mx_scores)
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
           "kernel_ms_bf16": kb, "kernel_ms_mx": km,
           "with_mx_scores": {
               "format": "also the attention's q.k in MXFP8 (q and k quantized along each "
                         "head's channels in one pass per layer); P V bf16",
               "ms": round(ms_s, 4), "speedup_vs_bf16": round(ms_b / ms_s, 3),
               "speedup_vs_mx_products": round(ms_m / ms_s, 3), "tflops": tf(lf, ms_s),
               "kernel_ms": ks}}
    log(f"mxfp8: {out}")
    return out


def bench_attn_mx(timer, configs=(3, 5, 4), reps=20):
    """Attention forward with the score product in MXFP8 (q and k quantized
    along each head's channels, the scaled FP8 MFMA for q.k, P V in bf16)
    against the bf16 attention on the same q, k, v: whole-call medians
    (quantization of q and k included on the MX side) and kernel times."""
    import numpy as np
    import torch

    import synth
    from hstu_sequential_transduction_amd import binding as B
    from hstu_sequential_transduction_amd import flops
    out = {}
    for ci in configs:
        cfg = synth.get_config(ci)
        a = synth.make_attn_inputs(cfg)
        T = a.q.shape[0]
        td = torch.bfloat16
        q = torch.from_numpy(a.q.reshape(T, -1)).to(td).cuda()
        k = torch.from_numpy(a.k.reshape(T, -1)).to(td).cuda()
        v = torch.from_numpy(a.v.reshape(T, -1)).to(td).cuda()
        offs = torch.from_numpy(a.seq_offsets.astype(np.int32)).cuda()
        ts = torch.from_numpy(a.timestamps.astype(np.int64)).cuda()
        rp, rt = torch.from_numpy(a.rab_pos).cuda(), torch.from_numpy(a.rab_time).cuda()
        nc = None if a.num_candidates is None else \
            torch.from_numpy(a.num_candidates.astype(np.int32)).cuda()
        ac = B.AttnConfig(H=cfg.H, d_qk=cfg.d_qk, d_v=cfg.d_v, norm_len=cfg.norm_len)
        ws = B.LayerWorkspace()
        o = torch.empty((T, cfg.H * cfg.d_v), dtype=td, device="cuda")

        def run_bf16():
            B.hstu_attn_fwd(q, k, v, offs, ts, rp, rt, ac, num_candidates=nc, out=o, workspace=ws)

        def run_mx():
            qc, qs = B.hstu_mx_quantize_heads(q, cfg.H, cfg.d_qk)
            kc, ks = B.hstu_mx_quantize_heads(k, cfg.H, cfg.d_qk)
            B.hstu_attn_fwd_mx(qc, qs, kc, ks, v, offs, ts, rp, rt, ac, num_candidates=nc,
                               out=o, workspace=ws)

        sb = time_region(run_bf16, reps, 2)
        sm = time_region(run_mx, reps, 2)
        kb, _ = instrumented(run_bf16, timer, reps, 4)
        km, _ = instrumented(run_mx, timer, reps, 8)
        per = lambda kern, tag: kern[tag][1] / reps if tag in kern else None
        fl = flops.attn_fwd_flops(a.lengths, a.num_candidates, cfg.H, cfg.d_qk, cfg.d_v)
        tf = lambda ms: round(fl / (ms * 1e-3) / 1e12, 1) if ms else None
        ab, am, qm = per(kb, "attn_fwd"), per(km, "attn_fwd"), per(km, "mx_quant")
        out[cfg.name] = {
            "d_qk": cfg.d_qk, "bf16_ms": round(sb["ms_median"], 4),
            "mx_ms": round(sm["ms_median"], 4),
            "speedup_whole_call": round(sb["ms_median"] / sm["ms_median"], 3),
            "attn_kernel_ms_bf16": round(ab, 4), "attn_kernel_ms_mx": round(am, 4),
            "quantize_q_and_k_ms": round(qm, 4) if qm else None,
            "attn_kernel_tflops_bf16": tf(ab), "attn_kernel_tflops_mx": tf(am),
            "attn_kernel_speedup": round(ab / am, 3)}
        log(f"attention mx {cfg.name}: {out[cfg.name]}")
    return out


def roofline(cfg, inp, kern, steps, traffic_dir):
    work = kernel_work(cfg, inp.lengths, inp.T)
    best = max(((ms, name, n) for name, (n, ms) in kern.items() if name in work), default=None)
    if best is None:
        return None, {}
    table = {}
    for name, (n, ms) in kern.items():
        per = ms / max(n, 1)
        # a tag's work is per step (a product may run as several launches)
        per_step = ms / max(steps, 1)
        entry = {"launches_per_step": n / max(steps, 1), "ms_per_launch": round(per, 5),
                 "ms_per_step": round(per_step, 5)}
        if name in work:
            kind, amt = work[name]
            if kind == "mfma":
                entry["tflops"] = round(amt / (per_step * 1e-3) / 1e12, 2)
            else:
                entry["gbs"] = round(amt / (per_step * 1e-3) / 1e9, 1)
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


def bench_fwd_configs(timer, configs=(2, 3, 5), reps=20):
    """Forward-only figures of the inference workloads (context for the forward
    kernel): uninstrumented median of `reps` runs, per-kernel times from an
    instrumented pass."""
    import numpy as np
    import torch

    import synth
    from hstu_sequential_transduction_amd import binding as B
    from hstu_sequential_transduction_amd import flops
    out = {}
    for ci in configs:
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

        st = time_region(run, reps, 2)
        kern, _ = instrumented(run, timer, reps, 64 * cfg.n_layers)
        ms = st["ms_median"]
        # the attention kernel, for comparison, with long blocks' keys split
        # in up to 4 workgroups, and with 128-row work items only (key_splits
        # 1; the default takes 64-row items whose key tiles two waves share
        # when the 128-row items would not fill the GPU)
        lc0, lc_r0, ws0 = lc, lc_r, ws
        alt = {}
        for ks in (4, 1):
            lc, lc_r = (dataclasses.replace(c, attn=dataclasses.replace(c.attn, key_splits=ks))
                        for c in (lc0, lc_r0))
            ws = B.LayerWorkspace()
            kern1, _ = instrumented(run, timer, reps, 64 * cfg.n_layers)
            alt[ks] = kern1.get("attn_fwd", (0, 0.0))
        lc, lc_r, ws = lc0, lc_r0, ws0
        n_a1, ms_a1 = alt[4]
        n_a2, ms_a2 = alt[1]
        lf = flops.layer_flops(inp.lengths, inp.num_candidates, cfg.D, cfg.H, cfg.d_qk, cfg.d_v,
                               backward=False)
        tot = lf["total"] * cfg.n_layers
        af = lf["attn_fwd"]
        n_a, ms_a = kern.get("attn_fwd", (0, 0.0))
        a_tf = af / (ms_a / max(n_a, 1) * 1e-3) / 1e12 if n_a else None
        out[cfg.name] = {
            "ms": ms, "ms_mean": st["ms_mean"], "ms_p10": st["ms_p10"], "ms_p90": st["ms_p90"],
            "reps": reps, "tokens": inp.T, "layers": cfg.n_layers,
            "tflops": round(tot / (ms * 1e-3) / 1e12, 2),
            "tokens_per_s": round(inp.T / (ms * 1e-3), 1),
            "attn_fwd_ms_per_layer": None if not n_a else round(ms_a / n_a, 5),
            "attn_fwd_ms_per_layer_key_splits_4": None if not n_a1 else round(ms_a1 / n_a1, 5),
            "attn_fwd_ms_per_layer_128_row_items": None if not n_a2 else round(ms_a2 / n_a2, 5),
            "attn_fwd_tflops": None if a_tf is None else round(a_tf, 2),
            "attn_fwd_frac_bf16_peak": None if a_tf is None else round(a_tf / PEAK_BF16_TFLOPS, 4),
            "kernel_ms": {k: round(v[1] / reps, 4) for k, v in kern.items()},
        }
        log(f"fwd {cfg.name}: {out[cfg.name]}")
    return out


def bench_epilogue(timer, reps=20):
    """Bandwidth of the LayerNorm + gating epilogue (forward) inside the
    inference forward of the training workload's batch: warm (calls back to
    back), after a 1 GiB write between calls (last-level cache flushed; O and
    U still come straight from the kernels of the same call that produced
    them), and on a batch of four times as many tokens, whose O, U and G
    (0.94 GB) exceed the 256 MB last-level cache."""
    import numpy as np
    import torch

    import synth
    from hstu_sequential_transduction_amd import binding as B
    cfg = synth.get_config(4)
    out = {}
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    for name, mult in (("warm", 1), ("flushed", 1), ("working_set_4x", 4)):
        inp = synth.make_inputs(cfg)
        X = torch.from_numpy(inp.X).to(torch.bfloat16).cuda()
        lengths = inp.lengths
        offs_np = inp.seq_offsets.astype(np.int64)
        ts_np = inp.timestamps
        if mult > 1:
            X = X.repeat(mult, 1)
            lengths = np.tile(lengths, mult)
            offs_np = np.concatenate([[0], np.cumsum(lengths)])
            ts_np = np.tile(ts_np, mult)
        offs = torch.from_numpy(offs_np.astype(np.int32)).cuda()
        ts = torch.from_numpy(ts_np).cuda()
        w = upload_layer(inp, cfg)
        lc = B.LayerConfig(D=cfg.D, attn=B.AttnConfig(H=cfg.H, d_qk=cfg.d_qk, d_v=cfg.d_v,
                                                      norm_len=cfg.norm_len))
        ws = B.LayerWorkspace()
        y = torch.empty_like(X)

        def run():
            B.hstu_layer_fwd(X, w["W1"], w["W2"], w["rp"], w["rt"], offs, ts, lc, y=y,
                             workspace=ws)

        run()
        torch.cuda.synchronize()
        timer.enable(64 * reps)
        timer.reset()
        for _ in range(reps):
            if name == "flushed":
                flush.fill_(1)
            run()
        torch.cuda.synchronize()
        kern = timer.read()
        timer.enable(0)
        n, ms = kern["ln_gate_fwd"]
        T = int(offs_np[-1])
        W = cfg.H * cfg.d_v
        byts = T * (4.0 * W + 2 * W + 2 * W)     # O fp32 + U read, G written (no stats)
        gbs = byts / (ms / n * 1e-3) / 1e9
        out[name] = {"tokens": T, "ms": round(ms / n, 5), "bytes": byts, "gbs": round(gbs, 1),
                     "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
        del X, y, ws
    log(f"LayerNorm-gate epilogue: {out}")
    return out


def bench_peaks(reps=10):
    """Measured MFMA rate (the library's MFMA-loop diagnostic) and device-copy
    bandwidth (a 2 GiB tensor copy), beside the nominal peaks."""
    import ctypes as C

    import torch

    from hstu_sequential_transduction_amd import _lib
    L = _lib.lib()
    wg, iters = 1024, 2000
    buf = torch.empty(4 * wg, dtype=torch.float32, device="cuda")
    st = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    run = lambda: _lib.check("hstu_diag_mfma_loop",
                             L.hstu_diag_mfma_loop(iters, wg, C.c_void_p(buf.data_ptr()), st))
    t = time_region(run, reps, 2)
    flop = wg * 4.0 * iters * 4 * 32768
    mfma = flop / (t["ms_median"] * 1e-3) / 1e12
    a = torch.empty(1 << 30, dtype=torch.uint16, device="cuda").fill_(1)
    b = torch.empty_like(a)
    tc = time_region(lambda: b.copy_(a), reps, 2)
    gbs = 2 * a.numel() * 2 / (tc["ms_median"] * 1e-3) / 1e9
    out = {"mfma_bf16_tflops_measured": round(mfma, 1), "mfma_bf16_tflops_nominal": PEAK_BF16_TFLOPS,
           "copy_gbs_measured": round(gbs, 1), "hbm_gbs_nominal": PEAK_HBM_GBS,
           "mfma_probe": f"{wg} workgroups x 4 waves x {iters} x 4 independent 32x32x16 bf16 MFMAs",
           "copy_probe": "2 GiB device-to-device tensor copy (read + write counted)"}
    log(f"peaks: {out}")
    return out


def _cores():
    try:
        from threadpoolctl import threadpool_info
        return max((p.get("num_threads", 1) for p in threadpool_info()), default=os.cpu_count())
    except Exception:
        return os.cpu_count()


CPU_SAMPLE_SEQS = 3


def cpu_baseline(cfg, inp):
    """The fp64 oracle on the CPU_SAMPLE_SEQS shortest sequences of the training
    batch (about 10 s of CPU work on 16 cores for the training workload)."""
    import numpy as np

    import synth
    from hstu_sequential_transduction_amd import flops
    from oracle import hstu as orc
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
    return {"value": round(lf["total"] / dt / 1e12, 5), "unit": "TFLOP/s", "cores": int(_cores()),
            "kind": "oracle", "seconds": round(dt, 2),
            "tokens_per_s": round(sub.T / dt, 1),
            "sample": f"the {len(idx)} shortest sequences ({sub.T} tokens) of the training "
                      f"batch, fwd+bwd of one layer, fp64 numpy"}


# Bounded oracle samples of the forward workloads: config -> (first sequences
# or None for the whole batch, layers); about 6 s on 16 host threads
CPU_FWD_SAMPLES = {1: (None, 1), 2: (None, 1), 3: (None, 1), 5: (4, 1)}


def cpu_baseline_configs():
    """The fp64 oracle's forward on a bounded sample of each inference workload
    (whole batch for the small fp32 workload, the first sequences otherwise,
    one layer), as GFLOP/s and tokens/s with the same algorithmic FLOPs."""
    import numpy as np

    import synth
    from hstu_sequential_transduction_amd import flops
    from oracle import hstu as orc
    out = {}
    for ci, (nseq, nl) in CPU_FWD_SAMPLES.items():
        cfg = synth.get_config(ci)
        inp = synth.make_inputs(cfg)
        sub = inp if nseq is None else synth.sub_batch(inp, list(range(nseq)))
        f = orc.LayerFlags(H=cfg.H, d_qk=cfg.d_qk, d_v=cfg.d_v, norm_len=cfg.norm_len, eps=1e-6)
        t0 = time.perf_counter()
        x = sub.X
        for li in range(nl):
            w = sub.layers[li]
            x, _ = orc.layer_fwd(x, w.W1, w.W2, w.rab_pos, w.rab_time, sub.seq_offsets,
                                 sub.timestamps, sub.num_candidates, f)
        dt = time.perf_counter() - t0
        lf = flops.layer_flops(sub.lengths, sub.num_candidates, cfg.D, cfg.H, cfg.d_qk, cfg.d_v,
                               backward=False)
        out[cfg.name] = {"seconds": round(dt, 3), "gflops": round(nl * lf["total"] / dt / 1e9, 3),
                         "tokens_per_s": round(sub.T * nl / dt, 1), "cores": int(_cores()),
                         "sample": ("whole batch" if nseq is None else f"first {nseq} sequences "
                                    f"({sub.T} tokens)") + f", {nl} layer(s), forward"}
    log(f"cpu oracle per workload: {out}")
    return out


ALL_PARTS = ("train", "recompute", "trainmx", "fwd", "semilocal", "trunc", "cached", "mx",
             "attnmx", "epilogue", "peaks", "cpu")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="only the training step (and the CPU baseline)")
    ap.add_argument("--reps", type=int, default=20,
                    help="timed runs of each forward-only workload")
    ap.add_argument("--only", default="",
                    help="comma list of parts to run (" + ",".join(ALL_PARTS) + "); "
                         "fwd and attnmx may name workloads, e.g. fwd3 or fwd2+fwd5")
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

    parts = set(ALL_PARTS)
    fwd_cfgs = (2, 3, 5)
    attnmx_cfgs = []
    if args.only:
        parts, picked = set(), []
        for tok in args.only.replace("+", ",").split(","):
            tok = tok.strip()
            if tok.startswith("attnmx") and tok != "attnmx":
                attnmx_cfgs.append(int(tok[6:]))
                parts.add("attnmx")
            elif tok.startswith("fwd") and tok != "fwd":
                picked.append(int(tok[3:]))
                parts.add("fwd")
            elif tok:
                parts.add(tok)
        if picked:
            fwd_cfgs = tuple(picked)
    if args.no_extra:
        parts &= {"train", "cpu"}
    if args.no_cpu_baseline:
        parts.discard("cpu")

    line = {"metric": METRIC, "value": None, "unit": "TFLOP/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": None,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded; inputs resident in HBM)"}
    ms = None
    if "train" in parts:
        cfg, inp, stats, kern, lf = bench_train(args, timer)
        ms = stats["ms_mean"]
        tflops = lf["total"] / (ms * 1e-3) / 1e12
        log(f"train step: {ms:.3f} ms (median {stats['ms_median']:.3f}, p10 {stats['ms_p10']:.3f},"
            f" p90 {stats['ms_p90']:.3f}), {tflops:.1f} TFLOP/s")
        roof, table = roofline(cfg, inp, kern, stats["instrumented_steps"],
                               os.path.join(ROOT, "profiles"))
        line.update({
            "value": round(tflops, 3), "ms_per_step": round(ms, 4),
            "config": {"workload": "1 HSTU layer fwd+bwd (training), bf16: batch 8, lengths "
                                   "U[4096,8192], d_model 512, 4 heads x 128, causal",
                       "global_batch": cfg.B, "tokens": inp.T, "seq_len": "U[4096,8192]",
                       "parallelism": "single GPU"},
            "step_ms": stats,
            "tokens_per_s": round(inp.T / (ms * 1e-3), 1),
            "frac_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
            "flops_per_step": {k: v for k, v in lf.items()},
            "kernels": table, "roofline": roof})
    if "recompute" in parts:
        line["train_dq_recomputed"] = bench_recompute(args, timer, ms or float("nan"))
    if "trainmx" in parts:
        line["train_mxfp8"] = bench_train_mx(args, timer, ms or float("nan"))
    if "fwd" in parts:
        line["forward_workloads"] = bench_fwd_configs(timer, fwd_cfgs, reps=args.reps)
    if "semilocal" in parts:
        line["semilocal"] = bench_semilocal(args, timer, ms or float("nan"))
    if "trunc" in parts:
        line["truncation"] = bench_truncation(timer)
    if "cached" in parts:
        line["cached_ranking"] = bench_cached(timer)
    if "mx" in parts:
        line["mxfp8"] = bench_mx(timer)
    if "attnmx" in parts:
        line["attention_mxfp8_scores"] = bench_attn_mx(
            timer, tuple(attnmx_cfgs) if attnmx_cfgs else (3, 5, 4), reps=args.reps)
    if "epilogue" in parts:
        line["ln_gate_epilogue"] = bench_epilogue(timer)
    if "peaks" in parts:
        line["measured_peaks"] = bench_peaks()
    if "cpu" in parts:
        import synth
        cfg4 = synth.get_config(4)
        line["cpu_baseline"] = cpu_baseline(cfg4, synth.make_inputs(cfg4))
        line["cpu_baseline"]["per_workload"] = cpu_baseline_configs()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
