"""HBM traffic of a kernel from rocprofv3 counters, calibrated on a plain copy.

Two sub-commands, each meant to run under `rocprofv3 --pmc <COUNTER>`:

  python -m hstu_sequential_transduction_amd.traffic copy [--mib N]
      device-to-device copy of N MiB (torch's copy of two contiguous buffers,
      the runtime's copy kernel), three times: the reference of known size.

and two that read counter CSVs afterwards (no GPU needed):

  python -m hstu_sequential_transduction_amd.traffic reduce \
      --fetch-run DIR --write-run DIR --copy-fetch DIR --copy-write DIR \
      --kernel attn_bwd_dkdv --workload c4-bf16-train --out profiles/

FETCH_SIZE and WRITE_SIZE are read in KiB per dispatch.  Each is scaled by the
ratio of the bytes the copy moves (read and written, N MiB each) to what the
same counter reports for it, and the per-launch traffic of the kernel is the
mean over its dispatches of scaled FETCH + scaled WRITE.

  python -m hstu_sequential_transduction_amd.traffic counters \
      --run DIR [--run DIR ...] --kernel k_attn_fwd_bf16 [--out FILE.json]

prints, for every kernel whose name contains the fragment, the number of
dispatches and the mean per dispatch of every counter found in the runs
(one run per rocprofv3 --pmc pass).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")

# kernel tag -> (symbol fragments in the trace, sources whose hash keys the
# record).  A tag's launch may run several kernels (dQ from a kept dS runs
# the product kernel, then the recomputing kernel, which exits at once when
# the kept dS was used): the first fragment names the kernel launched exactly
# once per tag launch, and the traffic of one launch is the sum over all the
# fragments' dispatches divided by the number of those launches.
_ATTN_SRC = ["attn_bwd.hip", "common.h", "bias.h", "lds.h"]
KERNELS = {
    "attn_fwd": (["k_attn_fwd_bf16"], ["attn_fwd.hip", "common.h", "bias.h", "lds.h"]),
    "attn_bwd_dkdv": (["k_attn_bwd_dkdv"], _ATTN_SRC),
    "attn_bwd_dq": (["k_attn_bwd_dq<", "k_attn_bwd_dq_ds"], _ATTN_SRC),
    "ln_gate_fwd": (["k_ln_gate_fwd"], ["ln_gate.hip", "common.h"]),
    "ln_gate_bwd": (["k_ln_gate_bwd"], ["ln_gate.hip", "common.h"]),
}
GEMM_SOURCES = ["gemm.hip", "common.h", "lds.h"]
COPY_SYMBOL = "copyBuffer"


def source_hash(kernel: str) -> str:
    files = KERNELS[kernel][1] if kernel in KERNELS else GEMM_SOURCES
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _rows(run_dir: str):
    paths = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not paths:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    for p in paths:
        with open(p) as fh:
            yield from csv.DictReader(fh)


def per_dispatch(run_dir: str, counter: str, symbol: str):
    """Counter value (summed over its instances) per dispatch of kernels matching symbol."""
    acc = {}
    for r in _rows(run_dir):
        if r["Counter_Name"] != counter or symbol not in r["Kernel_Name"]:
            continue
        key = (r["Dispatch_Id"], r["Kernel_Name"])
        acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
    return list(acc.values())


def cmd_counters(args) -> int:
    """Mean per dispatch of every counter, per kernel name matching args.kernel."""
    per = {}   # kernel -> counter -> {dispatch: value}
    for run in args.run:
        for r in _rows(run):
            if args.kernel not in r["Kernel_Name"]:
                continue
            d = per.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], {})
            key = (run, r["Dispatch_Id"])
            d[key] = d.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for k, cs in sorted(per.items()):
        n = max(len(v) for v in cs.values())
        out[k] = {"dispatches": n,
                  "mean_per_dispatch": {c: sum(v.values()) / len(v) for c, v in sorted(cs.items())}}
    text = json.dumps(out, indent=1)
    if args.out:
        with open(args.out, "w") as fh:
            fh.write(text + "\n")
    print(text)
    return 0 if out else 1


def cmd_copy(args) -> int:
    import torch
    n = args.mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "repeats": 3}))
    return 0


def cmd_reduce(args) -> int:
    syms = KERNELS.get(args.kernel, ([args.kernel],))[0]
    copy_bytes = args.mib << 20
    cf = per_dispatch(args.copy_fetch, "FETCH_SIZE", COPY_SYMBOL)
    cw = per_dispatch(args.copy_write, "WRITE_SIZE", COPY_SYMBOL)
    if not cf or not cw:
        print("no copy dispatches found", file=sys.stderr)
        return 1
    # the largest dispatches are the N MiB copies (small ones are the runtime's own)
    f_copy = sorted(cf)[-1] * 1024.0
    w_copy = sorted(cw)[-1] * 1024.0
    f_scale, w_scale = copy_bytes / f_copy, copy_bytes / w_copy
    kf = [per_dispatch(args.fetch_run, "FETCH_SIZE", s) for s in syms]
    kw = [per_dispatch(args.write_run, "WRITE_SIZE", s) for s in syms]
    if not kf[0] or not kw[0]:
        print(f"no dispatches of {syms[0]} found", file=sys.stderr)
        return 1
    nf, nw = len(kf[0]), len(kw[0])
    kf_sum, kw_sum = sum(map(sum, kf)), sum(map(sum, kw))
    fetch = kf_sum / nf * 1024.0 * f_scale
    write = kw_sum / nw * 1024.0 * w_scale
    rec = {
        "kernel": args.kernel, "workload": args.workload, "source_hash": source_hash(args.kernel),
        "bytes_per_launch": round(fetch + write), "fetch_bytes": round(fetch),
        "write_bytes": round(write), "dispatches": [nf, nw],
        "kernels": {s: [len(a), len(b)] for s, a, b in zip(syms, kf, kw)},
        "copy_scale": {"fetch": round(f_scale, 4), "write": round(w_scale, 4),
                       "copy_bytes": copy_bytes},
        "counters_kib_per_launch": {"FETCH_SIZE": round(kf_sum / nf, 1),
                                    "WRITE_SIZE": round(kw_sum / nw, 1)},
        "command": args.command,
    }
    os.makedirs(args.out, exist_ok=True)
    path = os.path.join(args.out, f"{args.kernel}_traffic.json")
    with open(path, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=512)
    r = sub.add_parser("reduce")
    for k in ("fetch-run", "write-run", "copy-fetch", "copy-write"):
        r.add_argument("--" + k, required=True)
    r.add_argument("--kernel", required=True)
    r.add_argument("--workload", required=True)
    r.add_argument("--mib", type=int, default=512)
    r.add_argument("--out", default=os.path.join(os.path.dirname(HERE), "profiles"))
    r.add_argument("--command", default="")
    k = sub.add_parser("counters")
    k.add_argument("--run", action="append", required=True)
    k.add_argument("--kernel", required=True)
    k.add_argument("--out", default="")
    args = ap.parse_args(argv)
    if args.cmd == "copy":
        return cmd_copy(args)
    return cmd_counters(args) if args.cmd == "counters" else cmd_reduce(args)


if __name__ == "__main__":
    sys.exit(main())
