"""Helpers that turn rocprofv3 output into the short text summaries kept under
profiles/, and the plain copy used to calibrate the HBM byte counters.

    # a device-to-device copy of known size, to be run under rocprofv3 --pmc
    python -m linear_attention_sequence_causal_amd.profiling copy --mib 1024

    # kernel-trace statistics -> markdown table
    python -m linear_attention_sequence_causal_amd.profiling stats \
        --csv <dir>/run_kernel_stats.csv --cmd "<command>" --out profiles/<name>.md

    # FETCH_SIZE / WRITE_SIZE passes of a workload and of the copy -> traffic
    python -m linear_attention_sequence_causal_amd.profiling traffic \
        --fetch <dir>/run_counter_collection.csv --write <dir>/run_counter_collection.csv \
        --copy-fetch <csv> --copy-write <csv> --copy-mib 1024 --calls-per-run N \
        --match chunk_ws_kernel --match chunk_loop_kernel --match seg_scan --match plan_kernel \
        --cmd "<commands>" --out profiles/<name>.md --json profiles/<name>.json

    # SQ counter passes -> per-kernel table (mean over each kernel's dispatches)
    python -m linear_attention_sequence_causal_amd.profiling counters \
        --csv <pass1>/run_counter_collection.csv --csv <pass2>/run_counter_collection.csv \
        --match grad_kernel --match dsr_kernel --cmd "<commands>" --out profiles/<name>.md

FETCH_SIZE and WRITE_SIZE are reported by rocprofv3 in KiB per dispatch.
Each is divided by what the same counter reads per byte of the plain copy
(which reads and writes exactly its size once), giving HBM bytes.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))


def source_digest() -> str:
    """SHA-256 over the HIP sources of libgdn: a stored traffic figure holds
    only for the kernels it was measured on."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(PKG, "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()


def _copy(mib: int, reps: int) -> None:
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("copied %d MiB x %d" % (mib, reps), flush=True)


def _read_counters(path: str):
    """{dispatch_id: (kernel_name, {counter: value})}"""
    out = {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            d = out.setdefault(r["Dispatch_Id"], [r["Kernel_Name"], {}])
            d[1][r["Counter_Name"]] = d[1].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def _per_byte(path: str, counter: str, mib: int) -> float:
    """Counter KiB per byte copied, from the largest dispatch of the copy run."""
    disp = _read_counters(path)
    vals = [c[counter] for _, c in disp.values() if counter in c]
    if not vals:
        raise SystemExit("no %s in %s" % (counter, path))
    return max(vals) * 1024.0 / (mib * (1 << 20))


def traffic(args) -> None:
    f_fetch = _per_byte(args.copy_fetch, "FETCH_SIZE", args.copy_mib)
    f_write = _per_byte(args.copy_write, "WRITE_SIZE", args.copy_mib)
    pats = [re.compile(m) for m in args.match]
    rows = {}
    for path, counter, f in ((args.fetch, "FETCH_SIZE", f_fetch), (args.write, "WRITE_SIZE", f_write)):
        per_kernel = defaultdict(lambda: [0, 0.0])
        for name, c in _read_counters(path).values():
            if counter in c and any(p.search(name) for p in pats):
                per_kernel[name][0] += 1
                per_kernel[name][1] += c[counter] * 1024.0 / f
        rows[counter] = per_kernel
    names = sorted(set(rows["FETCH_SIZE"]) | set(rows["WRITE_SIZE"]))
    calls = args.calls_per_run
    lines = ["# HBM traffic: %s" % args.title, "",
             "Commands (each under `timeout -s KILL 60`, from the repository root):", ""]
    lines += ["    %s" % c for c in args.cmd]
    lines += ["",
              "Calibration: a plain %d MiB device copy reads FETCH_SIZE = %.4f KiB and WRITE_SIZE = "
              "%.4f KiB per KiB copied; counters below are divided by these factors." %
              (args.copy_mib, f_fetch, f_write), "",
              "| kernel | dispatches | read MB / call | write MB / call |", "|---|---|---|---|"]
    tot_r = tot_w = 0.0
    for n in names:
        r = rows["FETCH_SIZE"].get(n, [0, 0.0])
        w = rows["WRITE_SIZE"].get(n, [0, 0.0])
        rb, wb = r[1] / calls, w[1] / calls
        tot_r += rb
        tot_w += wb
        short = n if len(n) < 90 else n[:87] + "..."
        lines.append("| `%s` | %d | %.1f | %.1f |" % (short, max(r[0], w[0]), rb / 1e6, wb / 1e6))
    lines += ["| **total per call** | | **%.1f** | **%.1f** |" % (tot_r / 1e6, tot_w / 1e6), ""]
    if args.algorithmic_bytes:
        lines.append("Algorithmic bytes per call: %.1f MB; measured / algorithmic = %.2f." %
                     (args.algorithmic_bytes / 1e6, (tot_r + tot_w) / args.algorithmic_bytes))
    text = "\n".join(lines) + "\n"
    with open(args.out, "w") as fh:
        fh.write(text)
    if args.json:
        with open(args.json, "w") as fh:
            json.dump({"bytes_per_call": tot_r + tot_w, "read_bytes_per_call": tot_r,
                       "write_bytes_per_call": tot_w, "source_sha256": source_digest(),
                       "calibration": {"fetch_per_byte": f_fetch, "write_per_byte": f_write}},
                      fh, indent=1)
    print(text)


def stats(args) -> None:
    rows = []
    with open(args.csv) as fh:
        for r in csv.DictReader(fh):
            rows.append(r)
    lines = ["# Kernel trace: %s" % args.title, "", "Command (from the repository root):", "",
             "    %s" % args.cmd, "", "| kernel | calls | total ms | average us | % |",
             "|---|---|---|---|---|"]
    for r in rows:
        n = r["Name"]
        short = n if len(n) < 100 else n[:97] + "..."
        lines.append("| `%s` | %s | %.3f | %.1f | %.2f |" % (
            short, r["Calls"], float(r["TotalDurationNs"]) / 1e6, float(r["AverageNs"]) / 1e3,
            float(r["Percentage"])))
    text = "\n".join(lines) + "\n"
    with open(args.out, "w") as fh:
        fh.write(text)
    print(text)


def counters(args) -> None:
    """SQ counters of several rocprofv3 --pmc passes: for each kernel whose name
    contains one of the --match strings, the mean over its dispatches of each
    counter (summed over the device as rocprofv3 reports it), and per wave."""
    per = defaultdict(lambda: defaultdict(list))  # kernel -> counter -> values
    for path in args.csv:
        for kname, vals in _read_counters(path).values():
            if not any(m in kname for m in args.match):
                continue
            for cn, v in vals.items():
                per[kname][cn].append(v)
    kernels = sorted(per)
    names = sorted({cn for k in kernels for cn in per[k]})
    short = [k if len(k) < 70 else k[:67] + "..." for k in kernels]
    lines = ["# SQ counters: %s" % args.title, "", "Commands (each under `timeout -s KILL 90`, from "
             "the repository root):", ""] + ["    %s" % c for c in args.cmd] + [
             "", "Values per dispatch (mean over the dispatches of each kernel in a run), summed "
             "over the device as rocprofv3 reports them; the second column of each kernel is per "
             "wave (SQ_WAVES).", "",
             "| counter | " + " | ".join("`%s` | per wave" % k for k in short) + " |",
             "|---|" + "---|---|" * len(kernels)]
    for cn in names:
        cells = []
        for k in kernels:
            v = per[k].get(cn, [])
            m = sum(v) / len(v) if v else float("nan")
            w = per[k].get("SQ_WAVES", [])
            waves = sum(w) / len(w) if w else float("nan")
            cells.append("%.4g | %.4g" % (m, m / waves if waves else float("nan")))
        lines.append("| `%s` | %s |" % (cn, " | ".join(cells)))
    text = "\n".join(lines) + "\n"
    with open(args.out, "w") as fh:
        fh.write(text)
    print(text)


def main(argv=None) -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=1024)
    c.add_argument("--reps", type=int, default=3)
    s = sub.add_parser("stats")
    s.add_argument("--csv", required=True)
    s.add_argument("--cmd", required=True)
    s.add_argument("--title", default="")
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    for k in ("fetch", "write", "copy_fetch", "copy_write", "out"):
        t.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    t.add_argument("--copy-mib", type=int, default=1024)
    t.add_argument("--calls-per-run", type=float, required=True)
    t.add_argument("--match", action="append", required=True)
    t.add_argument("--cmd", action="append", default=[])
    t.add_argument("--title", default="")
    t.add_argument("--json", default=None)
    t.add_argument("--algorithmic-bytes", type=float, default=0.0)
    q = sub.add_parser("counters")
    q.add_argument("--csv", action="append", required=True)
    q.add_argument("--match", action="append", required=True)
    q.add_argument("--cmd", action="append", default=[])
    q.add_argument("--title", default="")
    q.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.cmd_name == "copy":
        _copy(a.mib, a.reps)
    elif a.cmd_name == "stats":
        stats(a)
    elif a.cmd_name == "counters":
        counters(a)
    else:
        traffic(a)


if __name__ == "__main__":
    main(sys.argv[1:])
