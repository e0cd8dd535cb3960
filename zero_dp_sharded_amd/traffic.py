"""Summaries of rocprofv3 output for the profiles/ folder.

  stats   : a kernel-trace --stats CSV -> a short text table (calls, average
            and total duration per kernel), headed by the command that made it.
  traffic : two --pmc runs of bench.py (FETCH_SIZE, then WRITE_SIZE), each
            holding the plain copy kernel of known size and the step's kernels
            -> HBM bytes per launch of the update kernel (Adam or SGD) and of
            the reduce, the counters scaled by what they read for the copy
            (bytes moved / counter bytes), as JSON.

The JSON carries a hash of the kernels' code (zero_kernels.hip and the shapes
in zero_kernels.h, comments and whitespace left out); bench.py uses its byte
count only while that code is unchanged.
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

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_SOURCES = [os.path.join(ROOT, "zero_dp_sharded_amd", "csrc", name)
                  for name in ("zero_kernels.hip", "zero_kernels.h")]
COPY_BYTES = 8_000_000_000      # bytes read and bytes written by bench.py's copy


def _one_csv(path_or_dir: str, suffix: str) -> str:
    if os.path.isfile(path_or_dir):
        return path_or_dir
    hits = sorted(glob.glob(os.path.join(path_or_dir, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {path_or_dir}")
    return hits[0]


def counters_per_kernel(path: str, counter: str):
    """{kernel name: [counter value per dispatch]} from a counter-collection CSV."""
    per = defaultdict(float)
    names = {}
    with open(_one_csv(path, "counter_collection.csv"), newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter:
                continue
            key = row.get("Dispatch_Id") or row.get("Correlation_Id")
            per[key] += float(row["Counter_Value"])
            names[key] = row["Kernel_Name"]
    out = defaultdict(list)
    for key, val in per.items():
        out[names[key]].append(val)
    return out


def _match(d, needle):
    hits = [k for k in d if needle in k]
    if not hits:
        raise KeyError(f"no kernel matching {needle!r} among {list(d)[:8]}")
    vals = [v for k in hits for v in d[k]]
    return sum(vals) / len(vals), len(vals)


def code_only(text: str) -> str:
    """C++ source with comments removed and whitespace runs collapsed (the
    kernel sources hold no comment markers inside string literals)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_code_hash(texts=None) -> str:
    """First 16 hex digits of the SHA-256 of the kernels' code, by default of
    the files in KERNEL_SOURCES."""
    if texts is None:
        texts = []
        for path in KERNEL_SOURCES:
            with open(path) as f:
                texts.append(f.read())
    h = hashlib.sha256()
    for t in texts:
        h.update(code_only(t).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def traffic(args) -> int:
    fetch = counters_per_kernel(args.fetch, "FETCH_SIZE")
    write = counters_per_kernel(args.write, "WRITE_SIZE")
    cf, _ = _match(fetch, "hbm_copy_kernel")
    cw, _ = _match(write, "hbm_copy_kernel")
    ffac = COPY_BYTES / (cf * 1024.0)
    wfac = COPY_BYTES / (cw * 1024.0)
    out = {"command_fetch": args.cmd_fetch, "command_write": args.cmd_write,
           "kernel_code_sha256_16": kernel_code_hash(), "elems_per_launch": args.elems,
           "copy_calibration": {"bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES,
                                "fetch_kib": cf, "write_kib": cw,
                                "fetch_factor": ffac, "write_factor": wfac},
           "kernels": {}}
    for label, needle, algo in (("update", args.update_kernel,
                                 args.update_bytes_per_elem * args.elems),
                                ("reduce", args.reduce_kernel, None)):
        try:
            f, nf = _match(fetch, needle)
            w, nw = _match(write, needle)
        except KeyError:
            continue
        b = f * 1024.0 * ffac + w * 1024.0 * wfac
        out["kernels"][label] = {"fetch_kib_per_launch": f, "write_kib_per_launch": w,
                                 "dispatches": [nf, nw], "hbm_bytes_per_launch": b,
                                 "algorithmic_bytes_per_launch": algo}
    out["update_kernel"] = args.update_kernel
    out["hbm_bytes_per_launch"] = out["kernels"].get("update", {}).get("hbm_bytes_per_launch")
    with open(args.out, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))
    return 0


def stats(args) -> int:
    path = _one_csv(args.csv, "kernel_stats.csv")
    rows = []
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            rows.append(row)
    lines = [f"# rocprofv3 kernel-trace statistics", f"# command: {args.cmd}", "#",
             f"# {'calls':>6} {'avg_us':>11} {'total_ms':>10} {'pct':>6}  kernel"]
    for r in rows:
        name = r.get("Name", "")
        if args.filter and not any(k in name for k in args.filter):
            continue
        calls = int(float(r.get("Calls", 0)))
        avg_us = float(r.get("AverageNs", 0)) / 1e3
        tot_ms = float(r.get("TotalDurationNs", 0)) / 1e6
        pct = float(r.get("Percentage", 0))
        short = name if len(name) < 110 else name[:107] + "..."
        lines.append(f"  {calls:>6} {avg_us:>11.2f} {tot_ms:>10.3f} {pct:>6.2f}  {short}")
    text = "\n".join(lines) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    sys.stdout.write(text)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--elems", type=int, required=True,
                   help="shard elements one update launch processes")
    t.add_argument("--update-kernel", default="adam_vec_kernel",
                   help="name fragment of the update kernel (adam_vec_kernel, sgd_vec_kernel)")
    t.add_argument("--update-bytes-per-elem", type=int, default=28,
                   help="algorithmic bytes of the update per element")
    t.add_argument("--reduce-kernel", default="reduce_vec_kernel",
                   help="name fragment of the bucket reduce kernel (reduce_vec_kernel, or "
                        "reduce_shift_kernel for contributions off the output's phase)")
    t.add_argument("--cmd-fetch", required=True)
    t.add_argument("--cmd-write", required=True)
    t.add_argument("--out", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--csv", required=True)
    s.add_argument("--cmd", required=True)
    s.add_argument("--filter", nargs="*")
    s.add_argument("--out")
    args = ap.parse_args()
    return traffic(args) if args.what == "traffic" else stats(args)


if __name__ == "__main__":
    sys.exit(main())
