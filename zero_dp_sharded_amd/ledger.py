"""Per-rank memory ledger from the command line (no GPU needed).

    python -m zero_dp_sharded_amd.ledger PSI ND [--contrib R] [--bucket C_B]
                                         [--storage fp16|bf16|fp32] [--k K] [--hbm-gb 288]

Prints, from the library's zero_state_bytes_ex (host arithmetic only):
  - the analytic per-rank model-state bytes of ZeRO stages 0-3 for
    mixed-precision training with parameter width b and optimizer multiplier
    K ((2b+K) Psi; the blog.vllbc.top ZeRO/DeepSpeed page: stage formulas and
    Table 1), with their parameter / gradient / optimizer components and the
    per-step communication volume;
  - the device memory a handle of this library holds for one rank's shard
    (fp32 master and optimizer arrays, stored gradient, 2-byte parameter) and
    the staging of one bucket of R contributions, against the HBM of one
    MI355X (288 GB).
For example, 7.5e9 parameters at Nd = 64 give stages 1-3 of 31.4, 16.6 and
1.88 GB, and 128e9 at Nd = 64 give 536, 284 and 32 GB (the pages' Table 1).
"""
from __future__ import annotations

import argparse
import sys

from . import (ZERO_BF16, ZERO_FP16, ZERO_FP32, zero_state_bytes_ex)

STORAGE = {"fp16": ZERO_FP16, "bf16": ZERO_BF16, "fp32": ZERO_FP32}


def gb(x: float) -> str:
    """Decimal gigabytes, three significant digits below 100 GB."""
    v = x / 1e9
    return f"{v:,.0f}" if v >= 100 else f"{v:.3g}"


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(prog="python -m zero_dp_sharded_amd.ledger",
                                 description="per-rank ZeRO memory ledger")
    ap.add_argument("psi", type=float, help="model parameters (e.g. 7.5e9)")
    ap.add_argument("nd", type=int, help="data-parallel degree")
    ap.add_argument("--contrib", type=int, default=None,
                    help="contributions per bucket (default: Nd, at most 64)")
    ap.add_argument("--bucket", type=float, default=5e7, help="C_B elements (default 5e7)")
    ap.add_argument("--storage", choices=sorted(STORAGE), default="fp16")
    ap.add_argument("--k", type=int, default=12,
                    help="optimizer bytes per parameter: 12 mixed-precision Adam (default), "
                         "8 fp32 Adam, 4 SGD with momentum, 0 SGD")
    ap.add_argument("--hbm-gb", type=float, default=288.0, help="device memory (GB)")
    a = ap.parse_args(argv)
    psi, nd = int(round(a.psi)), a.nd
    r = a.contrib if a.contrib is not None else min(nd, 64)
    b = 4 if a.storage == "fp32" else 2
    led = zero_state_bytes_ex(psi, nd, r, int(round(a.bucket)), STORAGE[a.storage], b, a.k)
    print(f"Psi = {psi:,}, Nd = {nd}, b = {b}, K = {a.k}")
    print("stage  per-rank model states   params    grads  optimizer  comm/step (GB)")
    for s in range(4):
        print(f"{s:>5}  {gb(led['per_rank_stage'][s]):>20} GB  {gb(led['comp_params'][s]):>7}  "
              f"{gb(led['comp_grads'][s]):>7}  {gb(led['comp_optim'][s]):>9}  "
              f"{gb(led['comm_bytes_stage'][s]):>9}")
    print(f"stage 1 with the step-end parameter gather: {gb(led['comm_bytes_stage1_with_gather'])} GB"
          " per step")
    S = led["shard_elems"]
    total = led["bytes_shard_total"] + led["bytes_staging"]
    print(f"this library's shard on one rank: S = {S:,} elements")
    for k in ("master", "m", "v", "grad", "param"):
        print(f"  {k:<7}{gb(led['bytes_' + k]):>10} GB")
    print(f"  shard  {gb(led['bytes_shard_total']):>10} GB; one bucket of {r} contributions "
          f"{gb(led['bytes_staging'])} GB")
    fits = total <= a.hbm_gb * 1e9
    print(f"  {gb(total)} GB of {a.hbm_gb:g} GB HBM: {'fits' if fits else 'does not fit'}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
