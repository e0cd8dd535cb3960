"""Interleaved A/B of the bucket reduce or the update between builds of the library.

    python -m zero_dp_sharded_amd.ab_reduce WORKLOAD PHASE REPS NAME=LIB [NAME=LIB ...]
    python -m zero_dp_sharded_amd.ab_reduce --update WORKLOAD PHASE REPS NAME=LIB [...]

Loads every listed libzeroshard.so into one process (the binding once per
build), makes one handle per build over the same seeded shard and
contributions (contribution r at (r * PHASE) mod 16 bytes; 16 = aligned), and
times, with HIP events, all C_B bucket reduces of a step or (--update) the
step's update kernel (the synchronous-check flow's zero_adam_step), three
steps per build per round, the builds in alternating order over REPS rounds.
Each step is completed with the check and the update, so the handles stay in
step.  Prints one JSON line: per build the median time and the bandwidth of
the kernel's algorithmic bytes ((R + 1) x element size per shard element for
the reduce, 28 B for the Adam update) as
a percentage of 8 TB/s, with the range over the rounds.  Interleaving in one
process puts every build on the same box, placement and HBM temperature,
which sequential runs do not (on MI355X their spread was several points).

Variant builds come from `python -m zero_dp_sharded_amd.build --variant`.
"""
from __future__ import annotations

import importlib.util
import json
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def load_binding(name: str, lib: str):
    """The ctypes binding bound to `lib`, as a module of its own."""
    os.environ["ZERO_SHARD_LIB"] = lib
    spec = importlib.util.spec_from_file_location("zs_" + name, os.path.join(HERE, "__init__.py"))
    mod = importlib.util.module_from_spec(spec)
    sys.modules["zs_" + name] = mod
    spec.loader.exec_module(mod)
    mod.lib()
    return mod


def main(argv) -> int:
    update = bool(argv) and argv[0] == "--update"
    if update:
        argv = argv[1:]
    if len(argv) < 4:
        print(__doc__, file=sys.stderr)
        return 2
    sys.path.insert(0, ROOT)
    import torch
    from zero_dp_sharded_amd import synth

    wname, phase, reps = argv[0], int(argv[1]), int(argv[2])
    builds = [a.split("=", 1) for a in argv[3:]]
    mods = [(n, load_binding(n, p)) for n, p in builds]
    dev = torch.device("cuda", 0)
    w = synth.WORKLOADS[wname]
    S = w.shard
    master, m, v = synth.init_state(w, dev, 0)
    grad = torch.zeros(S, dtype=w.torch_lp, device=dev)
    param = None if w.lp == "fp32" else torch.zeros(S, dtype=w.torch_lp, device=dev)
    bufs = synth.alloc_contribs(w, dev, phase_step=phase)
    synth.fill_contribs(w, bufs, 0, w.scale, 0)
    handles = []
    for n, zs in mods:
        hp = zs.AdamHParams(lr=w.lr, weight_decay=w.weight_decay)
        ls = zs.LossScaleCfg(init_scale=w.scale, dynamic=0, growth_interval=1000, min_scale=1.0)
        handles.append((n, zs, zs.zero_shard_init(master, m, v, grad, param, psi=S, nd=1, rank=0,
                                                   bucket_elems=w.bucket_elems, hp=hp, ls=ls)))

    def step(zs, h):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if not update:
            e0.record()
        zs.reduce_buckets(h, bufs, S, w.bucket_elems)
        if not update:
            e1.record()
        zs.zero_overflow_check(h)
        if update:
            e0.record()
        zs.zero_adam_step(h)
        if update:
            e1.record()
        return e0, e1

    try:
        for _, zs, h in handles:
            step(zs, h)
            step(zs, h)
        torch.cuda.synchronize()
        times = {n: [] for n, _, _ in handles}
        for rep in range(reps):
            for n, zs, h in (handles if rep % 2 == 0 else handles[::-1]):
                evs = [step(zs, h) for _ in range(3)]
                torch.cuda.synchronize()
                times[n].append(sum(a.elapsed_time(b) for a, b in evs) / 3)
    finally:
        for _, zs, h in handles:
            zs.zero_shard_destroy(h)
    esz = grad.element_size()
    nbytes = S * 28 if update else S * (w.R + 1) * esz
    pct = lambda ms: round(nbytes / (ms * 1e-3) / 8e12 * 100, 2)
    out = {"workload": wname, "kernel": "update" if update else "reduce",
           "contrib_phase_bytes": phase, "rounds": reps}
    for n, x in times.items():
        med = statistics.median(x)
        out[n] = {"median_ms": round(med, 4), "pct_of_8tbs": pct(med),
                  "range_pct": [pct(max(x)), pct(min(x))]}
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
