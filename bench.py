#!/usr/bin/env python3
"""Throughput of the owner-rank ZeRO-DP step on one MI355X.

One step = every C_B bucket reduce of the owner's shard, the overflow check
and the fused Adam + cast, through the C ABI, on the 128B-parameter workload at
Nd = 64: a 2.0e9-element shard, 4 contributions, C_B = 2e8, fp16 storage, loss
scale 4096, AdamW lr 6e-5, wd 0.1.  Four flows run the same step and are all
timed: device-resident steps enqueued back to back (the reported value by
default: the decision and the counters stay on the GPU, no host round trip),
the same steps captured in a HIP graph (up to 10 per graph) and replayed, the
device-gated check (the host waits for a 16-byte result copy per step) and the
synchronous check.
Inputs are seeded synthetic tensors resident in HBM before timing starts; the
same contribution batch feeds every step (each step still reads and writes
every byte).

Prints one JSON line: params/s of the shard (Adam-updated parameters per
second), the step time, the dominant kernel's achieved HBM bandwidth against
the 8 TB/s peak (HIP events on the launch stream), and the CPU oracle timed on
a bounded sample of the same workload.

--workload picks another shape, among them the fp32-storage SGD cases of the
blog.vllbc.top page's extension group C (c1_7.5b_sgdm: SGD with momentum;
c2_1.5b_sgd: plain SGD); the update kernel is then the SGD one.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, AMD public spec
PROFILES = os.path.join(ROOT, "profiles")


def kernel_code_hash() -> str:
    from zero_dp_sharded_amd.traffic import kernel_code_hash as h
    return h()


def traffic_file(workload: str, contrib_phase: int = 16) -> str:
    tag = workload if contrib_phase == 16 else f"{workload}_phase{contrib_phase}"
    return os.path.join(PROFILES, f"traffic_{tag}.json")


def measured_traffic(workload: str, per_launch_elems: int, contrib_phase: int = 16):
    """HBM bytes per update launch from the committed rocprofv3 counter summary
    of this workload (and contribution phase), if it was taken on the current
    kernel source and the in-tree library is the one loaded (not a
    ZERO_SHARD_LIB variant); else None."""
    if os.environ.get("ZERO_SHARD_LIB"):
        return None
    try:
        with open(traffic_file(workload, contrib_phase)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_code_sha256_16") != kernel_code_hash():
        return None
    if t.get("elems_per_launch") != per_launch_elems:
        return None
    return t.get("hbm_bytes_per_launch")


def copy_ceiling(torch, nbytes: int, reps: int):
    """GB/s of the plain nontemporal copy kernel (read + write bytes / time),
    the achievable-bandwidth line beside the roofline peak."""
    import ctypes
    lib_path = os.path.join(ROOT, "zero_dp_sharded_amd", "libhbmcopy.so")
    if not os.path.exists(lib_path):
        raise RuntimeError(f"{lib_path} missing: build with `python -m zero_dp_sharded_amd.build`")
    lib = ctypes.CDLL(lib_path)
    lib.hbm_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.hbm_copy.restype = ctypes.c_int
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    src.normal_()                  # realistic bit patterns: HBM power depends on data
    stream = torch.cuda.current_stream()
    times = []
    for k in range(reps + 2):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        rc = lib.hbm_copy(dst.data_ptr(), src.data_ptr(), nbytes, stream.cuda_stream)
        b.record(stream)
        if rc != 0:
            raise RuntimeError(f"hbm_copy failed with {rc}")
        if k >= 2:
            times.append((a, b))
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in times)[len(times) // 2]
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / (ms * 1e-3) / 1e9


def update_bytes_per_elem(w) -> int:
    """Algorithmic HBM bytes of the update per shard element: the stored
    gradient read, each fp32 state array (master, then m / momentum and v where
    the optimizer keeps them) read and written, and the 2-byte parameter
    written (absent with fp32 storage, where the master is the parameter)."""
    esz = 4 if w.lp == "fp32" else 2
    fp32_arrays = 1 + int(w.has_m) + int(w.has_v)
    return esz + 8 * fp32_arrays + (0 if w.lp == "fp32" else 2)


def host_info() -> dict:
    """CPU model and the cores this process may run on (the oracle uses one)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0))}


def sample_parity(gpu, st, n, counters) -> dict:
    """One step of the benchmarked flow against the oracle's step from the same
    state, counters and contributions, on the first n shard elements: the
    stored gradient and the 2-byte params bitwise, the fp32 arrays bitwise and
    by max relative error (the parity bar is 1e-6)."""
    import numpy as np
    out = {"elements": n, "from_step": int(counters[0]), "loss_scale": counters[1]}
    out["grad_bitwise"] = bool(np.array_equal(gpu["grad"].view(np.uint8), st.grad.view(np.uint8)))
    rel = 0.0
    same = True
    for k, o in (("master", st.master), ("m", st.m), ("v", st.v)):
        g = gpu[k]
        if g is None:
            continue
        same &= bool(np.array_equal(g.view(np.uint32), o.view(np.uint32)))
        o64 = o.astype(np.float64)
        rel = max(rel, float(np.max(np.abs(g.astype(np.float64) - o64)
                                    / np.maximum(np.abs(o64), 1.1754944e-38))))
    out["fp32_state_bitwise"] = same
    out["fp32_state_max_rel"] = rel
    if gpu["param"] is not None:
        out["param_bitwise"] = bool(np.array_equal(gpu["param"], st.param))
    return out


def env_info(torch) -> dict:
    props = torch.cuda.get_device_properties(0)
    return {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None),
            "device": props.name, "arch": getattr(props, "gcnArchName", None)}


def _oracle_setup(w):
    import oracle
    if w.opt == "sgd":
        hp = oracle.SGDHP(lr=w.lr, momentum=w.momentum, weight_decay=w.weight_decay)
    else:
        hp = oracle.AdamHP(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                           weight_decay=w.weight_decay)
    ls = oracle.LossScale(init_scale=w.scale, dynamic=w.dynamic)
    lp = {"fp16": oracle.FP16, "bf16": oracle.BF16, "fp32": oracle.FP32}[w.lp]
    return oracle, hp, ls, lp


def _counters(st, counters):
    """Start an oracle state at the library's step count, loss scale and
    clean-step count (None: the workload's initial values)."""
    if counters is not None:
        st.t, st.scale, st.good_steps = counters
    return st


def cpu_baseline(w, state_host, contribs_host, bucket_elems, counters=None):
    """The oracle's step on the whole sample, on one core: (params/s, seconds,
    the oracle's state after the step)."""
    oracle, hp, ls, lp = _oracle_setup(w)
    master, m, v = state_host
    st = _counters(oracle.new_state(lp, master, m, v, hp, ls), counters)
    t0 = time.perf_counter()
    oracle.step(st, contribs_host, bucket_elems, hp, ls)
    dt = time.perf_counter() - t0
    return master.size / dt, dt, st


def cpu_baseline_threads(w, state_host, contribs_host, bucket_elems, threads, counters=None):
    """The same oracle step with the sample cut into `threads` contiguous
    chunks, one thread each (the oracle's C calls release the GIL).  Each chunk
    is a shard of its own, so the concatenated result equals the one-core
    result whenever no chunk overflows (no workload here plants an overflow in
    the timed step).  Returns (params/s, seconds, concatenated master)."""
    import threading

    import numpy as np
    oracle, hp, ls, lp = _oracle_setup(w)
    master, m, v = state_host
    n = master.size
    bounds = [n * k // threads for k in range(threads + 1)]
    parts = [slice(bounds[k], bounds[k + 1]) for k in range(threads) if bounds[k + 1] > bounds[k]]
    states = [_counters(oracle.new_state(lp, master[sl], None if m is None else m[sl],
                                         None if v is None else v[sl], hp, ls), counters)
              for sl in parts]
    chunks = [[c[sl] for c in contribs_host] for sl in parts]
    gate = threading.Barrier(len(parts) + 1)
    errors = []

    def work(k):
        gate.wait()
        try:
            oracle.step(states[k], chunks[k], bucket_elems, hp, ls)
        except Exception as e:   # reported after the join
            errors.append(e)

    pool = [threading.Thread(target=work, args=(k,)) for k in range(len(parts))]
    for t in pool:
        t.start()
    gate.wait()
    t0 = time.perf_counter()
    for t in pool:
        t.join()
    dt = time.perf_counter() - t0
    if errors:
        raise errors[0]
    return n / dt, dt, np.concatenate([s.master for s in states])


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="128b")
    ap.add_argument("--cpu-sample", type=int, default=1 << 29,
                    help="shard elements the CPU oracle runs on (0 = skip)")
    ap.add_argument("--only", choices=["copy"], default=None,
                    help="run only the plain copy kernel (byte-counter calibration)")
    ap.add_argument("--flow", choices=["gated", "sync", "device", "graph"], default="device",
                    help="flow whose step time is the reported value: device-gated check "
                         "(gated), synchronous check (sync), device-resident steps enqueued "
                         "back to back (device), or device-resident steps captured in a HIP "
                         "graph (up to 10 per graph) and replayed (graph); all four are timed")
    ap.add_argument("--contrib-phase", type=int, choices=[16, 8, 4, 2], default=16,
                    help="contribution r starts (r * P) mod 16 bytes past a 16-byte boundary "
                         "(16: every contribution aligned; 8, 4, 2: the phases of "
                         "contributions carved back to back from one buffer, which the "
                         "reduce reads at their own phase)")
    ap.add_argument("--mode", choices=["pos_g", "pos"], default="pos_g",
                    help="pos_g: gradient partitioning (bucket reduces + check + Adam); "
                         "pos: optimizer-state partitioning only (the owner's slice of an "
                         "already all-reduced gradient: scan check + Adam)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the owner-rank step on one GPU only; "
              "multi-GPU runs are not supported (use --gpus 1).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import zero_dp_sharded_amd as zs
    from zero_dp_sharded_amd import synth

    zs.lib()  # fails loudly when the HIP library is not built
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    copy_bytes = 8_000_000_000
    if args.only == "copy":
        copy_gbs = copy_ceiling(torch, copy_bytes, reps=3)
        print(f"[bench] plain copy of {copy_bytes} bytes: {copy_gbs:.0f} GB/s", file=sys.stderr,
              flush=True)
        return 0
    w = synth.WORKLOADS[args.workload]
    S, R, cb = w.shard, w.R, w.bucket_elems
    lp_t = w.torch_lp
    print(f"[bench] workload {w.name}: S={S} R={R} C_B={cb}", file=sys.stderr, flush=True)

    master, m, v = synth.init_state(w, dev, seed=0)
    m = m if w.has_m else None
    v = v if w.has_v else None
    grad = torch.zeros(S, dtype=lp_t, device=dev)
    param = None if w.lp == "fp32" else master.to(lp_t)
    esz = grad.element_size()
    sgd = w.opt == "sgd"
    if args.mode == "pos":
        # the caller's slice of the all-reduced gradient: one seeded draw
        bufs = []
        synth.fill_contribs(dataclasses.replace(w, R=1), [grad], 0, w.scale, seed=0)
    else:
        bufs = synth.alloc_contribs(w, dev, phase_step=args.contrib_phase)
        synth.fill_contribs(w, bufs, 0, w.scale, seed=0)
    torch.cuda.synchronize()
    print("[bench] inputs resident", file=sys.stderr, flush=True)

    ls = zs.LossScaleCfg(init_scale=w.scale, dynamic=w.dynamic)
    if sgd:
        hp = zs.SGDHParams(lr=w.lr, momentum=w.momentum, weight_decay=w.weight_decay)
        h = zs.zero_shard_init_sgd(master, m, grad, param, psi=w.psi, nd=w.nd, rank=w.rank,
                                   bucket_elems=cb, hp=hp, ls=ls)
        update_gated, update_sync = zs.zero_sgd_step_gated, zs.zero_sgd_step
    else:
        hp = zs.AdamHParams(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                            weight_decay=w.weight_decay)
        h = zs.zero_shard_init(master, m, v, grad, param, psi=w.psi, nd=w.nd, rank=w.rank,
                               bucket_elems=cb, hp=hp, ls=ls)
        update_gated, update_sync = zs.zero_adam_step_gated, zs.zero_adam_step
    stream = torch.cuda.current_stream()
    ptrs = [b.data_ptr() for b in bufs]
    offs = [(off, min(cb, S - off)) for off in range(0, S, cb)]

    def step(ev=None, flow="gated"):
        # four timing events per step: around all bucket reduces and around
        # the Adam enqueue (more events between kernels cost step time)
        if ev is not None:
            ev["r"][0].record(stream)
        if args.mode == "pos_g":
            for off, ln in offs:
                zs.zero_bucket_reduce(h, [p + esz * off for p in ptrs], off, ln, stream)
        if ev is not None:
            ev["r"][1].record(stream)
        if flow == "gated":
            # check, result copy and device-gated Adam in one enqueue; the
            # host waits only for the result copy
            if ev is not None:
                ev["a"][0].record(stream)
            update_gated(h, None, stream)
            if ev is not None:
                ev["a"][1].record(stream)
            return zs.zero_step_resolve(h)
        info = zs.zero_overflow_check(h, stream)
        if ev is not None:
            ev["a"][0].record(stream)
        update_sync(h, None, stream)
        if ev is not None:
            ev["a"][1].record(stream)
        return info

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup} done", file=sys.stderr, flush=True)

    mk = lambda: torch.cuda.Event(enable_timing=True)

    def timed(flow):
        evs = [{"r": (mk(), mk()), "a": (mk(), mk())} for _ in range(args.steps)]
        skipped = 0
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            info = step(evs[k], flow)
            skipped += info.overflow
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ms = (t1 - t0) * 1e3 / args.steps
        adam = [e["a"][0].elapsed_time(e["a"][1]) for e in evs]
        red = [e["r"][0].elapsed_time(e["r"][1]) for e in evs]
        return ms, sum(adam) / len(adam), sum(red) / len(red), skipped

    ms_step, adam_avg, red_avg, skipped = timed("gated")
    print(f"[bench] timed {args.steps} gated steps: {ms_step:.3f} ms/step, adam (with check "
          f"fold + copy) {adam_avg:.3f} ms, reduce {red_avg:.3f} ms, skipped {skipped}",
          file=sys.stderr, flush=True)
    ms_sync, adam_sync, red_sync, skipped_sync = timed("sync")
    print(f"[bench] timed {args.steps} synchronous-check steps: {ms_sync:.3f} ms/step, adam "
          f"{adam_sync:.3f} ms, reduce {red_sync:.3f} ms", file=sys.stderr, flush=True)

    def timed_device(use_graph):
        # device-resident flow: no host synchronisation inside the timed steps.
        # The graph holds g consecutive steps, g the largest divisor of K up to
        # 10, and is replayed K / g times: exactly K steps, with the graph
        # launch cost spread over g of them as a training loop would.
        contrib = bufs if args.mode == "pos_g" else None
        zs.zero_device_begin(h, stream)
        graph = None
        per_run = 1
        if use_graph:
            per_run = max(d for d in range(1, min(10, args.steps) + 1) if args.steps % d == 0)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for _ in range(per_run):
                    zs.zero_step_device(h, contrib)     # the capture stream is current here
            run = graph.replay
        else:
            run = lambda: zs.zero_step_device(h, contrib, stream)
        for _ in range(max(1, args.warmup // per_run)):
            run()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps // per_run):
            run()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps
        zs.zero_device_end(h, stream)
        del graph
        return ms

    ms_device = timed_device(False)
    ms_graph = timed_device(True)
    print(f"[bench] timed {args.steps} device-resident steps: {ms_device:.3f} ms/step; "
          f"graph replays: {ms_graph:.3f} ms/step", file=sys.stderr, flush=True)
    by_flow = {"gated": ms_step, "sync": ms_sync, "device": ms_device, "graph": ms_graph}
    ms_step = by_flow[args.flow]

    # The copy ceiling runs after the step timing: allocating and freeing its
    # 16 GB before the shard arrays were allocated slowed the Adam pass by ~5%
    # on MI355X (placement of the five streamed arrays).
    copy_gbs = copy_ceiling(torch, copy_bytes, reps=10)
    print(f"[bench] plain copy of {copy_bytes} bytes: {copy_gbs:.0f} GB/s", file=sys.stderr,
          flush=True)

    adam_bytes = update_bytes_per_elem(w) * S
    if args.mode == "pos_g":
        reduce_bytes = (R + 1) * esz * S       # R contributions read, the stored gradient written
    else:
        reduce_bytes = esz * S                 # the check's scan of the stored gradient
    # the update kernel alone: the synchronous-check flow brackets only its enqueue
    achieved = adam_bytes / (adam_sync * 1e-3) / 1e9
    step_bytes = adam_bytes + reduce_bytes
    traffic = measured_traffic(args.workload, S, args.contrib_phase)

    cpu = None
    parity = None
    if args.cpu_sample > 0 and args.mode == "pos_g":
        n = min(args.cpu_sample, S)
        host = lambda t: None if t is None else t[:n].cpu().numpy()
        bits = lambda t: (t[:n].cpu().numpy() if t.dtype == torch.float32
                          else t[:n].view(torch.int16).cpu().numpy().view(np.uint16))
        state_host = tuple(host(t) for t in (master, m, v))
        contribs_host = [bits(b) for b in bufs]
        counters = zs.zero_shard_get_counters(h)
        # one more step of the reported (device-resident) flow on the same
        # inputs: its first n elements are checked against the oracle's step
        zs.zero_device_begin(h, stream)
        zs.zero_step_device(h, bufs, stream)
        zs.zero_device_end(h, stream)
        gpu_after = {"grad": bits(grad), "master": host(master), "m": host(m), "v": host(v),
                     "param": None if param is None else bits(param)}
        # the one-core leg runs pinned to one core (this thread only; restored
        # before the all-cores leg starts its threads)
        affinity = os.sched_getaffinity(0)
        pinned = min(affinity)
        os.sched_setaffinity(0, {pinned})
        try:
            rate, dt, st1 = cpu_baseline(w, state_host, contribs_host, cb, counters)
        finally:
            os.sched_setaffinity(0, affinity)
        parity = sample_parity(gpu_after, st1, n, counters)
        del gpu_after
        print(f"[bench] parity of one more step on {n} elements: {parity}", file=sys.stderr,
              flush=True)
        threads = min(len(os.sched_getaffinity(0)), 16)
        prate, pdt, pmaster = cpu_baseline_threads(w, state_host, contribs_host, cb, threads,
                                                   counters)
        cpu = {"value": rate, "unit": "params/s", "cores": 1, "kind": "oracle",
               "sample": f"one full step (reduce of {R} contributions, flag/norm, "
                         f"{'SGD' if sgd else 'Adam'}) on the "
                         f"first {n} elements of the same shard; {dt:.1f} s single-threaded, "
                         f"pinned to core {pinned}",
               "host": host_info(),
               "all_cores": {"value": prate, "unit": "params/s", "cores": threads,
                             "seconds": pdt,
                             "equals_one_core": bool(np.array_equal(
                                 pmaster.view(np.uint32), st1.master.view(np.uint32))),
                             "how": "the same sample in contiguous chunks, one thread per "
                                    "chunk, each an oracle step of its own"}}
        del st1, pmaster
        del state_host, contribs_host
    zs.zero_shard_destroy(h)

    out = {
        "metric": ("SGD" if sgd else "Adam") + "-updated params/sec per rank shard + achieved "
                  "HBM GB/s vs MI355X peak",
        "value": S / (ms_step * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; same contribution batch every step)",
        "config": {"workload": w.name + (" -- P_os: scan check + Adam on the owner's slice of an "
                                          "all-reduced gradient" if args.mode == "pos" else "")
                               + (f", contribution r at (r*{args.contrib_phase}) mod 16 B"
                                  if args.contrib_phase != 16 and args.mode == "pos_g" else ""),
                   "mode": args.mode, "psi": w.psi, "nd": w.nd, "rank": w.rank,
                   "shard_elems": S, "contributions": R if args.mode == "pos_g" else 0,
                   "contrib_phase_bytes": args.contrib_phase,
                   "bucket_elems": cb,
                   "storage": w.lp, "optimizer": (f"sgd(momentum={w.momentum})" if sgd
                                                   else "adamw"),
                   "loss_scale": w.scale, "lr": w.lr, "weight_decay": w.weight_decay},
        "step_hbm_gbs": step_bytes / (ms_step * 1e-3) / 1e9,
        "copy_ceiling_gbs": copy_gbs,
        "step_frac_of_peak": step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        # the step against the plain copy measured on the same box in the same
        # run: separates the machine's HBM from the kernels' share of it
        "step_frac_of_copy_ceiling": step_bytes / (ms_step * 1e-3) / 1e9 / copy_gbs,
        "kernels_ms": {"update_gated_flow_incl_check": adam_avg, "update_sync_flow": adam_sync,
                       "reduce_all_buckets": red_avg,
                       "reduce_gbs": (reduce_bytes / (red_avg * 1e-3) / 1e9
                                      if args.mode == "pos_g" else None)},
        "flow": args.flow,
        "ms_per_step_by_flow": by_flow,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": (f"sgd_vec_kernel<{w.lp}, momentum={int(w.has_m)}>" if sgd
                                else f"adam_vec_kernel<{w.lp}, decoupled wd>"),
                     "algorithmic_bytes_per_launch": adam_bytes,
                     "launch_ms": adam_sync,
                     "timing": "HIP events around the update enqueue of the synchronous-check "
                               "flow, on the launch stream (the update kernel alone)"},
        "cpu_baseline": cpu,
        "parity_sample": parity,
        "env": env_info(torch),
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
