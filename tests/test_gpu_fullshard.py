"""Full-shard parity at the workloads' full sizes: every element, against the
oracle, in the device-resident flow bench.py times (one zero_device_begin,
one zero_step_device per step with fresh contributions, one zero_device_end).

The oracle evaluates the shard in chunks of one C_B bucket (oracle.ChunkedRun):
pass 1 per step reduces the step's contributions chunk by chunk (copied from
the GPU), takes the overflow flag, the norm and the next loss scale, and keeps
the reduced gradient; pass 2 evolves each chunk's state through all steps.
Compared bitwise: every step's whole stored gradient, and the final master,
m, v (SGD: the momentum buffer) and 2-byte params of the whole shard; exactly:
the final step count, loss scale and clean-step count and the last step's
flag; the last step's norm to relative 1e-5 (fixed-order fold against the
oracle's order).  Partitioning changes where the states live, not the math of
a step (the blog.vllbc.top ZeRO/DeepSpeed page), so the owner's full shard
must match the unsharded definition element for element.
"""
import dataclasses
import os
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import zero_dp_sharded_amd as zs
from gpu_common import LP_CODE, hp_of, ls_of, oracle_hp, oracle_ls, ulp_dist
from zero_dp_sharded_amd import synth

pytestmark = pytest.mark.gpu

CH = 1 << 26
THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def _host_dtype(t):
    return np.float32 if t.dtype == torch.float32 else np.uint16


def d2h(t, out=None):
    """Copy a 1-D GPU tensor to host storage values (2-byte bit patterns or
    fp32), in pieces, into `out` if given."""
    n = t.numel()
    if out is None:
        out = np.empty(n, _host_dtype(t))
    if t.dtype == torch.float32:
        src, dst = t, torch.from_numpy(out)
    else:
        src, dst = t.view(torch.int16), torch.from_numpy(out.view(np.int16))
    for off in range(0, n, CH):
        dst[off:off + CH].copy_(src[off:off + CH])
    return out


def mismatches(a, b):
    """Elements whose bit patterns differ, a NaN against a NaN not counted."""
    if a.dtype == np.float32:
        bad = a.view(np.uint32) != b.view(np.uint32)
        if bad.any():
            bad &= ~(np.isnan(a) & np.isnan(b))
    else:
        bad = a != b
    return int(np.count_nonzero(bad))


def worst_errors(a, b):
    """(max relative error with FLT_MIN floor, max 2-byte ulp distance) of a
    chunk; fp32 arrays give the first, 2-byte bit patterns the second."""
    if a.dtype == np.float32:
        a64, b64 = a.astype(np.float64), b.astype(np.float64)
        den = np.maximum(np.abs(b64), np.finfo(np.float32).tiny)
        return float(np.max(np.abs(a64 - b64) / den)) if a.size else 0.0
    return int(ulp_dist(a, b).max()) if a.size else 0


def par_mismatches(a, b):
    n = a.size
    parts = [(k * n // THREADS, (k + 1) * n // THREADS) for k in range(THREADS)]
    with ThreadPoolExecutor(THREADS) as ex:
        return sum(ex.map(lambda p: mismatches(a[p[0]:p[1]], b[p[0]:p[1]]), parts))


@pytest.mark.parametrize("name", ["tiny", "gpt2_1.5b", "7.5b_bf16", "13b_inf", "128b",
                                  "c1_7.5b_sgdm", "c2_1.5b_sgd"])
def test_full_shard_device_flow(name, capsys):
    _full_shard(name, capsys)


def test_full_shard_clipped_device_flow(capsys):
    """The GPT-2 workload with global-norm clipping to half its typical norm:
    the coefficient comes from the device's fixed-order fold and the oracle's
    bucket-ordered sum, so the state is held to the fp32 tolerance (max
    relative error 1e-6, 1 ulp on params); the stored gradients stay bitwise."""
    w = synth.WORKLOADS["gpt2_1.5b"]
    typical = w.grad_std / np.sqrt(w.R) * np.sqrt(w.shard)
    _full_shard("gpt2_1.5b", capsys, max_norm=0.5 * typical)


def test_full_shard_pos_scan_device_flow(capsys):
    """P_os on the 128B shard (the owner's slice of an already all-reduced
    gradient): each step the caller fills grad_shard, the device-resident step
    scans it (contribs = NULL) and updates; every element of the final state
    against the oracle's stored-gradient chunked evaluation."""
    _full_shard("128b", capsys, pos=True)


def _full_shard(name, capsys, max_norm=0.0, pos=False):
    w = synth.WORKLOADS[name]
    S, R, cb, lp_t = w.shard, w.R, w.bucket_elems, w.torch_lp
    lp = LP_CODE[w.lp]
    dev = torch.device("cuda", 0)
    t0 = time.time()

    def log(msg):
        with capsys.disabled():
            print(f"[fullshard {name} {time.time() - t0:6.1f}s] {msg}", flush=True)

    log(f"{w.name}: S={S} R={R} C_B={cb} steps={w.steps} max_norm={max_norm:.4g} pos={pos}, "
        f"oracle on {THREADS} threads")
    master, m, v = synth.init_state(w, dev, seed=0)
    m = m if w.has_m else None
    v = v if w.has_v else None
    grad = torch.zeros(S, dtype=lp_t, device=dev)
    param = None if lp_t == torch.float32 else master.to(lp_t)
    bufs = [] if pos else synth.alloc_contribs(w, dev)
    host0 = {k: None if t is None else d2h(t) for k, t in
             (("master", master), ("m", m), ("v", v), ("param", param))}
    hp, ls = hp_of(w), ls_of(w)
    run = oracle.ChunkedRun(lp, S, cb, oracle_hp(hp), oracle_ls(ls), max_norm=max_norm,
                            threads=THREADS)
    grads = [np.empty(S, _host_dtype(grad)) for _ in range(w.steps)]
    gpu_grad = np.empty(S, _host_dtype(grad))
    if w.opt == "sgd":
        h = zs.zero_shard_init_sgd(master, m, grad, param, psi=w.psi, nd=w.nd, rank=w.rank,
                                   bucket_elems=cb, hp=hp, ls=ls)
    else:
        h = zs.zero_shard_init(master, m, v, grad, param, psi=w.psi, nd=w.nd, rank=w.rank,
                               bucket_elems=cb, hp=hp, ls=ls)
    try:
        if max_norm:
            zs.zero_shard_set_clip(h, max_norm)
        zs.zero_device_begin(h)
        infos = []
        for s in range(w.steps):
            # the step's contributions (P_os: the gradient itself) carry the
            # scale the oracle's decisions so far leave (the device decides the
            # same scale on its own)
            if pos:
                synth.fill_contribs(dataclasses.replace(w, R=1), [grad], s, run.scale, seed=0)
                zs.zero_step_device(h, None)
                d2h(grad, grads[s])
                infos.append(run.check_step(lambda off, n: grads[s][off:off + n]))
            else:
                synth.fill_contribs(w, bufs, s, run.scale, seed=0)
                zs.zero_step_device(h, bufs)
                infos.append(run.scan_step(lambda off, n: [d2h(b[off:off + n]) for b in bufs],
                                           grads_out=grads[s]))
            torch.cuda.synchronize()
            bad = par_mismatches(d2h(grad, gpu_grad), grads[s])
            log(f"step {s}: overflow={infos[-1].overflow} t={infos[-1].step_t} "
                f"scale={infos[-1].scale_used} stored-gradient mismatches {bad} of {S}")
            assert bad == 0, (name, s, bad)
        end = zs.zero_device_end(h)
        counters = zs.zero_shard_get_counters(h)
    finally:
        zs.zero_shard_destroy(h)
    last = infos[-1]
    assert counters == (run.t, run.scale, run.good_steps), (counters, run.t, run.scale)
    assert (end.overflow, end.step_t, end.scale_used, end.scale_next) == \
        (last.overflow, last.step_t, last.scale_used, last.scale_next)
    if not last.overflow:
        assert end.grad_norm == pytest.approx(last.grad_norm, rel=1e-5)
    if w.inject_step is not None:
        assert run.steps[w.inject_step].overflow == 1 and run.t == w.steps - 1
    del bufs
    torch.cuda.empty_cache()

    final = {k: None if t is None else d2h(t) for k, t in
             (("master", master), ("m", m), ("v", v), ("param", param))}
    del master, m, v, grad, param
    torch.cuda.empty_cache()
    keys = [k for k in ("master", "m", "v", "param") if final[k] is not None]

    def chunk(c):
        off, n = c
        sl = slice(off, off + n)
        parts = {k: host0[k][sl].copy() for k in keys}
        run.evolve(parts["master"], parts.get("m"), parts.get("v"), parts.get("param"),
                   lambda s: grads[s][sl])
        return {k: (mismatches(parts[k], final[k][sl]), worst_errors(final[k][sl], parts[k]))
                for k in keys}

    with ThreadPoolExecutor(THREADS) as ex:
        results = list(ex.map(chunk, run.chunks()))
    total = {k: sum(r[k][0] for r in results) for k in keys}
    worst = {k: max(r[k][1] for r in results) for k in keys}
    log(f"final state mismatches over {S} elements: {total}; worst errors {worst}")
    if max_norm:
        # the fp32 tolerance: the clipping coefficient comes from two fp64 orders
        for k in keys:
            assert worst[k] <= (1 if k == "param" else 1e-6), (k, worst[k])
    else:
        assert all(v == 0 for v in total.values()), total
