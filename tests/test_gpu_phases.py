"""Bucket reduces whose contributions do not share one 16-byte address phase.

When every contribution and the output share their address phase modulo 16
bytes the reduce moves whole aligned 16-byte runs; otherwise the shift kernel
keeps the output runs aligned and cuts each contribution's runs out of the two
aligned 16-byte words around them (reduce_shift_kernel), with a scalar head
long enough to cover the largest phase and one whole run kept after the body.
Each case places the R contributions at their own byte offsets from a 16-byte
boundary (as a caller gets when it carves them back to back from one buffer of
a shard whose size is not a multiple of 8), runs several steps in the
synchronous, gated and device-resident flows, and compares every step's flag,
norm and stored gradient and the final state with the oracle, bitwise.
Buckets of an odd size start at a different phase each, so the layout changes
from bucket to bucket; one shard is above the small-shard limit (nontemporal
kernels with one and three runs per lane), one small enough for the
device-resident step to fold its partials inline, and a sweep of tiny buckets
covers the bodies of zero and one run."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import zero_dp_sharded_amd as zs
from gpu_common import (LP_CODE, GpuRun, compare, f32, hp_of, log, ls_of, oracle_hp, oracle_ls,
                        stored, u16)
from zero_dp_sharded_amd import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)
STEPS = 3

# byte offsets of the contributions from a 16-byte boundary, and of grad_shard
PHASES = {
    "8-byte phases": ([0, 8, 8, 0], 0),
    "4-byte phases": ([4, 8, 12, 0, 4], 8),
    "2-byte phases": ([0, 2, 6], 0),
    # output at 6 mod 16: head 5, then a phase of 6 elements moves it to 13
    "2-byte phases, output off": ([14, 2, 6, 0], 6),
    # nine contributions: two full batches of four and one more (a count the
    # kernel is not compiled for)
    "nine contributions": ([2, 4, 6, 8, 10, 12, 14, 0, 2], 4),
    # sixteen: the compiled-in count, four batches
    "sixteen contributions": ([(2 * r) % 16 for r in range(16)], 10),
    # the most the library takes: sixteen batches in the kernel's run-time loop
    "sixty-four contributions": ([(2 * (5 * r + r // 8)) % 16 for r in range(64)], 12),
}


def _make(lp, S, R, offs, goff, seed):
    w = dataclasses.replace(synth.WORKLOADS["gpt2_1.5b"], lp=lp, R=R, dynamic=1,
                            scale=1024.0 if lp != "fp32" else 1.0, steps=STEPS)
    t = w.torch_lp
    esz = torch.empty(0, dtype=t).element_size()

    def at(byte_off, n):
        assert byte_off % esz == 0
        base = torch.empty(n + 16, dtype=t, device=DEV)
        assert base.data_ptr() % 16 == 0
        k = byte_off // esz
        return base[k:k + n]

    master0, m0, v0 = synth.init_state(w, DEV, seed, elems=S)
    st = {"master": master0.clone(), "m": m0.clone(), "v": v0.clone(),
          "grad": at(goff, S), "param": None if lp == "fp32" else master0.to(t)}
    st["grad"].zero_()
    bufs = [at(o, S) for o in offs]
    return w, st, bufs, (f32(master0), f32(m0), f32(v0))


def _run(lp, S, cb, offs, goff, flow, seed=0):
    w, st, bufs, host0 = _make(lp, S, len(offs), offs, goff, seed)
    h = zs.zero_shard_init(st["master"], st["m"], st["v"], st["grad"], st["param"], psi=S, nd=1,
                           rank=0, bucket_elems=cb, hp=hp_of(w), ls=ls_of(w))
    infos, kept = [], []
    scale = w.scale
    try:
        for s in range(STEPS):
            synth.fill_contribs(w, bufs, s, scale, seed)
            kept.append([stored(b) for b in bufs])
            if flow == "device":
                zs.zero_device_begin(h)
                zs.zero_step_device(h, bufs)
                info = zs.zero_device_end(h)
            else:
                zs.reduce_buckets(h, bufs, S, cb)
                if flow == "gated":
                    zs.zero_adam_step_gated(h)
                    info = zs.zero_step_resolve(h)
                else:
                    zs.zero_overflow_check(h)
                    info = zs.zero_adam_step(h)
            infos.append(info)
            scale = info.scale_next
        torch.cuda.synchronize()
    finally:
        zs.zero_shard_destroy(h)
    ohp, ols = oracle_hp(hp_of(w)), oracle_ls(ls_of(w))
    ost = oracle.new_state(LP_CODE[lp], *host0, ohp, ols)
    oinfos = [oracle.step(ost, cs, cb, ohp, ols) for cs in kept]
    g = GpuRun(infos, kept, *host0, f32(st["master"]), f32(st["m"]), f32(st["v"]),
               stored(st["grad"]), None if st["param"] is None else u16(st["param"]))
    tag = f"{lp} S={S} cb={cb} offs={offs} grad+{goff} {flow}"
    log(f"[phases] {tag}")
    assert compare(w, g, ost, oinfos, tag)["bitwise"], tag


@pytest.mark.parametrize("phase", list(PHASES))
@pytest.mark.parametrize("lp", ["fp16", "bf16", "fp32"])
@pytest.mark.parametrize("flow", ["sync", "gated", "device"])
def test_contributions_at_distinct_phases(phase, lp, flow):
    offs, goff = PHASES[phase]
    if lp == "fp32":
        offs = [o - o % 4 for o in offs]           # fp32 arrays sit on 4-byte boundaries
        goff -= goff % 4
    _run(lp, 50_021, 10_007, offs, goff, flow)


def _fp32_offsets(offs, goff):
    return [o - o % 4 for o in offs], goff - goff % 4


@pytest.mark.parametrize("lp", ["fp16", "fp32"])
def test_shift_above_the_small_shard_limit(lp):
    """Nontemporal shift kernels: a shard past 8,388,608 elements, buckets of
    an odd size, 8-, 4- and 2-byte phase sets, with one run per lane (8 or
    more contributions) and three (fewer)."""
    for offs, goff in (([0, 8, 0, 8, 8, 0, 0, 8], 0), ([4, 0, 12], 8), ([0, 8, 8, 0], 8),
                       ([12, 4, 4, 8, 0, 4, 8, 12, 0], 0), ([2, 0, 14, 6], 10),
                       ([6, 2, 0, 14, 12, 10, 8, 4], 2), ([(6 * r) % 16 for r in range(16)], 14)):
        if lp == "fp32":
            offs, goff = _fp32_offsets(offs, goff)
        _run(lp, 8_400_017, 2_100_001, offs, goff, "device")


def test_shift_with_the_inline_fold():
    """A one-bucket device-resident step small enough to fold its partials in
    the update (aligned update arrays), its reduce in the shift kernel."""
    _run("fp16", 65_536, 65_536, [0, 8, 8], 0, "device")
    _run("bf16", 131_072, 131_072, [8, 0], 8, "device")
    _run("fp16", 65_536, 65_536, [2, 14, 0, 6], 0, "device")


@pytest.mark.parametrize("lp", ["bf16", "fp32"])
def test_shift_tiny_buckets(lp):
    """Buckets of 1 to 41 elements at 2-byte (fp32: 4-byte) phases: vector
    bodies of zero, one and a few runs after heads of up to 15 elements, and
    the head clipped to a bucket shorter than it."""
    offs, goff = ([2, 12, 6], 6) if lp != "fp32" else ([4, 12, 8], 4)
    for cb in (1, 2, 3, 7, 13, 16, 21, 24, 29, 31, 32, 37, 41):
        _run(lp, 97, cb, offs, goff, "sync")
