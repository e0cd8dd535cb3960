"""Stream discipline: every call enqueues on the stream it is given.

Two shards step at the same time on two non-default streams (default
priority), their enqueues interleaved step by step, in the synchronous,
device-gated and device-resident flows; the allocation-free step runs both
shards one after the other on one non-default stream (its static scratch is
shared per GPU, so only calls in order on one stream may follow each other).
One shard is above the small-shard limit (the streaming kernels), the other
below it (the cached shape, inline fold in the device-resident flow).  Each
shard's steps and final state equal the oracle's bitwise, as they do alone
on torch's default stream.  Every contribution batch is written before the
first step, so no fill is ordered against the step streams."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import zero_dp_sharded_amd as zs
from gpu_common import (LP_CODE, GpuRun, compare, f32, hp_of, log, oracle_hp, oracle_ls, stored,
                        u16)
from zero_dp_sharded_amd import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)
STEPS = 3
LS = zs.LossScaleCfg(init_scale=1024.0, dynamic=1, growth_interval=1000)


@dataclasses.dataclass
class Shard:
    w: synth.Workload
    S: int
    cb: int
    seed: int


SHARDS = [
    # streaming shapes: above the 8,388,608-element small-shard limit
    Shard(dataclasses.replace(synth.WORKLOADS["gpt2_1.5b"], R=4), 9_000_007, 2_000_000, 1),
    # cached small-shard shape
    Shard(dataclasses.replace(synth.WORKLOADS["7.5b_bf16"], R=8), 600_001, 600_001, 2),
]


def _setup(sh):
    w, S = sh.w, sh.S
    master0, m0, v0 = synth.init_state(w, DEV, sh.seed, elems=S)
    st = {"master": master0.clone(), "m": m0.clone(), "v": v0.clone(),
          "grad": torch.zeros(S, dtype=w.torch_lp, device=DEV),
          "param": master0.to(w.torch_lp)}
    batches = []
    for s in range(STEPS):
        bufs = synth.alloc_contribs(w, DEV, elems=S)
        synth.fill_contribs(w, bufs, s, LS.init_scale, sh.seed)
        batches.append(bufs)
    torch.cuda.synchronize()
    host0 = (f32(master0), f32(m0), f32(v0))
    return st, batches, host0


def _init(sh, st):
    return zs.zero_shard_init(st["master"], st["m"], st["v"], st["grad"], st["param"],
                              psi=sh.S, nd=1, rank=0, bucket_elems=sh.cb, hp=hp_of(sh.w),
                              ls=LS)


def _check(sh, st, batches, host0, infos, tag):
    w = sh.w
    lp = LP_CODE[w.lp]
    ohp, ols = oracle_hp(hp_of(w)), oracle_ls(LS)
    ost = oracle.new_state(lp, *host0, ohp, ols)
    kept = [[stored(b) for b in bufs] for bufs in batches]
    oinfos = [oracle.step(ost, cs, sh.cb, ohp, ols) for cs in kept]
    g = GpuRun(infos, kept, *host0, f32(st["master"]), f32(st["m"]), f32(st["v"]),
               stored(st["grad"]), u16(st["param"]))
    errs = compare(w, g, ost, oinfos, tag)
    assert errs["bitwise"], (tag, errs)


@pytest.mark.parametrize("flow", ["sync", "gated", "device"])
def test_two_shards_on_two_streams(flow):
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    setups = [_setup(sh) for sh in SHARDS]
    handles = [_init(sh, su[0]) for sh, su in zip(SHARDS, setups)]
    infos = [[], []]
    try:
        if flow == "device":
            for h, s in zip(handles, streams):
                zs.zero_device_begin(h, s)
        for step in range(STEPS):
            for k, (sh, (st, batches, _), h, s) in enumerate(zip(SHARDS, setups, handles,
                                                                  streams)):
                bufs = batches[step]
                if flow == "device":
                    zs.zero_step_device(h, bufs, stream=s)
                    continue
                zs.reduce_buckets(h, bufs, sh.S, sh.cb, stream=s)
                if flow == "gated":
                    zs.zero_adam_step_gated(h, stream=s)
                else:
                    zs.zero_overflow_check(h, stream=s)
                    infos[k].append(zs.zero_adam_step(h, stream=s))
            if flow == "gated":
                for k, h in enumerate(handles):
                    infos[k].append(zs.zero_step_resolve(h))
        if flow == "device":
            for k, (h, s) in enumerate(zip(handles, streams)):
                infos[k] = [None] * (STEPS - 1) + [zs.zero_device_end(h, s)]
        torch.cuda.synchronize()
    finally:
        for h in handles:
            zs.zero_shard_destroy(h)
    for k, (sh, (st, batches, host0)) in enumerate(zip(SHARDS, setups)):
        log(f"[streams] {flow}: shard {sh.S} ({sh.w.lp}, R={sh.w.R})")
        _check(sh, st, batches, host0, infos[k], f"{flow} shard {k}")


def test_noalloc_on_a_side_stream():
    s = torch.cuda.Stream()
    setups = [_setup(sh) for sh in SHARDS]
    infos = [[], []]
    counters = [(0, LS.init_scale, 0), (0, LS.init_scale, 0)]
    for step in range(STEPS):
        for k, (sh, (st, batches, _)) in enumerate(zip(SHARDS, setups)):
            info, counters[k] = zs.zero_adam_step_noalloc(
                st["master"], st["m"], st["v"], st["grad"], st["param"], psi=sh.S, nd=1,
                rank=0, bucket_elems=sh.cb, hp=hp_of(sh.w), ls=LS, counters=counters[k],
                contribs=batches[step], stream=s)
            infos[k].append(info)
    torch.cuda.synchronize()
    for k, (sh, (st, batches, host0)) in enumerate(zip(SHARDS, setups)):
        assert counters[k] == (STEPS, LS.init_scale, STEPS), counters[k]
        _check(sh, st, batches, host0, infos[k], f"noalloc shard {k}")
