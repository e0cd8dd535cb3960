"""Seeded random layouts for the bucket reduce against the oracle: every
contribution at its own address phase (a multiple of the element size modulo
16 bytes), the gradient output at another, sometimes contribution 0 being the
gradient itself (a reduce in place while the others are shifted), with the
contribution count, shard and bucket sizes, storage format and flow drawn at
random (fixed seeds: the same 32 small and 6 large cases every run).  Three
steps each, the dynamic loss scale moving between them; every step's flag,
norm and stored gradient and the final state must equal the oracle's bitwise.
The targeted phase tests pick layouts by hand; these reach the combinations
they do not list (counts the shift kernel is and is not compiled for, buckets
whose phases change from bucket to bucket, heads clipped to short buckets)."""
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
SMALL = [1, 7, 64, 1000, 4099, 50_021, 131_071, 250_001]
# past the 8,388,608 elements below which the kernels take the cached shape
LARGE = [8_400_017, 9_000_011]


def _case(k, sizes, seed0):
    rng = np.random.default_rng(seed0 + k)
    lp = ["fp16", "bf16", "fp32"][rng.integers(3)]
    esz = 4 if lp == "fp32" else 2
    R = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 9, 12, 16, 17, 24]))
    S = int(rng.choice(sizes))
    cb = S if rng.random() < 0.3 else int(rng.integers(1, S + 1))
    goff = int(rng.integers(0, 16 // esz)) * esz
    offs = [int(x) * esz for x in rng.integers(0, 16 // esz, size=R)]
    in_place = bool(rng.random() < 0.25)
    if in_place:
        offs[0] = goff
    flow = ["sync", "gated", "device"][rng.integers(3)]
    return lp, R, S, cb, goff, offs, in_place, flow


def _run(lp, R, S, cb, goff, offs, in_place, flow, seed):
    w = dataclasses.replace(synth.WORKLOADS["gpt2_1.5b"], lp=lp, R=R, dynamic=1,
                            scale=1024.0 if lp != "fp32" else 1.0, steps=STEPS)
    t = w.torch_lp
    esz = torch.empty(0, dtype=t).element_size()

    def at(byte_off, n):
        base = torch.empty(n + 16, dtype=t, device=DEV)
        assert base.data_ptr() % 16 == 0
        return base[byte_off // esz:byte_off // esz + n]

    master0, m0, v0 = synth.init_state(w, DEV, seed, elems=S)
    host0 = (f32(master0), f32(m0), f32(v0))
    master, m, v = master0.clone(), m0.clone(), v0.clone()
    grad = at(goff, S)
    grad.zero_()
    param = None if lp == "fp32" else master0.to(t)
    bufs = [grad if (in_place and r == 0) else at(o, S) for r, o in enumerate(offs)]
    h = zs.zero_shard_init(master, m, v, grad, param, psi=S, nd=1, rank=0, bucket_elems=cb,
                           hp=hp_of(w), ls=ls_of(w))
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
    g = GpuRun(infos, kept, *host0, f32(master), f32(m), f32(v), stored(grad),
               None if param is None else u16(param))
    return compare(w, g, ost, oinfos, f"random phases {lp} R={R} S={S} cb={cb}")


def _check(k, case):
    lp, R, S, cb, goff, offs, in_place, flow = case
    log(f"[random phases {k}] lp={lp} R={R} S={S} cb={cb} grad+{goff} offs={offs} "
        f"in_place={in_place} flow={flow}")
    errs = _run(lp, R, S, cb, goff, offs, in_place, flow, seed=k)
    assert errs["bitwise"], (k, errs)


@pytest.mark.parametrize("k", range(32))
def test_random_phase_case(k):
    _check(k, _case(k, SMALL, 5000))


@pytest.mark.parametrize("k", range(6))
def test_random_phase_large_case(k):
    """Shards past the cached-shape limit: nontemporal shift kernels with one
    run per lane (8 or more contributions) or two (fewer)."""
    _check(100 + k, _case(k, LARGE, 6000))
