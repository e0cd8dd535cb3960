"""Seeded random configurations against the oracle: shard size, contribution
count, bucket size, storage format, optimizer, flow, clipping, array offsets
and an overflow step drawn at random (fixed seed, so every run checks the same
48 cases), each a few steps at sizes the oracle finishes in well under a
second.  Catches interactions the targeted tests do not enumerate."""
import dataclasses

import numpy as np
import pytest

import zero_dp_sharded_amd as zs
from gpu_common import compare, hp_of, log, run_gpu, run_oracle
from zero_dp_sharded_amd import synth

pytestmark = pytest.mark.gpu

BASES = {"fp16": synth.WORKLOADS["gpt2_1.5b"], "bf16": synth.WORKLOADS["7.5b_bf16"],
         "fp32": synth.WORKLOADS["c1_7.5b_sgdm"]}


def _case(k: int):
    rng = np.random.default_rng(1000 + k)
    lp = ["fp16", "bf16", "fp32"][rng.integers(3)]
    opt = ["adam", "sgd_m", "sgd"][rng.integers(3)]
    elems = int(rng.choice([1, 5, 63, 64, 65, 1000, 4099, 65_537, 131_071, 250_000]))
    R = int(rng.integers(1, 21))
    cb = int(max(1, min(elems, rng.integers(1, elems + 1) if rng.random() < 0.5 else elems)))
    flow = ["sync", "gated", "device"][rng.integers(3)]
    clip = bool(rng.random() < 0.3)
    inject = int(rng.integers(0, 3)) if rng.random() < 0.3 else None
    names = ["master", "m", "v", "grad", "param", "contrib"]
    offsets = {n: int(rng.integers(0, 8)) for n in names} if rng.random() < 0.5 else {}
    w = dataclasses.replace(
        BASES[lp], name=f"random case {k}", R=R, steps=3, lp=lp, inject_step=inject,
        opt="adam" if opt == "adam" else "sgd", momentum=0.9 if opt == "sgd_m" else 0.0,
        scale=float(2 ** int(rng.integers(0, 12))), dynamic=int(rng.integers(0, 2)),
        weight_decay=float(rng.choice([0.0, 0.01])))
    return w, elems, cb, flow, clip, offsets


@pytest.mark.parametrize("k", range(48))
def test_random_case(k):
    w, elems, cb, flow, clip, offsets = _case(k)
    hp = hp_of(w)
    if w.opt == "adam" and k % 4 == 1:
        hp = dataclasses.replace(hp, wd_mode=zs.ZERO_WD_L2)
    norm = w.grad_std / np.sqrt(w.R) * np.sqrt(elems)
    max_norm = 0.5 * norm if clip else 0.0
    log(f"[random {k}] lp={w.lp} opt={w.opt} mom={w.momentum} elems={elems} R={w.R} cb={cb} "
        f"flow={flow} clip={clip} inject={w.inject_step} offsets={offsets} scale={w.scale} "
        f"dynamic={w.dynamic}")
    g = run_gpu(w, elems=elems, bucket_elems=cb, hp=hp, flow=flow, max_norm=max_norm,
                offsets=offsets)
    st, oi = run_oracle(w, g, bucket_elems=cb, hp=hp, max_norm=max_norm)
    errs = compare(w, g, st, oi, f"random {k}")
    if not clip:
        assert errs["bitwise"], (k, errs)
    if w.inject_step is not None:
        assert g.infos[w.inject_step].overflow == 1
