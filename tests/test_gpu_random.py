"""Seeded random configurations against the oracle: shard size, contribution
count, bucket size, storage format, optimizer, flow, clipping, array offsets
and an overflow step drawn at random (fixed seeds, so every run checks the same
48 small cases and 12 large ones), each a few steps at sizes the oracle
finishes in about a second.  Catches interactions the targeted tests do not
enumerate."""
import dataclasses

import numpy as np
import pytest

import zero_dp_sharded_amd as zs
from gpu_common import compare, expect_inline_folds, hp_of, log, run_gpu, run_oracle
from zero_dp_sharded_amd import synth

pytestmark = pytest.mark.gpu

BASES = {"fp16": synth.WORKLOADS["gpt2_1.5b"], "bf16": synth.WORKLOADS["7.5b_bf16"],
         "fp32": synth.WORKLOADS["c1_7.5b_sgdm"]}


SMALL = [1, 5, 63, 64, 65, 1000, 4099, 65_537, 131_071, 250_000]
# shards past the 8,388,608 elements below which every kernel takes its
# cache-resident 256-lane shape, whose buckets can reach the size at which the
# reduce gives each lane 3 runs (491,520 runs: 3,932,160 two-byte or 1,966,080
# fp32 elements)
LARGE = [8_388_609, 8_500_001, 9_000_007, 10_000_019]


def _case(k: int, sizes=SMALL, seed0: int = 1000, steps: int = 3, r_hi: int = 21):
    rng = np.random.default_rng(seed0 + k)
    lp = ["fp16", "bf16", "fp32"][rng.integers(3)]
    opt = ["adam", "sgd_m", "sgd"][rng.integers(3)]
    elems = int(rng.choice(sizes))
    R = int(rng.integers(1, r_hi))
    cb = int(max(1, min(elems, rng.integers(1, elems + 1) if rng.random() < 0.5 else elems)))
    flow = ["sync", "gated", "device"][rng.integers(3)]
    clip = bool(rng.random() < 0.3)
    inject = int(rng.integers(0, 3)) if rng.random() < 0.3 else None
    names = ["master", "m", "v", "grad", "param", "contrib"]
    offsets = {n: int(rng.integers(0, 8)) for n in names} if rng.random() < 0.5 else {}
    w = dataclasses.replace(
        BASES[lp], name=f"random case {k}", R=R, steps=steps, lp=lp,
        inject_step=None if inject is None else min(inject, steps - 1),
        opt="adam" if opt == "adam" else "sgd", momentum=0.9 if opt == "sgd_m" else 0.0,
        scale=float(2 ** int(rng.integers(0, 12))), dynamic=int(rng.integers(0, 2)),
        weight_decay=float(rng.choice([0.0, 0.01])))
    return w, elems, cb, flow, clip, offsets


def _run_case(k, case):
    w, elems, cb, flow, clip, offsets = case
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


@pytest.mark.parametrize("k", range(48))
def test_random_case(k):
    _run_case(k, _case(k))


@pytest.mark.parametrize("k", range(12))
def test_random_large_case(k):
    """Shards of 8.4-10M elements (the streaming shapes), where a bucket of up
    to the whole shard takes 3 runs per lane below 8 contributions; 2 steps
    each."""
    _run_case(100 + k, _case(k, LARGE, seed0=2000, steps=2, r_hi=8 if k % 3 else 21))


INLINE_SIZES = [8, 64, 1024, 4096, 32_768, 65_536]


@pytest.mark.parametrize("k", range(24))
def test_random_inline_fold_case(k):
    """Device-resident steps on aligned shards of 8-65,536 elements, where the
    update usually folds the partials itself: any storage format, optimizer,
    contribution count, bucket size, clipping and overflow step.  A single
    bucket of a multiple of 8 elements has at most 256 partials in every
    format, so there the inline fold must have run on every step."""
    w, elems, cb, _, clip, _ = _case(k, INLINE_SIZES, seed0=3000, steps=3)
    if k % 2 == 0:
        cb = elems
    hp = hp_of(w)
    norm = w.grad_std / np.sqrt(w.R) * np.sqrt(elems)
    max_norm = 0.5 * norm if clip else 0.0
    log(f"[random inline {k}] lp={w.lp} opt={w.opt} mom={w.momentum} elems={elems} R={w.R} "
        f"cb={cb} clip={clip} inject={w.inject_step} scale={w.scale} dynamic={w.dynamic}")
    n = []
    g = run_gpu(w, elems=elems, bucket_elems=cb, hp=hp, flow="device", max_norm=max_norm,
                inline_folds=n)
    st, oi = run_oracle(w, g, bucket_elems=cb, hp=hp, max_norm=max_norm)
    errs = compare(w, g, st, oi, f"random inline {k}")
    log(f"[random inline {k}] inline steps {n[0]} of {w.steps}")
    if not clip:
        assert errs["bitwise"], (k, errs)
    if w.inject_step is not None:
        assert g.infos[w.inject_step].overflow == 1
    if cb == elems:
        expect_inline_folds(n, [w.steps], k)
