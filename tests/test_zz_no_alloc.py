"""The allocation-free step (zero_adam_step_noalloc) against the handle flow it
is a variant of (zero_bucket_reduce over every bucket, zero_overflow_check,
zero_adam_step) on the same inputs, through the C ABI: stored gradient,
master, m, v and params bitwise, the step's result and the counters equal.

The no-alloc calls run back to back on one GPU, each next one on a smaller
shard, so every call after the first finds the previous call's partials in
the static scratch; the handle flows run afterwards on saved copies of the
same inputs."""
import dataclasses

import numpy as np
import pytest
import torch

import zero_dp_sharded_amd as zs
from gpu_common import log
from zero_dp_sharded_amd import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)


@dataclasses.dataclass
class Case:
    name: str
    S: int
    R: int                 # 0: scan of a caller-filled grad_shard
    lp: torch.dtype
    bucket: int
    counters: tuple        # (step_t, scale, good_steps) before the step
    max_norm: float = 0.0
    plant_inf: bool = False
    steps: int = 1
    phase: int = 16        # contribution r at (r * phase) mod 16 bytes (16: aligned)


def _make(case, seed):
    w = dataclasses.replace(synth.WORKLOADS["gpt2_1.5b"], R=max(case.R, 1),
                            lp={torch.float16: "fp16", torch.bfloat16: "bf16"}[case.lp])
    master, m, v = synth.init_state(w, DEV, seed, elems=case.S)
    m.normal_(0.0, 1e-4)
    v.copy_(torch.rand_like(v) * 1e-8)
    grad = torch.zeros(case.S, dtype=case.lp, device=DEV)
    contribs = []
    if case.R:
        contribs = synth.alloc_contribs(w, DEV, elems=case.S, phase_step=case.phase)
    steps = []
    for s in range(case.steps):
        if case.R:
            synth.fill_contribs(w, contribs, s, case.counters[1], seed)
            if case.plant_inf and s == case.steps - 1:
                contribs[case.R - 1][case.S - 3] = float("inf")
            kept = synth.alloc_contribs(w, DEV, elems=case.S, phase_step=case.phase)
            for d, c in zip(kept, contribs):
                d.copy_(c)
            steps.append(kept)
        else:
            g = torch.empty(case.S, dtype=case.lp, device=DEV)
            synth.fill_contribs(dataclasses.replace(w, R=1), [g], s, case.counters[1], seed)
            steps.append(g)
    return {"master": master, "m": m, "v": v, "grad": grad, "param": master.to(case.lp),
            "steps": steps}


def _clone(st):
    return {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in st.items()}


HP = zs.AdamHParams(lr=1e-3, weight_decay=0.01)
LS = zs.LossScaleCfg(init_scale=1.0, dynamic=1, growth_interval=4, min_scale=1.0)


def _noalloc(case, st):
    infos, counters = [], case.counters
    for s in range(case.steps):
        if case.R:
            contribs = st["steps"][s]
        else:
            st["grad"].copy_(st["steps"][s])
            contribs = None
        info, counters = zs.zero_adam_step_noalloc(
            st["master"], st["m"], st["v"], st["grad"], st["param"], psi=case.S, nd=1, rank=0,
            bucket_elems=case.bucket, hp=HP, ls=LS, counters=counters, contribs=contribs,
            max_grad_norm=case.max_norm)
        infos.append(info)
    torch.cuda.synchronize()
    return infos, counters


def _handle(case, st):
    h = zs.zero_shard_init(st["master"], st["m"], st["v"], st["grad"], st["param"], psi=case.S,
                           nd=1, rank=0, bucket_elems=case.bucket, hp=HP, ls=LS)
    infos = []
    try:
        zs.zero_shard_set_counters(h, *case.counters)
        if case.max_norm:
            zs.zero_shard_set_clip(h, case.max_norm)
        for s in range(case.steps):
            if case.R:
                zs.reduce_buckets(h, st["steps"][s], case.S, case.bucket)
            else:
                st["grad"].copy_(st["steps"][s])
            chk = zs.zero_overflow_check(h)
            info = zs.zero_adam_step(h)
            assert info.overflow == chk.overflow
            infos.append(info)
        torch.cuda.synchronize()
        counters = zs.zero_shard_get_counters(h)
    finally:
        zs.zero_shard_destroy(h)
    return infos, counters


def _bits(t):
    return t.view(torch.int32 if t.element_size() == 4 else torch.int16).cpu().numpy()


def _compare(case, a, b, ia, ib, ca, cb):
    for k in ("grad", "master", "m", "v", "param"):
        assert np.array_equal(_bits(a[k]), _bits(b[k])), (case.name, k)
    assert len(ia) == len(ib)
    for x, y in zip(ia, ib):
        assert (x.overflow, x.skipped, x.step_t, x.scale_used, x.scale_next) == \
            (y.overflow, y.skipped, y.step_t, y.scale_used, y.scale_next), (case.name, x, y)
        assert x.grad_norm == y.grad_norm or (np.isnan(x.grad_norm) and np.isnan(y.grad_norm))
    assert tuple(ca) == tuple(cb), (case.name, ca, cb)


CASES = [
    # every later case smaller than the one before it
    Case("fp16 R=4, 1,000,003 elements, clipping", 1_000_003, 4, torch.float16, 262_144,
         (0, 1024.0, 0), max_norm=0.05),
    Case("fp16 R=8, 500,009 elements, contributions at 2-byte phases", 500_009, 8,
         torch.float16, 131_072, (3, 256.0, 1), phase=2),
    Case("bf16 R=9, 300,007 elements, +inf: skipped, scale halved", 300_007, 9, torch.bfloat16,
         65_536, (5, 64.0, 3), plant_inf=True),
    Case("fp16 scan of a caller-filled grad_shard, 70,001 elements", 70_001, 0, torch.float16,
         70_001, (2, 8.0, 1)),
    Case("fp16 R=2, 4,099 elements, 3 steps (growth after 4 clean)", 4_099, 2, torch.float16,
         1_024, (7, 2.0, 2), steps=3),
]


def test_noalloc_back_to_back_equals_handle_flow():
    states = [_make(c, seed=11 + k) for k, c in enumerate(CASES)]
    saved = [_clone(st) for st in states]
    got = []
    for c, st in zip(CASES, states):          # the no-alloc calls, back to back
        log(f"[noalloc] {c.name}")
        got.append(_noalloc(c, st))
    for c, st, ref, (ia, ca) in zip(CASES, states, saved, got):
        ib, cb = _handle(c, ref)
        _compare(c, st, ref, ia, ib, ca, cb)
    assert got[2][0][-1].overflow == 1 and got[2][1] == (5, 32.0, 0)
    assert got[4][1][1] == 4.0                                   # grew 2 -> 4 after 4 clean


def test_noalloc_refuses_a_shard_beyond_its_scratch():
    """300M fp16 elements with 8 contributions need about 586K partial slots,
    more than the 523,232 the static scratch holds: refused before any launch,
    nothing written, counters unchanged."""
    S, R = 300_000_000, 8
    t = [torch.full((S,), 0.5, device=DEV) for _ in range(3)]
    g = torch.full((S,), 7.0, dtype=torch.float16, device=DEV)
    p = torch.full((S,), 3.0, dtype=torch.float16, device=DEV)
    cs = [torch.ones(S, dtype=torch.float16, device=DEV) for _ in range(R)]
    try:
        with pytest.raises(zs.ZeroError) as e:
            zs.zero_adam_step_noalloc(*t, g, p, psi=S, nd=1, rank=0, bucket_elems=50_000_000,
                                      hp=HP, ls=LS, counters=(0, 1.0, 0), contribs=cs)
        assert e.value.status == zs.ZERO_ERR_INVALID_ARG
        assert "scratch" in str(e.value)
        torch.cuda.synchronize()
        assert bool((g == 7.0).all()) and bool((p == 3.0).all())
        assert all(bool((x == 0.5).all()) for x in t)
    finally:
        del t, g, p, cs
        torch.cuda.empty_cache()


def test_noalloc_argument_checks():
    S = 1024
    t = [torch.zeros(S, device=DEV) for _ in range(3)]
    g = torch.zeros(S, dtype=torch.float16, device=DEV)
    p = torch.zeros(S, dtype=torch.float16, device=DEV)
    L = zs.lib()
    for counters, norm in (((-1, 1.0, 0), 0.0), ((0, 0.0, 0), 0.0), ((0, 1.0, -1), 0.0),
                           ((0, 1.0, 0), -1.0), ((0, 1.0, 0), float("nan"))):
        with pytest.raises(zs.ZeroError) as e:
            zs.zero_adam_step_noalloc(*t, g, p, psi=S, nd=1, rank=0, bucket_elems=S, hp=HP,
                                      ls=LS, counters=counters, max_grad_norm=norm)
        assert e.value.status == zs.ZERO_ERR_INVALID_ARG, (counters, norm)
    assert L.zero_adam_step_noalloc(None, None, None, 0.0, None, 0, None, None, None, None,
                                    None) == zs.ZERO_ERR_INVALID_ARG
