"""Parity at the workloads' full sizes, in the launch configuration bench.py
times (the workload's own shard, C_B and R through the C ABI).

Per step:
  - sampled elements (edges, both sides of every bucket boundary, the +inf
    event, 65,536 random positions) of the stored gradient against the oracle
    run on the same sampled contributions;
  - the whole stored gradient bitwise against an independent torch fp32
    reduce (sum in ascending r from +0, times 1/R, rounded to the storage
    format), a property that holds at any size;
  - the norm against a torch fp64 sum of the unscaled squares of the stored
    gradient;
  - flags, skips, t and scale exactly against the oracle.
After the last step: master, m, v (SGD: the momentum buffer) and the 2-byte
params at the sampled positions against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import zero_dp_sharded_amd as zs
from gpu_common import (LP_CODE, f32, hp_of, log, lp_is_nan, ls_of, max_rel, oracle_hp, oracle_ls,
                        stored, u16, ulp_dist)
from zero_dp_sharded_amd import synth

pytestmark = pytest.mark.gpu

CHUNK = 1 << 27


def sample_indices(w: synth.Workload, n_random: int = 65_536, seed: int = 1) -> np.ndarray:
    S, cb = w.shard, w.bucket_elems
    idx = {0, 1, 2, 3, 7, 8, 9, S - 1, S - 2, S - 3, S - 8, S - 9}
    for b in range(0, S, cb):
        idx.update({b - 1, b, b + 1})
    i = synth.inject_index(S)
    idx.update({i - 1, i, i + 1})
    rng = np.random.default_rng(seed)
    idx.update(rng.integers(0, S, size=n_random).tolist())
    return np.array(sorted(x for x in idx if 0 <= x < S), dtype=np.int64)


def torch_reduce_equal(bufs, grad, R, lp_t):
    """Bitwise compare of the stored gradient with a torch fp32 reduce."""
    inv_r = 1.0 / R
    S = grad.numel()
    for off in range(0, S, CHUNK):
        end = min(S, off + CHUNK)
        acc = torch.zeros(end - off, dtype=torch.float32, device=grad.device)
        for b in bufs:
            acc.add_(b[off:end].float())
        ref = (acc * inv_r).to(lp_t)
        got = grad[off:end]
        bits = torch.int32 if lp_t == torch.float32 else torch.int16
        same = (ref.view(bits) == got.view(bits)) | (torch.isnan(ref) & torch.isnan(got))
        if not bool(same.all()):
            bad = torch.nonzero(~same)[:4].flatten().tolist()
            return False, off + bad[0] if bad else -1
    return True, -1


def torch_sumsq(grad, inv_scale):
    s = torch.zeros((), dtype=torch.float64, device=grad.device)
    for off in range(0, grad.numel(), CHUNK):
        u = grad[off:off + CHUNK].float() * inv_scale
        s += (u.double() ** 2).sum()
    return float(s)


def _bits(x: np.ndarray) -> np.ndarray:
    return x.view(np.uint32) if x.dtype == np.float32 else x


@pytest.mark.parametrize("name,flow", [
    ("tiny", "sync"), ("gpt2_1.5b", "sync"), ("7.5b_bf16", "sync"), ("13b_inf", "sync"),
    ("128b", "sync"), ("c1_7.5b_sgdm", "sync"), ("c2_1.5b_sgd", "sync"),
    # the device-resident flow bench.py times, at full size
    ("gpt2_1.5b", "device"), ("7.5b_bf16", "device"), ("13b_inf", "device"), ("128b", "device"),
    ("c1_7.5b_sgdm", "device"), ("c2_1.5b_sgd", "device"),
])
def test_full_size_sampled(name, flow):
    w = synth.WORKLOADS[name]
    S, R, cb, lp_t = w.shard, w.R, w.bucket_elems, w.torch_lp
    lp = LP_CODE[w.lp]
    dev = torch.device("cuda", 0)
    log(f"[fullsize] {w.name}: S={S} R={R} C_B={cb} steps={w.steps} flow={flow}")
    idx = sample_indices(w)
    idx_t = torch.from_numpy(idx).to(dev)

    master, m, v = synth.init_state(w, dev, seed=0)
    m = m if w.has_m else None
    v = v if w.has_v else None
    grad = torch.zeros(S, dtype=lp_t, device=dev)
    param = None if lp_t == torch.float32 else master.to(lp_t)
    bufs = synth.alloc_contribs(w, dev)
    hp, ls = hp_of(w), ls_of(w)
    ohp, ols = oracle_hp(hp), oracle_ls(ls)
    sample = lambda t: None if t is None else f32(t[idx_t])
    ost = oracle.new_state(lp, f32(master[idx_t]), sample(m), sample(v), ohp, ols)
    if param is not None:
        assert np.array_equal(u16(param[idx_t]), ost.param)
    if w.opt == "sgd":
        h = zs.zero_shard_init_sgd(master, m, grad, param, psi=w.psi, nd=w.nd, rank=w.rank,
                                   bucket_elems=cb, hp=hp, ls=ls)
        step_fn = zs.zero_sgd_step
    else:
        h = zs.zero_shard_init(master, m, v, grad, param, psi=w.psi, nd=w.nd, rank=w.rank,
                               bucket_elems=cb, hp=hp, ls=ls)
        step_fn = zs.zero_adam_step
    try:
        scale = ls.init_scale
        for s in range(w.steps):
            synth.fill_contribs(w, bufs, s, scale, seed=0)
            cs = [stored(b[idx_t]) for b in bufs]
            if flow == "device":
                zs.zero_device_begin(h)
                zs.zero_step_device(h, bufs)
                chk = zs.zero_device_end(h)
            else:
                zs.reduce_buckets(h, bufs, S, cb)
                chk = zs.zero_overflow_check(h)
            ok, where = torch_reduce_equal(bufs, grad, R, lp_t)
            assert ok, (name, s, "full reduce differs at", where)
            oi = oracle.step(ost, cs, len(idx), ohp, ols)
            gs = stored(grad[idx_t])
            gn, on = lp_is_nan(gs, w.lp), lp_is_nan(ost.grad, w.lp)
            assert np.array_equal(gn, on), (name, s)
            assert np.array_equal(_bits(gs)[~gn], _bits(ost.grad)[~on]), (name, s)
            assert chk.overflow == oi.overflow, (name, s)
            if not chk.overflow:
                inv = float(np.float32(1.0 / chk.scale_used))
                tn = np.sqrt(torch_sumsq(grad, inv))
                assert chk.grad_norm == pytest.approx(tn, rel=1e-9), (name, s)
            info = chk if flow == "device" else step_fn(h)
            assert (info.overflow, info.skipped, info.step_t, info.scale_used, info.scale_next) == \
                (oi.overflow, oi.skipped, oi.step_t, oi.scale_used, oi.scale_next), (name, s)
            log(f"[fullsize] {name} step {s}: overflow={info.overflow} t={info.step_t} "
                f"norm={chk.grad_norm:.6g} scale={info.scale_used}")
            scale = info.scale_next
        torch.cuda.synchronize()
        assert max_rel(f32(master[idx_t]), ost.master) <= 1e-6
        for a, b in ((m, ost.m), (v, ost.v)):
            assert (a is None) == (b is None)
            if a is not None:
                assert max_rel(f32(a[idx_t]), b) <= 1e-6
        bit = np.array_equal(f32(master[idx_t]).view(np.uint32), ost.master.view(np.uint32))
        if param is not None:
            assert int(ulp_dist(u16(param[idx_t]), ost.param).max()) <= 1
            bit = bit and np.array_equal(u16(param[idx_t]), ost.param)
        if m is not None:
            bit = bit and np.array_equal(f32(m[idx_t]).view(np.uint32), ost.m.view(np.uint32))
        log(f"[fullsize] {name}: sampled state bitwise equal to the oracle: {bit}")
        assert bit
        if w.inject_step is not None:
            assert ost.t == w.steps - 1
    finally:
        zs.zero_shard_destroy(h)
        del master, m, v, grad, param, bufs
        torch.cuda.empty_cache()


def test_shard_beyond_2pow31_elements():
    """A 2^31 + 1001-element shard (64-bit element indices throughout): two
    steps, the second with +inf planted past index 2^31; sampled elements on
    both sides of 2^31 against the oracle, the whole stored gradient against a
    torch reduce."""
    S = (1 << 31) + 1001
    w = synth.Workload("2^31+1001-element shard, R=2, fp16", psi=S, nd=1, rank=0, R=2,
                       bucket_elems=1 << 30, lp="fp16", scale=256.0, dynamic=1, lr=1e-3,
                       weight_decay=0.01, steps=2)
    dev = torch.device("cuda", 0)
    log(f"[fullsize] {w.name}")
    idx = np.array(sorted({0, 1, (1 << 30) - 1, 1 << 30, (1 << 31) - 2, (1 << 31) - 1, 1 << 31,
                           (1 << 31) + 1, (1 << 31) + 7, S - 9, S - 2, S - 1}), dtype=np.int64)
    rng = np.random.default_rng(3)
    idx = np.unique(np.concatenate([idx, rng.integers(0, S, 4096)]))
    idx_t = torch.from_numpy(idx).to(dev)
    master, m, v = synth.init_state(w, dev, seed=0)
    grad = torch.zeros(S, dtype=torch.float16, device=dev)
    param = master.to(torch.float16)
    bufs = synth.alloc_contribs(w, dev)
    hp, ls = hp_of(w), ls_of(w)
    ohp, ols = oracle_hp(hp), oracle_ls(ls)
    ost = oracle.new_state(oracle.FP16, f32(master[idx_t]), f32(m[idx_t]), f32(v[idx_t]), ohp, ols)
    h = zs.zero_shard_init(master, m, v, grad, param, psi=S, nd=1, rank=0,
                           bucket_elems=w.bucket_elems, hp=hp, ls=ls)
    try:
        scale = w.scale
        for s in range(2):
            synth.fill_contribs(w, bufs, s, scale, seed=0)
            if s == 1:
                bufs[1][(1 << 31) + 7] = float("inf")
            cs = [u16(b[idx_t]) for b in bufs]
            zs.reduce_buckets(h, bufs, S, w.bucket_elems)
            chk = zs.zero_overflow_check(h)
            ok, where = torch_reduce_equal(bufs, grad, 2, torch.float16)
            assert ok, ("reduce differs at", where)
            oi = oracle.step(ost, cs, len(idx), ohp, ols)
            assert chk.overflow == oi.overflow == s
            gs = u16(grad[idx_t])
            gn = lp_is_nan(gs, "fp16")
            assert np.array_equal(gn, lp_is_nan(ost.grad, "fp16"))
            assert np.array_equal(gs[~gn], ost.grad[~gn])
            info = zs.zero_adam_step(h)
            assert (info.step_t, info.scale_next) == (oi.step_t, oi.scale_next)
            scale = info.scale_next
        torch.cuda.synchronize()
        assert np.array_equal(f32(master[idx_t]).view(np.uint32), ost.master.view(np.uint32))
        assert np.array_equal(u16(param[idx_t]), ost.param)
        assert ost.t == 1 and scale == 128.0
    finally:
        zs.zero_shard_destroy(h)
        del master, m, v, grad, param, bufs
        torch.cuda.empty_cache()
