"""Helpers shared by the GPU tests: run k owner-rank steps through the C ABI,
run the oracle on the same inputs, and compare them by the parity rules.

Comparison rules: overflow flags, skip decisions, t and the loss scale exact;
the stored gradient shard bitwise (any NaN matches any NaN); fp32 master / m /
v (or SGD momentum) within max relative error 1e-6; the 2-byte params within
1 ulp (ordered-integer distance, +0 and -0 at distance 0); the gradient norm
within relative 1e-5.  With fp32 storage there is no 2-byte param.
"""
from __future__ import annotations

import dataclasses
import os
import sys
from typing import List, Optional

import numpy as np
import torch

import oracle
import zero_dp_sharded_amd as zs
from zero_dp_sharded_amd import synth

LP_CODE = {"fp16": oracle.FP16, "bf16": oracle.BF16, "fp32": oracle.FP32}

# Which steps fold their partials inside the update depends on the launch
# shapes a build was compiled with; a variant build loaded through
# ZERO_SHARD_LIB (tuning shapes, or every launch split after 1024 work-items)
# may take the fold launch where the in-tree build does not.  Tests assert the
# inline-fold counts only for the in-tree library; parity holds for every build.
IN_TREE_BUILD = not os.environ.get("ZERO_SHARD_LIB")


def expect_inline_folds(got, expected, tag=""):
    if IN_TREE_BUILD:
        assert got == expected, (tag, got, expected)


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.float32, copy=False)


def stored(t: torch.Tensor) -> np.ndarray:
    """Host copy of stored values: 2-byte bit patterns, or fp32 values."""
    return f32(t) if t.dtype == torch.float32 else u16(t)


def hp_of(w: synth.Workload, **over):
    if w.opt == "sgd":
        return dataclasses.replace(zs.SGDHParams(lr=w.lr, momentum=w.momentum,
                                                 weight_decay=w.weight_decay), **over)
    hp = zs.AdamHParams(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                        weight_decay=w.weight_decay, bias_correction=1, wd_mode=0,
                        initial_step=0)
    return dataclasses.replace(hp, **over)


def oracle_hp(hp):
    if isinstance(hp, zs.SGDHParams):
        return oracle.SGDHP(lr=hp.lr, momentum=hp.momentum, weight_decay=hp.weight_decay,
                            initial_step=hp.initial_step)
    return oracle.AdamHP(lr=hp.lr, beta1=hp.beta1, beta2=hp.beta2, eps=hp.eps,
                         weight_decay=hp.weight_decay, bias_correction=hp.bias_correction,
                         wd_mode=hp.wd_mode, initial_step=hp.initial_step)


def ls_of(w: synth.Workload, **over) -> zs.LossScaleCfg:
    ls = zs.LossScaleCfg(init_scale=w.scale, dynamic=w.dynamic, growth_interval=1000,
                         min_scale=1.0)
    return dataclasses.replace(ls, **over)


def oracle_ls(ls: zs.LossScaleCfg) -> oracle.LossScale:
    return oracle.LossScale(init_scale=ls.init_scale, dynamic=ls.dynamic,
                            growth_interval=ls.growth_interval, min_scale=ls.min_scale)


@dataclasses.dataclass
class GpuRun:
    infos: List[zs.StepInfo]
    contribs: List[List[np.ndarray]]      # per step, R host copies (when kept)
    master0: np.ndarray
    m0: Optional[np.ndarray]              # None where the optimizer keeps no such array
    v0: Optional[np.ndarray]
    master: np.ndarray
    m: Optional[np.ndarray]
    v: Optional[np.ndarray]
    grad: np.ndarray                      # 2-byte bits, or fp32 values
    param: Optional[np.ndarray]           # 2-byte bits; None with fp32 storage


def run_gpu(w: synth.Workload, *, elems: Optional[int] = None, steps: Optional[int] = None,
            seed: int = 0, bucket_elems: Optional[int] = None, hp=None,
            ls: Optional[zs.LossScaleCfg] = None, keep_contribs: bool = True,
            offsets: Optional[dict] = None, hook=None, flow: str = "sync",
            max_norm: float = 0.0, scale_of=None, inline_folds: Optional[list] = None,
            init_hook=None) -> GpuRun:
    """Run `steps` owner-rank steps of workload w (its first `elems` shard
    elements) through the C ABI on cuda:0.  offsets maps an array name
    ('master', 'm', 'v', 'grad', 'param', 'contrib') to an element offset of its
    base pointer inside a larger allocation (alignment tests).  hook(step,
    bufs) may edit the contributions of a step before it runs.  flow "sync"
    uses zero_overflow_check + the step call, "gated" the gated step call +
    zero_step_resolve, "device" one zero_step_device per step between
    zero_device_begin and zero_device_end (ended after every step to read its
    result), "device_run" the same without ending between steps (only the last
    step's result is read; the others are None).  The workload's opt picks Adam
    or SGD; max_norm > 0 turns on global-norm clipping.  inline_folds, when
    given, receives the handle's count of device steps whose update folded the
    partials itself.  init_hook(master0, m0, v0) may edit the initial fp32
    state (m0 / v0 None where the optimizer keeps no such array) before it is
    copied into the shard; the 2-byte param starts as its rounding."""
    dev = torch.device("cuda", 0)
    S = w.shard if elems is None else elems
    steps = w.steps if steps is None else steps
    cb = w.bucket_elems if bucket_elems is None else bucket_elems
    hp = hp or hp_of(w)
    ls = ls or ls_of(w)
    offsets = offsets or {}
    lp_t = w.torch_lp

    def alloc(name, dtype):
        off = offsets.get(name, 0)
        base = torch.empty(S + off + 8, dtype=dtype, device=dev)
        return base[off:off + S]

    master0, m0, v0 = synth.init_state(w, dev, seed, elems=S)
    if not w.has_m:
        m0 = None
    if not w.has_v:
        v0 = None
    if init_hook is not None:
        init_hook(master0, m0, v0)
    master = alloc("master", torch.float32)
    master.copy_(master0)
    m = v = None
    if m0 is not None:
        m = alloc("m", torch.float32)
        m.copy_(m0)
    if v0 is not None:
        v = alloc("v", torch.float32)
        v.copy_(v0)
    grad = alloc("grad", lp_t)
    grad.zero_()
    param = None
    if lp_t != torch.float32:
        param = alloc("param", lp_t)
        param.copy_(master0.to(lp_t))
    coff = offsets.get("contrib", 0)
    cbase = [torch.empty(S + coff + 8, dtype=lp_t, device=dev) for _ in range(w.R)]
    bufs = [b[coff:coff + S] for b in cbase]
    psi = S * w.nd
    sgd = w.opt == "sgd"
    if sgd:
        h = zs.zero_shard_init_sgd(master, m, grad, param, psi=psi, nd=w.nd, rank=w.rank,
                                   bucket_elems=cb, hp=hp, ls=ls)
    else:
        h = zs.zero_shard_init(master, m, v, grad, param, psi=psi, nd=w.nd, rank=w.rank,
                               bucket_elems=cb, hp=hp, ls=ls)
    step_fn = zs.zero_sgd_step if sgd else zs.zero_adam_step
    gated_fn = zs.zero_sgd_step_gated if sgd else zs.zero_adam_step_gated
    infos, kept = [], []
    try:
        if max_norm:
            zs.zero_shard_set_clip(h, max_norm)
        scale = ls.init_scale
        if flow == "device_run":
            zs.zero_device_begin(h)
        for s in range(steps):
            if flow == "device_run" and scale_of is not None:
                scale = scale_of(s)
            synth.fill_contribs(w, bufs, s, scale, seed)
            if hook is not None:
                hook(s, bufs)
            if keep_contribs:
                kept.append([stored(b) for b in bufs])
            if flow == "device":
                zs.zero_device_begin(h)
                zs.zero_step_device(h, bufs)
                info = zs.zero_device_end(h)
                infos.append(info)
                scale = info.scale_next
                continue
            if flow == "device_run":
                zs.zero_step_device(h, bufs)
                infos.append(zs.zero_device_end(h) if s == steps - 1 else None)
                continue
            zs.reduce_buckets(h, bufs, S, cb)
            if flow == "gated":
                gated_fn(h)
                info = zs.zero_step_resolve(h)
            else:
                chk = zs.zero_overflow_check(h)
                info = step_fn(h)
                assert info.overflow == chk.overflow
                assert info.grad_norm == chk.grad_norm or (np.isnan(info.grad_norm) and np.isnan(chk.grad_norm))
            infos.append(info)
            scale = info.scale_next
        torch.cuda.synchronize()
        if inline_folds is not None:
            inline_folds.append(zs.zero_shard_inline_folds(h))
    finally:
        zs.zero_shard_destroy(h)
    opt = lambda t: None if t is None else f32(t)
    return GpuRun(infos, kept, f32(master0), opt(m0), opt(v0), f32(master), opt(m), opt(v),
                  stored(grad), None if param is None else u16(param))


def run_oracle(w: synth.Workload, g: GpuRun, *, bucket_elems: Optional[int] = None,
               hp=None, ls: Optional[zs.LossScaleCfg] = None, max_norm: float = 0.0):
    lp = LP_CODE[w.lp]
    cb = w.bucket_elems if bucket_elems is None else bucket_elems
    ohp = oracle_hp(hp or hp_of(w))
    ols = oracle_ls(ls or ls_of(w))
    st = oracle.new_state(lp, g.master0, g.m0, g.v0, ohp, ols)
    infos = [oracle.step(st, cs, cb, ohp, ols, max_norm=max_norm) for cs in g.contribs]
    return st, infos


def ulp_dist(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Ordered-integer distance of 2-byte encodings; +0 and -0 coincide."""
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x)
    return np.abs(ordered(a_bits) - ordered(b_bits))


def lp_is_nan(bits: np.ndarray, lp: str) -> np.ndarray:
    if lp == "fp32":
        return np.isnan(bits)
    if lp == "fp16":
        return ((bits & 0x7C00) == 0x7C00) & ((bits & 0x03FF) != 0)
    return ((bits & 0x7F80) == 0x7F80) & ((bits & 0x007F) != 0)


def max_rel(a: np.ndarray, b: np.ndarray) -> float:
    """Largest |a - b| / max(|b|, FLT_MIN); equal values (infinities of one
    sign included) and NaN against NaN count 0, any other non-finite pair inf."""
    if a.size == 0:
        return 0.0
    a64, b64 = a.astype(np.float64), b.astype(np.float64)
    den = np.maximum(np.abs(b64), np.finfo(np.float32).tiny)
    with np.errstate(invalid="ignore", over="ignore"):
        err = np.abs(a64 - b64) / den
    err = np.where((a64 == b64) | (np.isnan(a64) & np.isnan(b64)), 0.0, err)
    err = np.where(np.isnan(err), np.inf, err)
    return float(np.max(err))


def compare(w: synth.Workload, g: GpuRun, st, oinfos, tag: str = "") -> dict:
    """Assert the parity rules; return the observed worst errors."""
    assert len(g.infos) == len(oinfos)
    for k, (a, b) in enumerate(zip(g.infos, oinfos)):
        if a is None:                    # a device-resident step whose result was not read
            continue
        assert a.overflow == b.overflow, (tag, k, a, b)
        assert a.skipped == b.skipped, (tag, k)
        assert a.step_t == b.step_t, (tag, k, a.step_t, b.step_t)
        assert a.scale_used == b.scale_used and a.scale_next == b.scale_next, (tag, k)
        if not a.overflow:
            assert a.grad_norm == _approx(b.grad_norm, 1e-5), (tag, k, a.grad_norm, b.grad_norm)
    gn = lp_is_nan(g.grad, w.lp)
    on = lp_is_nan(st.grad, w.lp)
    assert np.array_equal(gn, on), tag
    bits = (lambda x: x.view(np.uint32)) if w.lp == "fp32" else (lambda x: x)
    bad = np.nonzero((bits(g.grad) != bits(st.grad)) & ~gn)[0]
    assert bad.size == 0, (tag, "grad", bad[:8], g.grad[bad[:8]], st.grad[bad[:8]])
    pairs = [("master", g.master, st.master), ("m", g.m, st.m), ("v", g.v, st.v)]
    errs = {}
    bitwise = True
    for k, a, b in pairs:
        assert (a is None) == (b is None), (tag, k)
        if a is None:
            continue
        errs[k] = max_rel(a, b)
        assert errs[k] <= 1e-6, (tag, k, errs[k])
        bitwise = bitwise and np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert (g.param is None) == (st.param is None), tag
    if g.param is not None:
        d = ulp_dist(g.param, st.param)
        errs["param_ulp"] = int(d.max()) if d.size else 0
        assert errs["param_ulp"] <= 1, (tag, "param", errs["param_ulp"])
        bitwise = bitwise and np.array_equal(g.param, st.param)
    errs["bitwise"] = bool(bitwise)
    return errs


def _approx(x, rel):
    import pytest
    return pytest.approx(x, rel=rel, abs=0)
