"""GPU parity at the edges of the arithmetic, in the synchronous, device-gated
and device-resident flows, bitwise against the oracle.

The path exists because 2-byte values underflow and overflow where fp32 does
not ("SC-2020 ZeRO" notes, "Where Did All the Memory Go?": the update runs on
fp32 master weights), so the cases here drive the fp32 update and the 2-byte
casts through their subnormal and overflow ranges:
  - a finite stored gradient that a loss scale below 1 unscales past FLT_MAX
    (an overflow: the step is skipped, the state is left bitwise unchanged);
  - gradients whose squares are fp32 subnormals, subnormal m and v;
  - whole buckets of fp16-subnormal gradients (the reduce rounds within the
    subnormal range);
  - fp32 params that round to fp16 subnormals, to +-65504 and past 65520 (inf);
  - gradients whose square overflows (v = inf, then u = m / inf);
  - eps-dominated updates (v = 0, tiny or zero gradients);
  - lr * u below the fp32 normal range (a subnormal lr).
Shard sizes: 65,536 (one vector launch per update; the device-resident flow
folds the partials inside the update) and 65,541 (element-wise tails; the fold
launch).
"""
import dataclasses

import numpy as np
import pytest
import torch

from gpu_common import compare, log, ls_of, hp_of, run_gpu, run_oracle
from zero_dp_sharded_amd import synth

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
FLOWS = ["sync", "gated", "device"]
SIZES = [65_536, 65_541]
CB = 16_384


def _randn(n, seed, dev):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    return torch.randn(n, generator=g, device=dev, dtype=torch.float32)


def _check(w, g, tag, **kw):
    st, oi = run_oracle(w, g, bucket_elems=CB, **kw)
    errs = compare(w, g, st, oi, tag)
    assert errs["bitwise"], (tag, errs)
    return st, oi


@pytest.mark.parametrize("flow", FLOWS)
@pytest.mark.parametrize("lp,R,scale,value", [
    ("bf16", 1, 0.5, 3e38),        # 3e38 * 2 > FLT_MAX
    ("bf16", 4, 0.125, 3e38),      # the mean 7.5e37 * 8 > FLT_MAX
    ("fp32", 1, 0.25, 1e38),       # 4e38
])
def test_unscaled_overflow_is_skipped(flow, lp, R, scale, value):
    """A finite stored gradient whose unscaled value is inf is an overflow: the
    step is skipped (state bitwise unchanged, t unchanged) and the scale halves."""
    w = dataclasses.replace(W["7.5b_bf16"], lp=lp, R=R, scale=scale, dynamic=1)
    ls = ls_of(w, min_scale=2.0 ** -6)
    n = 40_007

    def hook(s, bufs):
        if s == 1:
            bufs[0][12_345] = value
    log(f"[extremes] unscaled overflow {lp} R={R} scale={scale} flow={flow}")
    g = run_gpu(w, elems=n, steps=3, bucket_elems=CB, ls=ls, hook=hook, flow=flow)
    st, oi = _check(w, g, f"unscaled overflow {lp} {flow}", ls=ls)
    assert [i.overflow for i in g.infos] == [0, 1, 0]
    assert [i.step_t for i in g.infos] == [1, 1, 2]
    assert g.infos[1].scale_used == scale and g.infos[1].scale_next == scale / 2
    # the planted value is stored finite: only its unscaled value overflows
    c = g.contribs[1][0][12_345]
    assert np.isfinite(c) if lp == "fp32" else (int(c) & 0x7F80) != 0x7F80
    if flow == "sync":
        one = run_gpu(w, elems=n, steps=1, bucket_elems=CB, ls=ls)
        two = run_gpu(w, elems=n, steps=2, bucket_elems=CB, ls=ls, hook=hook)
        for k in ("master", "m", "v", "param"):
            a, b = getattr(one, k), getattr(two, k)
            if a is not None:
                assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), k


@pytest.mark.parametrize("flow", FLOWS)
@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("lp", ["bf16", "fp32"])
def test_subnormal_squares(flow, n, lp):
    """Gradients near 1e-20: g*g and (1-b2)*g*g are fp32 subnormals, so v, its
    bias-corrected value and the square root's input are subnormal."""
    w = dataclasses.replace(W["7.5b_bf16"], lp=lp, R=4, scale=1.0, dynamic=0, m_std=0.0,
                            v_std=0.0)

    def hook(s, bufs):
        for r, b in enumerate(bufs):
            b.copy_(_randn(b.numel(), 100 + 10 * s + r, b.device) * 1e-20)
    g = run_gpu(w, elems=n, steps=3, bucket_elems=CB, hook=hook, flow=flow)
    v = g.v[np.isfinite(g.v)]
    assert np.count_nonzero((v > 0) & (v < np.finfo(np.float32).tiny)) > n // 2
    _check(w, g, f"subnormal squares {lp} {n} {flow}")


@pytest.mark.parametrize("flow", FLOWS)
@pytest.mark.parametrize("n", SIZES)
def test_subnormal_moments(flow, n):
    """Subnormal m0 and v0 (and zeros of both signs) with gradients of 1e-19."""
    w = dataclasses.replace(W["7.5b_bf16"], R=3, scale=1.0, dynamic=0)

    def init(master, m, v):
        k = m.numel()
        m.copy_(_randn(k, 7, m.device) * 1e-39)
        v.copy_(_randn(k, 8, v.device).abs() * 1e-41)
        m[::97] = -0.0
        v[::89] = 0.0

    def hook(s, bufs):
        for r, b in enumerate(bufs):
            b.copy_(_randn(b.numel(), 200 + 10 * s + r, b.device) * 1e-19)
    g = run_gpu(w, elems=n, steps=3, bucket_elems=CB, hook=hook, init_hook=init, flow=flow)
    tiny = np.finfo(np.float32).tiny
    assert np.count_nonzero((np.abs(g.m0) > 0) & (np.abs(g.m0) < tiny)) > n // 2
    _check(w, g, f"subnormal moments {n} {flow}")


@pytest.mark.parametrize("flow", FLOWS)
@pytest.mark.parametrize("R", [3, 4])
def test_fp16_subnormal_buckets(flow, R):
    """Every contribution of every bucket an fp16 subnormal (k * 2^-24 for
    |k| < 1024): the fp32 sum is exact and the mean rounds within the fp16
    subnormal range (fp32(1/3) is inexact, 1/4 exact)."""
    w = dataclasses.replace(W["tiny"], R=R, scale=1.0, dynamic=0)
    n = 3 * CB + 5

    def hook(s, bufs):
        for r, b in enumerate(bufs):
            k = torch.randint(-1023, 1024, (b.numel(),), device=b.device,
                              generator=torch.Generator(device=b.device).manual_seed(
                                  300 + 10 * s + r))
            b.copy_(k.to(torch.float32) * 2.0 ** -24)
    g = run_gpu(w, elems=n, steps=3, bucket_elems=CB, hook=hook, flow=flow)
    e = (g.grad >> 10) & 0x1F
    assert np.all(e == 0)                               # every stored mean is subnormal or 0
    _check(w, g, f"fp16 subnormal buckets R={R} {flow}")


@pytest.mark.parametrize("flow", FLOWS)
@pytest.mark.parametrize("n", SIZES)
def test_params_at_fp16_limits(flow, n):
    """fp32 masters whose 2-byte copies are fp16 subnormals, sit at +-65504,
    or round past 65520 to +-inf (the cast of the definition: rne to fp16).
    lr 1e-8 keeps the masters in those ranges over the three steps."""
    w = dataclasses.replace(W["gpt2_1.5b"], R=4, lr=1e-8)

    def init(master, m, v):
        k = master.numel()
        q = k // 4
        x = _randn(k, 9, master.device)
        master[:q] = x[:q] * 3e-5                             # fp16 subnormal range
        master[q:2 * q] = 65504.0 + x[q:2 * q] * 12.0          # both sides of 65520
        master[2 * q:3 * q] = -65504.0 + x[2 * q:3 * q] * 12.0
        master[3 * q:] = x[3 * q:] * 6.1e-5                    # around the smallest normal
    g = run_gpu(w, elems=n, steps=3, bucket_elems=CB, hp=hp_of(w), init_hook=init, flow=flow)
    p = g.param
    assert np.count_nonzero((p & 0x7C00) == 0x7C00) > 0            # +-inf params
    assert np.count_nonzero(((p & 0x7C00) == 0) & ((p & 0x3FF) != 0)) > n // 8   # subnormals
    assert np.count_nonzero((p & 0x7FFF) == 0x7BFF) > 0            # +-65504
    _check(w, g, f"fp16 param limits {n} {flow}", hp=hp_of(w))


@pytest.mark.parametrize("flow", FLOWS)
@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("lp", ["bf16", "fp32"])
def test_gradient_square_overflows(flow, n, lp):
    """Finite gradients from 1e19 to 3e38: g*g overflows, v becomes inf, and
    the update takes u = m_hat / inf = 0 (plus the decoupled decay); v stays
    inf in later steps."""
    w = dataclasses.replace(W["7.5b_bf16"], lp=lp, R=4, scale=1.0, dynamic=0, weight_decay=0.01)

    def hook(s, bufs):
        b = bufs[s % len(bufs)]
        k = b.numel()
        mags = torch.tensor([1e19, 3e19, 1e25, 1e30, 1e35, 3e38], device=b.device)
        idx = torch.arange(0, k, 7, device=b.device)
        sign = torch.where(idx % 2 == 0, 1.0, -1.0)
        b[idx] = (mags[idx % 6] * sign).to(b.dtype)
    g = run_gpu(w, elems=n, steps=3, bucket_elems=CB, hook=hook, flow=flow)
    assert all(i.overflow == 0 for i in g.infos)
    assert np.count_nonzero(np.isinf(g.v)) > n // 20
    _check(w, g, f"square overflow {lp} {n} {flow}")


@pytest.mark.parametrize("flow", FLOWS)
@pytest.mark.parametrize("n", SIZES)
def test_eps_dominated_updates(flow, n):
    """m = v = 0 and gradients of 1e-12 or exactly 0: sqrt(v_hat) is far below
    eps, so the denominator is eps and zero gradients leave u = 0."""
    w = dataclasses.replace(W["7.5b_bf16"], R=2, scale=1.0, dynamic=0, m_std=0.0, v_std=0.0)

    def hook(s, bufs):
        for r, b in enumerate(bufs):
            b.copy_(_randn(b.numel(), 400 + 10 * s + r, b.device) * 1e-12)
            b[::5] = 0.0
    g = run_gpu(w, elems=n, steps=3, bucket_elems=CB, hook=hook, flow=flow)
    _check(w, g, f"eps dominated {n} {flow}")


@pytest.mark.parametrize("flow", FLOWS)
@pytest.mark.parametrize("n", SIZES)
def test_lr_times_update_underflows(flow, n):
    """A subnormal lr (fp32(1e-38)): lr * u is subnormal or 0 and vanishes
    against normal masters, but moves subnormal ones."""
    w = dataclasses.replace(W["gpt2_1.5b"], R=4, lr=1e-38, weight_decay=0.0)

    def init(master, m, v):
        master[::3] = _randn(master[::3].numel(), 11, master.device) * 1e-38
    g = run_gpu(w, elems=n, steps=3, bucket_elems=CB, hp=hp_of(w), init_hook=init, flow=flow)
    moved = g.master != g.master0
    assert np.count_nonzero(moved) > 0
    assert np.all(np.abs(g.master0[moved]) < 1e-30)
    _check(w, g, f"lr*u underflow {n} {flow}", hp=hp_of(w))
