"""GPU parity of the optimizer and storage variants against the oracle: 4-byte
storage (b = 4; fp32 grads, the fp32 master is the parameter) with Adam
(K = 8) and with SGD with and without momentum (K = 4 and K = 0, the
blog.vllbc.top page's extension group C), and SGD on 2-byte mixed-precision
storage.  Sizes span several tiles with ragged tails and ragged last buckets;
contribution counts cover the unrolled and the generic reduce; misaligned
bases cover the peeled heads; an injected +inf covers skip and loss-scale
halving."""
import dataclasses

import numpy as np
import pytest
import torch

import zero_dp_sharded_amd as zs
from gpu_common import compare, hp_of, log, ls_of, run_gpu, run_oracle
from zero_dp_sharded_amd import synth

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
C1, C2 = W["c1_7.5b_sgdm"], W["c2_1.5b_sgd"]


def _w(base, **over):
    return dataclasses.replace(base, **over)


FP32_ADAM = _w(W["gpt2_1.5b"], lp="fp32", scale=1.0, dynamic=0)
VARIANTS = {
    "c1_sgdm_fp32": C1,
    "c2_sgd_fp32": C2,
    "sgd_wd_fp32": _w(C2, weight_decay=1e-3),
    "adam_fp32": FP32_ADAM,
    "adam_l2_fp32": FP32_ADAM,
    "sgdm_fp16": _w(C1, lp="fp16", scale=1024.0, dynamic=1),
    "sgd_bf16": _w(C2, lp="bf16", weight_decay=1e-2),
    "sgdm_fp32_scaled": _w(C1, scale=512.0, dynamic=1),
}


def _hp(name, w):
    if name == "adam_l2_fp32":
        return hp_of(w, weight_decay=0.01, wd_mode=zs.ZERO_WD_L2)
    return hp_of(w)


@pytest.mark.parametrize("name", sorted(VARIANTS))
@pytest.mark.parametrize("elems,cb,R", [(300_007, 65_536, 4), (100_003, 33_333, 3)])
def test_variant_parity(name, elems, cb, R):
    w = _w(VARIANTS[name], R=R, steps=4)
    hp = _hp(name, w)
    log(f"[variants] {name} elems={elems} cb={cb} R={R}")
    g = run_gpu(w, elems=elems, bucket_elems=cb, hp=hp)
    st, oi = run_oracle(w, g, bucket_elems=cb, hp=hp)
    errs = compare(w, g, st, oi, name)
    log(errs)
    assert errs["bitwise"]


@pytest.mark.parametrize("name", ["c1_sgdm_fp32", "adam_fp32", "sgdm_fp16"])
def test_variant_overflow_skips(name):
    """+inf in contribution 0 at step 1: the step is skipped with every state
    unchanged, and with dynamic scaling the scale halves."""
    w = _w(VARIANTS[name], inject_step=1, steps=4, dynamic=1, scale=64.0)
    hp = _hp(name, w)
    g = run_gpu(w, elems=200_003, bucket_elems=50_000, hp=hp)
    st, oi = run_oracle(w, g, bucket_elems=50_000, hp=hp)
    compare(w, g, st, oi, name)
    assert [i.overflow for i in g.infos] == [0, 1, 0, 0]
    assert [i.step_t for i in g.infos] == [1, 1, 2, 3]
    assert [i.scale_used for i in g.infos] == [64.0, 64.0, 32.0, 32.0]


@pytest.mark.parametrize("name", ["c1_sgdm_fp32", "c2_sgd_fp32", "adam_fp32", "sgdm_fp16"])
def test_variant_misaligned(name):
    """Every array at an odd element offset: the peeled heads and tails and the
    element-wise fallback give the same result as the oracle."""
    w = _w(VARIANTS[name], steps=3)
    hp = _hp(name, w)
    offs = [dict(master=1, m=3, v=2, grad=1, param=3, contrib=2),
            dict(master=0, m=0, v=0, grad=1, param=0, contrib=1),
            dict(contrib=3)]
    for k, o in enumerate(offs):
        g = run_gpu(w, elems=70_001, bucket_elems=20_000, hp=hp, offsets=o)
        st, oi = run_oracle(w, g, bucket_elems=20_000, hp=hp)
        assert compare(w, g, st, oi, f"{name} offsets {k}")["bitwise"], (name, o)


@pytest.mark.parametrize("name", ["c1_sgdm_fp32", "c2_sgd_fp32", "adam_fp32", "sgdm_fp16"])
def test_variant_gated_equals_sync(name):
    w = _w(VARIANTS[name], inject_step=2, steps=4, dynamic=1, scale=8.0)
    hp = _hp(name, w)
    a = run_gpu(w, elems=150_001, bucket_elems=40_000, hp=hp, flow="sync")
    b = run_gpu(w, elems=150_001, bucket_elems=40_000, hp=hp, flow="gated")
    assert [(i.overflow, i.step_t, i.scale_next) for i in a.infos] == \
        [(i.overflow, i.step_t, i.scale_next) for i in b.infos]
    for k in ("master", "m", "v", "grad", "param"):
        x, y = getattr(a, k), getattr(b, k)
        assert (x is None) == (y is None), k
        if x is not None:
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), k
    st, oi = run_oracle(w, b, bucket_elems=40_000, hp=hp)
    assert compare(w, b, st, oi, f"{name} gated")["bitwise"]


@pytest.mark.parametrize("elems", [1, 3, 4, 5, 255, 2049, 4097])
def test_fp32_ragged_sizes(elems):
    for w in (C1, FP32_ADAM):
        w = _w(w, steps=2)
        cb = max(1, elems // 2)
        g = run_gpu(w, elems=elems, bucket_elems=cb)
        st, oi = run_oracle(w, g, bucket_elems=cb)
        assert compare(w, g, st, oi, f"fp32 ragged {elems}")["bitwise"]


def test_optimizer_mismatch_and_hparam_checks():
    dev = torch.device("cuda", 0)
    n = 4096
    master = torch.zeros(n, device=dev)
    mom = torch.zeros(n, device=dev)
    v = torch.zeros(n, device=dev)
    g32 = torch.ones(n, device=dev)
    ls = zs.LossScaleCfg(init_scale=1.0, dynamic=0)
    hs = zs.zero_shard_init_sgd(master, mom, g32, None, psi=n, nd=1, rank=0, bucket_elems=n,
                                hp=zs.SGDHParams(lr=0.1, momentum=0.9), ls=ls)
    ha = zs.zero_shard_init(torch.zeros(n, device=dev), torch.zeros(n, device=dev), v,
                            torch.ones(n, device=dev), None, psi=n, nd=1, rank=0, bucket_elems=n,
                            hp=zs.AdamHParams(), ls=ls)
    try:
        zs.zero_overflow_check(hs)
        zs.zero_overflow_check(ha)
        for fn, h in ((zs.zero_adam_step, hs), (zs.zero_sgd_step, ha)):
            with pytest.raises(zs.ZeroError) as e:
                fn(h)
            assert e.value.status == zs.ZERO_ERR_STATE
        with pytest.raises(zs.ZeroError) as e:
            zs.zero_sgd_step(hs, zs.SGDHParams(lr=0.1, momentum=1.5))
        assert e.value.status == zs.ZERO_ERR_INVALID_ARG
        info = zs.zero_sgd_step(hs)
        assert info.step_t == 1 and info.overflow == 0
        assert zs.zero_adam_step(ha).step_t == 1
        torch.cuda.synchronize()
        # p = 0 - 0.1 * (0.9 * 0 + 1)
        assert torch.equal(master, torch.full_like(master, np.float32(0.0) - np.float32(0.1)))
        assert torch.equal(mom, torch.ones_like(mom))
        with pytest.raises(zs.ZeroError) as e:
            zs.zero_adam_step_gated(hs)
        assert e.value.status == zs.ZERO_ERR_STATE
        with pytest.raises(zs.ZeroError) as e:
            zs.zero_sgd_step_gated(ha)
        assert e.value.status == zs.ZERO_ERR_STATE
    finally:
        zs.zero_shard_destroy(hs)
        zs.zero_shard_destroy(ha)


def test_plain_sgd_rejects_momentum_override():
    dev = torch.device("cuda", 0)
    n = 1000
    master = torch.zeros(n, device=dev)
    g = torch.ones(n, device=dev)
    h = zs.zero_shard_init_sgd(master, None, g, None, psi=n, nd=1, rank=0, bucket_elems=n,
                               hp=zs.SGDHParams(lr=0.5), ls=zs.LossScaleCfg(init_scale=2.0,
                                                                            dynamic=0))
    try:
        zs.zero_overflow_check(h)
        with pytest.raises(zs.ZeroError) as e:
            zs.zero_sgd_step(h, zs.SGDHParams(lr=0.5, momentum=0.5))
        assert e.value.status == zs.ZERO_ERR_INVALID_ARG
        zs.zero_sgd_step(h)
        torch.cuda.synchronize()
        # g = 1 * (1/2); p = 0 - 0.5 * 0.5
        assert torch.equal(master, torch.full_like(master, -0.25))
    finally:
        zs.zero_shard_destroy(h)
