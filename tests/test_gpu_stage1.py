"""P_os (optimizer-state partitioning, stage 1) on the GPU.

Every rank holds the full all-reduced gradient and updates only its 1/Nd
slice of the optimizer state, writing its slice of the full parameter
all-gather buffer ("ZeRO：大模型训练的内存优化革命" 3.1.1; the blog.vllbc.top page's
stage descriptions).  Here the Nd ranks are simulated on one GPU: each is a
handle whose grad_shard and param_shard point into the full gradient and the
full all-gather buffer at offset rank * S, and whose check scans that slice
(no bucket reduce).  The ranks share the skip decision through
zero_overflow_merge.  The pages' invariant: the concatenated slices equal one
unsharded update, bitwise.
"""
import numpy as np
import pytest
import torch

import oracle
import zero_dp_sharded_amd as zs
from gpu_common import f32, u16

pytestmark = pytest.mark.gpu


def _run_pos(psi, nd, steps, inject=None, seed=3, lr=1e-3, wd=0.01, scale=1024.0, max_norm=0.0):
    """Simulate nd P_os ranks; returns the all-gather buffer, fp32 states, infos
    per step (rank 0's) and the per-step full gradients (host bits)."""
    dev = torch.device("cuda", 0)
    S = -(-psi // nd)
    n = nd * S                                   # padded flat length
    gen = torch.Generator(device=dev).manual_seed(seed)
    master = torch.zeros(n, device=dev)
    master[:psi] = torch.randn(psi, generator=gen, device=dev) * 0.02
    m = torch.zeros(n, device=dev)
    v = torch.zeros(n, device=dev)
    grad = torch.zeros(n, dtype=torch.float16, device=dev)
    allgather = torch.zeros(n, dtype=torch.float16, device=dev)
    allgather.copy_(master.half())
    master0 = f32(master).copy()
    hp = zs.AdamHParams(lr=lr, weight_decay=wd)
    ls = zs.LossScaleCfg(init_scale=scale)
    hs = [zs.zero_shard_init(master[r * S:], m[r * S:], v[r * S:], grad[r * S:], allgather[r * S:],
                             psi=psi, nd=nd, rank=r, bucket_elems=S, hp=hp, ls=ls)
          for r in range(nd)]
    infos, grads = [], []
    try:
        for h in hs:
            if max_norm:
                zs.zero_shard_set_clip(h, max_norm)
        cur = scale
        for s in range(steps):
            g = torch.randn(psi, generator=gen, device=dev) * (1e-3 * cur)
            grad[:psi] = g.half()
            if inject is not None and inject[0] == s:
                grad[inject[1]] = float("inf")
            grads.append(u16(grad[:psi]))
            local = [zs.zero_overflow_check(h) for h in hs]
            flag = max(i.overflow for i in local)
            norm = float(np.sqrt(sum(i.grad_norm ** 2 for i in local))) if not flag else float("nan")
            merged = [zs.zero_overflow_merge(h, flag, norm) for h in hs]
            outs = [zs.zero_adam_step(h) for h in hs]
            assert len({(o.overflow, o.step_t, o.scale_next) for o in outs}) == 1
            infos.append((local, merged[0], outs[0]))
            cur = outs[0].scale_next
        torch.cuda.synchronize()
    finally:
        for h in hs:
            zs.zero_shard_destroy(h)
    return dict(allgather=u16(allgather[:psi]), master=f32(master[:psi]), m=f32(m[:psi]),
                v=f32(v[:psi]), pad=f32(master[psi:]), infos=infos, grads=grads,
                master0=master0[:psi])


@pytest.mark.parametrize("psi,nd", [(1_000_003, 4), (1_000_003, 7), (262_144, 1)])
def test_pos_ranks_concat_equals_unsharded_and_oracle(psi, nd):
    steps = 3
    got = _run_pos(psi, nd, steps)
    ref = _run_pos(psi, 1, steps)
    for k in ("allgather", "master", "m", "v"):
        assert np.array_equal(got[k].view(np.uint8), ref[k].view(np.uint8)), k
    assert np.all(got["pad"] == 0.0)              # padded tail of the last rank stays zero
    # oracle on the flat problem with the same gradients
    hp = oracle.AdamHP(lr=1e-3, weight_decay=0.01)
    ls = oracle.LossScale(init_scale=1024.0)
    st = oracle.new_state(oracle.FP16, got["master0"], np.zeros(psi), np.zeros(psi), hp, ls)
    for s, g in enumerate(got["grads"]):
        flag, ss = oracle.flag_sumsq(oracle.FP16, g, st.scale)
        assert flag == got["infos"][s][2].overflow
        assert got["infos"][s][1].grad_norm == pytest.approx(np.sqrt(ss), rel=1e-9)
        st.t += 1
        oracle.adam_update(oracle.FP16, g, st.master, st.m, st.v, st.param,
                           oracle.adam_scalars(hp, st.t, st.scale))
    assert np.array_equal(got["master"].view(np.uint32), st.master.view(np.uint32))
    assert np.array_equal(got["allgather"], st.param)


def test_pos_overflow_in_one_slice_skips_every_rank():
    psi, nd = 400_009, 4
    S = -(-psi // nd)
    where = 2 * S + 17                            # inside rank 2's slice
    got = _run_pos(psi, nd, 3, inject=(1, where))
    local, merged, out = got["infos"][1]
    assert [i.overflow for i in local] == [0, 0, 1, 0]
    assert merged.overflow == 1 and out.skipped == 1 and out.step_t == 1
    assert out.scale_next == 512.0
    ref = _run_pos(psi, 1, 3, inject=(1, where))
    for k in ("allgather", "master", "m", "v"):
        assert np.array_equal(got[k].view(np.uint8), ref[k].view(np.uint8)), k
    # step 2 (after the skip) is the second applied step
    assert got["infos"][2][2].step_t == 2


def test_merge_argument_checks():
    n = 4096
    dev = torch.device("cuda", 0)
    t = [torch.zeros(n, device=dev) for _ in range(3)]
    g = torch.zeros(n, dtype=torch.float16, device=dev)
    p = torch.zeros(n, dtype=torch.float16, device=dev)
    g[5] = float("inf")
    h = zs.zero_shard_init(*t, g, p, psi=n, nd=1, rank=0, bucket_elems=n,
                           hp=zs.AdamHParams(), ls=zs.LossScaleCfg(init_scale=8.0))
    try:
        with pytest.raises(zs.ZeroError) as e:
            zs.zero_overflow_merge(h, 1, 1.0)          # before the check
        assert e.value.status == zs.ZERO_ERR_STATE
        assert zs.zero_overflow_check(h).overflow == 1
        with pytest.raises(zs.ZeroError) as e:
            zs.zero_overflow_merge(h, 0, 1.0)          # cannot clear a local overflow
        assert e.value.status == zs.ZERO_ERR_INVALID_ARG
        with pytest.raises(zs.ZeroError):
            zs.zero_overflow_merge(h, 2, 1.0)
        info = zs.zero_overflow_merge(h, 1, 3.0)
        assert info.overflow == 1 and info.grad_norm == 3.0 and info.scale_next == 4.0
        assert zs.zero_adam_step(h).skipped == 1
    finally:
        zs.zero_shard_destroy(h)


def test_merge_refuses_bad_global_norms():
    """An applied step takes the global norm for its clipping coefficient, so a
    clean merge refuses a norm that is NaN, infinite, negative or below this
    rank's own norm (INVALID_ARG, the handle unchanged); an overflowing merge
    only reports it."""
    n = 4096
    dev = torch.device("cuda", 0)
    t = [torch.zeros(n, device=dev) for _ in range(3)]
    g = torch.full((n,), 0.5, dtype=torch.float16, device=dev)
    p = torch.zeros(n, dtype=torch.float16, device=dev)
    h = zs.zero_shard_init(*t, g, p, psi=n, nd=1, rank=0, bucket_elems=n,
                           hp=zs.AdamHParams(), ls=zs.LossScaleCfg(init_scale=1.0))
    try:
        zs.zero_shard_set_clip(h, 1.0)
        chk = zs.zero_overflow_check(h)
        own = chk.grad_norm
        assert chk.overflow == 0 and own == pytest.approx(32.0)     # sqrt(4096 * 0.25)
        for bad in (float("nan"), float("inf"), -1.0, 0.5 * own, own * (1 - 1e-6)):
            with pytest.raises(zs.ZeroError) as e:
                zs.zero_overflow_merge(h, 0, bad)
            assert e.value.status == zs.ZERO_ERR_INVALID_ARG, bad
            assert zs.zero_overflow_check(h).grad_norm == own          # handle unchanged
        info = zs.zero_overflow_merge(h, 0, own * 2.0)
        assert info.overflow == 0 and info.grad_norm == own * 2.0
        assert zs.zero_adam_step(h).step_t == 1
        # an overflowing global step: the norm is only reported
        zs.zero_overflow_check(h)
        info = zs.zero_overflow_merge(h, 1, float("nan"))
        assert info.overflow == 1 and np.isnan(info.grad_norm)
        assert zs.zero_adam_step(h).skipped == 1
    finally:
        zs.zero_shard_destroy(h)


def test_pos_clipping_uses_the_merged_global_norm():
    """With clipping on, every rank clips with the coefficient of the merged
    global norm: the concatenated slices match the oracle's unsharded clipped
    update (the coefficient comes from the host after the merge, so the bar is
    the fp32 tolerance), as does a single rank clipping with its own norm."""
    psi, nd, steps = 600_011, 4, 3
    max_norm = 0.2                       # well below the typical norm (~0.8 here)
    got = _run_pos(psi, nd, steps, max_norm=max_norm)
    hp = oracle.AdamHP(lr=1e-3, weight_decay=0.01)
    ls = oracle.LossScale(init_scale=1024.0)
    st = oracle.new_state(oracle.FP16, got["master0"], np.zeros(psi), np.zeros(psi), hp, ls)
    for s, g in enumerate(got["grads"]):
        flag, ss = oracle.flag_sumsq(oracle.FP16, g, st.scale)
        assert got["infos"][s][1].grad_norm == pytest.approx(np.sqrt(ss), rel=1e-9)
        assert oracle.clip_coef(ss, max_norm) < 1.0
        st.t += 1
        oracle.adam_update(oracle.FP16, g, st.master, st.m, st.v, st.param,
                           oracle.adam_scalars(hp, st.t, st.scale, oracle.clip_coef(ss, max_norm)))
    rel = np.max(np.abs(got["master"].astype(np.float64) - st.master) /
                 np.maximum(np.abs(st.master), 1.2e-38))
    assert rel <= 1e-6
    one = _run_pos(psi, 1, steps, max_norm=max_norm)       # one rank: its own norm is global
    assert np.max(np.abs(one["master"].astype(np.float64) - st.master) /
                  np.maximum(np.abs(st.master), 1.2e-38)) <= 1e-6
