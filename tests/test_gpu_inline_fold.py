"""GPU parity of the fold inside the update, the device-resident step of small
shards.  When a step has at most 1024 per-workgroup partials and the update is
one vector launch over the whole shard, every update workgroup folds the
partials itself in the fold kernel's order and decides the step from the state
snapshot the step's reduce took, and workgroup 0 advances the device counters.  The results must be bitwise
those of the synchronous flow (fold kernel, host decision) and match the
oracle, through skipped steps, loss-scale changes and clipping; shapes just
past the limits must take the fold launch instead; and graph replays of such
steps must equal eager ones after every replay.

The partial counts below follow the reduce's shape for shards of at most
8,388,608 elements: 256-lane workgroups with one run of 16 bytes per lane, so
2048 elements per workgroup with 2-byte storage and 1024 with fp32 storage,
for any contribution count."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import zero_dp_sharded_amd as zs
from gpu_common import (LP_CODE, compare, expect_inline_folds, f32, hp_of, log, ls_of, oracle_hp,
                        oracle_ls, run_gpu, run_oracle, stored)
from zero_dp_sharded_amd import synth

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _w(base, **over):
    return dataclasses.replace(base, **over)


# name -> (workload, shard elements, C_B): 256 partials (one partial per fold
# lane), 512 (two per lane), 513 (the first count folded with four loads per
# lane) or 1024 (four per lane, the limit)
CASES = {
    "adam_fp16_r4": (_w(W["tiny"], steps=5), 524_288, 131_072),       # 4 x 64
    "adam_fp16_r4_512": (_w(W["tiny"], steps=5), 1_048_576, 1_048_576),   # 512
    "adam_fp16_r4_513": (_w(W["tiny"], steps=5), 1_050_624, 1_050_624),   # 513
    "adam_fp16_r4_1024": (_w(W["tiny"], steps=5), 2_097_152, 2_097_152),  # 1024
    "adam_bf16_r8": (_w(W["7.5b_bf16"], steps=5), 524_288, 262_144),  # 2 x 128
    "adam_fp16_r16": (_w(W["13b_inf"], steps=5, inject_step=None), 524_288, 524_288),  # 256
    "sgdm_fp32_r8": (_w(W["c1_7.5b_sgdm"], steps=5), 262_144, 262_144),  # 256
    "sgdm_fp32_r8_512": (_w(W["c1_7.5b_sgdm"], steps=5), 524_288, 131_072),  # 4 x 128
    "sgd_fp32_r8": (_w(W["c2_1.5b_sgd"], steps=5), 262_144, 131_072),  # 2 x 128
    "sgdm_fp32_r8_1024": (_w(W["c1_7.5b_sgdm"], steps=5), 1_048_576, 262_144),  # 4 x 256
}


def _same(a, b, tag):
    assert [(i.overflow, i.step_t, i.scale_used, i.scale_next) for i in a.infos] == \
        [(i.overflow, i.step_t, i.scale_used, i.scale_next) for i in b.infos], tag
    for x, y in zip(a.infos, b.infos):
        assert x.grad_norm == y.grad_norm or (np.isnan(x.grad_norm) and np.isnan(y.grad_norm)), tag
    for k in ("master", "m", "v", "grad", "param"):
        x, y = getattr(a, k), getattr(b, k)
        assert (x is None) == (y is None), (tag, k)
        if x is not None:
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), (tag, k)


def _typical_norm(w, elems):
    return w.grad_std / np.sqrt(w.R) * np.sqrt(elems)


@pytest.mark.parametrize("clip", [False, True])
@pytest.mark.parametrize("name", sorted(CASES))
def test_inline_fold_equals_sync_and_oracle(name, clip):
    """An overflow at step 2 (skip, scale halved) among 5 steps, with and
    without clipping: the device-resident flow folds inside the update on
    every step and equals the synchronous flow bitwise and the oracle."""
    base, elems, cb = CASES[name]
    w = _w(base, inject_step=1, dynamic=1, scale=16.0)
    max_norm = 0.4 * _typical_norm(w, elems) if clip else 0.0
    log(f"[inline] {name} clip={clip} S={elems} C_B={cb}")
    n_sync, n_dev = [], []
    a = run_gpu(w, elems=elems, bucket_elems=cb, flow="sync", max_norm=max_norm,
                inline_folds=n_sync)
    b = run_gpu(w, elems=elems, bucket_elems=cb, flow="device", max_norm=max_norm,
                inline_folds=n_dev)
    assert n_sync == [0]
    expect_inline_folds(n_dev, [w.steps], name)
    assert [i.overflow for i in b.infos] == [0, 1, 0, 0, 0]
    _same(a, b, f"{name} clip={clip}")
    st, oi = run_oracle(w, b, bucket_elems=cb, max_norm=max_norm)
    compare(w, b, st, oi, f"inline {name} clip={clip}")


@pytest.mark.parametrize("name", sorted(CASES))
def test_inline_fold_uninterrupted_steps(name):
    """Five steps on the device alone (each step's snapshot must be the state
    the previous step left): the last step's result and the final state equal
    the synchronous flow's."""
    base, elems, cb = CASES[name]
    w = _w(base, inject_step=2, dynamic=1, scale=64.0)
    a = run_gpu(w, elems=elems, bucket_elems=cb, flow="sync")
    scales = [i.scale_used for i in a.infos]
    n = []
    c = run_gpu(w, elems=elems, bucket_elems=cb, flow="device_run",
                scale_of=lambda s: scales[s], inline_folds=n)
    expect_inline_folds(n, [w.steps], name)
    last, ref = c.infos[-1], a.infos[-1]
    assert (last.overflow, last.step_t, last.scale_used, last.scale_next, last.grad_norm) == \
        (ref.overflow, ref.step_t, ref.scale_used, ref.scale_next, ref.grad_norm)
    for k in ("master", "m", "v", "grad", "param"):
        x, y = getattr(a, k), getattr(c, k)
        if x is not None:
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), (name, k)


@pytest.mark.parametrize("elems,cb,why", [
    (2_099_200, 2_099_200, "1025 partials"),         # 262,400 runs / 256 per workgroup
    (200_002, 200_002, "update with a scalar tail"),  # 98 partials, S not a multiple of 4
])
def test_past_the_limits_takes_the_fold_launch(elems, cb, why):
    """Shapes just past the inline fold's limits use the fold launch and still
    equal the synchronous flow bitwise."""
    w = _w(W["tiny"], steps=3, inject_step=1, dynamic=1, scale=16.0)
    n = []
    a = run_gpu(w, elems=elems, bucket_elems=cb, flow="sync")
    b = run_gpu(w, elems=elems, bucket_elems=cb, flow="device", inline_folds=n)
    log(f"[inline] {why}: S={elems} inline steps {n}")
    assert n == [0], (why, n)
    _same(a, b, why)


def test_misaligned_update_takes_the_fold_launch():
    """A master array that starts one element past a 16-byte boundary gives the
    update a scalar head: no inline fold, same results as the host flow."""
    base, elems, cb = CASES["adam_fp16_r4"]
    w = _w(base, steps=3)
    n = []
    a = run_gpu(w, elems=elems, bucket_elems=cb, flow="sync", offsets={"master": 1})
    b = run_gpu(w, elems=elems, bucket_elems=cb, flow="device", offsets={"master": 1},
                inline_folds=n)
    assert n == [0]
    _same(a, b, "misaligned master")


@pytest.mark.parametrize("name", ["adam_fp16_r4", "sgdm_fp32_r8", "adam_fp16_r4_512",
                                  "adam_fp16_r4_1024"])
def test_inline_fold_graph_replays(name):
    """Three inline-fold steps captured in one CUDA graph, replayed twice with
    eager refills of the contributions between replays (an overflow planted
    in the second batch): after every replay the state equals six eager
    device-resident steps, bitwise, and the oracle's."""
    base, elems, cb = CASES[name]
    w = _w(base, steps=6, dynamic=1, scale=32.0)
    dev = torch.device("cuda", 0)
    hp = hp_of(w)
    K = 3

    def make():
        master0, m0, v0 = synth.init_state(w, dev, 0, elems=elems)
        master = master0.clone()
        m = m0.clone() if w.has_m else None
        v = v0.clone() if w.has_v else None
        grad = torch.zeros(elems, dtype=w.torch_lp, device=dev)
        param = None if w.lp == "fp32" else master0.to(w.torch_lp)
        if w.opt == "sgd":
            h = zs.zero_shard_init_sgd(master, m, grad, param, psi=elems * w.nd, nd=w.nd, rank=0,
                                       bucket_elems=cb, hp=hp, ls=ls_of(w))
        else:
            h = zs.zero_shard_init(master, m, v, grad, param, psi=elems * w.nd, nd=w.nd, rank=0,
                                   bucket_elems=cb, hp=hp, ls=ls_of(w))
        return h, dict(master=master, m=m, v=v, param=param, master0=master0, m0=m0, v0=v0)

    bufs = synth.alloc_contribs(w, dev, elems=elems)
    ha, A = make()
    hb, B = make()
    ohp, ols = oracle_hp(hp), oracle_ls(ls_of(w))
    ost = oracle.new_state(LP_CODE[w.lp], f32(A["master0"]), f32(A["m0"]) if w.has_m else None,
                           f32(A["v0"]) if w.has_v else None, ohp, ols)
    log(f"[inline graph x{K}] {name}")
    try:
        zs.zero_device_begin(ha)
        zs.zero_device_begin(hb)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(K):
                zs.zero_step_device(hb, bufs)
        torch.cuda.synchronize()
        scale = w.scale
        for rep in range(w.steps // K):
            synth.fill_contribs(w, bufs, rep, scale, seed=0)
            if rep == 1:
                bufs[0][elems // 2 + 1] = float("inf")
            torch.cuda.synchronize()
            cs = [stored(b) for b in bufs]
            for _ in range(K):
                zs.zero_step_device(ha, bufs)
                oi = oracle.step(ost, cs, cb, ohp, ols)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for k in ("master", "m", "v", "param"):
                if A[k] is not None:
                    view = torch.int32 if A[k].dtype == torch.float32 else torch.int16
                    assert torch.equal(A[k].view(view), B[k].view(view)), (name, rep, k)
            log(f"[inline graph] replay {rep}: oracle t={ost.t} scale={ost.scale}")
            scale = ost.scale
        ia, ib = zs.zero_device_end(ha), zs.zero_device_end(hb)
        expect_inline_folds(zs.zero_shard_inline_folds(ha), w.steps, name)
        expect_inline_folds(zs.zero_shard_inline_folds(hb), K, name)   # captured once, replayed twice
        assert (ia.overflow, ia.step_t, ia.scale_next) == (ib.overflow, ib.step_t, ib.scale_next)
        assert ia.overflow == 1 and np.isnan(ia.grad_norm) and np.isnan(ib.grad_norm)
        # three overflowing steps in the second batch: t stays at 3, the scale
        # halves three times
        assert (ib.step_t, ib.scale_next) == (ost.t, ost.scale) == (3, w.scale / 8)
        assert np.array_equal(f32(B["master"]).view(np.uint32), ost.master.view(np.uint32))
        del graph
    finally:
        zs.zero_shard_destroy(ha)
        zs.zero_shard_destroy(hb)


def test_inline_folds_needs_a_count_pointer():
    w = W["tiny"]
    dev = torch.device("cuda", 0)
    n = 4096
    master0, m0, v0 = synth.init_state(w, dev, 0, elems=n)
    grad = torch.zeros(n, dtype=torch.float16, device=dev)
    param = master0.to(torch.float16)
    h = zs.zero_shard_init(master0, m0, v0, grad, param, psi=n * w.nd, nd=w.nd, rank=0,
                           bucket_elems=n, hp=hp_of(w), ls=ls_of(w))
    try:
        assert zs.lib().zero_shard_inline_folds(h, None) == zs.ZERO_ERR_INVALID_ARG
        assert zs.zero_shard_inline_folds(h) == 0
    finally:
        zs.zero_shard_destroy(h)
