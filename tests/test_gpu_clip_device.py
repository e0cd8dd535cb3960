"""GPU parity of global-norm clipping and of the device-resident flow.

Clipping: every flow (synchronous check, device-gated, device-resident)
against the oracle with the coefficient active, including a skipped step.
The device computes the coefficient from its fixed-order norm and the oracle
from its sequential one, so the bar is the fp32 tolerance, not bitwise.

Device-resident flow: the same steps as the host flows, bitwise, whether the
flow is ended after every step or runs several steps on the device alone; the
state machine refuses host-flow calls while it is active; and a step captured
in a HIP graph (torch.cuda.CUDAGraph) and replayed, with eager refills of the
contributions and synchronisations between replays, equals the eager
device-resident run after every replay.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import zero_dp_sharded_amd as zs
from gpu_common import (LP_CODE, compare, expect_inline_folds, f32, hp_of, log, ls_of, oracle_hp,
                        oracle_ls, run_gpu, run_oracle, stored, u16)
from zero_dp_sharded_amd import synth

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _w(base, **over):
    return dataclasses.replace(base, **over)


CASES = {
    "adam_fp16": _w(W["gpt2_1.5b"], steps=4),
    "adam_bf16_l2": _w(W["7.5b_bf16"], steps=4),
    "sgdm_fp32": _w(W["c1_7.5b_sgdm"], steps=4),
    "sgd_fp32": _w(W["c2_1.5b_sgd"], steps=4),
}


def _hp(name, w):
    if name == "adam_bf16_l2":
        return hp_of(w, weight_decay=0.01, wd_mode=zs.ZERO_WD_L2)
    return hp_of(w)


def _typical_norm(w, elems):
    """Expected unscaled norm of a step's mean gradient: grad_std/sqrt(R) per
    element."""
    return w.grad_std / np.sqrt(w.R) * np.sqrt(elems)


@pytest.mark.parametrize("flow", ["sync", "gated", "device"])
@pytest.mark.parametrize("name", sorted(CASES))
def test_clipping_parity(name, flow):
    w = CASES[name]
    elems, cb = 200_003, 65_536
    hp = _hp(name, w)
    max_norm = 0.3 * _typical_norm(w, elems)
    log(f"[clip] {name} flow={flow} max_norm={max_norm:.4g}")
    g = run_gpu(w, elems=elems, bucket_elems=cb, hp=hp, flow=flow, max_norm=max_norm)
    st, oi = run_oracle(w, g, bucket_elems=cb, hp=hp, max_norm=max_norm)
    errs = compare(w, g, st, oi, f"clip {name} {flow}")
    log(errs)
    # the coefficient was active: the update differs from the unclipped one
    g0 = run_gpu(w, elems=elems, bucket_elems=cb, hp=hp, flow=flow)
    assert not np.array_equal(g.master, g0.master)


@pytest.mark.parametrize("flow", ["sync", "gated", "device"])
def test_clipping_with_overflow_step(flow):
    w = _w(CASES["adam_fp16"], inject_step=1, steps=4, scale=64.0)
    elems, cb = 100_003, 40_000
    max_norm = 0.5 * _typical_norm(w, elems)
    g = run_gpu(w, elems=elems, bucket_elems=cb, flow=flow, max_norm=max_norm)
    st, oi = run_oracle(w, g, bucket_elems=cb, max_norm=max_norm)
    compare(w, g, st, oi, f"clip overflow {flow}")
    assert [i.overflow for i in g.infos] == [0, 1, 0, 0]
    assert [i.scale_used for i in g.infos] == [64.0, 64.0, 32.0, 32.0]


def test_clip_off_and_huge_limit_are_bitwise_unclipped():
    w = CASES["adam_fp16"]
    a = run_gpu(w, elems=150_001, bucket_elems=50_000)
    b = run_gpu(w, elems=150_001, bucket_elems=50_000, max_norm=1e30)
    assert np.array_equal(a.master.view(np.uint32), b.master.view(np.uint32))
    assert np.array_equal(a.param, b.param)


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("clip", [False, True])
def test_device_flow_equals_sync_bitwise(name, clip):
    w = _w(CASES[name], inject_step=2, steps=5, dynamic=1, scale=16.0)
    elems, cb = 170_001, 50_000
    hp = _hp(name, w)
    max_norm = 0.4 * _typical_norm(w, elems) if clip else 0.0
    a = run_gpu(w, elems=elems, bucket_elems=cb, hp=hp, flow="sync", max_norm=max_norm)
    b = run_gpu(w, elems=elems, bucket_elems=cb, hp=hp, flow="device", max_norm=max_norm)
    assert [(i.overflow, i.step_t, i.scale_used, i.scale_next) for i in a.infos] == \
        [(i.overflow, i.step_t, i.scale_used, i.scale_next) for i in b.infos]
    for x, y in zip(a.infos, b.infos):
        assert x.grad_norm == y.grad_norm or (np.isnan(x.grad_norm) and np.isnan(y.grad_norm))
    for k in ("master", "m", "v", "grad", "param"):
        x, y = getattr(a, k), getattr(b, k)
        assert (x is None) == (y is None), k
        if x is not None:
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), (name, clip, k)
    # and several steps on the device alone, the scale of each step known only
    # on the device (the host mirrors it from the synchronous run)
    scales = [i.scale_used for i in a.infos]
    c = run_gpu(w, elems=elems, bucket_elems=cb, hp=hp, flow="device_run", max_norm=max_norm,
                scale_of=lambda s: scales[s])
    last = c.infos[-1]
    assert (last.overflow, last.step_t, last.scale_used, last.scale_next) == \
        (a.infos[-1].overflow, a.infos[-1].step_t, a.infos[-1].scale_used, a.infos[-1].scale_next)
    for k in ("master", "m", "v", "param"):
        x, y = getattr(a, k), getattr(c, k)
        if x is not None:
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), (name, clip, k, "run")


@pytest.mark.parametrize("name", ["adam_fp16", "sgdm_fp32"])
def test_device_flow_misaligned(name):
    """Arrays at odd element offsets (peeled heads and tails, and the
    element-wise fallback) in the device-resident flow, against the oracle."""
    w = _w(CASES[name], steps=3)
    hp = _hp(name, w)
    for o in (dict(master=1, m=3, v=2, grad=1, param=3, contrib=2), dict(grad=1, contrib=1)):
        g = run_gpu(w, elems=70_001, bucket_elems=20_000, hp=hp, offsets=o, flow="device",
                    max_norm=0.3 * _typical_norm(w, 70_001))
        st, oi = run_oracle(w, g, bucket_elems=20_000, hp=hp, max_norm=0.3 * _typical_norm(w, 70_001))
        compare(w, g, st, oi, f"device misaligned {name} {o}")


@pytest.mark.parametrize("n,inline", [(300_007, 0), (300_000, 1), (2_097_152, 1),
                                      (4_194_304, 1), (4_202_496, 1), (8_388_608, 1),
                                      (8_396_800, 0)])
def test_device_flow_scan_of_caller_filled_gradient(n, inline):
    """contribs = None: the device step scans grad_shard (the P_os case).  An
    aligned shard of at most 1024 scan workgroups of 8192 elements (2,097,152
    elements: 256; 4,194,304: 512; 4,202,496: 513; 8,388,608: 1024) folds the
    partials inside the update; 8,396,800 elements (1025 workgroups) take the
    fold launch, and so do 300,007 elements, which leave the update a scalar
    tail."""
    dev = torch.device("cuda", 0)
    gen = torch.Generator(device=dev).manual_seed(5)
    master = torch.randn(n, generator=gen, device=dev) * 0.02
    m, v = torch.zeros(n, device=dev), torch.zeros(n, device=dev)
    grad = (torch.randn(n, generator=gen, device=dev) * 4.0).half()
    param = master.half()
    master0 = f32(master).copy()
    hp = zs.AdamHParams(lr=1e-3, weight_decay=0.01)
    ls = zs.LossScaleCfg(init_scale=1024.0)
    h = zs.zero_shard_init(master, m, v, grad, param, psi=n, nd=1, rank=0, bucket_elems=n,
                           hp=hp, ls=ls)
    try:
        zs.zero_device_begin(h)
        zs.zero_step_device(h, None)
        info = zs.zero_device_end(h)
        expect_inline_folds(zs.zero_shard_inline_folds(h), inline, n)
    finally:
        zs.zero_shard_destroy(h)
    ohp = oracle.AdamHP(lr=1e-3, weight_decay=0.01)
    st = oracle.new_state(oracle.FP16, master0, np.zeros(n), np.zeros(n), ohp,
                          oracle.LossScale(init_scale=1024.0))
    g = u16(grad)
    flag, ss = oracle.flag_sumsq(oracle.FP16, g, 1024.0)
    oracle.adam_update(oracle.FP16, g, st.master, st.m, st.v, st.param,
                       oracle.adam_scalars(ohp, 1, 1024.0))
    assert info.overflow == flag == 0 and info.step_t == 1
    assert info.grad_norm == pytest.approx(np.sqrt(ss), rel=1e-9)
    assert np.array_equal(f32(master).view(np.uint32), st.master.view(np.uint32))
    assert np.array_equal(u16(param), st.param)


def test_device_flow_state_machine():
    dev = torch.device("cuda", 0)
    n = 4096
    t = [torch.zeros(n, device=dev) for _ in range(3)]
    g = torch.zeros(n, dtype=torch.float16, device=dev)
    p = torch.zeros(n, dtype=torch.float16, device=dev)
    c = [torch.zeros(n, dtype=torch.float16, device=dev)]
    h = zs.zero_shard_init(*t, g, p, psi=n, nd=1, rank=0, bucket_elems=n,
                           hp=zs.AdamHParams(), ls=zs.LossScaleCfg(init_scale=8.0))

    def status(fn, *a):
        with pytest.raises(zs.ZeroError) as e:
            fn(*a)
        return e.value.status

    try:
        assert status(zs.zero_step_device, h, c) == zs.ZERO_ERR_STATE      # before begin
        assert status(zs.zero_device_end, h) == zs.ZERO_ERR_STATE
        zs.zero_device_begin(h)
        assert status(zs.zero_device_begin, h) == zs.ZERO_ERR_STATE
        assert status(zs.zero_bucket_reduce, h, c, 0, n) == zs.ZERO_ERR_STATE
        assert status(zs.zero_overflow_check, h) == zs.ZERO_ERR_STATE
        assert status(zs.zero_adam_step_gated, h) == zs.ZERO_ERR_STATE
        assert status(zs.zero_adam_step, h) == zs.ZERO_ERR_STATE
        assert status(zs.zero_shard_set_clip, h, 1.0) == zs.ZERO_ERR_STATE
        assert status(zs.zero_shard_get_counters, h) == zs.ZERO_ERR_STATE
        assert status(zs.zero_shard_set_counters, h, 0, 1.0, 0) == zs.ZERO_ERR_STATE
        assert status(zs.zero_step_device, h, [c[0].data_ptr() + 1]) == zs.ZERO_ERR_INVALID_ARG
        info = zs.zero_device_end(h)                 # no step run
        assert (info.overflow, info.step_t, info.scale_used, info.scale_next) == (0, 0, 8.0, 8.0)
        zs.zero_device_begin(h)
        zs.zero_step_device(h, c)
        info = zs.zero_device_end(h)
        assert (info.overflow, info.step_t, info.grad_norm) == (0, 1, 0.0)
        assert zs.zero_shard_get_counters(h) == (1, 8.0, 1)
        # a step in progress refuses begin
        zs.zero_bucket_reduce(h, c, 0, n)
        assert status(zs.zero_device_begin, h) == zs.ZERO_ERR_STATE
        assert status(zs.zero_shard_set_clip, h, 1.0) == zs.ZERO_ERR_STATE
        zs.zero_overflow_check(h)
        zs.zero_adam_step(h)
        assert status(zs.zero_shard_set_clip, h, -1.0) == zs.ZERO_ERR_INVALID_ARG
        assert status(zs.zero_shard_set_clip, h, float("inf")) == zs.ZERO_ERR_INVALID_ARG
        zs.zero_shard_set_clip(h, 0.0)
    finally:
        zs.zero_shard_destroy(h)


@pytest.mark.parametrize("name", ["adam_fp16", "sgdm_fp32", "adam_bf16_l2", "sgd_fp32"])
def test_graph_captured_step_replays(name):
    """One zero_step_device captured in a CUDA graph, replayed 6 times with the
    contributions refilled eagerly (and an overflow planted before replay 3)
    between replays; after every replay the state equals an eager
    device-resident run of the same steps, bitwise, and the final counters
    and state equal the oracle's."""
    w = _w(CASES[name], steps=6, dynamic=1, scale=32.0, inject_step=3)
    dev = torch.device("cuda", 0)
    elems, cb = 120_011, 40_000
    hp = _hp(name, w)
    max_norm = 0.5 * _typical_norm(w, elems)

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
        zs.zero_shard_set_clip(h, max_norm)
        return h, dict(master=master, m=m, v=v, param=param, master0=master0, m0=m0, v0=v0)

    bufs = synth.alloc_contribs(w, dev, elems=elems)
    ha, A = make()          # eager device-resident run
    hb, B = make()          # graph replays
    ohp, ols = oracle_hp(hp), oracle_ls(ls_of(w))
    ost = oracle.new_state(LP_CODE[w.lp], f32(A["master0"]), f32(A["m0"]) if w.has_m else None,
                           f32(A["v0"]) if w.has_v else None, ohp, ols)
    try:
        zs.zero_device_begin(ha)
        zs.zero_device_begin(hb)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        # capture: the fill below is eager and outside the graph; the graph
        # holds only the library's launches on the capture stream
        with torch.cuda.graph(graph):
            zs.zero_step_device(hb, bufs)
        torch.cuda.synchronize()
        scale = w.scale
        for s in range(w.steps):
            synth.fill_contribs(w, bufs, s, scale, seed=0)
            torch.cuda.synchronize()
            zs.zero_step_device(ha, bufs)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for k in ("master", "m", "v", "param"):
                if A[k] is not None:
                    assert torch.equal(A[k].view(torch.int8 if A[k].dtype != torch.float32
                                                 else torch.int32),
                                       B[k].view(torch.int8 if B[k].dtype != torch.float32
                                                 else torch.int32)), (name, s, k)
            oi = oracle.step(ost, [stored(b) for b in bufs], cb, ohp, ols, max_norm=max_norm)
            log(f"[graph] {name} replay {s}: overflow={oi.overflow} t={oi.step_t} "
                f"scale={oi.scale_used}")
            scale = oi.scale_next
        ia, ib = zs.zero_device_end(ha), zs.zero_device_end(hb)
        assert (ia.overflow, ia.step_t, ia.scale_next) == (ib.overflow, ib.step_t, ib.scale_next)
        assert (ib.step_t, ib.scale_next) == (ost.t, ost.scale) == (w.steps - 1, w.scale / 2)
        assert np.allclose(f32(B["master"]), ost.master, rtol=1e-6, atol=0)
        del graph
    finally:
        zs.zero_shard_destroy(ha)
        zs.zero_shard_destroy(hb)


@pytest.mark.parametrize("name", ["adam_fp16", "sgdm_fp32"])
def test_graph_holding_several_steps(name):
    """Three zero_step_device calls captured in one CUDA graph: each replay runs
    three steps whose counters, bias corrections and loss scale evolve on the
    device.  Two replays equal six eager device-resident steps after every
    third step, bitwise, and the oracle's six steps on the same contributions."""
    w = _w(CASES[name], steps=6, dynamic=1, scale=64.0)
    dev = torch.device("cuda", 0)
    elems, cb, K = 70_001, 25_000, 3
    hp = _hp(name, w)

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
    synth.fill_contribs(w, bufs, 0, w.scale, seed=0)
    ha, A = make()
    hb, B = make()
    ohp, ols = oracle_hp(hp), oracle_ls(ls_of(w))
    ost = oracle.new_state(LP_CODE[w.lp], f32(A["master0"]), f32(A["m0"]) if w.has_m else None,
                           f32(A["v0"]) if w.has_v else None, ohp, ols)
    cs = [stored(b) for b in bufs]
    log(f"[graph x{K}] {name}")
    try:
        zs.zero_device_begin(ha)
        zs.zero_device_begin(hb)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(K):
                zs.zero_step_device(hb, bufs)
        torch.cuda.synchronize()
        for rep in range(w.steps // K):
            for _ in range(K):
                zs.zero_step_device(ha, bufs)
                oracle.step(ost, cs, cb, ohp, ols)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for k in ("master", "m", "v", "param"):
                if A[k] is not None:
                    view = torch.int32 if A[k].dtype == torch.float32 else torch.int16
                    assert torch.equal(A[k].view(view), B[k].view(view)), (name, rep, k)
        ia, ib = zs.zero_device_end(ha), zs.zero_device_end(hb)
        assert (ia.step_t, ia.scale_next) == (ib.step_t, ib.scale_next) == (w.steps, w.scale)
        assert ost.t == w.steps
        assert np.array_equal(f32(B["master"]).view(np.uint32), ost.master.view(np.uint32))
        if B["param"] is not None:
            assert np.array_equal(stored(B["param"]), ost.param)
        del graph
    finally:
        zs.zero_shard_destroy(ha)
        zs.zero_shard_destroy(hb)


@pytest.mark.parametrize("name", ["adam_fp16", "sgdm_fp32"])
def test_device_flow_after_counter_restore(name):
    """Counters restored with zero_shard_set_counters (t = 7, scale 64, 3 clean
    steps, as after a checkpoint): the device-resident flow starts from them
    (bias corrections of steps 8, 9, ...) exactly as the synchronous flow does."""
    w = _w(CASES[name], steps=3, dynamic=1, scale=64.0)
    dev = torch.device("cuda", 0)
    elems, cb = 90_001, 30_000
    hp = _hp(name, w)
    bufs = synth.alloc_contribs(w, dev, elems=elems)
    out = {}
    for flow in ("sync", "device"):
        master0, m0, v0 = synth.init_state(w, dev, 0, elems=elems)
        master = master0.clone()
        m = m0.clone() if w.has_m else None
        v = v0.clone() if w.has_v else None
        grad = torch.zeros(elems, dtype=w.torch_lp, device=dev)
        param = None if w.lp == "fp32" else master0.to(w.torch_lp)
        if w.opt == "sgd":
            h = zs.zero_shard_init_sgd(master, m, grad, param, psi=elems, nd=1, rank=0,
                                       bucket_elems=cb, hp=hp, ls=ls_of(w))
        else:
            h = zs.zero_shard_init(master, m, v, grad, param, psi=elems, nd=1, rank=0,
                                   bucket_elems=cb, hp=hp, ls=ls_of(w))
        try:
            zs.zero_shard_set_counters(h, 7, 64.0, 3)
            infos = []
            for s in range(w.steps):
                synth.fill_contribs(w, bufs, s, 64.0, seed=0)
                if flow == "sync":
                    zs.reduce_buckets(h, bufs, elems, cb)
                    zs.zero_overflow_check(h)
                    infos.append(zs.zero_sgd_step(h) if w.opt == "sgd" else zs.zero_adam_step(h))
                else:
                    zs.zero_device_begin(h)
                    zs.zero_step_device(h, bufs)
                    infos.append(zs.zero_device_end(h))
            torch.cuda.synchronize()
            out[flow] = (infos, f32(master), None if m is None else f32(m))
            assert zs.zero_shard_get_counters(h) == (10, 64.0, 6)
        finally:
            zs.zero_shard_destroy(h)
    (ia, ma, mma), (ib, mb, mmb) = out["sync"], out["device"]
    assert [(i.step_t, i.scale_next) for i in ia] == [(i.step_t, i.scale_next) for i in ib]
    assert np.array_equal(ma.view(np.uint32), mb.view(np.uint32))
    if mma is not None:
        assert np.array_equal(mma.view(np.uint32), mmb.view(np.uint32))
