"""GPU edge cases against the oracle: unaligned and mutually misaligned
buffers, inf/NaN at every kind of position, determinism, the stand-alone check
of a caller-filled gradient, per-step hyper-parameters, checkpoint/resume, and
the C-ABI state machine's error paths (no state change on error)."""
import ctypes
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import zero_dp_sharded_amd as zs
from gpu_common import (LP_CODE, compare, f32, hp_of, log, ls_of, oracle_hp, oracle_ls,
                        run_gpu, run_oracle, u16)
from zero_dp_sharded_amd import synth

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


@pytest.mark.parametrize("offsets", [
    {"contrib": 1, "grad": 1},                       # common head in the reduce
    {"contrib": 3, "grad": 5},                       # no common alignment: element-wise reduce
    {"master": 1, "m": 1, "v": 1, "grad": 1, "param": 1},   # common Adam head (3 elements)
    {"master": 1},                                   # fp32 arrays disagree: element-wise Adam
    {"param": 2},                                    # 2-byte arrays disagree
    {"grad": 4, "param": 4, "contrib": 4},           # 8-byte aligned only
])
@pytest.mark.parametrize("lp", ["fp16", "bf16"])
def test_misaligned_buffers(offsets, lp):
    w = dataclasses.replace(W["gpt2_1.5b"], lp=lp)
    cb = 10_007                                      # odd C_B: each bucket starts differently
    g = run_gpu(w, elems=50_021, steps=3, bucket_elems=cb, offsets=offsets)
    st, oi = run_oracle(w, g, bucket_elems=cb)
    assert compare(w, g, st, oi, f"{offsets} {lp}")["bitwise"]


def _plant(step_at, plants):
    """hook that writes 2-byte bit patterns into contributions at one step."""
    def hook(s, bufs):
        if s != step_at:
            return
        for r, idx, bits in plants:
            bufs[r].view(torch.int16)[idx] = int(np.array([bits], np.uint16).view(np.int16)[0])
    return hook


FP16_PINF, FP16_NINF, FP16_NAN = 0x7C00, 0xFC00, 0x7E00
BF16_PINF, BF16_NINF, BF16_NAN = 0x7F80, 0xFF80, 0x7FC0


@pytest.mark.parametrize("lp", ["fp16", "bf16"])
@pytest.mark.parametrize("where", ["first", "last", "bucket_edge_lo", "bucket_edge_hi", "tail",
                                   "middle_vector", "pinf_plus_ninf", "nan"])
def test_overflow_positions(lp, where):
    n, cb = 70_001, 16_384                          # tail: n % 8 == 1
    w = dataclasses.replace(W["tiny"], lp=lp, R=4)
    pinf, ninf, nan = (FP16_PINF, FP16_NINF, FP16_NAN) if lp == "fp16" else \
        (BF16_PINF, BF16_NINF, BF16_NAN)
    idx = {"first": 0, "last": n - 2, "bucket_edge_lo": cb - 1, "bucket_edge_hi": cb,
           "tail": n - 1, "middle_vector": 3 * cb + 517, "pinf_plus_ninf": 40_000,
           "nan": 12_345}[where]
    if where == "pinf_plus_ninf":
        plants = [(0, idx, pinf), (2, idx, ninf)]
    elif where == "nan":
        plants = [(3, idx, nan)]
    else:
        plants = [(1, idx, pinf if where != "tail" else ninf)]
    g = run_gpu(w, elems=n, steps=3, bucket_elems=cb, hook=_plant(1, plants))
    st, oi = run_oracle(w, g, bucket_elems=cb)
    compare(w, g, st, oi, f"{lp} {where}")
    assert [i.overflow for i in g.infos] == [0, 1, 0]
    assert [i.step_t for i in g.infos] == [1, 1, 2]
    assert g.infos[1].scale_next == g.infos[1].scale_used / 2


def test_skip_leaves_state_bitwise():
    """A skipped step is a bitwise no-op on master, m, v and param."""
    w = dataclasses.replace(W["tiny"], R=2)
    n = 33_333
    base = run_gpu(w, elems=n, steps=1, bucket_elems=8_192)
    skip = run_gpu(w, elems=n, steps=2, bucket_elems=8_192,
                   hook=_plant(1, [(0, 77, FP16_PINF)]))
    for a in ("master", "m", "v", "param"):
        assert np.array_equal(getattr(base, a).view(np.uint8), getattr(skip, a).view(np.uint8)), a
    assert skip.infos[1].skipped == 1


def test_static_scale_skip_keeps_scale():
    w = dataclasses.replace(W["7.5b_bf16"], R=4)
    g = run_gpu(w, elems=20_000, steps=3, bucket_elems=8_192,
                hook=_plant(1, [(2, 5, BF16_NAN)]))
    st, oi = run_oracle(w, g, bucket_elems=8_192)
    compare(w, g, st, oi, "static")
    assert [i.overflow for i in g.infos] == [0, 1, 0]
    assert all(i.scale_used == 1.0 and i.scale_next == 1.0 for i in g.infos)


def test_determinism_bitwise():
    w = W["gpt2_1.5b"]
    a = run_gpu(w, elems=1_000_003, steps=3, bucket_elems=262_144, seed=7)
    b = run_gpu(w, elems=1_000_003, steps=3, bucket_elems=262_144, seed=7)
    for k in ("master", "m", "v", "grad", "param"):
        assert np.array_equal(getattr(a, k).view(np.uint8), getattr(b, k).view(np.uint8)), k
    assert [i.grad_norm for i in a.infos] == [i.grad_norm for i in b.infos]


def test_bucket_size_invariance_gpu():
    w = W["gpt2_1.5b"]
    ref = run_gpu(w, elems=300_000, steps=2, bucket_elems=300_000)
    for cb in (1, 8, 4096, 65_537):
        if cb == 1:
            n = 3_000
            r1 = run_gpu(w, elems=n, steps=2, bucket_elems=n)
            o = run_gpu(w, elems=n, steps=2, bucket_elems=1)
        else:
            r1, o = ref, run_gpu(w, elems=300_000, steps=2, bucket_elems=cb)
        for k in ("master", "m", "v", "grad", "param"):
            assert np.array_equal(getattr(r1, k).view(np.uint8), getattr(o, k).view(np.uint8)), (cb, k)
        for x, y in zip(r1.infos, o.infos):
            assert x.grad_norm == pytest.approx(y.grad_norm, rel=1e-12)


def _handle(n, lp=torch.float16, cb=1000, hp=None, ls=None, psi_mul=4):
    dev = torch.device("cuda", 0)
    gen = torch.Generator(device=dev).manual_seed(11)
    master = (torch.randn(n, generator=gen, device=dev) * 0.02).float()
    m = torch.zeros(n, device=dev)
    v = torch.zeros(n, device=dev)
    grad = torch.zeros(n, dtype=lp, device=dev)
    param = master.to(lp)
    hp = hp or zs.AdamHParams(lr=1e-3)
    ls = ls or zs.LossScaleCfg(init_scale=1024.0)
    h = zs.zero_shard_init(master, m, v, grad, param, psi=n * psi_mul, nd=psi_mul, rank=0,
                           bucket_elems=cb, hp=hp, ls=ls)
    return h, dict(master=master, m=m, v=v, grad=grad, param=param)


def test_scan_path_caller_filled_gradient():
    """No bucket reduced: the check scans the caller's grad_shard (the P_os
    case, where the owner already holds the all-reduced gradient)."""
    n = 123_457
    h, t = _handle(n, cb=n)
    try:
        gen = torch.Generator(device="cuda").manual_seed(5)
        t["grad"].copy_((torch.randn(n, generator=gen, device="cuda") * 4.0).half())
        g_bits = u16(t["grad"])
        m0 = f32(t["master"]).copy()
        info = zs.zero_overflow_check(h)
        out = zs.zero_adam_step(h)
        torch.cuda.synchronize()
        hp = oracle.AdamHP(lr=1e-3)
        ls = oracle.LossScale(init_scale=1024.0)
        st = oracle.new_state(oracle.FP16, m0, np.zeros(n), np.zeros(n), hp, ls)
        flag, ss = oracle.flag_sumsq(oracle.FP16, g_bits, 1024.0)
        assert info.overflow == flag == 0
        assert info.grad_norm == pytest.approx(np.sqrt(ss), rel=1e-10)
        oracle.adam_update(oracle.FP16, g_bits, st.master, st.m, st.v, st.param,
                           oracle.adam_scalars(hp, 1, 1024.0))
        assert np.array_equal(f32(t["master"]).view(np.uint32), st.master.view(np.uint32))
        assert np.array_equal(u16(t["param"]), st.param)
        assert out.step_t == 1
        # a planted inf in the caller's gradient is found by the scan
        t["grad"][n - 1] = float("inf")
        assert zs.zero_overflow_check(h).overflow == 1
        assert zs.zero_adam_step(h).skipped == 1
    finally:
        zs.zero_shard_destroy(h)


def test_per_step_hparams_override():
    """zero_adam_step(h, hp) uses hp for that step only (an lr schedule)."""
    w = W["gpt2_1.5b"]
    n, cb, R = 40_000, 16_000, w.R
    dev = torch.device("cuda", 0)
    master0, m0, v0 = synth.init_state(w, dev, 3, elems=n)
    t = dict(master=master0.clone(), m=m0.clone(), v=v0.clone(),
             grad=torch.zeros(n, dtype=torch.float16, device=dev),
             param=master0.to(torch.float16))
    hp0 = hp_of(w)
    ls = ls_of(w)
    h = zs.zero_shard_init(t["master"], t["m"], t["v"], t["grad"], t["param"], psi=n * w.nd,
                           nd=w.nd, rank=0, bucket_elems=cb, hp=hp0, ls=ls)
    bufs = synth.alloc_contribs(w, dev, elems=n)
    ost = oracle.new_state(oracle.FP16, f32(master0), f32(m0), f32(v0), oracle_hp(hp0), oracle_ls(ls))
    try:
        scale = ls.init_scale
        for s, lr in enumerate([1e-3, 5e-4, 2.5e-4, 1e-3]):
            synth.fill_contribs(w, bufs, s, scale, 3)
            cs = [u16(b) for b in bufs]
            zs.reduce_buckets(h, bufs, n, cb)
            zs.zero_overflow_check(h)
            hp = dataclasses.replace(hp0, lr=lr, weight_decay=0.02 * (s + 1))
            info = zs.zero_adam_step(h, hp if s % 2 == 0 else None)
            ohp = oracle_hp(hp if s % 2 == 0 else hp0)
            oracle.step(ost, cs, cb, ohp, oracle_ls(ls))
            scale = info.scale_next
        torch.cuda.synchronize()
        assert np.array_equal(f32(t["master"]).view(np.uint32), ost.master.view(np.uint32))
        assert np.array_equal(u16(t["param"]), ost.param)
    finally:
        zs.zero_shard_destroy(h)


def test_checkpoint_resume_bitwise():
    """j steps, save arrays and counters, restore into a new handle, k - j more
    steps == k straight steps."""
    w = W["13b_inf"]
    n, cb, k, j = 30_011, 8_192, 5, 3          # the +inf lands in step 3 (index 2)
    full = run_gpu(w, elems=n, steps=k, bucket_elems=cb)
    dev = torch.device("cuda", 0)
    master0, m0, v0 = synth.init_state(w, dev, 0, elems=n)
    t = dict(master=master0.clone(), m=m0.clone(), v=v0.clone(),
             grad=torch.zeros(n, dtype=torch.float16, device=dev),
             param=master0.to(torch.float16))
    bufs = synth.alloc_contribs(w, dev, elems=n)
    hp, ls = hp_of(w), ls_of(w)

    def run(h, steps, scale):
        for s in steps:
            synth.fill_contribs(w, bufs, s, scale, 0)
            zs.reduce_buckets(h, bufs, n, cb)
            zs.zero_overflow_check(h)
            scale = zs.zero_adam_step(h).scale_next
        return scale

    h = zs.zero_shard_init(t["master"], t["m"], t["v"], t["grad"], t["param"], psi=n * w.nd,
                           nd=w.nd, rank=w.rank, bucket_elems=cb, hp=hp, ls=ls)
    scale = run(h, range(j), ls.init_scale)
    counters = zs.zero_shard_get_counters(h)
    zs.zero_shard_destroy(h)
    saved = {a: v.clone() for a, v in t.items()}
    assert counters[0] == 2 and counters[1] == w.scale / 2          # one skip so far
    t2 = {a: v.clone() for a, v in saved.items()}
    h2 = zs.zero_shard_init(t2["master"], t2["m"], t2["v"], t2["grad"], t2["param"],
                            psi=n * w.nd, nd=w.nd, rank=w.rank, bucket_elems=cb, hp=hp, ls=ls)
    try:
        zs.zero_shard_set_counters(h2, *counters)
        run(h2, range(j, k), counters[1])
        torch.cuda.synchronize()
    finally:
        zs.zero_shard_destroy(h2)
    for a in ("master", "m", "v", "param"):
        x = t2[a].view(torch.int16 if t2[a].dtype == torch.float16 else torch.int32).cpu().numpy()
        y = getattr(full, a).view(np.int16 if a == "param" else np.int32)
        assert np.array_equal(x, y), a


def _status(fn, *args):
    return fn(*args)


def test_abi_state_machine_errors_leave_state_unchanged():
    n, cb = 10_000, 4_096
    h, t = _handle(n, cb=cb)
    master0 = f32(t["master"]).copy()
    L = zs.lib()
    R = 4
    bufs = [torch.randn(n, device="cuda").half() for _ in range(R)]
    arr = lambda off: (ctypes.c_void_p * R)(*[b.data_ptr() + 2 * off for b in bufs])
    info = zs.ZeroStepInfo()
    try:
        # Adam and a second check before anything was reduced
        assert L.zero_adam_step(h, None, None, ctypes.byref(info)) == zs.ZERO_ERR_STATE
        # wrong first bucket, bad sizes, bad counts
        assert L.zero_bucket_reduce(h, arr(cb), R, cb, cb, None) == zs.ZERO_ERR_STATE
        assert L.zero_bucket_reduce(h, arr(0), R, 0, cb + 1, None) == zs.ZERO_ERR_INVALID_ARG
        assert L.zero_bucket_reduce(h, arr(0), R, 0, 100, None) == zs.ZERO_ERR_STATE  # short, not last
        assert L.zero_bucket_reduce(h, arr(0), 0, 0, cb, None) == zs.ZERO_ERR_INVALID_ARG
        assert L.zero_bucket_reduce(h, arr(0), 65, 0, cb, None) == zs.ZERO_ERR_INVALID_ARG
        assert L.zero_bucket_reduce(h, arr(0), R, n, 1, None) == zs.ZERO_ERR_INVALID_ARG
        assert L.zero_bucket_reduce(h, arr(0), R, -1, 1, None) == zs.ZERO_ERR_INVALID_ARG
        assert L.zero_bucket_reduce(h, None, R, 0, cb, None) == zs.ZERO_ERR_INVALID_ARG
        odd = (ctypes.c_void_p * R)(*[b.data_ptr() + 1 for b in bufs])
        assert L.zero_bucket_reduce(h, odd, R, 0, cb, None) == zs.ZERO_ERR_INVALID_ARG
        # a contribution over a shard array, or over grad_shard other than as
        # the bucket's own slice
        for name, shift in (("master", 0), ("m", 4 * 7), ("v", 0), ("param", 2 * (n - 1)),
                            ("grad", 2), ("grad", 2 * cb)):
            over = (ctypes.c_void_p * R)(*([t[name].data_ptr() + shift] +
                                           [b.data_ptr() for b in bufs[1:]]))
            assert L.zero_bucket_reduce(h, over, R, 0, cb, None) == zs.ZERO_ERR_INVALID_ARG, name
            assert "overlaps" in zs.zero_last_error(), name
        assert L.zero_overflow_check(h, None, None) == zs.ZERO_ERR_INVALID_ARG
        # a valid first bucket, then errors mid-step
        assert L.zero_bucket_reduce(h, arr(0), R, 0, cb, None) == zs.ZERO_OK
        assert L.zero_overflow_check(h, None, ctypes.byref(info)) == zs.ZERO_ERR_STATE  # partial
        assert L.zero_adam_step(h, None, None, ctypes.byref(info)) == zs.ZERO_ERR_STATE
        assert L.zero_bucket_reduce(h, arr(0), R, 0, cb, None) == zs.ZERO_ERR_STATE   # repeat
        assert L.zero_shard_set_counters(h, 5, 2.0, 0) == zs.ZERO_ERR_STATE          # mid-step
        assert L.zero_bucket_reduce(h, arr(cb), R, cb, cb, None) == zs.ZERO_OK
        assert L.zero_bucket_reduce(h, arr(2 * cb), R, 2 * cb, n - 2 * cb, None) == zs.ZERO_OK
        assert L.zero_overflow_check(h, None, ctypes.byref(info)) == zs.ZERO_OK
        again = zs.ZeroStepInfo()
        assert L.zero_overflow_check(h, None, ctypes.byref(again)) == zs.ZERO_OK
        assert bytes(again) == bytes(info)
        assert L.zero_bucket_reduce(h, arr(0), R, 0, cb, None) == zs.ZERO_ERR_STATE   # after check
        bad = zs.AdamHParams(lr=-1.0).to_c()
        assert L.zero_adam_step(h, ctypes.byref(bad), None, ctypes.byref(info)) == zs.ZERO_ERR_INVALID_ARG
        assert zs.zero_shard_get_counters(h) == (0, 1024.0, 0)
        assert L.zero_adam_step(h, None, None, ctypes.byref(info)) == zs.ZERO_OK
        assert info.step_t == 1
        torch.cuda.synchronize()
        # the step equals the oracle's: the errors changed nothing
        cs = [u16(b) for b in bufs]
        ohp, ols = oracle.AdamHP(lr=1e-3), oracle.LossScale(init_scale=1024.0)
        st = oracle.new_state(oracle.FP16, master0, np.zeros(n), np.zeros(n), ohp, ols)
        oi = oracle.step(st, cs, cb, ohp, ols)
        assert oi.overflow == info.overflow == 0
        assert np.array_equal(u16(t["grad"]), st.grad)
        assert np.array_equal(f32(t["master"]).view(np.uint32), st.master.view(np.uint32))
        assert np.array_equal(u16(t["param"]), st.param)
    finally:
        zs.zero_shard_destroy(h)
    assert L.zero_shard_destroy(h) == zs.ZERO_ERR_STATE
    assert L.zero_bucket_reduce(h, arr(0), R, 0, cb, None) == zs.ZERO_ERR_STATE


@pytest.mark.parametrize("flow", ["sync", "device"])
def test_in_place_reduce(flow):
    """Contribution 0 is grad_shard itself (a reduce in place of the first
    contribution's buffer): bucket by bucket in the synchronous flow, the
    whole shard in one device-resident step; bitwise equal to the oracle fed
    the original contributions."""
    n, cb, R = 100_003, 30_000, 4
    h, t = _handle(n, cb=cb)
    master0 = f32(t["master"]).copy()
    gen = torch.Generator(device="cuda").manual_seed(21)
    bufs = [(torch.randn(n, generator=gen, device="cuda") * 4.0).half() for _ in range(R)]
    cs = [u16(b) for b in bufs]
    t["grad"].copy_(bufs[0])
    srcs = [t["grad"]] + bufs[1:]
    log(f"in-place reduce, {flow} flow")
    try:
        if flow == "sync":
            zs.reduce_buckets(h, srcs, n, cb)
            zs.zero_overflow_check(h)
            info = zs.zero_adam_step(h)
        else:
            zs.zero_device_begin(h)
            zs.zero_step_device(h, srcs)
            info = zs.zero_device_end(h)
        torch.cuda.synchronize()
    finally:
        zs.zero_shard_destroy(h)
    ohp, ols = oracle.AdamHP(lr=1e-3), oracle.LossScale(init_scale=1024.0)
    st = oracle.new_state(oracle.FP16, master0, np.zeros(n), np.zeros(n), ohp, ols)
    oi = oracle.step(st, cs, cb, ohp, ols)
    assert info.overflow == oi.overflow == 0 and info.step_t == 1
    assert np.array_equal(u16(t["grad"]), st.grad)
    assert np.array_equal(f32(t["master"]).view(np.uint32), st.master.view(np.uint32))
    assert np.array_equal(u16(t["param"]), st.param)


def _hip():
    h = ctypes.CDLL("libamdhip64.so")
    h.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
    h.hipFree.argtypes = [ctypes.c_void_p]
    return h


def test_host_memory_and_short_allocations_refused():
    """Arrays the runtime reports as pageable host memory, or that run past the
    end of their allocation, are refused before anything is launched.  Each
    case is tried first at zero_shard_init, which launches nothing, and only
    then as a contribution."""
    n = (1 << 19) + 1                    # 4n bytes = 2 MiB + 4
    L = zs.lib()
    hip = _hip()
    dev = torch.device("cuda", 0)
    host = torch.zeros(n, dtype=torch.float32)                 # pageable host memory
    raw = ctypes.c_void_p()
    assert hip.hipMalloc(ctypes.byref(raw), 1 << 21) == 0      # 2 MiB: one fp32 element short
    try:
        m = torch.zeros(n, device=dev)
        v = torch.zeros(n, device=dev)
        grad = torch.zeros(n, dtype=torch.float16, device=dev)
        param = torch.zeros(n, dtype=torch.float16, device=dev)
        hp, ls = zs.AdamHParams(lr=1e-3).to_c(), zs.LossScaleCfg(init_scale=1.0).to_c()
        for master_ptr, what in ((host.data_ptr(), "not device-accessible"), (raw.value, "past the end")):
            d = zs.ZeroShardDesc(n * 4, 4, 0, n, zs.ZERO_FP16, master_ptr, m.data_ptr(),
                                 v.data_ptr(), grad.data_ptr(), param.data_ptr())
            out = ctypes.c_void_p()
            st = L.zero_shard_init(ctypes.byref(d), ctypes.byref(hp), ctypes.byref(ls),
                                   ctypes.byref(out))
            if st == zs.ZERO_OK:
                zs.zero_shard_destroy(out.value)
            assert st == zs.ZERO_ERR_INVALID_ARG and what in zs.zero_last_error(), what
        # the same checks guard the contributions
        h, t = _handle(n, cb=n)
        try:
            good = [torch.zeros(n, dtype=torch.float16, device=dev) for _ in range(3)]
            host16 = torch.zeros(n, dtype=torch.float16)
            # n fp16 elements from raw + 1 MiB end 2 bytes past the 2 MiB allocation
            for bad, what in ((host16.data_ptr(), "not device-accessible"),
                              (raw.value + (1 << 20), "past the end")):
                ptrs = (ctypes.c_void_p * 4)(bad, *[g.data_ptr() for g in good])
                assert L.zero_bucket_reduce(h, ptrs, 4, 0, n, None) == zs.ZERO_ERR_INVALID_ARG
                assert what in zs.zero_last_error(), what
            with pytest.raises(ValueError):
                zs.zero_bucket_reduce(h, [host16] + good, 0, n)
            # nothing was launched or recorded: a valid step still runs
            zs.reduce_buckets(h, good + [good[0]], n, n)
            assert zs.zero_overflow_check(h).overflow == 0
            assert zs.zero_adam_step(h).step_t == 1
        finally:
            zs.zero_shard_destroy(h)
    finally:
        torch.cuda.synchronize()
        hip.hipFree(raw)


def test_device_step_refuses_overlapping_contribution():
    n, cb, R = 20_000, 8_192, 4
    h, t = _handle(n, cb=cb)
    bufs = [torch.randn(n, device="cuda").half() for _ in range(R)]
    L = zs.lib()
    try:
        zs.zero_device_begin(h)
        for name, shift in (("master", 0), ("grad", 2)):
            ptrs = (ctypes.c_void_p * R)(*([t[name].data_ptr() + shift] +
                                           [b.data_ptr() for b in bufs[1:]]))
            assert L.zero_step_device(h, ptrs, R, None) == zs.ZERO_ERR_INVALID_ARG, name
        info = zs.zero_device_end(h)
        assert info.step_t == 0
    finally:
        zs.zero_shard_destroy(h)


@pytest.mark.parametrize("name,elems,cb", [("gpt2_1.5b", 300_007, 65_536), ("13b_inf", 120_013, 16_384),
                                           ("7.5b_bf16", 90_001, 30_000)])
def test_gated_flow_matches_oracle(name, elems, cb):
    """The device-gated check + Adam gives the synchronous flow's results,
    including the skipped overflow step of the 13B workload."""
    w = W[name]
    g = run_gpu(w, elems=elems, bucket_elems=cb, flow="gated")
    st, oi = run_oracle(w, g, bucket_elems=cb)
    assert compare(w, g, st, oi, f"gated {name}")["bitwise"]
    s = run_gpu(w, elems=elems, bucket_elems=cb, flow="sync")
    for k in ("master", "m", "v", "grad", "param"):
        assert np.array_equal(getattr(g, k).view(np.uint8), getattr(s, k).view(np.uint8)), k
    assert [(i.overflow, i.step_t, i.scale_next) for i in g.infos] == \
        [(i.overflow, i.step_t, i.scale_next) for i in s.infos]


def test_gated_skip_and_state_errors():
    n, cb = 20_000, 8_192
    h, t = _handle(n, cb=cb)
    L = zs.lib()
    R = 2
    bufs = [torch.randn(n, device="cuda").half() for _ in range(R)]
    bufs[1][n // 3] = float("inf")
    info = zs.ZeroStepInfo()
    try:
        before = {k: v.clone() for k, v in t.items()}
        # gated step with partial coverage is refused
        zs.reduce_buckets(h, bufs, cb, cb)        # only the first bucket
        assert L.zero_adam_step_gated(h, None, None) == zs.ZERO_ERR_STATE
        for off in range(cb, n, cb):
            ln = min(cb, n - off)
            zs.zero_bucket_reduce(h, [b.data_ptr() + 2 * off for b in bufs], off, ln)
        assert L.zero_step_resolve(h, ctypes.byref(info)) == zs.ZERO_ERR_STATE   # nothing pending
        zs.zero_adam_step_gated(h)
        # everything else is refused while the step is pending
        arr = (ctypes.c_void_p * R)(*[b.data_ptr() for b in bufs])
        assert L.zero_bucket_reduce(h, arr, R, 0, cb, None) == zs.ZERO_ERR_STATE
        assert L.zero_overflow_check(h, None, ctypes.byref(info)) == zs.ZERO_ERR_STATE
        assert L.zero_adam_step(h, None, None, ctypes.byref(info)) == zs.ZERO_ERR_STATE
        assert L.zero_adam_step_gated(h, None, None) == zs.ZERO_ERR_STATE
        assert L.zero_shard_set_counters(h, 0, 1.0, 0) == zs.ZERO_ERR_STATE
        res = zs.zero_step_resolve(h)
        assert res.overflow == 1 and res.skipped == 1 and res.step_t == 0
        assert res.scale_next == 512.0
        torch.cuda.synchronize()
        for k in ("master", "m", "v", "param"):
            assert torch.equal(before[k], t[k]), k
        # a clean gated step after the skip applies t = 1
        bufs[1][n // 3] = 0.5
        zs.reduce_buckets(h, bufs, n, cb)
        zs.zero_adam_step_gated(h)
        res = zs.zero_step_resolve(h)
        assert res.overflow == 0 and res.step_t == 1
        torch.cuda.synchronize()
        assert not torch.equal(before["master"], t["master"])
    finally:
        zs.zero_shard_destroy(h)
