"""C-ABI checks that need no GPU: the library loads, exports every function
include/zero_shard.h declares, its pure-host ledger equals the oracle's, and
argument validation rejects bad calls before any device work."""
import ctypes
import os
import re

import pytest

import zero_dp_sharded_amd as zs
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "zero_shard.h")


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zero_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = zs.lib()
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(zs.ABI_SYMBOLS)


def test_abi_version_and_status_strings():
    assert zs.zero_abi_version() == 1
    for code, name in [(0, "ZERO_OK"), (1, "ZERO_ERR_INVALID_ARG"), (2, "ZERO_ERR_STATE"),
                       (3, "ZERO_ERR_HIP"), (4, "ZERO_ERR_OOM"), (5, "ZERO_ERR_UNSUPPORTED")]:
        assert zs.zero_status_str(code) == name


def test_struct_layouts_match_header():
    # sizes fixed by the header's field order on x86-64
    assert ctypes.sizeof(zs.ZeroShardDesc) == 72
    assert ctypes.sizeof(zs.ZeroAdamHParams) == 56
    assert ctypes.sizeof(zs.ZeroLossScaleCfg) == 24
    assert ctypes.sizeof(zs.ZeroStepInfo) == 40
    assert ctypes.sizeof(zs.ZeroSgdHParams) == 32
    assert ctypes.sizeof(zs.ZeroStateBytes) == 8 * 8 + 8 * 4 * 2 + 8 + 8 * 4 * 3


CASES = [(1_048_576, 4, 4, 50_000_000), (1_500_000_000, 8, 8, 50_000_000),
         (7_500_000_000, 64, 8, 50_000_000), (13_000_000_000, 16, 16, 50_000_000),
         (128_000_000_000, 64, 4, 200_000_000), (10, 4, 1, 1), (10**12, 1024, 64, 7),
         (999_999_937, 3, 5, 12345)]


@pytest.mark.parametrize("psi,nd,R,cb", CASES)
def test_state_bytes_equals_oracle(oracle, psi, nd, R, cb):
    a = zs.zero_state_bytes(psi, nd, R, cb, zs.ZERO_FP16)
    b = oracle.state_bytes(psi, nd, R, cb)
    assert a == b


@pytest.mark.parametrize("b,K", [(2, 12), (4, 8), (4, 4), (4, 0), (2, 8), (2, 4)])
@pytest.mark.parametrize("lp,lp_bytes", [(zs.ZERO_BF16, 2), (zs.ZERO_FP32, 4)])
def test_state_bytes_ex_equals_oracle(oracle, b, K, lp, lp_bytes):
    for psi, nd, R, cb in CASES:
        a = zs.zero_state_bytes_ex(psi, nd, R, cb, lp, b, K)
        o = oracle.state_bytes(psi, nd, R, cb, lp_bytes=lp_bytes, param_bytes=b, k_optim=K)
        assert a == o


def test_state_bytes_128b_allocation():
    d = zs.zero_state_bytes(128_000_000_000, 64, 4, 200_000_000, zs.ZERO_FP16)
    assert d["shard_elems"] == 2_000_000_000
    assert d["bytes_shard_total"] == 32_000_000_000 == d["per_rank_stage"][3]


@pytest.mark.parametrize("args", [(0, 4, 1, 1), (10, 0, 1, 1), (10, 4, 0, 1), (10, 4, 65, 1),
                                  (10, 4, 1, 0)])
def test_state_bytes_rejects(args):
    with pytest.raises(zs.ZeroError) as e:
        zs.zero_state_bytes(*args, zs.ZERO_FP16)
    assert e.value.status == zs.ZERO_ERR_INVALID_ARG
    with pytest.raises(zs.ZeroError):
        zs.zero_state_bytes(10, 4, 1, 1, 7)
    with pytest.raises(zs.ZeroError):
        zs.zero_state_bytes_ex(10, 4, 1, 1, zs.ZERO_FP16, 3, 12)


def _desc(**over):
    d = dict(psi=1000, nd=4, rank=0, bucket_elems=100, lp=zs.ZERO_FP16, master=0x1000,
             exp_avg=0x20000, exp_avg_sq=0x40000, grad_shard=0x60000, param_shard=0x80000)
    d.update(over)
    return zs.ZeroShardDesc(**d)


GOOD_HP = zs.ZeroAdamHParams(1e-3, 0.9, 0.999, 1e-8, 0.0, 1, 0, 0)
GOOD_LS = zs.ZeroLossScaleCfg(1024.0, 1, 1000, 1.0)


@pytest.mark.parametrize("over", [
    dict(psi=0), dict(nd=0), dict(rank=4), dict(rank=-1), dict(bucket_elems=0), dict(lp=7),
    dict(master=0), dict(exp_avg=0), dict(exp_avg_sq=0), dict(grad_shard=0), dict(param_shard=0),
    dict(master=0x1002), dict(grad_shard=0x60001), dict(exp_avg=0x1100),  # misaligned, overlap
])
def test_init_rejects_bad_desc_before_device_work(over):
    h = ctypes.c_void_p()
    s = zs.lib().zero_shard_init(ctypes.byref(_desc(**over)), ctypes.byref(GOOD_HP),
                                 ctypes.byref(GOOD_LS), ctypes.byref(h))
    assert s == zs.ZERO_ERR_INVALID_ARG, zs.zero_last_error()
    assert h.value is None
    assert zs.zero_last_error()


@pytest.mark.parametrize("field,val", [("lr", -1.0), ("lr", float("nan")), ("beta1", 1.0),
                                       ("beta2", -0.1), ("eps", 0.0), ("eps", 1e-50),
                                       ("weight_decay", -0.1), ("bias_correction", 2),
                                       ("wd_mode", 5), ("initial_step", -1),
                                       # below 1 in fp64 but 1.0 after rounding to fp32
                                       ("beta1", 0.99999999), ("beta2", 1.0 - 1e-9)])
def test_init_rejects_bad_hparams(field, val):
    hp = zs.ZeroAdamHParams(1e-3, 0.9, 0.999, 1e-8, 0.0, 1, 0, 0)
    setattr(hp, field, val)
    h = ctypes.c_void_p()
    s = zs.lib().zero_shard_init(ctypes.byref(_desc()), ctypes.byref(hp), ctypes.byref(GOOD_LS),
                                 ctypes.byref(h))
    assert s == zs.ZERO_ERR_INVALID_ARG


@pytest.mark.parametrize("field,val", [("init_scale", 0.0), ("init_scale", float("inf")),
                                       ("init_scale", float("nan")),
                                       ("dynamic", 2), ("growth_interval", 0), ("min_scale", -1.0),
                                       # fp32(1/scale) would be inf, or 0
                                       ("init_scale", 1e-40), ("min_scale", 2e-39),
                                       ("init_scale", 2e45), ("min_scale", 1e46)])
def test_init_rejects_bad_loss_scale(field, val):
    ls = zs.ZeroLossScaleCfg(1024.0, 1, 1000, 1.0)
    setattr(ls, field, val)
    h = ctypes.c_void_p()
    s = zs.lib().zero_shard_init(ctypes.byref(_desc()), ctypes.byref(GOOD_HP), ctypes.byref(ls),
                                 ctypes.byref(h))
    assert s == zs.ZERO_ERR_INVALID_ARG


def test_null_and_dead_handles():
    L = zs.lib()
    h = ctypes.c_void_p()
    assert L.zero_shard_init(None, ctypes.byref(GOOD_HP), ctypes.byref(GOOD_LS),
                             ctypes.byref(h)) == zs.ZERO_ERR_INVALID_ARG
    assert L.zero_shard_init(ctypes.byref(_desc()), None, ctypes.byref(GOOD_LS),
                             ctypes.byref(h)) == zs.ZERO_ERR_INVALID_ARG
    assert L.zero_shard_init(ctypes.byref(_desc()), ctypes.byref(GOOD_HP), None,
                             ctypes.byref(h)) == zs.ZERO_ERR_INVALID_ARG
    assert L.zero_shard_destroy(None) == zs.ZERO_ERR_STATE
    bogus = ctypes.c_void_p(0xDEAD0)
    info = zs.ZeroStepInfo()
    arr = (ctypes.c_void_p * 1)(0x1000)
    assert L.zero_bucket_reduce(bogus, arr, 1, 0, 1, None) == zs.ZERO_ERR_STATE
    assert L.zero_overflow_check(bogus, None, ctypes.byref(info)) == zs.ZERO_ERR_STATE
    assert L.zero_adam_step(bogus, None, None, ctypes.byref(info)) == zs.ZERO_ERR_STATE
    n = ctypes.c_int64(-1)
    assert L.zero_shard_inline_folds(bogus, ctypes.byref(n)) == zs.ZERO_ERR_STATE
    assert L.zero_shard_inline_folds(None, ctypes.byref(n)) == zs.ZERO_ERR_STATE
    assert n.value == -1                                   # untouched on error
    assert L.zero_shard_destroy(bogus) == zs.ZERO_ERR_STATE


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(zs, "_lib", None)
    monkeypatch.setattr(zs, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="no fallback"):
        zs.zero_abi_version()


def test_init_rejects_too_many_buckets_before_device_work():
    """C_B = 1 on a 2^31-element shard would need 2^32 partial slots: refused
    during validation, before any device call (addresses are never touched)."""
    d = zs.ZeroShardDesc(1 << 31, 1, 0, 1, zs.ZERO_FP16, 1 << 40, 2 << 40, 3 << 40, 4 << 40,
                         5 << 40)
    h = ctypes.c_void_p()
    s = zs.lib().zero_shard_init(ctypes.byref(d), ctypes.byref(GOOD_HP), ctypes.byref(GOOD_LS),
                                 ctypes.byref(h))
    assert s == zs.ZERO_ERR_UNSUPPORTED
    assert "bucket" in zs.zero_last_error()
    assert h.value is None


@pytest.mark.parametrize("psi,nd,R,cb", CASES[:4])
def test_state_bytes_fp32_storage_equals_oracle(oracle, psi, nd, R, cb):
    a = zs.zero_state_bytes(psi, nd, R, cb, zs.ZERO_FP32)
    b = oracle.state_bytes(psi, nd, R, cb, lp_bytes=4)
    assert a == b
    assert a["bytes_param"] == 0 and a["bytes_grad"] == 4 * a["shard_elems"]
    assert a["bytes_shard_total"] == 16 * a["shard_elems"]


def _desc32(**over):
    d = dict(lp=zs.ZERO_FP32, param_shard=0)
    d.update(over)
    return _desc(**d)


GOOD_SGD = zs.ZeroSgdHParams(1e-2, 0.9, 0.0, 0)


@pytest.mark.parametrize("over", [
    dict(param_shard=0x80000),          # fp32 storage takes no 2-byte param
    dict(grad_shard=0x60002),           # fp32 grads must be 4-byte aligned
    dict(exp_avg_sq=0), dict(master=0),
])
def test_init_fp32_storage_rejects(over):
    h = ctypes.c_void_p()
    s = zs.lib().zero_shard_init(ctypes.byref(_desc32(**over)), ctypes.byref(GOOD_HP),
                                 ctypes.byref(GOOD_LS), ctypes.byref(h))
    assert s == zs.ZERO_ERR_INVALID_ARG, zs.zero_last_error()
    assert h.value is None


@pytest.mark.parametrize("desc_over,hp", [
    (dict(exp_avg=0), zs.ZeroSgdHParams(1e-2, 0.9, 0.0, 0)),    # momentum without a buffer
    (dict(), zs.ZeroSgdHParams(1e-2, 1.0, 0.0, 0)),            # momentum outside [0, 1)
    (dict(), zs.ZeroSgdHParams(-1.0, 0.9, 0.0, 0)),
    (dict(), zs.ZeroSgdHParams(float("nan"), 0.9, 0.0, 0)),
    (dict(), zs.ZeroSgdHParams(1e-2, 0.9, -1.0, 0)),
    (dict(), zs.ZeroSgdHParams(1e-2, 0.9, 0.0, -3)),
    (dict(exp_avg_sq=0x40000), GOOD_SGD),                       # SGD takes no second moment
    (dict(grad_shard=0x20001), GOOD_SGD),
])
def test_init_sgd_rejects(desc_over, hp):
    d = dict(exp_avg_sq=0)
    d.update(desc_over)
    h = ctypes.c_void_p()
    s = zs.lib().zero_shard_init_sgd(ctypes.byref(_desc(**d)), ctypes.byref(hp),
                                     ctypes.byref(GOOD_LS), ctypes.byref(h))
    assert s == zs.ZERO_ERR_INVALID_ARG, zs.zero_last_error()
    assert h.value is None


def test_sgd_entry_points_reject_dead_handles():
    L = zs.lib()
    bogus = ctypes.c_void_p(0xDEAD0)
    info = zs.ZeroStepInfo()
    assert L.zero_sgd_step(bogus, None, None, ctypes.byref(info)) == zs.ZERO_ERR_STATE
    assert L.zero_sgd_step_gated(bogus, None, None) == zs.ZERO_ERR_STATE
    h = ctypes.c_void_p()
    assert L.zero_shard_init_sgd(None, ctypes.byref(GOOD_SGD), ctypes.byref(GOOD_LS),
                                 ctypes.byref(h)) == zs.ZERO_ERR_INVALID_ARG
    assert L.zero_shard_init_sgd(ctypes.byref(_desc(exp_avg_sq=0)), None, ctypes.byref(GOOD_LS),
                                 ctypes.byref(h)) == zs.ZERO_ERR_INVALID_ARG


def test_init_accepts_scales_at_the_fp32_reciprocal_limits():
    """3e-39 and 1.4e45 keep a finite, non-zero fp32 reciprocal: the loss-scale
    check passes them, and init goes on to the device queries (which fail here
    without a GPU, with another status than INVALID_ARG for the scale)."""
    for init, mn in ((3e-39, 3e-39), (1.4e45, 1.0)):
        ls = zs.ZeroLossScaleCfg(init, 1, 1000, mn)
        h = ctypes.c_void_p()
        s = zs.lib().zero_shard_init(ctypes.byref(_desc()), ctypes.byref(GOOD_HP),
                                     ctypes.byref(ls), ctypes.byref(h))
        assert "loss scale" not in zs.zero_last_error(), (init, s, zs.zero_last_error())


def test_binding_refuses_bad_contribution_tensors():
    """The binding checks each contribution tensor against the handle's storage
    dtype and the elements the call reads, before any address crosses the ABI
    (the library's own range check sees whole allocations, not tensors)."""
    import torch
    h = 0x5EED0
    zs._handles[h] = (torch.float16, 1000)
    try:
        good = torch.zeros(1000, dtype=torch.float16)
        cases = [
            (lambda: zs.zero_bucket_reduce(h, [torch.zeros(100, dtype=torch.float32)], 0, 100),
             TypeError),
            (lambda: zs.zero_bucket_reduce(h, [good[:50]], 0, 100), ValueError),
            (lambda: zs.zero_bucket_reduce(h, [good[::2]], 0, 100), ValueError),
            (lambda: zs.zero_step_device(h, [good, good[:999]]), ValueError),
            (lambda: zs.zero_step_device(h, [good.to(torch.bfloat16)]), TypeError),
            (lambda: zs.reduce_buckets(h, [good[:999]], 1000, 100), ValueError),
        ]
        for call, err in cases:
            with pytest.raises(err):
                call()
        # the right dtype, shape and size passes the binding's checks and
        # fails only at the device test (a CPU tensor here)
        with pytest.raises(ValueError, match="GPU"):
            zs.zero_bucket_reduce(h, [good[:100]], 0, 100)
    finally:
        zs._handles.pop(h, None)


def _noalloc(desc=None, hp=None, ls=None, max_norm=0.0, counters=(0, 1024.0, 0)):
    t, sc, g = ctypes.c_int64(counters[0]), ctypes.c_double(counters[1]), \
        ctypes.c_int64(counters[2])
    return zs.lib().zero_adam_step_noalloc(
        None if desc is False else ctypes.byref(desc or _desc()),
        None if hp is False else ctypes.byref(hp or GOOD_HP),
        None if ls is False else ctypes.byref(ls or GOOD_LS),
        max_norm, None, 0, ctypes.byref(t), ctypes.byref(sc), ctypes.byref(g), None, None), \
        (t.value, sc.value, g.value)


@pytest.mark.parametrize("kw", [
    dict(desc=False), dict(hp=False), dict(ls=False),
    dict(desc=_desc(psi=0)), dict(desc=_desc(rank=4)), dict(desc=_desc(lp=7)),
    dict(desc=_desc(master=0)), dict(desc=_desc(grad_shard=0x60001)),
    dict(hp=zs.ZeroAdamHParams(1e-3, 1.0, 0.999, 1e-8, 0.0, 1, 0, 0)),
    dict(ls=zs.ZeroLossScaleCfg(0.0, 1, 1000, 1.0)),
    dict(counters=(-1, 1024.0, 0)), dict(counters=(0, 0.0, 0)),
    dict(counters=(0, float("inf"), 0)), dict(counters=(0, 1e-40, 0)),
    dict(counters=(0, 1024.0, -1)),
    dict(max_norm=-1.0), dict(max_norm=float("nan")), dict(max_norm=float("inf")),
], ids=lambda kw: ",".join(f"{k}={v}" for k, v in kw.items()))
def test_noalloc_rejects_bad_arguments_before_device_work(kw):
    """The allocation-free step validates its desc, hyper-parameters, loss-scale
    configuration, counters and clipping limit before it touches a device (the
    same rules as zero_shard_init and zero_shard_set_counters), and leaves the
    caller's counters untouched when it refuses."""
    counters = kw.get("counters", (0, 1024.0, 0))
    s, after = _noalloc(**kw)
    assert s == zs.ZERO_ERR_INVALID_ARG, (s, zs.zero_last_error())
    assert zs.zero_last_error()
    assert after == counters


def test_noalloc_null_counters():
    L = zs.lib()
    t, sc = ctypes.c_int64(0), ctypes.c_double(1.0)
    for args in ((None, ctypes.byref(sc), ctypes.byref(t)),
                 (ctypes.byref(t), None, ctypes.byref(t)),
                 (ctypes.byref(t), ctypes.byref(sc), None)):
        assert L.zero_adam_step_noalloc(ctypes.byref(_desc()), ctypes.byref(GOOD_HP),
                                        ctypes.byref(GOOD_LS), 0.0, None, 0, *args, None,
                                        None) == zs.ZERO_ERR_INVALID_ARG
