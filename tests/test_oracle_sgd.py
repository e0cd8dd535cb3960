"""Pins of the oracle's optimizer and storage variants: SGD with and without
momentum (the K = 4 and K = 0 optimizers of the blog.vllbc.top page's
extension group C) and 4-byte storage of grads and params (b = 4).

The pages give no SGD formula; the oracle follows textbook heavy-ball SGD with
L2 weight decay.  Pins: closed forms for constant gradients, special cases that
reduce to plain SGD or to no update, the loss-scale and sign symmetries, and
the invariant that the storage format changes where values live, not the
update (fp32-stored gradients that hold fp16 values give the fp16 update)."""
import numpy as np
import pytest

FP16, BF16, FP32 = 1, 2, 3


def f16_bits(x):
    return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


def f16_vals(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def ulp32(x):
    return np.spacing(np.abs(np.asarray(x, np.float32))).astype(np.float64)


G = np.array([1e-3, -1e-3, 0.5, -2.0, 3e-6, -7e-7, 1e-4, 60.0], np.float32)


def _sgd(oracle, lp, g, p0, buf0, hp, steps, scale=1.0):
    p = np.array(p0, np.float32)
    buf = None if buf0 is None else np.array(buf0, np.float32)
    for _ in range(steps):
        oracle.sgd_update(lp, g, p, buf, None, oracle.sgd_scalars(hp, scale))
    return p, buf


def test_plain_sgd_constant_gradient(oracle):
    hp = oracle.SGDHP(lr=1e-2, momentum=0.0)
    p0 = np.linspace(-1, 1, 8).astype(np.float32)
    for t in (1, 2, 10):
        p, _ = _sgd(oracle, FP32, G, p0, None, hp, t)
        want = p0.astype(np.float64) - t * np.float64(np.float32(1e-2)) * G
        assert np.all(np.abs(p - want) <= 2 * t * ulp32(want) + 1e-12), t


def test_momentum_closed_form(oracle):
    """Constant g from buf = 0: buf_t = g (1 - mu^t) / (1 - mu) and
    p_t = p_0 - lr * sum_s buf_s."""
    mu = np.float64(np.float32(0.9))
    lr = np.float64(np.float32(1e-2))
    hp = oracle.SGDHP(lr=1e-2, momentum=0.9)
    p0 = np.linspace(-1, 1, 8).astype(np.float32)
    p = p0.copy()
    buf = np.zeros(8, np.float32)
    acc = np.zeros(8)
    for t in range(1, 11):
        oracle.sgd_update(FP32, G, p, buf, None, oracle.sgd_scalars(hp, 1.0))
        bt = G * (1 - mu**t) / (1 - mu)
        acc += bt
        assert np.allclose(buf, bt, rtol=3e-6, atol=0), t
        assert np.allclose(p, p0 - lr * acc, rtol=2e-6, atol=1e-6), t


def test_zero_momentum_equals_plain_sgd(oracle):
    rng = np.random.default_rng(1)
    g = rng.standard_normal(1000).astype(np.float32)
    p0 = rng.standard_normal(1000).astype(np.float32)
    a, _ = _sgd(oracle, FP32, g, p0, np.zeros(1000), oracle.SGDHP(lr=0.1, momentum=0.0), 3)
    b, _ = _sgd(oracle, FP32, g, p0, None, oracle.SGDHP(lr=0.1, momentum=0.0), 3)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_weight_decay_only(oracle):
    """g = 0: the L2 term alone gives p1 = p0 (1 - lr wd)."""
    hp = oracle.SGDHP(lr=1e-2, momentum=0.0, weight_decay=0.1)
    p0 = np.linspace(-1, 1, 8).astype(np.float32)
    p, _ = _sgd(oracle, FP32, np.zeros(8, np.float32), p0, None, hp, 1)
    want = p0.astype(np.float64) * (1 - np.float64(np.float32(1e-2)) * np.float64(np.float32(0.1)))
    assert np.all(np.abs(p - want) <= 2 * ulp32(want))
    # with momentum the decayed gradient enters the buffer
    p, buf = _sgd(oracle, FP32, np.zeros(8, np.float32), p0, np.zeros(8),
                  oracle.SGDHP(lr=1e-2, momentum=0.5, weight_decay=0.1), 1)
    assert np.allclose(buf, 0.1 * p0, rtol=1e-6)


def test_lr_zero_and_sign_symmetry(oracle):
    rng = np.random.default_rng(2)
    g = rng.standard_normal(256).astype(np.float32)
    p0 = rng.standard_normal(256).astype(np.float32)
    p, buf = _sgd(oracle, FP32, g, p0, np.zeros(256), oracle.SGDHP(lr=0.0, momentum=0.9), 2)
    assert np.array_equal(p, p0) and np.all(buf != 0)
    a, ba = _sgd(oracle, FP32, g, np.zeros(256), np.zeros(256), oracle.SGDHP(lr=0.1), 3)
    b, bb = _sgd(oracle, FP32, -g, np.zeros(256), np.zeros(256), oracle.SGDHP(lr=0.1), 3)
    assert np.array_equal(a, -b) and np.array_equal(ba, -bb)


def test_sgd_loss_scale_transparency(oracle):
    rng = np.random.default_rng(3)
    g = rng.standard_normal(512).astype(np.float32)
    p0 = rng.standard_normal(512).astype(np.float32)
    hp = oracle.SGDHP(lr=0.05, momentum=0.9, weight_decay=0.01)
    a, ba = _sgd(oracle, FP32, g, p0, np.zeros(512), hp, 3, scale=1.0)
    b, bb = _sgd(oracle, FP32, g * np.float32(1024.0), p0, np.zeros(512), hp, 3, scale=1024.0)
    assert np.array_equal(a, b) and np.array_equal(ba, bb)


def test_mixed_precision_sgd_casts_master(oracle):
    hp = oracle.SGDHP(lr=1e-2, momentum=0.9)
    g = f16_bits(G)
    p = np.linspace(-1, 1, 8).astype(np.float32)
    buf = np.zeros(8, np.float32)
    param = np.zeros(8, np.uint16)
    oracle.sgd_update(FP16, g, p, buf, param, oracle.sgd_scalars(hp, 1.0))
    assert np.array_equal(param, f16_bits(p))
    assert np.array_equal(buf, f16_vals(g).astype(np.float32))


def test_fp32_storage_reduce_and_flags(oracle):
    rng = np.random.default_rng(4)
    for R in (1, 2, 4, 8):
        ints = rng.integers(-1 << 20, 1 << 20, size=(R, 3001)).astype(np.float32)
        got = oracle.bucket_reduce(FP32, list(ints))
        assert got.dtype == np.float32
        assert np.array_equal(got, (ints.astype(np.float64).sum(0) / R).astype(np.float32))
    x = rng.standard_normal(5000).astype(np.float32)
    f, s = oracle.flag_sumsq(FP32, x, 4.0)
    assert f == 0 and np.sqrt(s) == pytest.approx(np.linalg.norm(x.astype(np.float64) / 4.0), rel=1e-12)
    for bad in (np.inf, -np.inf, np.nan):
        y = x.copy()
        y[4999] = bad
        assert oracle.flag_sumsq(FP32, y, 1.0)[0] == 1
    cs = [rng.standard_normal(10007).astype(np.float32) for _ in range(4)]
    a = oracle.reduce_shard(FP32, cs, 10007)
    for cb in (1, 9, 4096):
        assert np.array_equal(oracle.reduce_shard(FP32, cs, cb), a)


def test_storage_changes_where_values_live_not_the_update(oracle):
    """fp32-stored gradients holding fp16 values give the fp16-storage update,
    for Adam and for SGD with momentum, bitwise."""
    rng = np.random.default_rng(5)
    n, R = 4096, 4
    c16 = [f16_bits(rng.standard_normal(n) * 4) for _ in range(R)]
    c32 = [f16_vals(c).astype(np.float32) for c in c16]
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    ls = oracle.LossScale(init_scale=4.0)
    for hp, mv in ((oracle.AdamHP(lr=1e-3, weight_decay=0.01), True),
                   (oracle.SGDHP(lr=1e-2, momentum=0.9, weight_decay=0.01), False)):
        z = np.zeros(n)
        a = oracle.new_state(FP16, master, z, z if mv else None, hp, ls)
        b = oracle.new_state(FP32, master, z, z if mv else None, hp, ls)
        # R contributions whose mean is an fp16 value on both sides: R identical copies
        for s in range(3):
            oracle.step(a, [c16[s]] * R, 1000, hp, ls)
            oracle.step(b, [c32[s]] * R, 1000, hp, ls)
        assert np.array_equal(a.master.view(np.uint32), b.master.view(np.uint32))
        assert np.array_equal(a.m.view(np.uint32), b.m.view(np.uint32))
        assert b.param is None


def test_sgd_shard_concat_equals_unsharded(oracle):
    hp = oracle.SGDHP(lr=1e-2, momentum=0.9, weight_decay=0.01)
    ls = oracle.LossScale(init_scale=1.0, dynamic=0)
    rng = np.random.default_rng(6)
    psi, R = 1003, 4
    flat = rng.standard_normal(psi).astype(np.float32)
    cs = [[rng.standard_normal(psi).astype(np.float32) for _ in range(R)] for _ in range(3)]
    full = oracle.new_state(FP32, flat, np.zeros(psi), None, hp, ls)
    for s in range(3):
        oracle.step(full, cs[s], 128, hp, ls)
    for nd in (2, 5):
        parts = []
        for r in range(nd):
            sm = oracle.take_shard(flat, nd, r)
            st = oracle.new_state(FP32, sm, np.zeros(sm.size), None, hp, ls)
            for s in range(3):
                oracle.step(st, [oracle.take_shard(c, nd, r) for c in cs[s]], 50, hp, ls)
            parts.append(st)
        for a in ("master", "m", "grad"):
            cat = np.concatenate([getattr(p, a) for p in parts])[:psi]
            assert np.array_equal(cat.view(np.uint32), getattr(full, a).view(np.uint32)), (nd, a)
