"""Pins of the oracle's step arithmetic: reduce, overflow flag, norm, Adam, loss
scale and the flat partition.

The pages print no Adam example, so Adam is pinned by closed forms of the
textbook algorithm (Kingma & Ba 2015, Algorithm 1) that hold for special
inputs, by special cases, and by invariants the pages state (the blog.vllbc.top
ZeRO/DeepSpeed page: partitioning changes where states live, not the math of a
step).  The reduce is pinned by exact sums and by numpy's float16 rounding of
the exact mean; the norm by numpy.linalg.norm.
"""
from fractions import Fraction

import numpy as np
import pytest

FP16, BF16, FP32 = 1, 2, 3


def f16_bits(x):
    return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


def f16_vals(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def ulp32(x):
    x = np.abs(np.asarray(x, np.float32))
    return np.spacing(x).astype(np.float64)


# ------------------------------------------------------------------ reduce

def test_reduce_exact_integer_sums(oracle):
    """Integer-valued fp16 contributions: every fp32 partial sum is exact, so the
    result is the exact mean rounded once to fp16."""
    rng = np.random.default_rng(0)
    for R in (1, 2, 3, 4, 8, 16):
        ints = rng.integers(-1000, 1000, size=(R, 4097))
        cs = [f16_bits(c) for c in ints]
        got = oracle.bucket_reduce(FP16, cs)
        mean = ints.sum(axis=0) / R
        # divisor is R as fp32 reciprocal; exact for powers of two
        if R & (R - 1) == 0:
            assert np.array_equal(got, f16_bits(mean.astype(np.float32)))
        else:
            inv = np.float32(1.0 / R)
            want = (ints.sum(axis=0).astype(np.float32) * inv).astype(np.float16).view(np.uint16)
            assert np.array_equal(got, want)


def test_reduce_scales_by_fp32_reciprocal(oracle):
    """The mean is the fp32 sum times fp32(1/R) (one fp32 rounding), not the sum
    divided by R; the two differ in the last fp32 bit for some sums when R is not
    a power of two.  fp32 storage keeps that bit.  Integer contributions make
    every partial sum exact, and sum * fp32(1/R) is exact in fp64, so rounding
    it once to fp32 gives the expected value."""
    rng = np.random.default_rng(3)
    for R in (3, 5, 6, 7):
        ints = rng.integers(-1000, 1000, size=(R, 4099))
        cs = [c.astype(np.float32) for c in ints]
        got = oracle.bucket_reduce(FP32, cs)
        sums = ints.sum(axis=0).astype(np.float64)
        want = (sums * np.float64(np.float32(1.0 / R))).astype(np.float32)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), R
        divided = (sums / R).astype(np.float32)
        assert np.any(want != divided), R          # the pin tells the two apart


def test_reduce_brute_force_fractions(oracle):
    """Tiny inputs, exact rational mean, one rounding to fp16 (numpy)."""
    rng = np.random.default_rng(1)
    R = 4
    x = rng.standard_normal((R, 257)).astype(np.float32) * 3
    cs = [f16_bits(c) for c in x]
    got = oracle.bucket_reduce(FP16, cs)
    for i in range(257):
        exact = sum(Fraction(float(f16_vals(cs[r][i:i + 1])[0])) for r in range(R)) / R
        # fp32 partial sums of 4 fp16 values within a 2^12 range are exact
        want = np.float64(exact).astype(np.float16).view(np.uint16)
        assert got[i] == want


def test_reduce_identical_contributions(oracle):
    rng = np.random.default_rng(2)
    x = f16_bits(rng.standard_normal(1000))
    for R in (1, 2, 4, 8, 16, 64):
        assert np.array_equal(oracle.bucket_reduce(FP16, [x] * R), x)
    xb = (rng.standard_normal(1000).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(oracle.bucket_reduce(BF16, [xb] * 8), xb)


def test_reduce_is_mean_not_sum(oracle):
    c = [f16_bits(np.full(8, 2.0))] * 4
    assert np.all(f16_vals(oracle.bucket_reduce(FP16, c)) == 2.0)


def test_reduce_bucket_size_invariance(oracle):
    rng = np.random.default_rng(3)
    cs = [f16_bits(rng.standard_normal(10007)) for _ in range(8)]
    a = oracle.reduce_shard(FP16, cs, 10007)
    for cb in (1, 7, 8, 9, 1000, 4096):
        assert np.array_equal(oracle.reduce_shard(FP16, cs, cb), a)


def test_reduce_signed_zero_starts_from_plus_zero(oracle):
    # acc starts at +0: the mean of -0 contributions is +0
    z = np.array([0x8000], np.uint16)
    assert oracle.bucket_reduce(FP16, [z, z])[0] == 0x0000


def test_reduce_overflow_and_nan(oracle):
    big = f16_bits([60000.0, 60000.0, 1.0, 1.0])
    assert f16_vals(oracle.bucket_reduce(FP16, [big, big])).tolist()[:2] == [60000.0, 60000.0]
    # the mean of finite fp16 values is never beyond the largest of them, so the
    # cast back to fp16 cannot overflow: the mean of maxima stays 65504
    mx = np.array([0x7BFF], np.uint16)
    assert oracle.bucket_reduce(FP16, [mx] * 16)[0] == 0x7BFF
    # a non-finite contribution reaches the stored value
    pinf, ninf = np.array([0x7C00], np.uint16), np.array([0xFC00], np.uint16)
    assert oracle.bucket_reduce(FP16, [mx, pinf, mx, mx])[0] == 0x7C00
    assert np.isnan(f16_vals(oracle.bucket_reduce(FP16, [pinf, ninf]))[0])
    # bf16: same, with its own encodings
    b_inf = np.array([0x7F80], np.uint16)
    b_one = np.array([0x3F80], np.uint16)
    assert oracle.bucket_reduce(BF16, [b_one, b_inf])[0] == 0x7F80


# ------------------------------------------------------------------ flag and norm

def test_flag_and_norm(oracle):
    rng = np.random.default_rng(4)
    g = f16_bits(rng.standard_normal(5000) * 8)
    for scale in (1.0, 1024.0, 65536.0):
        f, s = oracle.flag_sumsq(FP16, g, scale)
        assert f == 0
        ref = np.linalg.norm(f16_vals(g) / scale)
        assert np.sqrt(s) == pytest.approx(ref, rel=1e-12)
    for pos in (0, 2500, 4999):
        for bad in (0x7C00, 0xFC00, 0x7E00):
            h = g.copy()
            h[pos] = bad
            assert oracle.flag_sumsq(FP16, h, 1.0)[0] == 1
    # bf16 inf / nan
    b = np.full(16, 0x3F80, np.uint16)
    assert oracle.flag_sumsq(BF16, b, 1.0) == (0, 16.0)
    b[7] = 0x7F80
    assert oracle.flag_sumsq(BF16, b, 1.0)[0] == 1
    b[7] = 0x7FC1
    assert oracle.flag_sumsq(BF16, b, 1.0)[0] == 1


def test_flag_on_unscaled_overflow(oracle):
    """The check runs on the unscaled values: with a loss scale below 1 a finite
    stored gradient can unscale past the fp32 range, and that is an overflow.
    bf16 0x7EFF is 0x1.FEp126, twice it is 0x1.FEp127 (below FLT_MAX, finite);
    bf16 0x7F00 is 2^127, twice it is 2^128 (inf)."""
    b = np.full(8, 0x3F80, np.uint16)
    b[3] = 0x7EFF
    f, s = oracle.flag_sumsq(BF16, b, 0.5)
    assert f == 0
    big = 2.0 * float(np.array([0x7EFF << 16], np.uint32).view(np.float32)[0])
    assert big == float.fromhex("0x1.FEp127")
    assert s == 7 * 4.0 + big * big
    b[3] = 0x7F00
    assert oracle.flag_sumsq(BF16, b, 0.5)[0] == 1
    # fp32 storage: 1e38 unscaled by 4 is 4e38 > FLT_MAX
    x = np.array([1.0, 1e38, -2.0], np.float32)
    assert oracle.flag_sumsq(FP32, x, 0.25)[0] == 1
    assert oracle.flag_sumsq(FP32, x, 1.0)[0] == 0
    # fp16: 65504 * 2^120 > FLT_MAX, 65504 * 2^100 is not
    h = f16_bits([65504.0, 1.0])
    assert oracle.flag_sumsq(FP16, h, 2.0 ** -120)[0] == 1
    assert oracle.flag_sumsq(FP16, h, 2.0 ** -100)[0] == 0


def test_unscaled_overflow_skips_the_step(oracle):
    """A whole step whose only fault is a finite gradient that unscales to inf:
    skipped, state bitwise unchanged, t unchanged, the scale halved."""
    hp = oracle.AdamHP(lr=1e-3)
    ls = oracle.LossScale(init_scale=0.5, dynamic=1, min_scale=0.125)
    rng = np.random.default_rng(11)
    n = 64
    master = rng.standard_normal(n).astype(np.float32) * 0.02
    st = oracle.new_state(BF16, master, np.zeros(n, np.float32), np.zeros(n, np.float32), hp, ls)
    before = st.copy()
    c0 = oracle.f32_to_lp(BF16, rng.standard_normal(n).astype(np.float32) * 1e-3)
    c0[17] = oracle.f32_to_lp(BF16, np.array([3e38], np.float32))[0]
    info = oracle.step(st, [c0], n, hp, ls)
    assert (info.overflow, info.skipped, info.step_t) == (1, 1, 0)
    assert (info.scale_used, info.scale_next) == (0.5, 0.25)
    assert not np.isfinite(info.grad_norm)
    for a, b in ((st.master, before.master), (st.m, before.m), (st.v, before.v)):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.array_equal(st.param, before.param)
    # the same gradient at scale 1 is an ordinary step
    st2 = oracle.new_state(BF16, master, np.zeros(n, np.float32), np.zeros(n, np.float32), hp,
                           oracle.LossScale(init_scale=1.0))
    info2 = oracle.step(st2, [c0], n, hp, oracle.LossScale(init_scale=1.0))
    assert (info2.overflow, info2.step_t) == (0, 1) and np.isfinite(info2.grad_norm)
    # two such contributions overflow the fp32 accumulator itself (6e38): the
    # stored mean is inf, an overflow at any scale
    st3 = oracle.new_state(BF16, master, np.zeros(n, np.float32), np.zeros(n, np.float32), hp,
                           oracle.LossScale(init_scale=1.0))
    info3 = oracle.step(st3, [c0, c0.copy()], n, hp, oracle.LossScale(init_scale=1.0))
    assert st3.grad[17] == 0x7F80 and info3.overflow == 1


# ------------------------------------------------------------------ Adam

def _adam_once(oracle, g_bits, master, m, v, hp, t, scale=1.0, lp=FP16):
    master = np.array(master, np.float32)
    m = np.array(m, np.float32)
    v = np.array(v, np.float32)
    param = np.zeros(master.size, np.uint16)
    sc = oracle.adam_scalars(hp, t, scale)
    oracle.adam_update(lp, np.asarray(g_bits, np.uint16), master, m, v, param, sc, hp.wd_mode)
    return master, m, v, param


G_TEST = [1e-3, -1e-3, 0.5, -2.0, 3e-6, -7e-7, 1e-4, 60.0]


def test_adam_first_step_closed_form(oracle):
    """m0 = v0 = 0, bias correction on, wd = 0: p1 = p0 - lr g / (|g| + eps)."""
    hp = oracle.AdamHP(lr=1e-3, eps=1e-8)
    g = f16_bits(G_TEST)
    gv = f16_vals(g)
    p0 = np.linspace(-0.05, 0.05, len(G_TEST)).astype(np.float32)
    p1, m1, v1, par = _adam_once(oracle, g, p0, np.zeros(8), np.zeros(8), hp, t=1)
    want = p0.astype(np.float64) - 1e-3 * gv / (np.abs(gv) + 1e-8)
    step = 1e-3 * np.abs(gv) / (np.abs(gv) + 1e-8)
    assert np.all(np.abs(p1 - want) <= 4e-6 * step + 2 * ulp32(want))
    # the betas are the fp32 roundings of 0.9 and 0.999
    omb1 = 1 - np.float64(np.float32(0.9))
    omb2 = 1 - np.float64(np.float32(0.999))
    assert np.allclose(m1, omb1 * gv, rtol=1e-6, atol=0)
    assert np.allclose(v1, omb2 * gv * gv, rtol=1e-6, atol=0)
    assert np.array_equal(par, f16_bits(p1))


def test_adam_constant_gradient_closed_form(oracle):
    """Constant g from m0 = v0 = 0: the bias-corrected moments are g and g^2
    exactly in real arithmetic, so every step moves p by lr g / (|g| + eps)."""
    hp = oracle.AdamHP(lr=1e-3, eps=1e-8, beta1=0.9, beta2=0.999)
    g = f16_bits(G_TEST)
    gv = f16_vals(g)
    p = np.full(8, 0.5, np.float32)
    m = np.zeros(8, np.float32)
    v = np.zeros(8, np.float32)
    for t in range(1, 11):
        p, m, v, _ = _adam_once(oracle, g, p, m, v, hp, t)
        want = 0.5 - t * 1e-3 * gv / (np.abs(gv) + 1e-8)
        step = t * 1e-3 * np.abs(gv) / (np.abs(gv) + 1e-8)
        assert np.all(np.abs(p - want) <= 2e-5 * step + 4 * t * ulp32(want)), t
        b1t = np.float64(np.float32(0.9)) ** t
        b2t = np.float64(np.float32(0.999)) ** t
        assert np.allclose(m, (1 - b1t) * gv, rtol=2e-5, atol=0)
        assert np.allclose(v, (1 - b2t) * gv * gv, rtol=5e-5, atol=0)


def test_adam_nonzero_moments_closed_form(oracle):
    """m_t = b1^t m0 + (1 - b1^t) g and v_t = b2^t v0 + (1 - b2^t) g^2 for a
    constant g (the recurrences unrolled)."""
    hp = oracle.AdamHP(lr=1e-4)
    rng = np.random.default_rng(5)
    g = f16_bits(rng.standard_normal(64) * 1e-3)
    gv = f16_vals(g)
    m0 = (rng.standard_normal(64) * 1e-4).astype(np.float32)
    v0 = np.abs(rng.standard_normal(64) * 1e-8).astype(np.float32)
    p = (rng.standard_normal(64) * 0.02).astype(np.float32)
    m, v = m0.copy(), v0.copy()
    p_ref = p.astype(np.float64)
    b1 = np.float64(np.float32(0.9))
    b2 = np.float64(np.float32(0.999))
    for t in range(1, 11):
        p, m, v, _ = _adam_once(oracle, g, p, m, v, hp, t)
        mt = b1**t * m0 + (1 - b1**t) * gv
        vt = b2**t * v0 + (1 - b2**t) * gv * gv
        assert np.allclose(m, mt, rtol=1e-5, atol=1e-12)
        assert np.allclose(v, vt, rtol=1e-5, atol=1e-18)
        p_ref = p_ref - 1e-4 * (mt / (1 - b1**t)) / (np.sqrt(vt / (1 - b2**t)) + 1e-8)
    assert np.allclose(p, p_ref, rtol=0, atol=1e-8)


def test_adam_lr_zero_keeps_params(oracle):
    hp = oracle.AdamHP(lr=0.0)
    g = f16_bits(G_TEST)
    p0 = np.linspace(-1, 1, 8).astype(np.float32)
    p1, m1, v1, _ = _adam_once(oracle, g, p0, np.zeros(8), np.zeros(8), hp, t=1)
    assert np.array_equal(p1.view(np.uint32), p0.view(np.uint32))
    assert np.all(m1 != 0) and np.all(v1 > 0)


def test_adam_zero_gradient_zero_moments(oracle):
    hp = oracle.AdamHP(lr=1e-3)
    p0 = np.linspace(-1, 1, 8).astype(np.float32)
    p1, m1, v1, _ = _adam_once(oracle, np.zeros(8, np.uint16), p0, np.zeros(8), np.zeros(8), hp, t=1)
    assert np.array_equal(p1.view(np.uint32), p0.view(np.uint32))
    assert np.all(m1 == 0) and np.all(v1 == 0)


def test_adam_beta1_zero_momentum_is_gradient(oracle):
    hp = oracle.AdamHP(beta1=0.0)
    g = f16_bits(G_TEST)
    _, m1, _, _ = _adam_once(oracle, g, np.zeros(8), np.full(8, 5.0), np.zeros(8), hp, t=3)
    assert np.array_equal(m1, f16_vals(g).astype(np.float32))


def test_adam_bias_correction_off(oracle):
    hp = oracle.AdamHP(lr=1e-3, bias_correction=0)
    g = f16_bits(G_TEST)
    gv = f16_vals(g)
    p1, _, _, _ = _adam_once(oracle, g, np.zeros(8), np.zeros(8), np.zeros(8), hp, t=1)
    omb1 = 1 - np.float64(np.float32(0.9))
    omb2 = 1 - np.float64(np.float32(0.999))
    want = -1e-3 * (omb1 * gv) / (np.sqrt(omb2 * gv * gv) + 1e-8)
    assert np.allclose(p1, want, rtol=2e-6, atol=0)


def test_adam_decoupled_weight_decay(oracle):
    """g = 0, m = v = 0: only the decay acts, p1 = p0 (1 - lr wd)."""
    hp = oracle.AdamHP(lr=1e-3, weight_decay=0.1, wd_mode=0)
    p0 = np.linspace(-1, 1, 8).astype(np.float32)
    p1, m1, _, _ = _adam_once(oracle, np.zeros(8, np.uint16), p0, np.zeros(8), np.zeros(8), hp, t=1)
    want = p0.astype(np.float64) * (1 - 1e-4)
    assert np.all(np.abs(p1 - want) <= 2 * ulp32(want))
    assert np.all(m1 == 0)


def test_adam_l2_weight_decay(oracle):
    """L2 mode folds wd p into g: with g = 0 the first step is
    p1 = p0 - lr (wd p0) / (|wd p0| + eps)."""
    hp = oracle.AdamHP(lr=1e-3, weight_decay=0.1, wd_mode=1)
    p0 = np.array([-1, -0.5, 0.25, 1, 2, -3, 0.125, 4], np.float32)
    p1, m1, _, _ = _adam_once(oracle, np.zeros(8, np.uint16), p0, np.zeros(8), np.zeros(8), hp, t=1)
    gd = 0.1 * p0.astype(np.float64)
    want = p0 - 1e-3 * gd / (np.abs(gd) + 1e-8)
    assert np.all(np.abs(p1 - want) <= 4 * ulp32(want))
    assert np.allclose(m1, (1 - np.float64(np.float32(0.9))) * gd, rtol=1e-6)


def test_adam_sign_symmetry(oracle):
    hp = oracle.AdamHP(lr=1e-3)
    rng = np.random.default_rng(6)
    g = f16_bits(rng.standard_normal(256) * 1e-2)
    m0 = (rng.standard_normal(256) * 1e-3).astype(np.float32)
    v0 = np.abs(rng.standard_normal(256) * 1e-6).astype(np.float32)
    a = _adam_once(oracle, g, np.zeros(256), m0, v0, hp, t=2)
    b = _adam_once(oracle, g ^ np.uint16(0x8000), np.zeros(256), -m0, v0, hp, t=2)
    assert np.array_equal(a[0], -b[0]) and np.array_equal(a[1], -b[1]) and np.array_equal(a[2], b[2])


def test_loss_scale_is_transparent(oracle):
    """Contributions scaled by a power of two, then unscaled: same update bitwise."""
    hp = oracle.AdamHP(lr=1e-3, weight_decay=0.01)
    ls1 = oracle.LossScale(init_scale=1.0)
    ls2 = oracle.LossScale(init_scale=4096.0)
    rng = np.random.default_rng(7)
    n, R = 4096, 4
    raw = [rng.standard_normal(n).astype(np.float32) * 1e-3 for _ in range(R)]
    c1 = [f16_bits(x) for x in raw]
    c2 = [f16_bits(f16_vals(x) * 4096.0) for x in c1]
    # keep only values that stay normal in fp16 on both sides
    ok = np.ones(n, bool)
    for x in c1:
        ok &= np.abs(f16_vals(x)) >= 2.0**-14
    c1 = [x[ok] for x in c1]
    c2 = [x[ok] for x in c2]
    n = int(ok.sum())
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    s1 = oracle.new_state(FP16, master, np.zeros(n), np.zeros(n), hp, ls1)
    s2 = oracle.new_state(FP16, master, np.zeros(n), np.zeros(n), hp, ls2)
    oracle.step(s1, c1, 1000, hp, ls1)
    oracle.step(s2, c2, 1000, hp, ls2)
    # the reduced means that stay normal in fp16 unscale exactly
    g1 = f16_vals(s1.grad)
    keep = np.abs(g1) >= 2.0**-14
    assert np.array_equal(s1.master[keep], s2.master[keep])
    assert np.array_equal(s1.m[keep], s2.m[keep])


# ------------------------------------------------------------------ steps, skip, scale

def test_skip_is_bitwise_noop_and_halves_scale(oracle):
    hp = oracle.AdamHP(lr=1e-3)
    ls = oracle.LossScale(init_scale=32768.0, dynamic=1)
    rng = np.random.default_rng(8)
    n, R = 1000, 4
    st = oracle.new_state(FP16, (rng.standard_normal(n) * 0.02).astype(np.float32),
                          np.zeros(n), np.zeros(n), hp, ls)

    def contribs(s, scale):
        cs = [f16_bits(rng.standard_normal(n) * 1e-3 * scale) for _ in range(R)]
        if s == 2:
            cs[0][n // 2 + 1] = 0x7C00
        return cs

    snaps = []
    infos = []
    for s in range(8):
        infos.append(oracle.step(st, contribs(s, st.scale), 300, hp, ls))
        snaps.append(st.copy())
    assert [i.overflow for i in infos] == [0, 0, 1, 0, 0, 0, 0, 0]
    assert [i.scale_used for i in infos] == [32768.0] * 3 + [16384.0] * 5
    assert [i.step_t for i in infos] == [1, 2, 2, 3, 4, 5, 6, 7]
    for a in ("master", "m", "v", "param"):
        assert np.array_equal(getattr(snaps[1], a), getattr(snaps[2], a))


def test_scale_growth_and_floor(oracle):
    ls = oracle.LossScale(init_scale=4.0, dynamic=1, growth_interval=3, min_scale=1.0)
    s, g = 4.0, 0
    seq = []
    for f in (0, 0, 0, 1, 1, 1, 1, 0):
        s, g = oracle.loss_scale_next(f, ls, s, g)
        seq.append(s)
    assert seq == [4.0, 4.0, 8.0, 4.0, 2.0, 1.0, 1.0, 1.0]
    st = oracle.LossScale(init_scale=1.0, dynamic=0)
    assert oracle.loss_scale_next(1, st, 1.0, 0) == (1.0, 0)


def test_scale_clean_count_restarts(oracle):
    """The loss-scale reading (halve on overflow down to min_scale, double
    after growth_interval clean steps) counts clean steps since the scale last
    changed: the count restarts after a growth and after an overflow.
    Hand-computed for interval 2 from 8.0: clean, overflow, then four clean
    steps (two growths), two overflows, one clean step."""
    ls = oracle.LossScale(init_scale=8.0, dynamic=1, growth_interval=2, min_scale=1.0)
    s, g = 8.0, 0
    scales, goods = [], []
    for f in (0, 1, 0, 0, 0, 0, 1, 1, 0):
        s, g = oracle.loss_scale_next(f, ls, s, g)
        scales.append(s)
        goods.append(g)
    assert scales == [8.0, 4.0, 4.0, 8.0, 8.0, 16.0, 8.0, 4.0, 4.0]
    assert goods == [1, 0, 1, 0, 1, 0, 0, 0, 1]


def test_static_scale_never_changes(oracle):
    """A static loss scale (the 7.5B workload's) stays put on an overflow and on
    clean steps, above the floor too, and the clean count is left alone."""
    st = oracle.LossScale(init_scale=8.0, dynamic=0, growth_interval=1, min_scale=1.0)
    assert oracle.loss_scale_next(1, st, 8.0, 3) == (8.0, 3)
    assert oracle.loss_scale_next(0, st, 8.0, 3) == (8.0, 3)


def test_shard_concat_equals_unsharded(oracle):
    """The pages' invariant: partitioning over Nd ranks changes only where the
    states live; concatenating the Nd owner updates equals the Nd = 1 update."""
    hp = oracle.AdamHP(lr=1e-3, weight_decay=0.01)
    ls = oracle.LossScale(init_scale=1024.0)
    rng = np.random.default_rng(9)
    psi, R = 1003, 4
    flat_master = (rng.standard_normal(psi) * 0.02).astype(np.float32)
    flat_c = [[f16_bits(rng.standard_normal(psi) * 1e-3 * 1024) for _ in range(R)] for _ in range(3)]
    full = oracle.new_state(FP16, flat_master, np.zeros(psi), np.zeros(psi), hp, ls)
    for s in range(3):
        oracle.step(full, flat_c[s], 128, hp, ls)
    for nd in (2, 4, 7):
        parts = []
        for r in range(nd):
            sm = oracle.take_shard(flat_master, nd, r)
            st = oracle.new_state(FP16, sm, np.zeros(sm.size), np.zeros(sm.size), hp, ls)
            for s in range(3):
                cs = [oracle.take_shard(c, nd, r) for c in flat_c[s]]
                oracle.step(st, cs, 50, hp, ls)
            parts.append(st)
        cat = lambda a: np.concatenate([getattr(p, a) for p in parts])[:psi]
        for a in ("master", "m", "v", "param", "grad"):
            assert np.array_equal(cat(a).view(np.uint8), getattr(full, a).view(np.uint8)), (nd, a)


def test_partition_layout(oracle):
    assert oracle.partition(1_048_576, 4, 0) == (262_144, 0, 262_144)
    assert oracle.partition(13_000_000_000, 16, 1) == (812_500_000, 812_500_000, 812_500_000)
    assert oracle.partition(128_000_000_000, 64, 63) == (2_000_000_000, 126_000_000_000, 2_000_000_000)
    # ragged: 10 over 4 ranks -> S = 3, last rank holds 1 real element
    assert [oracle.partition(10, 4, r) for r in range(4)] == [(3, 0, 3), (3, 3, 3), (3, 6, 3), (3, 9, 1)]
    flat = np.arange(1, 11, dtype=np.float32)
    shards = [oracle.take_shard(flat, 4, r) for r in range(4)]
    assert np.array_equal(np.concatenate(shards), np.r_[flat, np.zeros(2, np.float32)])
