"""Pins of the chunked evaluation (oracle.ChunkedRun): k steps evaluated one
C_B bucket at a time give the whole-shard steps' results bitwise, because
everything but the overflow decision and the norm is per element (the
blog.vllbc.top ZeRO/DeepSpeed page: partitioning changes where states live,
not the math of a step; here the partition is into chunks of one shard).

Each case runs the same seeded contributions through oracle.step on the whole
shard and through ChunkedRun (pass 1 per step, then pass 2 per chunk, chunks
in shuffled order), and compares every step's flag, t, norm and scales, every
step's stored gradient and the final master / m / v / param, bitwise.  Pass 2
takes the reduced gradients either stored by pass 1 or recomputed from the
contributions chunk by chunk (the form whose memory is one bucket)."""
import dataclasses

import numpy as np
import pytest

FP16, BF16, FP32 = 1, 2, 3


@dataclasses.dataclass
class Shape:
    name: str
    lp: int
    S: int
    R: int
    cb: int
    steps: int
    scale: float
    dynamic: int = 1
    growth: int = 1000
    opt: str = "adam"
    lr: float = 1e-3
    wd: float = 0.0
    mom: float = 0.0
    m_std: float = 0.0
    v_std: float = 0.0
    inf_step: int = -1
    max_norm: float = 0.0


SHAPES = [
    # the tiny workload's shape, with a planted +inf (a skipped step)
    Shape("tiny", FP16, 262_144, 4, 65_536, 3, 1024.0, inf_step=1),
    # the GPT-2 1.5B shape scaled by 1/1000: 3 full buckets and a 37,500 tail
    Shape("gpt2-shaped", FP16, 187_500, 8, 50_000, 10, 65536.0, wd=0.01),
    Shape("gpt2-shaped, clipped", FP16, 187_500, 8, 50_000, 4, 65536.0, wd=0.01, max_norm=0.02),
    Shape("bf16 static, moments", BF16, 117_187, 8, 50_000, 4, 1.0, dynamic=0, lr=1e-4,
          m_std=1e-4, v_std=1e-8),
    Shape("fp16, growth every 2 clean steps", FP16, 60_001, 3, 16_384, 6, 8.0, growth=2,
          inf_step=3),
    Shape("fp32 SGD with momentum", FP32, 117_187, 8, 50_000, 4, 1.0, dynamic=0, opt="sgd",
          lr=1e-2, wd=1e-4, mom=0.9),
]


def _contribs(oracle, sh, step, scale):
    out = []
    for r in range(sh.R):
        rng = np.random.default_rng(1000 * step + r)
        x = (rng.standard_normal(sh.S) * 1e-3 * scale).astype(np.float32)
        if step == sh.inf_step and r == 0:
            x[sh.S // 2 + 1] = np.inf
        out.append(x if sh.lp == FP32 else oracle.f32_to_lp(sh.lp, x))
    return out


def _hp(oracle, sh):
    if sh.opt == "sgd":
        return oracle.SGDHP(lr=sh.lr, momentum=sh.mom, weight_decay=sh.wd)
    return oracle.AdamHP(lr=sh.lr, weight_decay=sh.wd)


def _state0(sh):
    rng = np.random.default_rng(7)
    master = (rng.standard_normal(sh.S) * 0.02).astype(np.float32)
    m = (rng.standard_normal(sh.S) * sh.m_std).astype(np.float32)
    v = np.abs(rng.standard_normal(sh.S) * sh.v_std).astype(np.float32)
    if sh.opt == "sgd":
        return master, (m if sh.mom else None), None
    return master, m, v


def _bits(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a


@pytest.mark.parametrize("sh", SHAPES, ids=[s.name for s in SHAPES])
@pytest.mark.parametrize("threads,stored", [(1, True), (4, False)])
def test_chunked_equals_unchunked(oracle, sh, threads, stored):
    hp = _hp(oracle, sh)
    ls = oracle.LossScale(init_scale=sh.scale, dynamic=sh.dynamic, growth_interval=sh.growth)
    master0, m0, v0 = _state0(sh)

    # whole shard
    st = oracle.new_state(sh.lp, master0, m0, v0, hp, ls)
    infos, grads, batches = [], [], []
    for s in range(sh.steps):
        cs = _contribs(oracle, sh, s, st.scale)
        batches.append(cs)
        infos.append(oracle.step(st, cs, sh.cb, hp, ls, max_norm=sh.max_norm))
        grads.append(st.grad.copy())

    # chunked: pass 1 per step
    run = oracle.ChunkedRun(sh.lp, sh.S, sh.cb, hp, ls, max_norm=sh.max_norm, threads=threads)
    cgrads = []
    for s in range(sh.steps):
        assert run.scale == infos[s].scale_used
        cs = _contribs(oracle, sh, s, run.scale)
        g = np.empty(sh.S, grads[0].dtype)
        ci = run.scan_step(lambda off, n: [c[off:off + n] for c in cs], grads_out=g)
        cgrads.append(g)
        a, b = infos[s], ci
        assert (a.overflow, a.skipped, a.step_t, a.scale_used, a.scale_next) == \
            (b.overflow, b.skipped, b.step_t, b.scale_used, b.scale_next), (sh.name, s)
        assert np.array_equal(np.float64(a.grad_norm), np.float64(b.grad_norm)) or \
            (np.isnan(a.grad_norm) and np.isnan(b.grad_norm)), (sh.name, s)
        assert np.array_equal(_bits(g), _bits(grads[s])), (sh.name, s)
    if sh.inf_step >= 0:
        assert run.steps[sh.inf_step].overflow == 1

    # pass 2 per chunk, chunks in shuffled order
    master = master0.copy()
    m = None if m0 is None else m0.copy()
    v = None if v0 is None else v0.copy()
    param = None if sh.lp == FP32 else oracle.f32_to_lp(sh.lp, master0)
    chunks = run.chunks()
    order = np.random.default_rng(3).permutation(len(chunks))
    for k in order:
        off, n = chunks[k]
        sl = slice(off, off + n)
        parts = [None if a is None else a[sl].copy() for a in (master, m, v, param)]
        if stored:
            grad_of = lambda s: cgrads[s][sl]
        else:
            grad_of = lambda s: oracle.bucket_reduce(sh.lp, [c[sl] for c in batches[s]])
        run.evolve(*parts, grad_of)
        for a, p in zip((master, m, v, param), parts):
            if a is not None:
                a[sl] = p
    for name, a, b in (("master", master, st.master), ("m", m, st.m), ("v", v, st.v),
                       ("param", param, st.param)):
        assert (a is None) == (b is None), name
        if a is not None:
            assert np.array_equal(_bits(a), _bits(b)), (sh.name, name)
    assert (run.t, run.scale, run.good_steps) == (st.t, st.scale, st.good_steps)


def test_chunked_norm_order_is_the_bucket_order(oracle):
    """The whole-shard norm adds one fp64 sum per bucket in bucket order: it
    equals math.fsum of the squares to the fp64 rounding, and it is exactly
    the sum of the per-bucket sums."""
    import math
    rng = np.random.default_rng(5)
    g = oracle.f32_to_lp(FP16, (rng.standard_normal(100_003) * 3).astype(np.float32))
    f, s = oracle.bucket_flag_sumsq(FP16, g, 4.0, 8_192)
    parts = [oracle.flag_sumsq(FP16, g[o:o + 8_192], 4.0)[1] for o in range(0, g.size, 8_192)]
    acc = 0.0
    for p in parts:
        acc += p
    assert f == 0 and s == acc
    u = oracle.lp_to_f32(FP16, g).astype(np.float64) / 4.0
    assert s == pytest.approx(math.fsum(u * u), rel=1e-13)


@pytest.mark.parametrize("lp,max_norm", [(FP16, 0.0), (BF16, 0.0), (FP16, 0.3)])
def test_chunked_check_of_stored_gradient(oracle, lp, max_norm):
    """The stored-gradient form (no reduce: the owner's slice of an all-reduced
    gradient) chunked, against the same steps written out with the oracle's
    primitives on the whole shard: flag and squared norm per bucket
    (bucket_flag_sumsq), the decision, the update.  A planted inf in one step
    is skipped."""
    n, cb, steps = 100_003, 16_384, 4
    hp = oracle.AdamHP(lr=1e-3, weight_decay=0.01)
    ls = oracle.LossScale(init_scale=1024.0)
    rng = np.random.default_rng(9)
    master0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    grads = []
    for s in range(steps):
        x = (rng.standard_normal(n) * 1e-3 * 1024.0).astype(np.float32)
        if s == 2:
            x[n - 5] = np.inf
        grads.append(oracle.f32_to_lp(lp, x))
    # whole shard, by hand
    st = oracle.new_state(lp, master0, np.zeros(n, np.float32), np.zeros(n, np.float32), hp, ls)
    flags = []
    for g in grads:
        flag, ss = oracle.bucket_flag_sumsq(lp, g, st.scale, cb)
        flags.append(flag)
        if not flag:
            st.t += 1
            sc = oracle.adam_scalars(hp, st.t, st.scale, oracle.clip_coef(ss, max_norm))
            oracle.adam_update(lp, g, st.master, st.m, st.v, st.param, sc, hp.wd_mode)
        st.scale, st.good_steps = oracle.loss_scale_next(flag, ls, st.scale, st.good_steps)
    assert flags == [0, 0, 1, 0]
    # chunked
    run = oracle.ChunkedRun(lp, n, cb, hp, ls, max_norm=max_norm, threads=3)
    for g in grads:
        run.check_step(lambda off, k: g[off:off + k])
    master, m, v = master0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    param = oracle.f32_to_lp(lp, master0)
    for off, k in reversed(run.chunks()):
        sl = slice(off, off + k)
        parts = [master[sl].copy(), m[sl].copy(), v[sl].copy(), param[sl].copy()]
        run.evolve(*parts, lambda s: grads[s][sl])
        master[sl], m[sl], v[sl], param[sl] = parts
    for a, b in ((master, st.master), (m, st.m), (v, st.v)):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.array_equal(param, st.param)
    assert (run.t, run.scale, run.good_steps) == (st.t, st.scale, st.good_steps)
