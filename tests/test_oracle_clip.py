"""Pins of the oracle's global-norm clipping and of its optimizers against
library routines.

The pages name no clipping; the oracle follows the textbook rule (PyTorch's
clip_grad_norm_): the unscaled gradient is multiplied by
min(1, max_norm / (norm + 1e-6)).  Pins:
  - torch.nn.utils.clip_grad_norm_ on the CPU in float64, through a plain SGD
    step with lr = 1 (the update is then the clipped gradient itself), for
    limits below and above the norm and for norms near 1e-6, where the 1e-6
    term matters;
  - below the limit nothing changes, bitwise;
  - the norm is the unscaled one: a power-of-two loss scale changes nothing;
  - whole trajectories of SGD (momentum, weight decay) and of AdamW with
    clipping against torch.optim.SGD / torch.optim.AdamW after clip_grad_norm_,
    in float64 on the CPU (the oracle runs in fp32, so rel 1e-5);
  - Adam's step is invariant to a positive gradient scale when eps is
    negligible, so clipping leaves a constant-gradient Adam trajectory unchanged.
"""
import numpy as np
import pytest
import torch

FP16, BF16, FP32 = 1, 2, 3


def _torch_clipped(g: np.ndarray, max_norm: float) -> np.ndarray:
    t = torch.tensor(g.astype(np.float64), requires_grad=True)
    t.grad = torch.tensor(g.astype(np.float64))
    torch.nn.utils.clip_grad_norm_([t], max_norm)
    return t.grad.numpy()


def _oracle_clipped(oracle, g: np.ndarray, max_norm: float, scale: float = 1.0) -> np.ndarray:
    """The clipped unscaled gradient through one plain SGD step with lr = 1 from
    p = 0 (p1 = -coef * g)."""
    gs = (g.astype(np.float64) * scale).astype(np.float32)
    _, sumsq = oracle.flag_sumsq(FP32, gs, scale)
    coef = oracle.clip_coef(sumsq, max_norm)
    p = np.zeros(g.size, np.float32)
    oracle.sgd_update(FP32, gs, p, None, None,
                      oracle.sgd_scalars(oracle.SGDHP(lr=1.0, momentum=0.0), scale, coef))
    return -p.astype(np.float64)


@pytest.mark.parametrize("ratio", [0.01, 0.3, 0.999, 1.0, 1.5, 1e6])
@pytest.mark.parametrize("mag", [1.0, 1e-3, 3e-8])
def test_clip_matches_torch_clip_grad_norm(oracle, ratio, mag):
    rng = np.random.default_rng(int(ratio * 1000) + int(-np.log10(mag)))
    g = (rng.standard_normal(4099) * mag).astype(np.float32)
    norm = float(np.linalg.norm(g.astype(np.float64)))
    max_norm = ratio * norm
    got = _oracle_clipped(oracle, g, max_norm)
    want = _torch_clipped(g, max_norm)
    assert np.allclose(got, want, rtol=2e-7 * 8, atol=0), (ratio, mag)
    clipped_norm = np.linalg.norm(got)
    assert clipped_norm <= max_norm * (1 + 1e-6)
    if max_norm >= (norm + 1e-6) * (1 + 1e-9):
        # at or above the limit (plus the 1e-6) the gradient passes unchanged, bitwise
        assert np.array_equal(got.astype(np.float32), g), (ratio, mag)
    else:
        assert clipped_norm == pytest.approx(max_norm * norm / (norm + 1e-6), rel=1e-6)


def test_tiny_norm_uses_the_epsilon(oracle):
    """norm = 1e-6 exactly: coef = max_norm / 2e-6, half of max_norm / norm."""
    g = np.zeros(4, np.float32)
    g[0] = np.float32(1e-6)
    sumsq = float(np.float64(g[0]) ** 2)
    c = oracle.clip_coef(sumsq, 1e-7)
    assert c == pytest.approx(1e-7 / (float(g[0]) + 1e-6), rel=1e-7)
    assert c == pytest.approx(0.05, rel=1e-6)
    assert oracle.clip_coef(sumsq, 0.0) == 1.0
    assert oracle.clip_coef(sumsq, -1.0) == 1.0
    assert oracle.clip_coef(4.0, 1.0) == pytest.approx(0.5, rel=1e-6)


def test_clip_uses_the_unscaled_norm(oracle):
    rng = np.random.default_rng(7)
    g = (rng.standard_normal(2000) * 1e-2).astype(np.float32)
    norm = float(np.linalg.norm(g.astype(np.float64)))
    a = _oracle_clipped(oracle, g, 0.25 * norm, scale=1.0)
    b = _oracle_clipped(oracle, g, 0.25 * norm, scale=4096.0)
    assert np.array_equal(a, b)


def _step_oracle(oracle, hp, lp, p0, m0, v0, grads, max_norm):
    ls = oracle.LossScale(init_scale=1.0, dynamic=0)
    st = oracle.new_state(lp, p0, m0, v0, hp, ls)
    for g in grads:
        oracle.step(st, [g], 1 << 30, hp, ls, max_norm=max_norm)
    return st


@pytest.mark.parametrize("mom,wd", [(0.0, 0.0), (0.9, 0.0), (0.9, 0.01), (0.5, 0.1)])
def test_sgd_clip_trajectory_matches_torch(oracle, mom, wd):
    rng = np.random.default_rng(11)
    n, steps, lr, max_norm = 3001, 4, 0.05, 0.5
    p0 = rng.standard_normal(n).astype(np.float32)
    grads = [(rng.standard_normal(n) * (0.003 if k % 2 else 0.05)).astype(np.float32)
             for k in range(steps)]
    hp = oracle.SGDHP(lr=lr, momentum=mom, weight_decay=wd)
    st = _step_oracle(oracle, hp, FP32, p0, np.zeros(n) if mom else None, None, grads, max_norm)
    # torch reference in float64 with the fp32-rounded hyper-parameters
    f = lambda x: float(np.float32(x))
    p = torch.tensor(p0.astype(np.float64), requires_grad=True)
    opt = torch.optim.SGD([p], lr=f(lr), momentum=f(mom), weight_decay=f(wd))
    for g in grads:
        p.grad = torch.tensor(g.astype(np.float64))
        torch.nn.utils.clip_grad_norm_([p], max_norm)
        opt.step()
    want = p.detach().numpy()
    assert np.allclose(st.master, want, rtol=1e-5, atol=1e-7)
    moved = np.abs(want - p0) > 1e-4
    assert moved.any()


@pytest.mark.parametrize("max_norm", [0.0, 0.05, 1e9])
def test_adamw_clip_trajectory_matches_torch(oracle, max_norm):
    rng = np.random.default_rng(12)
    n, steps = 2003, 5
    lr, b1, b2, eps, wd = 1e-2, 0.9, 0.999, 1e-8, 0.1
    p0 = (rng.standard_normal(n) * 0.1).astype(np.float32)
    grads = [(rng.standard_normal(n) * 0.01).astype(np.float32) for _ in range(steps)]
    hp = oracle.AdamHP(lr=lr, beta1=b1, beta2=b2, eps=eps, weight_decay=wd)
    z = np.zeros(n)
    st = _step_oracle(oracle, hp, FP32, p0, z, z, grads, max_norm)
    f = lambda x: float(np.float32(x))
    p = torch.tensor(p0.astype(np.float64), requires_grad=True)
    opt = torch.optim.AdamW([p], lr=f(lr), betas=(f(b1), f(b2)), eps=f(eps), weight_decay=f(wd))
    for g in grads:
        p.grad = torch.tensor(g.astype(np.float64))
        if max_norm > 0:
            torch.nn.utils.clip_grad_norm_([p], max_norm)
        opt.step()
    want = p.detach().numpy()
    assert np.allclose(st.master, want, rtol=1e-5, atol=1e-8)


@pytest.mark.parametrize("max_norm", [0.0, 0.05, 1e9])
def test_adam_l2_clip_trajectory_matches_torch(oracle, max_norm):
    """L2 weight decay (wd_mode 1) adds wd * p to the gradient after clipping,
    as torch.optim.Adam's weight_decay does to a gradient that
    clip_grad_norm_ has already scaled (float64, CPU)."""
    rng = np.random.default_rng(13)
    n, steps = 2003, 5
    lr, b1, b2, eps, wd = 1e-2, 0.9, 0.999, 1e-8, 0.1
    p0 = (rng.standard_normal(n) * 0.1).astype(np.float32)
    grads = [(rng.standard_normal(n) * 0.01).astype(np.float32) for _ in range(steps)]
    hp = oracle.AdamHP(lr=lr, beta1=b1, beta2=b2, eps=eps, weight_decay=wd, wd_mode=1)
    z = np.zeros(n)
    st = _step_oracle(oracle, hp, FP32, p0, z, z, grads, max_norm)
    f = lambda x: float(np.float32(x))
    p = torch.tensor(p0.astype(np.float64), requires_grad=True)
    opt = torch.optim.Adam([p], lr=f(lr), betas=(f(b1), f(b2)), eps=f(eps), weight_decay=f(wd))
    for g in grads:
        p.grad = torch.tensor(g.astype(np.float64))
        if max_norm > 0:
            torch.nn.utils.clip_grad_norm_([p], max_norm)
        opt.step()
    want = p.detach().numpy()
    assert np.allclose(st.master, want, rtol=1e-5, atol=1e-8)


def test_clipping_leaves_constant_gradient_adam_unchanged(oracle):
    """Adam with eps -> 0 sees g and c*g (c > 0) alike, so a clipped constant
    gradient gives the unclipped trajectory up to rounding."""
    rng = np.random.default_rng(13)
    n = 1000
    g = (rng.standard_normal(n) * 0.1).astype(np.float32)
    p0 = rng.standard_normal(n).astype(np.float32)
    hp = oracle.AdamHP(lr=1e-3, eps=1e-30)
    z = np.zeros(n)
    a = _step_oracle(oracle, hp, FP32, p0, z, z, [g] * 4, 0.0)
    norm = float(np.linalg.norm(g.astype(np.float64)))
    b = _step_oracle(oracle, hp, FP32, p0, z, z, [g] * 4, 0.01 * norm)
    assert np.allclose(a.master, b.master, rtol=1e-6, atol=0)
    assert np.allclose(b.m, 0.01 * a.m, rtol=1e-4)      # the moments do carry the factor


def test_clip_skipped_step_and_global_norm(oracle):
    """An overflowing step stays skipped with clipping; clip_sumsq takes the
    coefficient from a global norm (the sum over shards), not the shard's."""
    hp = oracle.SGDHP(lr=1.0, momentum=0.0)
    ls = oracle.LossScale(init_scale=1.0, dynamic=0)
    g = np.array([3.0, 4.0, 0.0, 0.0], np.float32)
    st = oracle.new_state(FP32, np.zeros(4, np.float32), None, None, hp, ls)
    bad = g.copy()
    bad[2] = np.inf
    info = oracle.step(st, [bad], 4, hp, ls, max_norm=1.0)
    assert info.skipped == 1 and np.all(st.master == 0)
    info = oracle.step(st, [g], 4, hp, ls, max_norm=1.0)
    assert info.grad_norm == 5.0
    assert np.allclose(-st.master, g / 5.0, rtol=1e-6)
    st2 = oracle.new_state(FP32, np.zeros(4, np.float32), None, None, hp, ls)
    oracle.step(st2, [g], 4, hp, ls, max_norm=1.0, clip_sumsq=100.0)   # global norm 10
    assert np.allclose(-st2.master, g / 10.0, rtol=1e-6)
