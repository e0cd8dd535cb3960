"""The seeded input generator (test infrastructure shared by the oracle side
and the GPU side), checked on the CPU: the stated distributions hold (mean and
standard deviation within 4 sigma of their sampling error), draws are
reproducible and independent across steps, contributions and seeds, the +inf
event lands where the workload says, and the shapes follow the workloads."""
import dataclasses

import numpy as np
import pytest
import torch

from zero_dp_sharded_amd import synth

N = 1 << 20


def _stats(x: torch.Tensor):
    a = x.double().numpy()
    return a.mean(), a.std()


@pytest.mark.parametrize("name", ["tiny", "gpt2_1.5b", "7.5b_bf16", "c1_7.5b_sgdm"])
def test_contributions_follow_the_stated_normal(name):
    w = synth.WORKLOADS[name]
    bufs = [torch.empty(N, dtype=w.torch_lp) for _ in range(2)]
    synth.fill_contribs(w, bufs, 0, w.scale, seed=0)
    s = w.grad_std * w.scale
    for b in bufs:
        mean, std = _stats(b)
        assert abs(mean) < 4 * s / np.sqrt(N)
        assert abs(std - s) < 4 * s / np.sqrt(2 * N) + 1e-2 * s    # + storage rounding
        assert torch.isfinite(b).all()
    assert not torch.equal(bufs[0], bufs[1])                         # r = 0 and r = 1 differ


def test_draws_are_reproducible_and_independent():
    w = synth.WORKLOADS["tiny"]
    a = [torch.empty(4096, dtype=w.torch_lp) for _ in range(w.R)]
    b = [torch.empty(4096, dtype=w.torch_lp) for _ in range(w.R)]
    synth.fill_contribs(w, a, 3, w.scale, seed=7)
    synth.fill_contribs(w, b, 3, w.scale, seed=7)
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    seeds = {synth.contribution_seed(s, st, r) for s in range(3) for st in range(10)
             for r in range(64)}
    assert len(seeds) == 3 * 10 * 64
    synth.fill_contribs(w, b, 4, w.scale, seed=7)
    x, y = a[0].float().numpy(), b[0].float().numpy()
    assert abs(np.corrcoef(x, y)[0, 1]) < 0.1                        # steps draw afresh


def test_inject_event_position():
    w = synth.WORKLOADS["13b_inf"]
    n = 1001
    bufs = [torch.empty(n, dtype=w.torch_lp) for _ in range(3)]
    synth.fill_contribs(w, bufs, w.inject_step, w.scale, seed=0)
    bad = torch.nonzero(~torch.isfinite(bufs[0])).flatten().tolist()
    assert bad == [synth.inject_index(n)] == [n // 2 + 1]
    assert float(bufs[0][n // 2 + 1]) == float("inf")
    assert all(torch.isfinite(b).all() for b in bufs[1:])
    synth.fill_contribs(w, bufs, w.inject_step + 1, w.scale, seed=0)
    assert all(torch.isfinite(b).all() for b in bufs)


def test_initial_state_distributions():
    w = synth.WORKLOADS["7.5b_bf16"]
    master, m, v = synth.init_state(w, torch.device("cpu"), seed=0, elems=N)
    for x, s in ((master, w.master_std), (m, w.m_std)):
        mean, std = _stats(x)
        assert abs(mean) < 4 * s / np.sqrt(N) and abs(std - s) < 4 * s / np.sqrt(2 * N)
    assert (v >= 0).all()
    # |N(0, s)| has mean s * sqrt(2 / pi)
    assert abs(v.double().mean().item() - w.v_std * np.sqrt(2 / np.pi)) < 4 * w.v_std / np.sqrt(N)
    w0 = synth.WORKLOADS["gpt2_1.5b"]
    master, m, v = synth.init_state(w0, torch.device("cpu"), seed=0, elems=4096)
    assert not m.any() and not v.any()


def test_13b_rank1_shard_state_follows_the_layout():
    w = synth.WORKLOADS["13b_inf"]
    layout = synth.layout_13b(psi=w.psi)
    lo = w.begin
    n = 50_000
    master, _, _ = synth.init_state(w, torch.device("cpu"), seed=0, elems=n)
    for name, start, size in layout:
        a, b = max(lo, start), min(lo + n, start + size)
        if a >= b:
            continue
        seg = master[a - lo:b - lo]
        if name.endswith("ln1.w") or name.endswith("ln2.w"):
            assert (seg == 1).all(), name
        elif name.endswith(".b"):
            assert (seg == 0).all(), name
        else:
            assert seg.std().item() == pytest.approx(w.master_std, rel=0.05), name


def test_workload_shapes():
    for name, w in synth.WORKLOADS.items():
        assert w.shard == -(-w.psi // w.nd)
        assert 1 <= w.R <= 64 and w.bucket_elems >= 1
        assert w.opt in ("adam", "sgd")
        assert w.torch_lp in (torch.float16, torch.bfloat16, torch.float32)
        if w.opt == "sgd":
            assert not w.has_v and w.has_m == (w.momentum > 0)
        else:
            assert w.has_m and w.has_v
    assert synth.WORKLOADS["128b"].shard == 2_000_000_000
    assert synth.WORKLOADS["c1_7.5b_sgdm"].shard == 117_187_500


@pytest.mark.parametrize("lp,step", [("fp16", 2), ("bf16", 4), ("fp16", 8), ("fp32", 4),
                                     ("fp32", 8)])
def test_contributions_at_carved_phases(lp, step):
    """phase_step p puts contribution r at (r * p) mod 16 bytes past a 16-byte
    boundary, each a full buffer of its own; 16 keeps them aligned; an fp32
    buffer cannot start 2 bytes off."""
    w = dataclasses.replace(synth.WORKLOADS["gpt2_1.5b"], lp=lp, R=9)
    bufs = synth.alloc_contribs(w, "cpu", elems=1001, phase_step=step)
    assert [b.data_ptr() % 16 for b in bufs] == [(r * step) % 16 for r in range(9)]
    assert all(b.numel() == 1001 and b.dtype == w.torch_lp for b in bufs)
    assert all(b.data_ptr() % 16 == 0 for b in synth.alloc_contribs(w, "cpu", elems=5))
    with pytest.raises(ValueError):
        synth.alloc_contribs(dataclasses.replace(w, lp="fp32"), "cpu", elems=5, phase_step=2)
