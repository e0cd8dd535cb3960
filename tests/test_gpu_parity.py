"""GPU parity: the HIP path through the C ABI against the CPU oracle, element by
element, on seeded inputs of every workload shape at sizes the oracle finishes
in seconds (several tiles plus a ragged tail)."""
import dataclasses

import pytest

from gpu_common import compare, log, run_gpu, run_oracle, hp_of, ls_of
from zero_dp_sharded_amd import synth

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


@pytest.mark.parametrize("cb", [50_000_000, 65_536, 100_003])
def test_tiny_full(cb):
    """The tiny workload at full size: 262,144 elements, 4 contributions, 3 steps."""
    w = W["tiny"]
    log(f"tiny full cb={cb}")
    g = run_gpu(w, bucket_elems=cb)
    st, oi = run_oracle(w, g, bucket_elems=cb)
    errs = compare(w, g, st, oi, f"tiny cb={cb}")
    log(errs)
    assert errs["bitwise"]


@pytest.mark.parametrize("name,elems,cb", [
    ("gpt2_1.5b", 300_007, 65_536),
    ("7.5b_bf16", 250_001, 100_000),
    ("13b_inf", 120_013, 16_384),
    ("128b", 400_009, 131_072),
])
def test_workload_reduced(name, elems, cb):
    """Each workload's R, format, loss scale, hyper-parameters, step count and
    overflow event, on a shard the oracle handles in seconds."""
    w = W[name]
    log(f"{name} reduced elems={elems} cb={cb}")
    g = run_gpu(w, elems=elems, bucket_elems=cb)
    st, oi = run_oracle(w, g, bucket_elems=cb)
    errs = compare(w, g, st, oi, name)
    log(errs)
    assert errs["bitwise"]
    if w.inject_step is not None:
        flags = [i.overflow for i in g.infos]
        assert flags == [1 if s == w.inject_step else 0 for s in range(w.steps)]
        assert [i.scale_used for i in g.infos] == \
            [w.scale] * (w.inject_step + 1) + [w.scale / 2] * (w.steps - w.inject_step - 1)


@pytest.mark.parametrize("elems", [1, 2, 7, 8, 9, 15, 16, 17, 255, 256, 257, 2049, 1_000_003])
def test_ragged_sizes(elems):
    w = W["gpt2_1.5b"]
    cb = max(1, elems // 3) if elems > 8 else elems
    g = run_gpu(w, elems=elems, steps=3, bucket_elems=cb)
    st, oi = run_oracle(w, g, bucket_elems=cb)
    assert compare(w, g, st, oi, f"ragged {elems}")["bitwise"]


@pytest.mark.parametrize("R", [1, 2, 3, 5, 8, 16, 17, 64])
def test_contribution_counts(R):
    w = dataclasses.replace(W["tiny"], R=R)
    g = run_gpu(w, elems=70_001, steps=2, bucket_elems=30_000)
    st, oi = run_oracle(w, g, bucket_elems=30_000)
    assert compare(w, g, st, oi, f"R={R}")["bitwise"]


HP_VARIANTS = [
    dict(weight_decay=0.1, wd_mode=0), dict(weight_decay=0.1, wd_mode=1),
    dict(bias_correction=0), dict(beta1=0.0), dict(lr=0.0), dict(initial_step=5),
    dict(beta1=0.5, beta2=0.75, eps=1e-3),
]


@pytest.mark.parametrize("flow", ["sync", "gated", "device"])
@pytest.mark.parametrize("over", HP_VARIANTS)
def test_hparam_variants(over, flow):
    """Each hyper-parameter variant in the synchronous, device-gated and
    device-resident flows (the last computes the step count and the bias
    corrections on the device)."""
    w = W["gpt2_1.5b"]
    hp = hp_of(w, **over)
    g = run_gpu(w, elems=50_001, steps=4, bucket_elems=20_000, hp=hp, flow=flow)
    st, oi = run_oracle(w, g, bucket_elems=20_000, hp=hp)
    assert compare(w, g, st, oi, f"{over} {flow}")["bitwise"]
