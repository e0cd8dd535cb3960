"""GPU parity at the sizes where the streaming kernels change shape, element by
element against the oracle.

In a shard of more than 8,388,608 elements (smaller shards run every kernel in
their cache-resident 256-lane shape), a bucket reduce below 8 contributions
gives each lane 3 runs of 16 bytes once the bucket holds at least 491,520 runs
(256 CUs x 10 workgroups x 64 lanes x 3 runs: 3,932,160 two-byte or 1,966,080
fp32 elements) and 2 runs below that; from 8 contributions it gives 1 run.
The stand-alone scan gives each lane 4 runs.  Each case below fills a shard
past 8,388,608 elements with buckets exactly at that threshold and ends it
with one just under it (with a ragged element-wise tail), with every
contribution-count class and storage format, and with base pointers off the
16-byte grid.  The last case steps shards just at and just past the
small-shard limit.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import zero_dp_sharded_amd as zs
from gpu_common import compare, f32, log, run_gpu, run_oracle, u16
from zero_dp_sharded_amd import synth

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
THRESHOLD_RUNS = 256 * 10 * 64 * 3
SMALL_SHARD = 1 << 23               # shards up to this size take the 256-lane shape


def _two_buckets(run_width: int):
    """(shard elements, bucket elements): buckets of exactly THRESHOLD_RUNS
    runs until the shard passes SMALL_SHARD, then one of a run fewer plus a
    ragged tail of run_width - 1."""
    cb = THRESHOLD_RUNS * run_width
    full = SMALL_SHARD // cb + 1
    return full * cb + cb - 1, cb


@pytest.mark.parametrize("R", [1, 2, 3, 4, 5, 7, 8])
def test_reduce_threshold_fp16(R):
    w = dataclasses.replace(W["gpt2_1.5b"], R=R, steps=2)
    S, cb = _two_buckets(8)
    log(f"shapes fp16 R={R} S={S} cb={cb}")
    g = run_gpu(w, elems=S, bucket_elems=cb)
    st, oi = run_oracle(w, g, bucket_elems=cb)
    assert compare(w, g, st, oi, f"fp16 R={R}")["bitwise"]


def test_reduce_threshold_bf16():
    w = dataclasses.replace(W["7.5b_bf16"], R=4, steps=2)
    S, cb = _two_buckets(8)
    log(f"shapes bf16 R=4 S={S} cb={cb}")
    g = run_gpu(w, elems=S, bucket_elems=cb)
    st, oi = run_oracle(w, g, bucket_elems=cb)
    assert compare(w, g, st, oi, "bf16 R=4")["bitwise"]


@pytest.mark.parametrize("R", [3, 4, 8])
def test_reduce_threshold_fp32(R):
    w = dataclasses.replace(W["c1_7.5b_sgdm"], R=R, steps=2)
    S, cb = _two_buckets(4)
    log(f"shapes fp32 R={R} S={S} cb={cb}")
    g = run_gpu(w, elems=S, bucket_elems=cb)
    st, oi = run_oracle(w, g, bucket_elems=cb)
    assert compare(w, g, st, oi, f"fp32 R={R}")["bitwise"]


def test_reduce_threshold_misaligned():
    """Every base 3 elements (6 bytes) off the 16-byte grid: each bucket
    starts with a 5-element head; bucket 0's vector body is then exactly at
    the threshold, bucket 1's one run short of it, with a 1-element tail."""
    w = dataclasses.replace(W["gpt2_1.5b"], R=4, steps=2)
    cb = THRESHOLD_RUNS * 8 + 8
    S = 2 * cb + THRESHOLD_RUNS * 8 - 2
    assert S > SMALL_SHARD
    offs = dict(master=3, m=3, v=3, grad=3, param=3, contrib=3)
    log(f"shapes misaligned S={S} cb={cb}")
    g = run_gpu(w, elems=S, bucket_elems=cb, offsets=offs)
    st, oi = run_oracle(w, g, bucket_elems=cb)
    assert compare(w, g, st, oi, "misaligned")["bitwise"]


def test_scan_multi_block_with_planted_inf():
    """The stand-alone scan (4 runs per lane) over a caller-filled gradient of
    several thousand workgroups and a ragged tail: flag and norm against the
    oracle, then a +inf planted in the last vector run is found."""
    n = 3 * 1024 * 8 * 1000 + 13
    dev = torch.device("cuda", 0)
    master = torch.zeros(n, device=dev)
    m = torch.zeros(n, device=dev)
    v = torch.zeros(n, device=dev)
    grad = torch.empty(n, dtype=torch.float16, device=dev)
    param = torch.zeros(n, dtype=torch.float16, device=dev)
    gen = torch.Generator(device="cuda").manual_seed(11)
    grad.copy_((torch.randn(n, generator=gen, device=dev) * 4.0).half())
    log(f"scan n={n}")
    h = zs.zero_shard_init(master, m, v, grad, param, psi=n * 8, nd=8, rank=0, bucket_elems=n,
                           hp=zs.AdamHParams(lr=1e-3), ls=zs.LossScaleCfg(init_scale=1024.0))
    try:
        info = zs.zero_overflow_check(h)
        flag, ss = oracle.flag_sumsq(oracle.FP16, u16(grad), 1024.0)
        assert info.overflow == flag == 0
        # fp64 sums of 24.6M positive terms in two orders
        assert info.grad_norm == pytest.approx(np.sqrt(ss), rel=1e-9)
        assert zs.zero_adam_step(h).step_t == 1
        last_vec = (n // 8) * 8 - 1
        grad[last_vec] = float("inf")
        assert zs.zero_overflow_check(h).overflow == 1
        assert zs.zero_adam_step(h).skipped == 1
        grad[last_vec] = 0.0
        grad[0] = float("nan")
        assert zs.zero_overflow_check(h).overflow == 1
        assert zs.zero_adam_step(h).skipped == 1
        assert np.isfinite(f32(master)).all()
    finally:
        zs.zero_shard_destroy(h)


@pytest.mark.parametrize("S", [SMALL_SHARD, SMALL_SHARD + 4, SMALL_SHARD + 1])
@pytest.mark.parametrize("flow", ["sync", "device"])
def test_small_shard_limit(S, flow):
    """Shards at the small-shard limit (256-lane cached shape) and just past it
    (the streaming shapes; +1 also with an element-wise tail): bitwise against
    the oracle in the synchronous and device-resident flows."""
    w = dataclasses.replace(W["gpt2_1.5b"], R=4, steps=2)
    log(f"shapes small-shard limit S={S} flow={flow}")
    g = run_gpu(w, elems=S, bucket_elems=3_000_000, flow=flow)
    st, oi = run_oracle(w, g, bucket_elems=3_000_000)
    assert compare(w, g, st, oi, f"S={S} {flow}")["bitwise"]
