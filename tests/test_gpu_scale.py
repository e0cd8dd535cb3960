"""GPU parity of the dynamic loss scale over a long trajectory, in every flow:
the scale halves on each overflowing step down to min_scale, and doubles after
growth_interval clean steps in a row, the counter restarting after an overflow
and after each doubling.  The workloads never reach their growth interval
(1000), so this test shortens it to 4 and plants overflows so that the scale
hits the floor, grows back in several doublings, and halves again.  Every
step's flag, t, scale used and next scale, and the final state, are compared
with the oracle."""
import dataclasses

import pytest
import torch

from gpu_common import compare, log, ls_of, run_gpu, run_oracle
from zero_dp_sharded_amd import synth

pytestmark = pytest.mark.gpu

ELEMS, CB = 50_001, 20_000
INJECT = {3, 4, 5, 17}          # steps (0-based) with a +inf in contribution 0


def _setup():
    w = dataclasses.replace(synth.WORKLOADS["tiny"], steps=30, scale=8.0, dynamic=1,
                            inject_step=None)
    ls = ls_of(w, growth_interval=4, min_scale=2.0)
    return w, ls


def _plant(step, bufs):
    if step in INJECT:
        bufs[0][ELEMS // 2] = float("inf")


def _check_trajectory(infos):
    """The scale sequence this schedule must produce, step by step."""
    used = [i.scale_used for i in infos]
    assert used[:4] == [8.0] * 4                    # overflow at step 3
    assert used[4:7] == [4.0, 2.0, 2.0]             # halved at 3 and 4, held at the floor at 5
    assert used[6:10] == [2.0] * 4 and used[10] == 4.0   # 4 clean steps (6-9), then doubled
    assert used[10:14] == [4.0] * 4 and used[14] == 8.0
    assert used[14:18] == [8.0] * 4 and used[18] == 4.0  # overflow at 17 halves it again
    assert used[-1] == 16.0 and infos[-1].scale_next == 32.0


@pytest.mark.parametrize("flow", ["sync", "gated", "device"])
def test_scale_growth_floor_and_halving(flow):
    w, ls = _setup()
    log(f"scale trajectory, {flow} flow")
    g = run_gpu(w, elems=ELEMS, bucket_elems=CB, ls=ls, flow=flow, hook=_plant)
    st, oi = run_oracle(w, g, bucket_elems=CB, ls=ls)
    assert compare(w, g, st, oi, f"scale {flow}")["bitwise"]
    assert [i.overflow for i in g.infos] == [int(s in INJECT) for s in range(w.steps)]
    _check_trajectory(g.infos)
    assert g.infos[-1].step_t == w.steps - len(INJECT)


def test_scale_trajectory_device_run():
    """The device-resident flow run as one uninterrupted sequence of steps: the
    host learns the counters only at the end, and the contributions of each
    step are drawn with the scale the synchronous flow used at that step."""
    w, ls = _setup()
    ref = run_gpu(w, elems=ELEMS, bucket_elems=CB, ls=ls, flow="sync", hook=_plant)
    scales = [i.scale_used for i in ref.infos]
    log("scale trajectory, uninterrupted device-resident flow")
    g = run_gpu(w, elems=ELEMS, bucket_elems=CB, ls=ls, flow="device_run", hook=_plant,
                scale_of=lambda s: scales[s])
    st, oi = run_oracle(w, g, bucket_elems=CB, ls=ls)
    assert compare(w, g, st, oi, "scale device_run")["bitwise"]
    last = g.infos[-1]
    assert (last.step_t, last.scale_next) == (st.t, st.scale)
    assert torch.equal(torch.from_numpy(g.master), torch.from_numpy(ref.master))
