"""The consecutive-launch path.  A launch whose work-item count would pass
2^31 is split into consecutive launches over consecutive runs and partial
slots; real shards reach that only beyond 8.6e9 elements (2-byte Adam, about
138 GB of state, which one MI355X holds).  __graft_entry__.build() also builds
the library with every launch split after 1024 work-items
(zero_dp_sharded_amd/variants/split_launch/), and these tests run the parity
test files against that build in a child process through ZERO_SHARD_LIB:
Adam and SGD, 2-byte and fp32 storage, the synchronous, gated and
device-resident flows and graph replays, against the oracle ("ZeRO：大模型训练的
内存优化革命" 3.1.1: each rank updates its 1/Nd partition, however large)."""
import os
import re
import subprocess
import sys

import pytest

from conftest import ROOT

pytestmark = pytest.mark.gpu

SPLIT_LIB = os.path.join(ROOT, "zero_dp_sharded_amd", "variants", "split_launch",
                         "libzeroshard.so")
FILES = ["test_gpu_parity.py", "test_gpu_edges.py", "test_gpu_variants.py", "test_gpu_phases.py",
         "test_gpu_random_phases.py", "test_gpu_clip_device.py", "test_gpu_inline_fold.py",
         "test_gpu_random.py", "test_gpu_shapes.py", "test_gpu_scale.py", "test_gpu_stage1.py",
         "test_gpu_extremes.py", "test_zz_no_alloc.py"]

PROBE = r"""
import torch, zero_dp_sharded_amd as zs
from zero_dp_sharded_amd import synth
print("library", zs.LIB_PATH)
w = synth.WORKLOADS["tiny"]
S = 65536
dev = torch.device("cuda", 0)
master, m, v = synth.init_state(w, dev, elems=S)
grad = torch.zeros(S, dtype=torch.float16, device=dev)
param = master.to(torch.float16)
bufs = synth.alloc_contribs(w, dev, elems=S)
synth.fill_contribs(w, bufs, 0, w.scale)
h = zs.zero_shard_init(master, m, v, grad, param, psi=S * 4, nd=4, rank=0, bucket_elems=S,
                       hp=zs.AdamHParams(), ls=zs.LossScaleCfg(init_scale=w.scale))
zs.zero_device_begin(h)
zs.zero_step_device(h, bufs)
info = zs.zero_device_end(h)
print("inline_folds", zs.zero_shard_inline_folds(h), "step_t", info.step_t)
zs.zero_shard_destroy(h)
"""


def _child(args, timeout):
    if not os.path.exists(SPLIT_LIB):
        pytest.fail(f"{SPLIT_LIB} is missing: run __graft_entry__.build()")
    env = dict(os.environ, ZERO_SHARD_LIB=SPLIT_LIB,
               PYTHONPATH=os.pathsep.join([ROOT, os.environ.get("PYTHONPATH", "")]))
    return subprocess.run([sys.executable, *args], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=timeout)


def test_split_launch_build_is_the_one_loaded():
    """The child loads the split build, and that build splits: a 65,536-element
    device-resident step, whose update the in-tree build runs as one launch that
    folds the partials itself, takes the fold launch (256 update workgroups of
    64 lanes are 16 launches of 1024 work-items)."""
    r = _child(["-c", PROBE], 120)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert f"library {SPLIT_LIB}" in r.stdout
    assert "inline_folds 0 step_t 1" in r.stdout, r.stdout


def test_split_launch_build_parity():
    r = _child(["-u", "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "gpu",
                *[os.path.join("tests", f) for f in FILES]], 600)
    tail = (r.stdout[-3000:] + r.stderr[-2000:])
    print(tail)
    assert r.returncode == 0, tail
    m = re.search(r"(\d+) passed", r.stdout)
    assert m and int(m.group(1)) > 300 and " failed" not in r.stdout, tail
