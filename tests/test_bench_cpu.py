"""bench.py's host-side contract, without a GPU: more than one GPU is refused
with a message, the algorithmic byte counts match the kernels' definitions,
and the traffic lookup only accepts counters taken on the current kernels."""
import json
import os
import subprocess
import sys

import pytest

from conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402
from zero_dp_sharded_amd import synth  # noqa: E402


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_is_refused(args, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                       env=dict(os.environ, **env), capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_update_bytes_per_element():
    W = synth.WORKLOADS
    assert bench.update_bytes_per_elem(W["128b"]) == 28        # 2 + 12 read, 12 + 2 written
    assert bench.update_bytes_per_elem(W["7.5b_bf16"]) == 28
    assert bench.update_bytes_per_elem(W["c1_7.5b_sgdm"]) == 20  # 4 + 8 read, 8 written
    assert bench.update_bytes_per_elem(W["c2_1.5b_sgd"]) == 12   # 4 + 4 read, 4 written


def test_traffic_only_from_counters_of_the_current_kernels(tmp_path, monkeypatch):
    assert bench.measured_traffic("no_such_workload", 1) is None
    d = {"kernel_code_sha256_16": bench.kernel_code_hash(), "elems_per_launch": 10,
         "hbm_bytes_per_launch": 123.0}
    (tmp_path / "traffic_w.json").write_text(json.dumps(d))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.measured_traffic("w", 10) == 123.0
    assert bench.measured_traffic("w", 11) is None              # another shard size
    assert bench.measured_traffic("w", 10, contrib_phase=2) is None   # no phase-2 counters
    (tmp_path / "traffic_w_phase2.json").write_text(json.dumps(dict(d, hbm_bytes_per_launch=7.0)))
    assert bench.measured_traffic("w", 10, contrib_phase=2) == 7.0
    assert bench.measured_traffic("w", 10) == 123.0
    d["kernel_code_sha256_16"] = "0" * 16
    (tmp_path / "traffic_w.json").write_text(json.dumps(d))
    assert bench.measured_traffic("w", 10) is None              # stale kernels


def test_kernel_code_hash_ignores_comments_only():
    from zero_dp_sharded_amd.traffic import kernel_code_hash
    src = "int f(int x)\n{\n    return x * 3;   // triple\n}\n"
    assert kernel_code_hash([src]) == kernel_code_hash(["/* note */ int f(int x) { return x * 3; }"])
    assert kernel_code_hash([src]) != kernel_code_hash([src.replace("3", "4")])
    assert kernel_code_hash([src, "a"]) != kernel_code_hash([src + "a"])      # file boundaries count
    assert len(kernel_code_hash()) == 16


def test_variant_builds_and_traffic_of_variants(monkeypatch, tmp_path):
    from zero_dp_sharded_amd import build as B
    with pytest.raises(ValueError):
        B.build_variant({"NOT_A_SHAPE": 1}, "/nonexistent")      # refused before compiling
    d = {"kernel_code_sha256_16": bench.kernel_code_hash(), "elems_per_launch": 2_000_000_000,
         "hbm_bytes_per_launch": 5.6e10}
    (tmp_path / "traffic_128b.json").write_text(json.dumps(d))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.measured_traffic("128b", 2_000_000_000) == 5.6e10
    monkeypatch.setenv("ZERO_SHARD_LIB", "/some/variant/libzeroshard.so")
    assert bench.measured_traffic("128b", 2_000_000_000) is None  # counters are the in-tree build's


@pytest.mark.parametrize("wname,threads", [("128b", 3), ("7.5b_bf16", 4), ("c1_7.5b_sgdm", 5),
                                           ("c2_1.5b_sgd", 2)])
def test_threaded_oracle_timing_equals_one_core(wname, threads):
    """The all-cores CPU baseline runs the oracle on contiguous chunks of the
    sample; with no overflow that is the one-core step, bitwise."""
    import numpy as np
    w = synth.WORKLOADS[wname]
    n, cb = 40_003, 8_192
    rng = np.random.default_rng(5)
    master = rng.normal(0, 0.02, n).astype(np.float32)
    m = rng.normal(0, 1e-4, n).astype(np.float32) if w.has_m else None
    v = np.abs(rng.normal(0, 1e-8, n)).astype(np.float32) if w.has_v else None
    R = w.R
    g = rng.normal(0, 1e-3, (R, n)) * w.scale
    if w.lp == "fp32":
        contribs = [row.astype(np.float32) for row in g]
    elif w.lp == "fp16":
        contribs = [row.astype(np.float16).view(np.uint16) for row in g]
    else:
        import torch
        contribs = [torch.from_numpy(row.astype(np.float32)).to(torch.bfloat16)
                    .view(torch.int16).numpy().view(np.uint16) for row in g]
    rate, dt, st = bench.cpu_baseline(w, (master, m, v), contribs, cb)
    prate, pdt, pmaster = bench.cpu_baseline_threads(w, (master, m, v), contribs, cb, threads)
    assert rate > 0 and prate > 0
    assert np.array_equal(pmaster.view(np.uint32), st.master.view(np.uint32))
    assert not np.array_equal(st.master, master)                 # the step did update


def test_sample_parity_reports_bitwise_and_relative_error():
    import numpy as np
    from types import SimpleNamespace
    rng = np.random.default_rng(1)
    n = 1000
    st = SimpleNamespace(grad=rng.integers(0, 2**16, n, dtype=np.uint16),
                         master=rng.normal(0, 0.02, n).astype(np.float32),
                         m=rng.normal(0, 1e-4, n).astype(np.float32),
                         v=np.abs(rng.normal(0, 1e-8, n)).astype(np.float32),
                         param=rng.integers(0, 2**16, n, dtype=np.uint16))
    gpu = {k: getattr(st, k).copy() for k in ("grad", "master", "m", "v", "param")}
    p = bench.sample_parity(gpu, st, n, (7, 4096.0, 7))
    assert p["grad_bitwise"] and p["fp32_state_bitwise"] and p["param_bitwise"]
    assert p["fp32_state_max_rel"] == 0.0 and p["from_step"] == 7
    gpu["v"][3] = np.nextafter(gpu["v"][3], np.float32(1))      # one ulp off
    gpu["grad"][5] ^= 1
    p = bench.sample_parity(gpu, st, n, (7, 4096.0, 7))
    assert not p["fp32_state_bitwise"] and not p["grad_bitwise"] and p["param_bitwise"]
    assert 0.0 < p["fp32_state_max_rel"] < 1e-6
    gpu["m"] = None                                              # SGD without momentum
    gpu["v"] = None
    assert bench.sample_parity(gpu, st, n, (7, 4096.0, 7))["fp32_state_bitwise"]


def test_copy_helper_refuses_bad_arguments_before_device_work():
    """bench.py's copy kernel (its bandwidth ceiling and counter calibration)
    refuses NULL pointers, sizes that are not a positive multiple of 16 or
    exceed 2^34 bytes (at most 2^30 work-items), and misaligned pointers,
    returning 1 before any HIP call."""
    import ctypes
    path = os.path.join(ROOT, "zero_dp_sharded_amd", "libhbmcopy.so")
    if not os.path.exists(path):
        pytest.skip("libhbmcopy.so is not built")
    lib = ctypes.CDLL(path)
    lib.hbm_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.hbm_copy.restype = ctypes.c_int
    a, b = 0x10000, 0x20000
    for dst, src, n in ((None, b, 16), (a, None, 16), (a, b, 0), (a, b, -16), (a, b, 24),
                        (a + 8, b, 16), (a, b + 4, 16), (a, b, (1 << 34) + 16)):
        assert lib.hbm_copy(dst, src, n, None) == 1, (dst, src, n)


def test_ab_reduce_prints_usage_without_builds(capsys):
    from zero_dp_sharded_amd import ab_reduce
    assert ab_reduce.main([]) == 2
    assert "ab_reduce" in capsys.readouterr().err
