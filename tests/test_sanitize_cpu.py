"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).  zero_shard.cpp and zero_state_bytes.cpp are rebuilt with both
sanitizers on their host code (the device code is the in-tree build's kernel
object, unsanitized), and tests/test_abi_cpu.py runs against that library in a
child process (ZERO_SHARD_LIB, the clang ASan runtime preloaded): argument
validation, overlap and alignment checks, the ledger, the state-machine error
paths on dead handles.  Any sanitizer report fails the run (UBSan reports are
fatal; leak detection is off, the HIP runtime's own allocations at exit are
not the library's)."""
import glob
import os
import subprocess
import sys

import pytest

from conftest import ROOT

SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined " \
      "-Xarch_host -fno-sanitize-recover=undefined -Xarch_host -fno-omit-frame-pointer"


def _asan_runtime(hipcc):
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "lib", "llvm", "bin",
                         "amdclang++")
    cands = []
    for c in (clang, "/opt/rocm/lib/llvm/bin/amdclang++", "/opt/rocm/llvm/bin/amdclang++"):
        if os.path.exists(c):
            r = subprocess.run([c, "-print-resource-dir"], capture_output=True, text=True)
            if r.returncode == 0:
                cands.append(os.path.join(r.stdout.strip(), "lib", "linux",
                                          "libclang_rt.asan-x86_64.so"))
    cands += glob.glob("/opt/rocm*/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    for c in cands:
        if os.path.exists(c):
            return c
    return None


def test_library_host_code_under_asan_and_ubsan(tmp_path):
    from zero_dp_sharded_amd import build as B
    if not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not available")
    rt = _asan_runtime(B.HIPCC)
    if rt is None:
        pytest.skip("clang ASan runtime not found")
    kern = os.path.join(ROOT, "_build", "zeroshard", "zero_kernels.o")
    if not os.path.exists(kern):
        kern = B._compile(["zero_kernels.hip"], str(tmp_path), False)[0]
    objs = []
    for src in ("zero_shard.cpp", "zero_state_bytes.cpp"):
        obj = str(tmp_path / (src[:-4] + ".o"))
        cmd = [B.HIPCC, *B.FLAGS, "-O1", "-g", *SAN.split(), "-c", os.path.join(B.CSRC, src),
               "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(obj)
    lib = str(tmp_path / "libzeroshard.so")
    r = subprocess.run([B.HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-shared-libasan",
                        *SAN.split()[:4], "-o", lib, *objs, kern], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ZERO_SHARD_LIB=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    # -s: a sanitizer report goes to stderr even when it ends the process
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-s", "-p", "no:cacheprovider",
                        "tests/test_abi_cpu.py"], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout
