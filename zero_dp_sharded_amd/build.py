"""Build libzeroshard.so for gfx950 with hipcc, in-tree.

Floating-point flags: no contraction into fused multiply-adds, correctly
rounded fp32 divide and square root, fp32 denormals kept, and no packed-fp32
instructions.  hipcc's host pass warns that it does not know the packed-fp32
feature; the warning is harmless.
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libzeroshard.so")
SOURCES = ["zero_kernels.hip", "zero_shard.cpp", "zero_state_bytes.cpp"]
# benchmark helper: plain HBM copy (ceiling and counter calibration)
COPY_LIB = os.path.join(HERE, "libhbmcopy.so")
COPY_SOURCES = ["hbm_copy.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _compile(sources, objdir, verbose):
    objs = []
    for src in sources:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [HIPCC, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        err = "\n".join(line for line in r.stderr.splitlines()
                        if "packed-fp32-ops" not in line)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)
        objs.append(obj)
    return objs


def _link(objs, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def device_asm(src: str = "zero_kernels.hip") -> str:
    """gfx950 assembly of one source under the build flags (for inspection and
    for tests of what the compiler emitted)."""
    objdir = os.path.join(ROOT, "_build", "zeroshard")
    os.makedirs(objdir, exist_ok=True)
    out = os.path.join(objdir, os.path.splitext(src)[0] + ".s")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "--cuda-device-only", "-S", os.path.join(CSRC, src),
           "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{r.stderr}")
    with open(out, encoding="utf-8") as f:
        return f.read()


def build(verbose: bool = False) -> str:
    objdir = os.path.join(ROOT, "_build", "zeroshard")
    os.makedirs(objdir, exist_ok=True)
    _link(_compile(SOURCES, objdir, verbose), LIB, verbose)
    _link(_compile(COPY_SOURCES, objdir, verbose), COPY_LIB, verbose)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
