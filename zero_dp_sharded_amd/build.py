"""Build libzeroshard.so for gfx950 with hipcc, in-tree.

Floating-point flags: no contraction into fused multiply-adds, correctly
rounded fp32 divide and square root, fp32 denormals kept, and no packed-fp32
instructions.  hipcc's host pass warns that it does not know the packed-fp32
feature; the warning is harmless.

    python -m zero_dp_sharded_amd.build [-v]
    python -m zero_dp_sharded_amd.build --variant OUT_DIR NAME=VALUE ...

The second form builds a tuning variant (the ZK_* shape macros of
csrc/zero_kernels.h overridden) into OUT_DIR and leaves the in-tree library
alone; point ZERO_SHARD_LIB at OUT_DIR/libzeroshard.so to run the tests or
bench.py against it.
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
# test build: every launch split after 1024 work-items, so the consecutive-
# launch path that only shards beyond 8.6e9 elements reach runs in the tests
SPLIT_LAUNCH_DIR = os.path.join(HERE, "variants", "split_launch")
SPLIT_LAUNCH_DEFINES = {"ZK_MAX_LAUNCH_ITEMS": 1024}

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


def _compile(sources, objdir, verbose, extra=()):
    objs = []
    for src in sources:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [HIPCC, *FLAGS, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
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
    build_variant(SPLIT_LAUNCH_DEFINES, SPLIT_LAUNCH_DIR, verbose,
                  objdir=os.path.join(ROOT, "_build", "split_launch"))
    return LIB


def build_variant(defines: dict, out_dir: str, verbose: bool = False,
                  objdir: str = None) -> str:
    """libzeroshard.so with shape macros overridden ({"ZK_RED_PER_CU": 3, ...})
    into out_dir (objects in objdir, default out_dir/obj), for A/B
    measurements and the split-launch test build."""
    for name in defines:
        if not name.startswith("ZK_"):
            raise ValueError(f"{name}: only the ZK_* shape macros may be overridden")
    out_dir = os.path.abspath(out_dir)
    objdir = objdir or os.path.join(out_dir, "obj")
    os.makedirs(out_dir, exist_ok=True)
    os.makedirs(objdir, exist_ok=True)
    extra = [f"-D{k}={v}" for k, v in defines.items()]
    lib = os.path.join(out_dir, "libzeroshard.so")
    _link(_compile(SOURCES, objdir, verbose, extra), lib, verbose)
    return lib


if __name__ == "__main__":
    args = [a for a in sys.argv[1:] if a != "-v"]
    if args and args[0] == "--variant":
        defs = dict(a.split("=", 1) for a in args[2:])
        print(build_variant(defs, args[1], verbose="-v" in sys.argv))
    else:
        build(verbose="-v" in sys.argv)
