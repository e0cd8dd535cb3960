"""Build the native test programs, C++ users of libzeroshard.so through its C
header with plain HIP memory, streams and the HIP graph API:
  abi_example  : every flow checked against the oracle (test infrastructure,
                 linked in from oracle/);
  step_latency : microseconds per device-resident step, direct and in graphs."""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
OUT = os.path.join(HERE, "abi_example")
LATENCY = os.path.join(HERE, "step_latency")
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")


def build(verbose: bool = False) -> str:
    sys.path.insert(0, os.path.join(ROOT, "oracle"))
    from build import CFLAGS as ORACLE_CFLAGS          # the oracle's own flags
    objdir = os.path.join(ROOT, "_build", "native")
    os.makedirs(objdir, exist_ok=True)
    oracle_obj = os.path.join(objdir, "zero_oracle.o")
    cflags = [f for f in ORACLE_CFLAGS if f not in ("-shared",)]
    main_obj = os.path.join(objdir, "abi_example.o")
    cmds = [
        ["gcc", *cflags, "-c", os.path.join(ROOT, "oracle", "zero_oracle.c"), "-o", oracle_obj],
        # host-only C++: hipcc for the HIP runtime headers, no device code
        [HIPCC, "-O2", "-std=c++17", "-Wall", f"-I{os.path.join(ROOT, 'include')}", "-c",
         os.path.join(HERE, "abi_example.cpp"), "-o", main_obj],
        [HIPCC, main_obj, oracle_obj, f"-L{os.path.join(ROOT, 'zero_dp_sharded_amd')}",
         "-lzeroshard", "-lm", "-Wl,-rpath,$ORIGIN/../../zero_dp_sharded_amd", "-o", OUT + ".tmp"],
    ]
    lat_obj = os.path.join(objdir, "step_latency.o")
    cmds += [
        [HIPCC, "-O2", "-std=c++17", "-Wall", f"-I{os.path.join(ROOT, 'include')}", "-c",
         os.path.join(HERE, "step_latency.cpp"), "-o", lat_obj],
        [HIPCC, lat_obj, f"-L{os.path.join(ROOT, 'zero_dp_sharded_amd')}", "-lzeroshard",
         "-Wl,-rpath,$ORIGIN/../../zero_dp_sharded_amd", "-o", LATENCY + ".tmp"],
    ]
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"{cmd[0]} failed:\n{r.stderr}")
    os.replace(OUT + ".tmp", OUT)
    os.replace(LATENCY + ".tmp", LATENCY)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
