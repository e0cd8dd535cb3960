"""The C ABI used natively (plain HIP memory and streams, the HIP graph API, no
torch): tests/native/abi_example runs fp16 Adam steps through the synchronous
flow, the device-resident flow, graph replays of a captured device-resident
step and the allocation-free step, and checks each against the oracle
bitwise;
tests/native/step_latency times device-resident steps enqueued directly and
replayed from graphs of one and ten steps."""
import os
import subprocess

import pytest

from conftest import ROOT

pytestmark = pytest.mark.gpu

EXE = os.path.join(ROOT, "tests", "native", "abi_example")


def test_native_abi_example():
    if not os.path.exists(EXE):
        pytest.skip("tests/native/abi_example is not built (python -c 'import __graft_entry__ as "
                    "g; g.build()')")
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    print(r.stderr)
    assert r.returncode == 0, r.stderr
    lines = r.stdout.strip().splitlines()
    assert lines[-1] == "abi_example ok"
    assert sum("bitwise equal to the oracle: yes" in ln for ln in lines) == 4


LATENCY = os.path.join(ROOT, "tests", "native", "step_latency")


@pytest.mark.parametrize("elems", [262_144, 4_194_304])
def test_native_step_latency(elems):
    """Runs to completion with every one of its 6150 steps counted once by the
    device state; prints microseconds per step of each launch mode."""
    if not os.path.exists(LATENCY):
        pytest.skip("tests/native/step_latency is not built")
    r = subprocess.run([LATENCY, str(elems)], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stderr
    f = dict(kv.split("=") for kv in r.stdout.split())
    assert int(f["S"]) == elems and int(f["step_t"]) == 6150 and int(f["overflow"]) == 0
    for k in ("direct_us", "graph1_us", "graph10_us"):
        assert 0 < float(f[k]) < 10_000, (k, f[k])
