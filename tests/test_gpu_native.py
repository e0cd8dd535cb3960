"""The C ABI used natively: tests/native/abi_example (plain HIP memory and
streams, the HIP graph API, no torch) runs fp16 Adam steps through the
synchronous flow, the device-resident flow and graph replays of a captured
device-resident step, and checks each against the oracle bitwise."""
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
    assert sum("bitwise equal to the oracle: yes" in ln for ln in lines) == 3
