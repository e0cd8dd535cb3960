"""bench.py's output contract on the GPU: a short run on the small workload
prints one JSON line with every field the measurement contract names, of the
right types, with the roofline and CPU-baseline objects filled in."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("flow", ["device", "graph"])
def test_bench_json_line(flow):
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny", "--steps", "3",
           "--warmup", "1", "--cpu-sample", "65536", "--flow", flow]
    print("running", " ".join(cmd), flush=True)
    out = subprocess.run(cmd, capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert out.returncode == 0, out.stderr[-2000:]
    lines = [l for l in out.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, out.stdout
    d = json.loads(lines[0])
    for key, typ in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int),
                     ("steps", int), ("warmup", int), ("ms_per_step", float),
                     ("higher_is_better", bool), ("scaling", str), ("dtype", str),
                     ("data", str), ("config", dict), ("roofline", dict),
                     ("cpu_baseline", dict)):
        assert isinstance(d[key], typ), (key, d.get(key))
    assert "vs_baseline" in d and d["vs_baseline"] is None
    assert d["flow"] == flow and d["ms_per_step"] == d["ms_per_step_by_flow"][flow]
    assert (d["n_gpus"], d["steps"], d["warmup"]) == (1, 3, 1)
    assert d["higher_is_better"] is True and d["scaling"] in ("weak", "strong")
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert abs(d["step_frac_of_copy_ceiling"] -
               d["step_hbm_gbs"] / d["copy_ceiling_gbs"]) < 1e-9
    assert isinstance(d["config"]["workload"], str)
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["achieved"] > 0 and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-9
    assert "traffic" in r
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["cores"] >= 1 and c["value"] > 0
    assert isinstance(c["unit"], str) and isinstance(c["sample"], str)
    a = c["all_cores"]
    assert a["cores"] >= 1 and a["value"] > 0 and a["equals_one_core"] is True
    p = d["parity_sample"]
    assert p["elements"] == 65536 and p["from_step"] > 0
    assert p["grad_bitwise"] and p["fp32_state_bitwise"] and p["param_bitwise"]
    assert p["fp32_state_max_rel"] == 0.0
    assert d["env"]["arch"].startswith("gfx950")
