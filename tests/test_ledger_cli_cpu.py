"""The ledger command line (python -m zero_dp_sharded_amd.ledger): the
library's host ledger printed per stage, checked against the pages' Table 1
cells for the 7.5B and 128B models at Nd = 64 (blog.vllbc.top ZeRO/DeepSpeed
page, Table 1: stages 1-3 of 31.4 / 16.6 / 1.88 GB and 536 / 284 / 32 GB),
the shard this library allocates, and the HBM fit."""
import re

from zero_dp_sharded_amd import ledger


def _stages(out):
    rows = {}
    for ln in out.splitlines():
        m = re.match(r"\s+(\d)\s+([\d.,]+) GB", ln)
        if m:
            rows[int(m.group(1))] = m.group(2)
    return rows


def test_table1_cells(capsys):
    assert ledger.main(["7.5e9", "64"]) == 0
    rows = _stages(capsys.readouterr().out)
    assert [rows[s] for s in (1, 2, 3)] == ["31.4", "16.6", "1.88"]
    assert rows[0] == "120"
    assert ledger.main(["128e9", "64", "--bucket", "2e8", "--contrib", "4"]) == 0
    out = capsys.readouterr().out
    rows = _stages(out)
    assert [rows[s] for s in (1, 2, 3)] == ["536", "284", "32"]
    # the 128B shard: 2.0e9 elements, 16 B each = 32 GB, plus one bucket of 4 x 2e8 x 2 B
    assert "S = 2,000,000,000 elements" in out
    assert re.search(r"shard\s+32 GB; one bucket of 4 contributions 1.6 GB", out)
    assert "33.6 GB of 288 GB HBM: fits" in out


def test_fit_and_variants(capsys):
    # one rank holding a 1T-parameter model's whole Adam state does not fit
    assert ledger.main(["1e12", "1", "--contrib", "1"]) == 0
    assert "does not fit" in capsys.readouterr().out
    # fp32 storage with plain SGD (b = 4, K = 0): stage 3 is 8 Psi / Nd
    assert ledger.main(["1.5e9", "8", "--storage", "fp32", "--k", "0"]) == 0
    rows = _stages(capsys.readouterr().out)
    assert rows[3] == "1.5"
