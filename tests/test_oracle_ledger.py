"""Pins of the oracle's per-rank byte ledger against the pages' printed tables.

Table 1, worked examples A/B/C1/C2 and the theoretical columns of Table 2 are
on the blog.vllbc.top ZeRO/DeepSpeed page; the 24 GB / 16 TB totals are in
section 01 of the Tencent "AI论文陪读·ZeRO" page.
"""
from fractions import Fraction

import pytest

from conftest import read_golden

MODELS = [7.5e9, 128e9, 1e12]


def exact_stage_bytes(psi, nd, b=2, K=12):
    P, N = Fraction(int(psi)), Fraction(nd)
    return [(2 * b + K) * P, 2 * b * P + K * P / N, b * P + (b + K) * P / N,
            (2 * b + K) * P / N]


@pytest.mark.parametrize("row", read_golden("table1_model_state_gb.txt"))
def test_table1_cells(oracle, row):
    nd = int(row[0])
    cells = row[1:]
    assert len(cells) == 9
    for mi, psi in enumerate(MODELS):
        d = oracle.state_bytes(int(psi), nd)
        for st in range(3):
            printed = cells[3 * mi + st]
            got = d["per_rank_stage"][st + 1]
            # the ledger value is an exact double here: compare exactly
            exact = exact_stage_bytes(psi, nd)[st + 1]
            assert Fraction(got) == exact or abs(got - float(exact)) <= 1e-6 * float(exact)
            assert oracle.display_gb(Fraction(got)) == printed, (nd, psi, st)
        # stage 0 is 16 Psi for every Nd (Table 1 row Nd=1 equals all three)
        assert d["per_rank_stage"][0] == 16 * psi


def test_table1_has_54_cells():
    rows = read_golden("table1_model_state_gb.txt")
    assert sum(len(r) - 1 for r in rows) == 54


@pytest.mark.parametrize("row", read_golden("worked_examples_gb.txt"))
def test_worked_examples(oracle, row):
    group, psi, nd, b, K, st = row[0], float(row[1]), int(row[2]), int(row[3]), int(row[4]), int(row[5])
    params, grads, optim, total, comm, comm_g = row[6:12]
    d = oracle.state_bytes(int(psi), nd, param_bytes=b, k_optim=K)
    assert oracle.display_gb(Fraction(d["per_rank_stage"][st])) == total
    if params != "-":
        assert oracle.display_gb(Fraction(d["comp_params"][st])) == params
        assert oracle.display_gb(Fraction(d["comp_grads"][st])) == grads
        assert oracle.display_gb(Fraction(d["comp_optim"][st])) == optim
        # components add up to the total (the page rounds parts separately)
        s = d["comp_params"][st] + d["comp_grads"][st] + d["comp_optim"][st]
        assert s == pytest.approx(d["per_rank_stage"][st], rel=1e-15)
    if comm != "-":
        assert oracle.display_gb(Fraction(d["comm_bytes_stage"][st])) == comm
    if comm_g != "-":
        assert st == 1
        assert oracle.display_gb(Fraction(d["comm_bytes_stage1_with_gather"])) == comm_g


def test_worked_example_bytes_exact(oracle):
    # group A at Nd=64: exact byte counts behind 31.4 / 16.6 / 1.88
    d = oracle.state_bytes(7_500_000_000, 64)
    assert d["per_rank_stage"][1:] == [31_406_250_000.0, 16_640_625_000.0, 1_875_000_000.0]
    # group B at Nd=64: 536 / 284 / 32 GB
    d = oracle.state_bytes(128_000_000_000, 64)
    assert d["per_rank_stage"][1:] == [536e9, 284e9, 32e9]


@pytest.mark.parametrize("row", read_golden("table2_max_model_size.txt"))
def test_table2_theoretical(oracle, row):
    """Largest Psi with per-rank bytes <= 32 GB at Nd = 64.  The page's MP > 1
    rows are MP times the one-decimal MP = 1 value (15.2 = 2 x 7.6)."""
    mp = int(row[0])
    printed = [Fraction(x) for x in row[2:6]]
    per_param = oracle.state_bytes(1, 64)  # bytes per parameter, exact
    # per_rank_stage at Psi = 1 is the per-parameter cost; baseline is stage 0
    for col, st in enumerate([0, 1, 2, 3]):
        cost = Fraction(per_param["per_rank_stage"][st])
        psi_max_b = Fraction(32) / cost          # billions, at MP = 1
        one_dec = (psi_max_b * 10 + Fraction(1, 2)).__floor__() / Fraction(10)
        assert mp * one_dec == printed[col], (mp, st)
    # GPU count is MP x 64
    assert int(row[1]) == mp * 64


def test_headline_totals(oracle):
    for row in read_golden("headline_ledger.txt"):
        psi, nd, what, val = float(row[0]), int(row[1]), row[2], float(row[3])
        approx = len(row) > 4
        d = oracle.state_bytes(int(psi), nd)
        got = d["comp_params"][0] if what == "weights_fp16" else d["per_rank_stage"][int(what)]
        if approx:
            assert got == pytest.approx(val, rel=0.05)
        else:
            assert got == val


def test_stage_asymptotes(oracle):
    """P2 section 1.2 and 3.1: 4x for P_os, 8x for P_os+g as Nd grows, Nd x for
    P_os+g+p."""
    nd = 1 << 20
    d = oracle.state_bytes(10**12, nd)
    s0 = d["per_rank_stage"][0]
    assert s0 / d["per_rank_stage"][1] == pytest.approx(4, rel=1e-4)
    assert s0 / d["per_rank_stage"][2] == pytest.approx(8, rel=1e-4)
    assert s0 / d["per_rank_stage"][3] == nd


def test_allocation_and_staging(oracle):
    # 128B at Nd=64: the owner shard is 2.0e9 elements; allocation 16 S bytes
    d = oracle.state_bytes(128_000_000_000, 64, n_contrib=4, bucket_elems=200_000_000)
    assert d["shard_elems"] == 2_000_000_000
    assert d["bytes_shard_total"] == 32_000_000_000
    assert d["bytes_shard_total"] == d["per_rank_stage"][3]
    assert d["bytes_staging"] == 4 * 200_000_000 * 2
    # a Psi that Nd does not divide: S is rounded up
    d = oracle.state_bytes(10, 4)
    assert d["shard_elems"] == 3


@pytest.mark.parametrize("val,shown", [
    (Fraction(31406250000), "31.4"), (Fraction(1875000000), "1.88"),
    (Fraction(41250000000), "41.3"), (Fraction(4187500000000), "4187"),
    (Fraction(31000000000), "31"), (Fraction(1500000000), "1.5"),
    (Fraction(468750000), "0.47"), (Fraction(100 * 10**9), "100"),
    (Fraction(99_990_000_000), "100.0".rstrip("0").rstrip(".")),
])
def test_display_rule(oracle, val, shown):
    assert oracle.display_gb(val) == shown


@pytest.mark.parametrize("psi,nd,lp_bytes,b,K", [
    (7_500_000_000, 64, 2, 2, 12),     # example A: mixed-precision Adam
    (128_000_000_000, 64, 2, 2, 12),   # example B
    (7_500_000_000, 64, 4, 4, 4),      # C1: fp32 SGD with momentum
    (1_500_000_000, 8, 4, 4, 0),       # C2: fp32 plain SGD
    (1_500_000_000, 8, 4, 4, 8),       # fp32 Adam
    (1_500_000_000, 8, 2, 2, 8),       # mixed-precision SGD with momentum (master + buffer)
])
def test_allocation_equals_stage3_bytes(oracle, psi, nd, lp_bytes, b, K):
    """The shard one rank allocates is the Stage-3 per-rank share (2b+K)Psi/Nd
    of the page's ledger, for every storage/optimizer pair of its examples."""
    d = oracle.state_bytes(psi, nd, 1, 1, lp_bytes=lp_bytes, param_bytes=b, k_optim=K)
    assert psi % nd == 0
    assert d["bytes_shard_total"] == d["per_rank_stage"][3] == (2 * b + K) * psi // nd
