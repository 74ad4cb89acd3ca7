"""The GPU library's C++ schedule tables, checked on the CPU against the schedule oracle.

* In the paper's normalisation (one group of n lanes, m heads) the C++ tables equal
  the oracle's reference schedules task for task, ranks included.
* At every workload shape and the measured MI355X topology (8 XCDs x 32 CUs) the
  tables pass the oracle validator (coverage, KV contiguity, rank order,
  acyclicity, conflict-freedom for the timestamp schedules), keep every dQ tile's
  contributors on one XCD, and reach the makespan the oracle simulator predicts.
"""
import numpy as np
import pytest

from oracle import schedule as osch
from scheduling_fa_attn_amd import dash

RULE = {"naive": "kv_index", "descending": "kv_index", "shift": "timestamp", "sym_shift": "timestamp"}

WORKLOADS = {
    # name: (B, H, Hkv, N, mask, schedules)
    "tiny-full": (1, 2, 2, 256, "full", ("naive", "descending", "shift")),
    "tiny-causal": (1, 2, 2, 256, "causal", ("naive", "descending", "sym_shift")),
    "full-d128-N2048": (8, 16, 16, 2048, "full", ("naive", "descending", "shift")),
    "causal-d64-N4096": (4, 32, 32, 4096, "causal", ("naive", "descending", "sym_shift")),
    "causal-d128-N16384": (1, 16, 16, 16384, "causal", ("naive", "descending", "sym_shift")),
    "gqa-causal-N8192": (1, 32, 8, 8192, "causal", ("naive", "descending", "sym_shift")),
}


def to_table(records, B, H, Hkv, N, mask, schedule, workers):
    n = -(-N // dash.dash_tile_size(N))
    lanes = [[] for _ in range(workers)]
    for w, b, h, g, i, j, rank in records.tolist():
        lanes[w].append((b, h, g, i, j, rank))
    return {"lanes": lanes, "n": n, "causal": mask == "causal", "B": B, "H": H, "Hkv": Hkv,
            "rule": RULE[schedule]}


@pytest.mark.parametrize("kind,causal", [("naive", False), ("naive", True), ("descending", False),
                                         ("descending", True), ("shift", False), ("sym_shift", True)])
@pytest.mark.parametrize("n,m", [(4, 1), (4, 2), (8, 4), (8, 3), (16, 2)])
def test_equals_reference_in_paper_normalisation(kind, causal, n, m):
    if kind == "sym_shift" and m % 2:
        m += 1
    N = n * (64 if n * 64 < 512 else 128)
    assert -(-N // dash.dash_tile_size(N)) == n
    rec, local = dash.dash_schedule_table(1, m, m, N, "causal" if causal else "full", kind, 1, n)
    ref = osch.reference_schedule(kind, n, m, causal)
    got = to_table(rec, 1, m, m, N, "causal" if causal else "full", kind, n)
    assert got["lanes"] == ref["lanes"]
    assert local


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_tables_valid(name):
    B, H, Hkv, N, mask, scheds = WORKLOADS[name]
    for s in scheds:
        rec, local = dash.dash_schedule_table(B, H, Hkv, N, mask, s, 8, 32)
        table = to_table(rec, B, H, Hkv, N, mask, s, 256)
        osch.validate(table)
        assert local, (name, s)
        # every dQ tile's contributors share one XCD (workers xcd*32 .. xcd*32+31)
        xcd = rec[:, 0] // 32
        chain = (rec[:, 1].astype(np.int64) * H + rec[:, 2]) * 4096 + rec[:, 5]
        order = np.lexsort((xcd, chain))
        c, x = chain[order], xcd[order]
        same = c[1:] == c[:-1]
        assert np.all(x[1:][same] == x[:-1][same])


def _lane_work(table):
    return max(len(lane) for lane in table["lanes"])


@pytest.mark.parametrize("name,schedule", [("full-d128-N2048", "shift"), ("causal-d64-N4096", "sym_shift"),
                                           ("causal-d128-N16384", "sym_shift"), ("gqa-causal-N8192", "sym_shift")])
def test_optimal_schedules_reach_the_work_bound(name, schedule):
    """Shift / symmetric shift tables: makespan = busiest lane's work (no bubbles), for any c, r."""
    B, H, Hkv, N, mask, _ = WORKLOADS[name]
    rec, _ = dash.dash_schedule_table(B, H, Hkv, N, mask, schedule, 8, 32)
    table = to_table(rec, B, H, Hkv, N, mask, schedule, 256)
    work = _lane_work(table)
    expected = {"full-d128-N2048": 128, "causal-d64-N4096": 264, "causal-d128-N16384": 516,
                "gqa-causal-N8192": 260}[name]
    assert work == expected
    for c, r in ((1.0, 0.0), (3.0, 1.0), (1.0, 2.0)):
        assert osch.simulate(table, c, r) == pytest.approx(work * (c + r))


def test_naive_baseline_has_the_startup_term():
    B, H, Hkv, N, mask, _ = WORKLOADS["full-d128-N2048"]
    rec, _ = dash.dash_schedule_table(B, H, Hkv, N, mask, "naive", 8, 32)
    table = to_table(rec, B, H, Hkv, N, mask, "naive", 256)
    n, m = 16, 8
    assert osch.simulate(table, 3.0, 1.0) == pytest.approx(m * n * 4.0 + (n - 1) * 1.0)


@pytest.mark.parametrize("args,status", [
    ((1, 2, 2, 256, "causal", "shift"), dash.DASH_ERR_UNSUPPORTED),
    ((1, 2, 2, 256, "full", "sym_shift"), dash.DASH_ERR_UNSUPPORTED),
    ((1, 2, 2, 192, "causal", "sym_shift"), dash.DASH_ERR_UNSUPPORTED),  # 3 tiles: odd
    ((1, 3, 2, 256, "full", "naive"), dash.DASH_ERR_INVALID_ARG),       # H % Hkv != 0
    ((1, 2, 2, 256, "full", 7), dash.DASH_ERR_INVALID_ARG),
    ((-1, 2, 2, 256, "full", "naive"), dash.DASH_ERR_INVALID_ARG),
])
def test_table_argument_errors(args, status):
    with pytest.raises(dash.DashError) as e:
        dash.dash_schedule_table(*args, 8, 32)
    assert e.value.status == status


def test_ragged_and_empty():
    # N not a multiple of the tile: ceil(N / tile) tiles, same invariants.
    rec, _ = dash.dash_schedule_table(2, 4, 2, 1000, "causal", "descending", 8, 32)
    osch.validate(to_table(rec, 2, 4, 2, 1000, "causal", "descending", 256))
    rec, _ = dash.dash_schedule_table(0, 4, 2, 1000, "full", "shift", 8, 32)
    assert len(rec) == 0


@pytest.mark.parametrize("schedule,lanes", [("sym_shift", 64), ("naive", 128), ("descending", 128)])
def test_spread_placement_of_the_long_causal_head(schedule, lanes):
    """C4 (n = 128 KV tiles per head): with the spread placement a head's group takes one
    CU per lane over several XCDs (the paper's n-SM layout), its chains cross XCDs, and
    the table stays valid; the symmetric shift still reaches the work bound (each CU then
    runs its single lane for every unit of its group: 16 units over 4 groups of 64 CUs).
    The default (aggregate) placement keeps every chain on one XCD."""
    B, H, Hkv, N, mask, _ = WORKLOADS["causal-d128-N16384"]
    assert dash.dash_set_placement("spread") == 0
    try:
        rec, local = dash.dash_schedule_table(B, H, Hkv, N, mask, schedule, 8, 32)
    finally:
        assert dash.dash_set_placement("aggregate") == 0
    table = to_table(rec, B, H, Hkv, N, mask, schedule, 256)
    osch.validate(table)
    assert not local
    # one lane per CU: every CU that works has the KV tiles of one lane of each unit
    workers = np.unique(rec[:, 0])
    assert len(workers) == 256
    per_unit = {}
    for w, b, h, g, i, j, rank in rec.tolist():
        per_unit.setdefault((w, b, g), set()).add(i)
    assert max(len(v) for v in per_unit.values()) == (2 if schedule == "sym_shift" else 1)
    if schedule == "sym_shift":
        work = _lane_work(table)
        assert work == 516
        assert osch.simulate(table, 3.0, 1.0) == pytest.approx(work * 4.0)
    rec2, local2 = dash.dash_schedule_table(B, H, Hkv, N, mask, schedule, 8, 32)
    assert local2


def test_placement_argument_errors():
    assert dash.dash_set_placement(2) == dash.DASH_ERR_INVALID_ARG
    assert dash.dash_set_placement(-1) == dash.DASH_ERR_INVALID_ARG


@pytest.mark.parametrize("N,mask,resolved", [
    (2048, "full", "shift"),
    (4096, "causal", "sym_shift"),
    (1000, "causal", "sym_shift"),     # 8 tiles of 128
    (1100, "causal", "descending"),    # 9 tiles: symmetric shift is not defined
    (448, "causal", "descending"),     # 7 tiles of 64
    (256, "full", "shift"),
])
def test_auto_schedule_resolves_to_the_measured_best(N, mask, resolved):
    """schedule=auto gives the same table as the schedule it resolves to."""
    auto, local_a = dash.dash_schedule_table(2, 4, 2, N, mask, "auto", 8, 32)
    ref, local_r = dash.dash_schedule_table(2, 4, 2, N, mask, resolved, 8, 32)
    assert np.array_equal(auto, ref) and local_a == local_r
