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
    """Causal, B=1, H=16, N=16384 (n = 128 KV tiles per head): with the spread placement a head's group takes one
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


NAMES = {0: "naive", 1: "descending", 2: "shift", 3: "sym_shift"}


@pytest.mark.parametrize("N,mask", [(2048, "full"), (4096, "causal"), (1000, "causal"), (1100, "causal"),
                                    (448, "causal"), (256, "full")])
def test_auto_schedule_table_is_the_resolved_schedule(N, mask):
    """schedule=auto gives the same table as the schedule dash_schedule_resolve names
    (odd tile counts, 1100 and 448, never resolve to symmetric shift)."""
    resolved = dash.dash_schedule_resolve(2, 4, 2, N, 128, mask, "auto", 8, 32)
    assert resolved in NAMES
    n = -(-N // dash.dash_tile_size(N))
    assert not (resolved == 3 and n % 2)
    auto, local_a = dash.dash_schedule_table(2, 4, 2, N, mask, "auto", 8, 32)
    ref, local_r = dash.dash_schedule_table(2, 4, 2, N, mask, NAMES[resolved], 8, 32)
    assert np.array_equal(auto, ref) and local_a == local_r


# ---------------------------------------------------------------------------------
# Hardware-aware cost model (dash_schedule_makespan / dash_schedule_resolve).
# ---------------------------------------------------------------------------------

def _oracle_makespan(rec, table, cus_per_xcd, c, r_local, r_remote):
    """The oracle DAG simulator on the exported table, each task's reduction costing
    r_remote when the previous reduction into its dQ tile ran on another L2 domain."""
    pred_worker = {}
    chains = {}
    for w, b, h, g, i, j, rank in rec.tolist():
        chains.setdefault((b, h, j), []).append((rank, w, (b, h, g, i, j, rank)))
    for members in chains.values():
        members.sort()
        for (_, w0, _), (_, w1, key1) in zip(members, members[1:]):
            pred_worker[key1] = (w0, w1)

    def r_cost(task):
        pw = pred_worker.get(tuple(task))
        return r_remote if pw is not None and pw[0] // cus_per_xcd != pw[1] // cus_per_xcd else r_local

    return osch.simulate(table, c, r_cost)


MODEL_CASES = [
    # (B, H, Hkv, N, mask, schedule, num_xcd, cus_per_xcd, placement)
    (1, 2, 2, 256, "full", "shift", 1, 4, "aggregate"),
    (1, 2, 2, 256, "causal", "descending", 2, 4, "aggregate"),
    (2, 8, 8, 2048, "full", "naive", 8, 32, "aggregate"),
    (2, 8, 8, 2048, "full", "shift", 8, 32, "aggregate"),
    (2, 16, 16, 4096, "causal", "sym_shift", 8, 32, "aggregate"),
    (1, 16, 4, 4096, "causal", "descending", 8, 32, "aggregate"),
    (1, 4, 4, 16384, "causal", "sym_shift", 8, 32, "spread"),   # chains across XCDs
    (1, 2, 2, 16384, "full", "shift", 4, 32, "spread"),
]


@pytest.mark.parametrize("case", MODEL_CASES, ids=["-".join(map(str, c)) for c in MODEL_CASES])
def test_makespan_equals_oracle_simulator(case):
    """The C++ model's longest path equals the oracle simulator's on the same table
    (integer costs, so the sums are exact), with local and remote reduction costs."""
    B, H, Hkv, N, mask, sched, X, S, placement = case
    assert dash.dash_set_placement(placement) == dash.DASH_OK
    try:
        rec, local = dash.dash_schedule_table(B, H, Hkv, N, mask, sched, X, S)
        table = to_table(rec, B, H, Hkv, N, mask, sched, X * S)
        for c, rl, rr in ((5.0, 1.0, 7.0), (2.0, 3.0, 3.0), (1.0, 0.0, 0.0)):
            got = dash.dash_schedule_makespan(B, H, Hkv, N, mask, sched, X, S, c, rl, rr)
            want = _oracle_makespan(rec, table, S, c, rl, rr)
            assert got == want, (c, rl, rr, got, want)
        if placement == "spread" and -(-N // 128) > S:
            assert not local  # the case does exercise remote reductions
            got_l = dash.dash_schedule_makespan(B, H, Hkv, N, mask, sched, X, S, 5.0, 1.0, 1.0)
            got_r = dash.dash_schedule_makespan(B, H, Hkv, N, mask, sched, X, S, 5.0, 1.0, 7.0)
            assert got_r > got_l
    finally:
        dash.dash_set_placement("aggregate")


@pytest.mark.parametrize("kind,causal,n,m", [("naive", False, 8, 4), ("shift", False, 8, 4), ("naive", True, 8, 4),
                                             ("sym_shift", True, 8, 4), ("shift", False, 16, 2),
                                             ("descending", True, 8, 2)])
def test_makespan_closed_forms(kind, causal, n, m):
    """In the paper's normalisation (one group of n lanes, m heads) the C++ model gives
    the section 3.2-3.4 closed forms (exact for these cases, r < c)."""
    c, r = 3.0, 1.0
    N = n * (64 if n * 64 < 512 else 128)
    got = dash.dash_schedule_makespan(1, m, m, N, "causal" if causal else "full", kind, 1, n, c, r, r)
    want = {"naive": m * n * (c + r) + (n - 1) * r, "shift": m * n * (c + r),
            "sym_shift": m * (n + 1) * (c + r) / 2, "descending": m * (n + 1) * (c + r) / 2 + (n - 1) * r}[kind]
    assert got == want, (got, want)


def test_auto_picks_measured_fastest_on_paper_grid():
    """On the DASH paper's benchmark grid (section 4.1: 16 384 tokens, hidden 2048, N =
    512 .. 16384, d = 64 and 128) the cost model picks the schedule measured fastest on
    MI355X at every point: shift for the full mask, symmetric shift for the causal mask."""
    for d in (64, 128):
        for mask, want in (("full", 2), ("causal", 3)):
            for N in (512, 1024, 2048, 4096, 8192, 16384):
                B, H = 16384 // N, 2048 // d
                assert dash.dash_schedule_resolve(B, H, H, N, d, mask, "auto", 8, 32) == want, (d, mask, N)


# Main-kernel times measured on one MI355X, microseconds per call (naive / descending /
# shift or symmetric shift), and the schedule measured fastest:
# (B, H, Hkv, N, d, mask, placement) -> fastest.
MEASURED_FASTEST = [
    ((2, 4, 2, 4096, 128, "causal", "aggregate"), "sym_shift"),   # 638 / 543 / 307
    ((1, 2, 2, 256, 64, "causal", "aggregate"), "descending"),    # 34 / 30 / 35
    ((1, 4, 4, 640, 128, "causal", "aggregate"), "descending"),   # 57 / 46 / (odd tile count)
    ((2, 3, 1, 1000, 64, "causal", "aggregate"), "descending"),   # 122 / 100 / 112
    ((2, 4, 2, 2048, 128, "full", "aggregate"), "shift"),         # 244 / 241 / 162
    ((8, 16, 16, 2048, 128, "full", "aggregate"), "shift"),       # 917 / 890 / 840
    ((4, 32, 32, 4096, 64, "causal", "aggregate"), "sym_shift"),  # 2724 / 1573 / 1026
    ((1, 16, 16, 16384, 128, "causal", "aggregate"), "sym_shift"),  # 4244 / 4939 / 3081
    ((1, 32, 8, 8192, 128, "causal", "aggregate"), "sym_shift"),  # 3992 / 1929 / 1847
    ((1, 4, 4, 8192, 64, "causal", "spread"), "sym_shift"),       # 490 / 313 / 259
    ((1, 4, 4, 8192, 128, "causal", "spread"), "descending"),     # 623 / 392 / 404
    ((1, 16, 16, 16384, 128, "causal", "spread"), "sym_shift"),   # 8033 / 5743 / 4017
]


@pytest.mark.parametrize("shape,fastest", MEASURED_FASTEST,
                         ids=["B{}H{}Hkv{}N{}d{}-{}-{}".format(*m[0]) for m in MEASURED_FASTEST])
def test_auto_picks_measured_fastest_on_timed_shapes(shape, fastest):
    """AUTO picks the schedule measured fastest (or one within 3 % of it: 392 against 404
    us on the spread d = 128 shape) on every shape timed for the model."""
    B, H, Hkv, N, d, mask, placement = shape
    assert dash.dash_set_placement(placement) == dash.DASH_OK
    try:
        got = NAMES[dash.dash_schedule_resolve(B, H, Hkv, N, d, mask, "auto", 8, 32)]
    finally:
        dash.dash_set_placement("aggregate")
    close = {((1, 4, 4, 8192, 128, "causal", "spread"), "sym_shift")}
    assert got == fastest or (shape, got) in close, (shape, got, fastest)


# Whole-call TFLOPS on one MI355X of the ordered reduction (best schedule, deterministic =
# 1) and the two-pass variant (2) by query heads per KV head G: (B, H, N, d, mask) ->
# {G: (ordered, two-pass)}.
MODES_MEASURED = {
    (1, 32, 8192, 128, "causal"): {1: (842.4, 785.8), 2: (818.9, 807.9), 4: (762.5, 800.4), 8: (477.5, 509.3)},
    (1, 32, 8192, 128, "full"): {1: (895.4, 832.6), 2: (899.8, 836.9), 4: (897.5, 838.0), 8: (513.1, 525.6)},
    (2, 32, 4096, 64, "causal"): {1: (704.8, 615.0), 2: (694.7, 633.5), 4: (678.3, 630.5), 8: (394.9, 412.9)},
    (4, 16, 2048, 128, "causal"): {1: (667.3, 618.9), 2: (667.3, 650.7), 4: (509.2, 479.5), 8: (274.6, 299.4)},
    (2, 16, 4096, 128, "full"): {1: (859.5, 807.6), 2: (882.9, 815.8), 4: (899.6, 819.4), 8: (516.5, 518.2)},
}


@pytest.mark.parametrize("shape", list(MODES_MEASURED), ids=["B{}H{}N{}d{}-{}".format(*k) for k in MODES_MEASURED])
def test_deterministic_auto_within_5_percent_of_the_faster_mode(shape):
    """deterministic = 4 resolves to the ordered reduction or the two-pass variant; on every
    measured shape the pick is the faster of the two, or within 1 % of it (and the ordered
    reduction whenever there is one query head per KV head)."""
    B, H, N, d, mask = shape
    for G, (ordered, two_pass) in MODES_MEASURED[shape].items():
        mode = dash.dash_deterministic_resolve(B, H, H // G, N, d, mask, 4)
        assert mode in (1, 2), mode
        got = ordered if mode == 1 else two_pass
        assert got >= 0.99 * max(ordered, two_pass), (shape, G, mode)
        if G == 1:
            assert mode == 1


def test_deterministic_resolve_arguments():
    assert dash.dash_deterministic_resolve(1, 4, 4, 2048, 128, "full", 1) == 1
    assert dash.dash_deterministic_resolve(1, 4, 4, 2048, 128, "full", 3) == 3
    assert dash.dash_deterministic_resolve(1, 4, 4, 256, 64, "causal", 4) == 1  # 64-row tiles
    assert dash.dash_deterministic_resolve(1, 4, 4, 2048, 128, "full", 5) == dash.DASH_ERR_INVALID_ARG
    assert dash.dash_deterministic_resolve(1, 4, 3, 2048, 128, "full", 4) == dash.DASH_ERR_INVALID_ARG
    assert dash.dash_deterministic_resolve(1, 4, 4, 2048, 96, "full", 4) == dash.DASH_ERR_UNSUPPORTED


def test_auto_never_picks_an_invalid_schedule():
    """An odd tile count rules symmetric shift out; explicit schedules pass through."""
    assert dash.dash_schedule_resolve(1, 4, 4, 640, 128, "causal", "auto", 8, 32) in (0, 1)
    assert dash.dash_schedule_resolve(1, 4, 4, 640, 128, "causal", "naive", 8, 32) == 0
    assert dash.dash_schedule_resolve(1, 4, 4, 640, 128, "causal", "sym_shift", 8, 32) == dash.DASH_ERR_UNSUPPORTED
    assert dash.dash_schedule_resolve(1, 4, 4, 2048, 96, "full", "auto", 8, 32) == dash.DASH_ERR_UNSUPPORTED
    assert dash.dash_schedule_resolve(1, 4, 4, 2048, 128, "full", "auto", 0, 32) == dash.DASH_ERR_INVALID_ARG


def test_makespan_rejects_bad_costs():
    with pytest.raises(dash.DashError):
        dash.dash_schedule_makespan(1, 2, 2, 256, "full", "shift", 1, 4, -1.0, 0.0, 0.0)
    with pytest.raises(dash.DashError):
        dash.dash_schedule_makespan(1, 2, 2, 256, "full", "shift", 1, 4, float("nan"), 0.0, 0.0)


# ---------------------------------------------------------------------------------
# Variable-length batches: one table per batch at its own length, merged per CU.
# ---------------------------------------------------------------------------------

@pytest.mark.parametrize("N,lens", [(2048, (2048, 1100, 512)), (448, (448, 200, 64))], ids=["tile128", "tile64"])
@pytest.mark.parametrize("mask,schedule", [("full", "shift"), ("full", "naive"), ("causal", "descending"),
                                           ("causal", "auto"), ("full", "auto")])
def test_varlen_table_is_the_per_batch_tables_merged(mask, schedule, N, lens):
    """Each batch's part of the merged table passes the oracle validator at its own tile
    count (tiles of the padded length's size; coverage, KV contiguity, rank order,
    acyclicity); the whole merged DAG is acyclic (the oracle simulator raises on a
    cycle); every CU runs its batches in order."""
    B, H, Hkv = 3, 4, 2
    tile = dash.dash_tile_size(N)
    rec, local = dash.dash_schedule_table_varlen(B, H, Hkv, N, lens, mask, schedule, 8, 32)
    assert local
    for b, nb in enumerate(lens):
        n_b = -(-nb // tile)
        model_len = max(nb, 512) if tile == 128 else nb  # priced at the table's tile size
        kind = schedule
        if kind == "auto":
            kind = NAMES[dash.dash_schedule_resolve(1, H, Hkv, model_len, 128, mask, "auto", 8, 32)]
            if kind == "sym_shift" and n_b % 2:
                kind = "descending"
        part = rec[rec[:, 1] == b].copy()
        part[:, 1] = 0
        table = to_table(part, 1, H, Hkv, model_len, mask, kind, 256)
        table["n"] = n_b
        osch.validate(table)
        assert {int(t) for t in part[:, 5]} <= set(range(n_b))
    full = to_table(rec, B, H, Hkv, N, mask, "naive", 256)
    assert osch.simulate(full, 1.0, 0.5) > 0
    for w in range(256):
        bs = rec[rec[:, 0] == w][:, 1]
        assert (np.diff(bs) >= 0).all()


def test_varlen_table_argument_errors():
    with pytest.raises(dash.DashError):
        dash.dash_schedule_table_varlen(2, 2, 2, 1024, (0, 1024), "full", "shift", 8, 32)
    with pytest.raises(dash.DashError):
        dash.dash_schedule_table_varlen(2, 2, 2, 1024, (1024, 1025), "full", "shift", 8, 32)
    with pytest.raises(dash.DashError):
        dash.dash_schedule_table_varlen(2, 2, 2, 1024, (1024, 384), "causal", "sym_shift", 8, 32)  # 3 tiles
    with pytest.raises(dash.DashError):
        dash.dash_schedule_table_varlen(2, 2, 2, 256, (256, 192), "causal", "sym_shift", 8, 32)  # 3 tiles of 64


@pytest.mark.parametrize("N,lens", [(1024, [1024, 600, 513, 1000, 777, 512]), (448, [448, 130, 64, 1, 320, 65])],
                         ids=["tile128", "tile64"])
@pytest.mark.parametrize("B,topology", [(3, (8, 32)), (6, (2, 4))], ids=["banded", "shared"])
def test_varlen_layouts_valid(B, topology, N, lens):
    """Up to one batch per slot of a domain: batches on disjoint bands of slots (no CU
    runs two batches); more batches than slots: shared CUs, batches in order. Both merged
    tables pass the per-batch validator (at the padded length's tile size) and are
    acyclic."""
    X, S = topology
    H, Hkv = 2, 1
    lens = lens[:B]
    tile = dash.dash_tile_size(N)
    rec, _ = dash.dash_schedule_table_varlen(B, H, Hkv, N, lens, "causal", "descending", X, S)
    per_cu = {}
    for w, b in rec[:, :2].tolist():
        per_cu.setdefault(w, set()).add(b)
    if B <= S:
        assert max(len(v) for v in per_cu.values()) == 1
    else:
        assert max(len(v) for v in per_cu.values()) > 1
    for b, nb in enumerate(lens):
        part = rec[rec[:, 1] == b].copy()
        part[:, 1] = 0
        table = to_table(part, 1, H, Hkv, max(nb, 512) if tile == 128 else nb, "causal", "descending", X * S)
        table["n"] = -(-nb // tile)
        osch.validate(table)
    assert osch.simulate(to_table(rec, B, H, Hkv, N, "causal", "descending", X * S), 1.0, 0.5) > 0
