"""Pins of the schedule oracle (reference schedules, DAG simulator, validator).

Pinned against:
* the paper's closed-form makespans (DASH, sections 3.2-3.4),
* the work / lanes lower bound (a theorem: no schedule beats it),
* Lemma 1 of section 3.4 (brute force over random isomorphic-chain DAGs),
* hand-written schedules from the text (tests/golden/*.txt),
* planted corruptions of a table, each of which the validator must reject.
"""
import os
import random

import pytest

from oracle import schedule as osch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
PARAMS = [(8, 4, 3.0, 1.0), (16, 6, 2.0, 0.7), (32, 8, 5.0, 2.0)]


# Closed forms, DASH section 3.2 (naive), 3.3 (descending), 3.4 summary (shift, symmetric shift).
def naive_full(n, m, c, r):
    return m * n * (c + r) + (n - 1) * r


def naive_causal(n, m, c, r):
    return m * n * (c + r) + (n - 1) * r


def descending_causal(n, m, c, r):
    return m * (n + 1) * (c + r) / 2 + (n - 1) * r


def shift_full(n, m, c, r):
    return m * n * (c + r)


def sym_shift_causal(n, m, c, r):
    return m * (n + 1) * (c + r) / 2


@pytest.mark.parametrize("n,m,c,r", PARAMS)
def test_closed_forms(n, m, c, r):
    cases = [
        ("naive", False, naive_full),
        ("naive", True, naive_causal),
        ("descending", True, descending_causal),
        ("shift", False, shift_full),
        ("sym_shift", True, sym_shift_causal),
    ]
    for kind, causal, formula in cases:
        table = osch.reference_schedule(kind, n, m, causal)
        osch.validate(table)
        assert osch.simulate(table, c, r) == pytest.approx(formula(n, m, c, r), rel=1e-12), (kind, causal)


def test_descending_extra_case_and_approximation():
    # Exact also with r > c at (8, 2, 0.5, 4); the paper writes "approximately" and
    # assumes an even head count, and the simulated value never beats the optimum.
    t = osch.reference_schedule("descending", 8, 2, True)
    assert osch.simulate(t, 0.5, 4.0) == pytest.approx(descending_causal(8, 2, 0.5, 4.0))
    for n, m, c, r in ((8, 4, 1.0, 3.0), (8, 3, 3.0, 1.0)):
        t = osch.reference_schedule("descending", n, m, True)
        assert osch.simulate(t, c, r) >= sym_shift_causal(n, m, c, r) - 1e-9


@pytest.mark.parametrize("kind,causal", [("naive", False), ("naive", True), ("descending", False),
                                         ("descending", True), ("shift", False), ("sym_shift", True)])
def test_work_lower_bound(kind, causal):
    rng = random.Random(5)
    for _ in range(10):
        n = rng.choice([2, 4, 6, 8, 10])
        m = rng.randint(1, 5) * (2 if kind == "sym_shift" else 1)
        c, r = rng.uniform(0.1, 3), rng.uniform(0.1, 3)
        t = osch.reference_schedule(kind, n, m, causal)
        osch.validate(t)
        tasks = m * (n * (n + 1) // 2 if causal else n * n)
        assert osch.simulate(t, c, r) >= tasks * (c + r) / n - 1e-9


def test_lemma1_brute_force():
    """Lemma 1: zero-weight edges keep the critical path iff depth(u) <= depth(v) for all of them."""
    rng = random.Random(1234)
    checked = 0
    while checked < 1500:
        L = rng.randint(1, 5)
        nc = rng.randint(2, 4)
        weights = [rng.choice([0.5, 1.0, 1.5, 2.0, 3.0]) for _ in range(L)]
        edges = []
        for _ in range(rng.randint(1, 4)):
            k1, k2 = rng.sample(range(nc), 2)
            edges.append(((k1, rng.randint(0, L)), (k2, rng.randint(0, L))))
        try:
            cp0, cp1, monotone = osch.lemma_holds(weights, nc, edges)
        except osch.ScheduleError:
            continue  # the added edges made a cycle: not a DAG, outside the lemma
        assert (abs(cp1 - cp0) < 1e-12) == monotone, (weights, edges, cp0, cp1)
        checked += 1


def _read_golden(name):
    lanes = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                lanes.append([tuple(int(x) for x in e.split(":")) for e in line.split()])
    return lanes


def test_shift_matches_text():
    t = osch.reference_schedule("shift", 4, 1, False)
    assert [[(x[3], x[4]) for x in lane] for lane in t["lanes"]] == _read_golden("shift_n4.txt")
    # Ranks follow the timestamps: dQ tile j is reduced by KV j, j-1, ... (mod n).
    for lane in t["lanes"]:
        for (_, _, _, i, j, rank) in lane:
            assert rank == (j - i) % 4


def test_sym_shift_matches_text():
    t = osch.reference_schedule("sym_shift", 8, 1, True)
    assert [[(x[3], x[4]) for x in lane] for lane in t["lanes"][:4]] == _read_golden("sym_shift_n8.txt")
    assert all(len(lane) == 0 for lane in t["lanes"][4:])


def test_descending_matches_text():
    t = osch.reference_schedule("descending", 4, 2, True)
    assert [[(x[1], x[3], x[4]) for x in lane] for lane in t["lanes"]] == _read_golden("descending_n4_m2.txt")


def _corruptions(table):
    """Yield (name, corrupted table) pairs; each breaks one invariant."""
    import copy

    t = copy.deepcopy(table)
    t["lanes"][0] = t["lanes"][0][:-1]
    yield "dropped task", t

    t = copy.deepcopy(table)
    t["lanes"][1] = t["lanes"][1] + [t["lanes"][0][0]]
    yield "duplicated task", t

    # swap the ranks of two contributors of one dQ tile (the first tile with two)
    t = copy.deepcopy(table)
    where = {}
    done = False
    for li, lane in enumerate(t["lanes"]):
        for p, x in enumerate(lane):
            key = (x[0], x[1], x[4])
            if key in where and not done:
                lj, pj = where[key]
                y = t["lanes"][lj][pj]
                t["lanes"][lj][pj] = y[:5] + (x[5],)
                t["lanes"][li][p] = x[:5] + (y[5],)
                done = True
            where.setdefault(key, (li, p))
    assert done
    yield "swapped ranks", t

    # move one lane's last KV item to another lane (splits or breaks contiguity)
    t = copy.deepcopy(table)
    t["lanes"][2] = t["lanes"][2] + [t["lanes"][1][0]]
    t["lanes"][1] = t["lanes"][1][1:]
    yield "split KV item", t

    # rank gap
    t = copy.deepcopy(table)
    x = t["lanes"][3][-1]
    t["lanes"][3][-1] = x[:5] + (x[5] + 100,)
    yield "rank gap", t

    # task in the masked triangle / out of range
    t = copy.deepcopy(table)
    x = t["lanes"][0][0]
    t["lanes"][0][0] = x[:4] + (table["n"],) + x[5:]
    yield "out of range", t


@pytest.mark.parametrize("kind,causal", [("naive", True), ("shift", False), ("sym_shift", True),
                                         ("descending", True)])
def test_validator_rejects_corruptions(kind, causal):
    table = osch.reference_schedule(kind, 8, 2, causal)
    osch.validate(table)
    for name, bad in _corruptions(table):
        with pytest.raises(osch.ScheduleError):
            osch.validate(bad)
            raise AssertionError(f"{name} was accepted")


def test_validator_rejects_conflict_and_cycle():
    # Two lanes reducing the same dQ tile at the same timestamp (the corollary of Lemma 1).
    t = {"lanes": [[(0, 0, 0, 0, 0), (0, 0, 0, 0, 1)], [(0, 0, 0, 1, 0), (0, 0, 0, 1, 1)]],
         "n": 2, "causal": False, "B": 1, "H": 1, "Hkv": 1, "rule": "timestamp"}
    with pytest.raises(osch.ScheduleError):
        osch.validate(osch.assign_ranks(t))
    # A cycle: lane 0 reduces tile 0 second in order (after lane 1's last task) before its
    # own tile-1 task, which lane 1's first task waits for.
    cyc = {"lanes": [[(0, 0, 0, 0, 0, 1), (0, 0, 0, 0, 1, 0)], [(0, 0, 0, 1, 1, 1), (0, 0, 0, 1, 0, 0)]],
           "n": 2, "causal": False, "B": 1, "H": 1, "Hkv": 1, "rule": "timestamp"}
    with pytest.raises(osch.ScheduleError):
        osch.simulate(cyc, 1.0, 1.0)
