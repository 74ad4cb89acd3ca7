"""DASH reference schedules, DAG critical-path simulator and schedule-table validator (test infrastructure only).

Source: DASH paper (arXiv 2601.21824), section 3.

Model (section 3.1, "Graph Construction"): every tile task (KV tile i, Q tile j)
is a chain of two weighted edges, computation c then global reduction r. A lane
(an SM in the paper, a CU here) runs its tasks back to back. The reductions into
one dQ tile happen one after the other in a fixed order; each such ordering
constraint is a zero-weight edge from the end of one reduction to the start of
the next. The makespan is the longest path; a cycle is a deadlock.

Constraint (section 3.1, "Optimization Constraint"): all tasks of one KV tile run
contiguously on one lane, so its dK/dV stay in registers.

Schedules in the paper's normalisation (section 3 opening: n KV tiles per head,
n lanes, m heads processed one after another):

naive       (section 3.2, the FlashAttention-3 deterministic baseline): lane i
            owns KV tile i of every head and visits Q tiles in ascending order
            (causal: i .. n-1). dQ tiles are reduced in ascending KV index
            ("ordered by CTA index", section 1).
descending  (section 3.3): Q tiles in descending order (n-1 .. 0, causal
            n-1 .. i); dQ order ascending KV index. The (head, KV tile) items go,
            in head-major order, to the lane that becomes free first; this
            module reads "first" under unit task cost, ties to the lowest lane.
shift       (section 3.4, full mask, Fig. 6): lane i visits Q tiles
            i, i+1, .., n-1, 0, .., i-1 (the text says "KV blocks" there, the
            figure caption says Q tiles per SM; the KV-contiguity constraint
            only allows the latter). dQ order = ascending timestamp.
sym_shift   (section 3.4, causal mask, Fig. 7): lanes work in pairs of KV tiles
            (p, n-1-p); n/2 lanes serve one head, so n lanes serve two heads
            at a time (head h goes to half h % 2). Lane p runs
            phase 1: KV p against rows n/2 + ((p + t) mod n/2), t = 0..n/2-1
                     (cyclic shift over the dense lower-left rectangle);
            phase 2: KV p against rows p .. n/2-1 (left triangle, top-down from
                     the diagonal), then KV n-1-p against rows n-1 down to n-1-p
                     (right triangle, bottom-up to the diagonal).
            dQ order = ascending timestamp.

Closed forms (sections 3.2-3.4): naive full m n (c+r) + (n-1) r; naive causal
~ m n (c+r) + (n-1) r; descending causal ~ m (n+1)(c+r)/2 + (n-1) r (even m);
shift m n (c+r); symmetric shift m (n+1)(c+r)/2.

Tables
------
A table is a dict with keys
  lanes  : list (one per lane) of task tuples (b, h, g, i, j, rank)
           b batch, h query head, g KV head, i KV tile, j Q tile, rank = place of
           this task in the reduction order of dQ tile (b, h, j);
  n      : KV tiles (= Q tiles) per head;
  causal : bool;
  B, H, Hkv : sizes (query head h reads KV head h // (H // Hkv));
  rule   : "kv_index" (dQ order by ascending KV tile) or
           "timestamp" (ascending position in the lane, ties to the lower lane).
The same format is produced by the GPU library's C++ table builder, which this
module checks.
"""
from __future__ import annotations

from collections import defaultdict, deque

__all__ = [
    "reference_schedule",
    "assign_ranks",
    "simulate",
    "validate",
    "critical_path",
    "lemma_holds",
    "ScheduleError",
]


class ScheduleError(ValueError):
    """A table breaks one of the schedule invariants."""


# ----------------------------------------------------------------------------
# Reference schedules in the paper's normalisation (one batch, m heads, Hkv = H).
# ----------------------------------------------------------------------------

def _q_tiles(n, i, causal):
    return list(range(i, n)) if causal else list(range(n))


def reference_schedule(kind: str, n: int, m: int, causal: bool) -> dict:
    """Per-lane task lists of schedule `kind` for m heads of n KV tiles on n lanes."""
    lanes = [[] for _ in range(n)]
    if kind == "naive":
        rule = "kv_index"
        for h in range(m):
            for i in range(n):
                for j in _q_tiles(n, i, causal):
                    lanes[i].append((0, h, h, i, j))
    elif kind == "descending":
        rule = "kv_index"
        free = [0] * n  # unit-cost finish time of each lane
        for h in range(m):
            for i in range(n):
                qs = _q_tiles(n, i, causal)[::-1]
                lane = min(range(n), key=lambda x: (free[x], x))
                for j in qs:
                    lanes[lane].append((0, h, h, i, j))
                free[lane] += len(qs)
    elif kind == "shift":
        if causal:
            raise ValueError("shift scheduling is defined for the full mask")
        rule = "timestamp"
        for h in range(m):
            for i in range(n):
                for t in range(n):
                    lanes[i].append((0, h, h, i, (i + t) % n))
    elif kind == "sym_shift":
        if not causal:
            raise ValueError("symmetric shift scheduling is defined for the causal mask")
        if n % 2:
            raise ValueError("symmetric shift needs an even number of KV tiles")
        rule = "timestamp"
        half = n // 2
        for h in range(m):
            base = (h % 2) * half
            for p in range(half):
                lane = lanes[base + p]
                for t in range(half):
                    lane.append((0, h, h, p, half + (p + t) % half))
                for j in range(p, half):
                    lane.append((0, h, h, p, j))
                for j in range(n - 1, n - 2 - p, -1):
                    lane.append((0, h, h, n - 1 - p, j))
    else:
        raise ValueError(f"unknown schedule {kind!r}")
    table = {"lanes": lanes, "n": n, "causal": causal, "B": 1, "H": m, "Hkv": m, "rule": rule}
    return assign_ranks(table)


def assign_ranks(table: dict) -> dict:
    """Fill in each task's rank in its dQ tile's reduction order, following table['rule']."""
    chains = defaultdict(list)
    for lane_id, lane in enumerate(table["lanes"]):
        for pos, task in enumerate(lane):
            b, h, g, i, j = task[:5]
            if table["rule"] == "kv_index":
                key = (i,)
            elif table["rule"] == "timestamp":
                key = (pos, lane_id)
            else:
                raise ValueError(f"unknown rule {table['rule']!r}")
            chains[(b, h, j)].append((key, lane_id, pos))
    rank = {}
    for members in chains.values():
        for r, (_, lane_id, pos) in enumerate(sorted(members)):
            rank[(lane_id, pos)] = r
    lanes = [[tuple(task[:5]) + (rank[(li, p)],) for p, task in enumerate(lane)]
             for li, lane in enumerate(table["lanes"])]
    out = dict(table)
    out["lanes"] = lanes
    return out


# ----------------------------------------------------------------------------
# DAG simulator (section 3.1): longest path over compute/reduce chains.
# ----------------------------------------------------------------------------

def simulate(table: dict, c, r) -> float:
    """Critical-path length (makespan) of the table's DAG.

    `c` and `r` are the compute and reduction costs, either numbers or callables
    of the task tuple. Raises ScheduleError on a cycle (a deadlock).
    Nodes per task: compute start, reduction start, reduction end.
    """
    cost_c = c if callable(c) else (lambda task: c)
    cost_r = r if callable(r) else (lambda task: r)
    # node ids: 3 * task_index + {0: compute start, 1: reduction start, 2: reduction end}
    tasks = []
    for lane in table["lanes"]:
        for task in lane:
            tasks.append(task)
    nt = len(tasks)
    adj = [[] for _ in range(3 * nt)]
    indeg = [0] * (3 * nt)

    def edge(u, v, w):
        adj[u].append((v, w))
        indeg[v] += 1

    idx = 0
    chain_members = defaultdict(list)
    for lane in table["lanes"]:
        prev = None
        for task in lane:
            edge(3 * idx, 3 * idx + 1, float(cost_c(task)))
            edge(3 * idx + 1, 3 * idx + 2, float(cost_r(task)))
            if prev is not None:
                edge(3 * prev + 2, 3 * idx, 0.0)
            b, h, g, i, j, rank = task
            chain_members[(b, h, j)].append((rank, idx))
            prev = idx
            idx += 1
    for members in chain_members.values():
        members.sort()
        for (_, u), (_, v) in zip(members, members[1:]):
            edge(3 * u + 2, 3 * v + 1, 0.0)
    return _longest_path(adj, indeg)


def _longest_path(adj, indeg) -> float:
    """Longest path from the sources of a weighted DAG (Kahn's order); raises on a cycle."""
    n = len(adj)
    indeg = list(indeg)
    dist = [0.0] * n
    queue = deque(u for u in range(n) if indeg[u] == 0)
    seen = 0
    while queue:
        u = queue.popleft()
        seen += 1
        for v, w in adj[u]:
            if dist[u] + w > dist[v]:
                dist[v] = dist[u] + w
            indeg[v] -= 1
            if indeg[v] == 0:
                queue.append(v)
    if seen != n:
        raise ScheduleError("dependency cycle: the schedule deadlocks")
    return max(dist) if dist else 0.0


def critical_path(num_nodes: int, edges) -> float:
    """Longest path of a DAG given as (u, v, weight) edges over nodes 0..num_nodes-1."""
    adj = [[] for _ in range(num_nodes)]
    indeg = [0] * num_nodes
    for u, v, w in edges:
        adj[u].append((v, float(w)))
        indeg[v] += 1
    return _longest_path(adj, indeg)


def lemma_holds(chain_weights, n_chains: int, extra_edges) -> tuple:
    """Lemma 1 (section 3.4) on n isomorphic chains from one source to one sink.

    Chain k has nodes (k, 0) .. (k, L) with edge weights chain_weights (all > 0);
    (k, 0) is joined to a common source and (k, L) to a common sink by zero-weight
    edges. extra_edges are zero-weight ((k, a), (k2, b)) pairs. Returns
    (critical path of G0, critical path of G_k, all depth(u) <= depth(v)).
    Raises ScheduleError if the extra edges create a cycle.
    """
    L = len(chain_weights)
    src, sink = 0, 1

    def node(k, a):
        return 2 + k * (L + 1) + a

    nn = 2 + n_chains * (L + 1)
    base = []
    for k in range(n_chains):
        base.append((src, node(k, 0), 0.0))
        for a in range(L):
            base.append((node(k, a), node(k, a + 1), chain_weights[a]))
        base.append((node(k, L), sink, 0.0))
    cp0 = critical_path(nn, base)
    extra = [(node(k, a), node(k2, b2), 0.0) for (k, a), (k2, b2) in extra_edges]
    cp1 = critical_path(nn, base + extra)
    monotone = all(a <= b2 for (_, a), (_, b2) in extra_edges)
    return cp0, cp1, monotone


# ----------------------------------------------------------------------------
# Validator
# ----------------------------------------------------------------------------

def validate(table: dict, conflict_free: bool | None = None) -> None:
    """Check a schedule table; raise ScheduleError naming the first broken invariant.

    1. coverage: every valid task (b, h, i, j) appears exactly once
       (causal: j >= i), with g = h // (H // Hkv);
    2. KV contiguity (section 3.1): the tasks of one KV item (b, g, i) form a
       single contiguous run on a single lane;
    3. ranks: in every dQ tile the ranks are 0 .. count-1, each once;
    4. order rule: ranks follow the table's rule (ascending KV tile, or
       ascending (position, lane));
    5. acyclic: the lane order plus the reduction order has no cycle;
    6. conflict-free and depth-monotone (Lemma 1 and its corollary, section
       3.4), checked when `conflict_free` is true (default: rule == "timestamp"):
       no two tasks of one dQ tile share a position, and every reduction edge
       goes from a smaller to a larger position.
    """
    n, causal = table["n"], table["causal"]
    B, H, Hkv = table["B"], table["H"], table["Hkv"]
    if H % Hkv:
        raise ScheduleError("H must be a multiple of Hkv")
    G = H // Hkv
    rule = table["rule"]
    if conflict_free is None:
        conflict_free = rule == "timestamp"

    seen = set()
    item_lane = {}
    chains = defaultdict(list)
    for lane_id, lane in enumerate(table["lanes"]):
        closed = set()
        current = None
        for pos, task in enumerate(lane):
            b, h, g, i, j, rank = task
            if not (0 <= b < B and 0 <= h < H and 0 <= i < n and 0 <= j < n):
                raise ScheduleError(f"task {task} out of range")
            if g != h // G:
                raise ScheduleError(f"task {task}: KV head {g} is not h // G = {h // G}")
            if causal and j < i:
                raise ScheduleError(f"task {task} lies in the masked upper triangle")
            key = (b, h, i, j)
            if key in seen:
                raise ScheduleError(f"task {key} appears twice")
            seen.add(key)
            item = (b, g, i)
            if item != current:
                if item in closed:
                    raise ScheduleError(f"KV item {item} is not contiguous on lane {lane_id}")
                if current is not None:
                    closed.add(current)
                current = item
                if item in item_lane and item_lane[item] != lane_id:
                    raise ScheduleError(f"KV item {item} is split across lanes")
                item_lane[item] = lane_id
            chains[(b, h, j)].append((rank, lane_id, pos, i))
    expected = B * H * (n * (n + 1) // 2 if causal else n * n)
    if len(seen) != expected:
        raise ScheduleError(f"coverage: {len(seen)} tasks, expected {expected}")

    for key, members in chains.items():
        ranks = sorted(m[0] for m in members)
        if ranks != list(range(len(members))):
            raise ScheduleError(f"dQ tile {key}: ranks {ranks} are not 0..{len(members) - 1}")
        members.sort()
        if rule == "kv_index":
            order = [m[3] for m in members]
            if order != sorted(order):
                raise ScheduleError(f"dQ tile {key}: order is not ascending KV index")
        elif rule == "timestamp":
            order = [(m[2], m[1]) for m in members]
            if order != sorted(order):
                raise ScheduleError(f"dQ tile {key}: order is not ascending timestamp")
        else:
            raise ScheduleError(f"unknown rule {rule!r}")
        if conflict_free:
            positions = [m[2] for m in members]
            if len(set(positions)) != len(positions):
                raise ScheduleError(f"dQ tile {key}: two contributors share a timestamp (conflict)")
            if positions != sorted(positions):
                raise ScheduleError(f"dQ tile {key}: a reduction edge decreases depth")

    simulate(table, 1.0, 1.0)  # raises ScheduleError on a cycle
