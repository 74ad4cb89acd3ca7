"""GPU parity and determinism at the benchmark's full configuration sizes.

The HIP path runs every configuration in the launch configuration bench.py times
(same shapes, seeds, schedules and workspace sizing). The fp64 oracle cannot
afford every head at these sizes, so the check samples (batch, query head) units:
for a sampled unit the GPU receives the O and LSE of the oracle forward, and the
oracle backward of that unit (dQ of its query heads, dK/dV of its KV head, summed
over the KV head's whole query-head group) is compared element by element with the
GPU result. Other heads get O/LSE from the library's forward (dash_attn_fwd); their
gradients are not compared.

Bars: max|GPU - oracle| / max|oracle| <= 1e-2 per tensor (dQ, dK, dV) of every
sampled unit and every schedule, deterministic and atomic; dQ/dK/dV bitwise equal
over 20 repeated runs of each deterministic schedule.

DASH paper (arXiv 2601.21824) section 4.1 "Benchmark Settings" (16 384 tokens,
hidden 2048, head dim 64/128, bf16 random inputs) and section 4.5 Table 1 (runs of
identical backward passes: deterministic schedules deviate by exactly zero).
"""
import math
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import attention as oa  # noqa: E402
from scheduling_fa_attn_amd import dash, inputs  # noqa: E402

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

TOL = 1e-2
REPEATS = 20

# workload -> sampled KV groups (b, g): every query head of the group is checked.
SAMPLES = {
    "full-d128-N2048": [(0, 0), (7, 15)],
    "causal-d64-N4096": [(0, 0), (3, 31)],
    "causal-d128-N16384": [(0, 9)],
    "gqa-causal-d128-N8192": [(0, 7)],
}
SCHEDULES = {False: ("shift", "naive"), True: ("sym_shift", "descending", "naive")}


def _bits_to_dev(bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


@pytest.fixture(scope="module", params=list(SAMPLES), ids=list(SAMPLES))
def workload(request):
    """Seeded inputs of a workload on the GPU, O/LSE of the sampled heads from the oracle
    (the other heads get theirs from the library's forward, dash_attn_fwd)."""
    name = request.param
    B, H, Hkv, N, d, causal, best, others, ci = bench.WORKLOADS[name]
    seed = 1000 + ci
    G = H // Hkv
    scale = 1.0 / math.sqrt(d)
    print(f"\n[{name}] inputs seed={seed}", flush=True)
    bits = inputs.make_qkvdo(B, H, Hkv, N, d, seed)
    dev = {k: _bits_to_dev(v) for k, v in bits.items()}
    dev["o"] = torch.empty_like(dev["q"])
    dev["lse"] = torch.empty(B, H, N, dtype=torch.float32, device="cuda")
    st = dash.dash_attn_fwd(dev["q"], dev["k"], dev["v"], dev["o"], dev["lse"], scale, "causal" if causal else "full")
    assert st == dash.DASH_OK, dash.dash_status_string(st)
    refs = []
    for (b, g) in SAMPLES[name]:
        hs = slice(g * G, (g + 1) * G)
        f = {k: inputs.bf16_bits_to_f32(bits[k][b:b + 1, hs if k in ("q", "do") else slice(g, g + 1)])
             .astype(np.float64) for k in ("q", "k", "v", "do")}
        print(f"[{name}] oracle forward/backward b={b} kv_head={g}", flush=True)
        o, lse = oa.forward(f["q"], f["k"], f["v"], causal, scale)
        o_bits = inputs.bf16_round_bits(o.astype(np.float32))
        lse32 = lse.astype(np.float32)
        dev["o"][b, hs] = _bits_to_dev(o_bits)[0]
        dev["lse"][b, hs] = torch.from_numpy(lse32[0]).cuda()
        dq, dk, dv = oa.backward(f["q"], f["k"], f["v"], inputs.bf16_bits_to_f32(o_bits).astype(np.float64),
                                 f["do"], lse32.astype(np.float64), causal, scale)
        refs.append(((b, g, hs), (dq[0], dk[0, 0], dv[0, 0])))
    torch.cuda.synchronize()
    ws = torch.empty(dash.dash_attn_bwd_workspace_size(B, H, Hkv, N, d), dtype=torch.uint8, device="cuda")
    return {"name": name, "shape": (B, H, Hkv, N, d), "causal": causal, "scale": scale, "dev": dev,
            "refs": refs, "ws": ws}


def _ws(w, det):
    if det != 3:
        return w["ws"]
    if "ws3" not in w:
        B, H, Hkv, N, d = w["shape"]
        size = dash.dash_attn_bwd_partials_workspace_size(B, H, Hkv, N, d, "causal" if w["causal"] else "full")
        w["ws3"] = torch.empty(size, dtype=torch.uint8, device="cuda")
    return w["ws3"]


def _run(w, schedule, det):
    dev = w["dev"]
    dq = torch.empty_like(dev["q"])
    dk = torch.empty_like(dev["k"])
    dv = torch.empty_like(dev["v"])
    st = dash.dash_attn_bwd(dev["q"], dev["k"], dev["v"], dev["o"], dev["do"], dev["lse"], dq, dk, dv, w["scale"],
                            "causal" if w["causal"] else "full", schedule, det, _ws(w, det))
    assert st == dash.DASH_OK, dash.dash_status_string(st)
    torch.cuda.synchronize()
    err = dash.dash_last_kernel_error()
    assert err == dash.DASH_OK, dash.dash_status_string(err)
    return dq, dk, dv


def _rel(got, ref):
    g = got.float().cpu().numpy().astype(np.float64)
    return float(np.abs(g - ref).max() / max(np.abs(ref).max(), 1e-30))


def test_sampled_parity_all_schedules(workload):
    w = workload
    for sched in SCHEDULES[w["causal"]]:
        # Ordered and atomic reductions for every schedule; the two-pass variant
        # (deterministic = 2) and the per-tile partials (3) with the first (best) schedule.
        for det in (1, 0, 2, 3) if sched == SCHEDULES[w["causal"]][0] else (1, 0):
            print(f"[{w['name']}] schedule={sched} det={det}", flush=True)
            dq, dk, dv = _run(w, sched, det)
            for (b, g, hs), (rq, rk, rv) in w["refs"]:
                errs = (_rel(dq[b, hs], rq), _rel(dk[b, g], rk), _rel(dv[b, g], rv))
                assert max(errs) <= TOL, (sched, det, b, g, errs)


def test_bitwise_repeatable_at_full_size(workload):
    w = workload
    runs = [(s, 1) for s in SCHEDULES[w["causal"]]] + [(SCHEDULES[w["causal"]][0], 2), (SCHEDULES[w["causal"]][0], 3)]
    for sched, det in runs:
        print(f"[{w['name']}] {REPEATS} runs of schedule={sched} det={det}", flush=True)
        first = [t.clone() for t in _run(w, sched, det)]
        for rep in range(REPEATS - 1):
            out = _run(w, sched, det)
            for a, b_ in zip(first, out):
                assert torch.equal(a.view(torch.int16), b_.view(torch.int16)), (sched, det, rep)


def test_atomic_run_to_run_deviation(workload):
    """Table 1 analogue: M_r = max|g_r - g_1| over runs of the atomic variant (reported,
    not asserted: atomics may happen to land in the same order), and the deterministic
    schedule's M_r, which must be exactly 0."""
    w = workload
    best = SCHEDULES[w["causal"]][0]
    for det in (0, 1):
        first = [t.float() for t in _run(w, best, det)]
        dev_max = 0.0
        for _ in range(4):
            out = _run(w, best, det)
            dev_max = max(dev_max, max(float((a - b_.float()).abs().max()) for a, b_ in zip(first, out)))
        print(f"[{w['name']}] schedule={best} det={det} max run-to-run deviation {dev_max:.3g}", flush=True)
        if det:
            assert dev_max == 0.0


def _spread_checks(w, schedules):
    assert dash.dash_set_placement("spread") == 0
    try:
        for sched in schedules:
            print(f"[{w['name']}] spread placement, schedule={sched}, {REPEATS} runs", flush=True)
            first = [t.clone() for t in _run(w, sched, 1)]
            for (b, g, hs), (rq, rk, rv) in w["refs"]:
                errs = (_rel(first[0][b, hs], rq), _rel(first[1][b, g], rk), _rel(first[2][b, g], rv))
                assert max(errs) <= TOL, (sched, b, g, errs)
            for rep in range(REPEATS - 1):
                out = _run(w, sched, 1)
                for a, b_ in zip(first, out):
                    assert torch.equal(a.view(torch.int16), b_.view(torch.int16)), (sched, rep)
    finally:
        assert dash.dash_set_placement("aggregate") == 0


def test_spread_placement_parity_and_determinism(workload):
    """The long causal head (n = 128 KV tiles, 64 lanes for the symmetric shift) with the
    spread placement: the group spans XCDs and its dQ chains cross L2 domains (device-
    scope ordering). Same bars for every deterministic schedule: parity on the sampled
    heads, 20 bitwise-identical runs."""
    w = workload
    if w["name"] != "causal-d128-N16384":
        pytest.skip("only this workload has groups larger than one XCD")
    _spread_checks(w, ("sym_shift", "descending", "naive"))


@pytest.fixture(scope="module")
def spread_full():
    """A full-mask shape whose groups span XCDs under the spread placement: 64 KV tiles
    per head (64 lanes for shift, naive and descending, two XCDs); both heads sampled."""
    B, H, Hkv, N, d, causal = 1, 2, 2, 8192, 64, False
    scale = 1.0 / math.sqrt(d)
    bits = inputs.make_qkvdo(B, H, Hkv, N, d, 1234)
    dev = {k: _bits_to_dev(v) for k, v in bits.items()}
    f = {k: inputs.bf16_bits_to_f32(v).astype(np.float64) for k, v in bits.items()}
    print("\n[spread-full-d64-N8192] oracle forward/backward", flush=True)
    o, lse = oa.forward(f["q"], f["k"], f["v"], causal, scale)
    o_bits = inputs.bf16_round_bits(o.astype(np.float32))
    lse32 = lse.astype(np.float32)
    dev["o"] = _bits_to_dev(o_bits)
    dev["lse"] = torch.from_numpy(lse32).cuda()
    dq, dk, dv = oa.backward(f["q"], f["k"], f["v"], inputs.bf16_bits_to_f32(o_bits).astype(np.float64), f["do"],
                             lse32.astype(np.float64), causal, scale)
    refs = [((0, g, slice(g, g + 1)), (dq[0, g:g + 1], dk[0, g], dv[0, g])) for g in range(H)]
    ws = torch.empty(dash.dash_attn_bwd_workspace_size(B, H, Hkv, N, d), dtype=torch.uint8, device="cuda")
    return {"name": "spread-full-d64-N8192", "shape": (B, H, Hkv, N, d), "causal": causal, "scale": scale,
            "dev": dev, "refs": refs, "ws": ws}


def test_spread_placement_full_mask(spread_full):
    _spread_checks(spread_full, ("shift", "descending", "naive"))
