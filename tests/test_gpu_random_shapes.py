"""GPU parity over seeded random shapes: the HIP path through the C ABI against the fp64
oracle, element by element, beyond the hand-picked cases of the other parity tests.

Each case draws a batch size, query and KV head counts (grouped-query ratios 1, 2, 3, 4),
a sequence length in [1, 1100] (so both tile sizes, the switch between them at 512 rows,
odd and even tile counts and ragged tails all occur), a head dimension, a mask, one valid
schedule, a reduction mode and a main kernel, from a fixed seed. Bar: the same per-tensor
tolerance as every parity test, and for the deterministic modes a second call with the
same workspace must give the same bytes.
"""
import numpy as np
import pytest

from gpu_helpers import bf16_bytes, make_case, oracle_grads, rel_errs, run, to_device

TOL = 1e-2
N_CASES = 64


def _draw_cases():
    rng = np.random.default_rng(20261203)
    cases = []
    for i in range(N_CASES):
        d = int(rng.choice([64, 128]))
        G = int(rng.choice([1, 2, 3, 4]))
        Hkv = int(rng.integers(1, 3))
        B = int(rng.integers(1, 3))
        # lengths: a third below 512 rows (64-row tiles), the rest up to 1100
        N = int(rng.integers(1, 512)) if i % 3 == 0 else int(rng.integers(512, 1101))
        causal = bool(rng.integers(0, 2))
        tile = 64 if N < 512 else 128
        n_tiles = -(-N // tile)
        scheds = ["naive", "descending"]
        if causal and n_tiles % 2 == 0:
            scheds.append("sym_shift")
        if not causal:
            scheds.append("shift")
        sched = str(rng.choice(scheds))
        det = int(rng.choice([1, 1, 0, 2, 3, 4]))
        kernel = str(rng.choice(["auto", "one_wave"]))
        cases.append((B, G * Hkv, Hkv, N, d, causal, sched, det, kernel, 5000 + i))
    return cases


CASES = _draw_cases()


def _id(c):
    B, H, Hkv, N, d, causal, sched, det, kernel, seed = c
    return f"B{B}H{H}Hkv{Hkv}N{N}d{d}-{'causal' if causal else 'full'}-{sched}-det{det}-{kernel}"


def test_draw_covers_the_cases_it_is_meant_to():
    """The seeded draw spans both tile sizes, both masks, grouped-query heads, odd tile
    counts, every reduction mode and both kernels (so a change of seed cannot silently
    narrow the sweep)."""
    tiles = {64 if c[3] < 512 else 128 for c in CASES}
    assert tiles == {64, 128}
    assert {c[5] for c in CASES} == {False, True}
    assert any(c[1] > c[2] for c in CASES)
    assert any((-(-c[3] // (64 if c[3] < 512 else 128))) % 2 for c in CASES)
    assert {c[7] for c in CASES} == {0, 1, 2, 3, 4}
    assert {c[8] for c in CASES} == {"auto", "one_wave"}
    assert {c[4] for c in CASES} == {64, 128}


@pytest.mark.gpu
@pytest.mark.parametrize("c", CASES, ids=[_id(c) for c in CASES])
def test_random_shape_parity(c):
    pytest.importorskip("torch")
    from scheduling_fa_attn_amd import dash
    B, H, Hkv, N, d, causal, sched, det, kernel, seed = c
    print(f"case {_id(c)} seed={seed}", flush=True)
    case = make_case(B, H, Hkv, N, d, causal, seed=seed)
    refs = oracle_grads(case)
    dev = to_device(case)
    assert dash.dash_set_kernel(kernel) == dash.DASH_OK
    try:
        out, ws = run(case, dev, sched, det)
        errs = rel_errs(out, refs)
        assert max(errs) <= TOL, (errs, _id(c))
        if det != 0:
            again, _ = run(case, dev, sched, det, workspace=ws)
            assert [bf16_bytes(t) for t in again] == [bf16_bytes(t) for t in out], _id(c)
    finally:
        dash.dash_set_kernel("auto")
