"""Exact check of the ordered dQ reduction, in the replay build of the library.

DASH paper (arXiv 2601.21824) section 1 and Table 1: the deterministic backward adds
the dQ partials of one tile in an order fixed by the schedule, so a CPU that adds the
same partials in the same order reproduces the GPU's sums bit for bit. The replay
build (libdash_mi355x_replay.so, -DDASH_REPLAY) dumps every fp32 partial of every
contribution at its rank and adds it to the running sum with one fp32 addition. Here
the CPU adds the dumped partials of every 32x32 dQ block in rank order, in float32 from
+0, and requires:
  - the sums equal the final fp32 accumulator of the workspace bitwise;
  - the bf16 dQ the cast wrote equals bf16_RNE(scale * sum) bitwise;
  - every rank slot up to the tile's contributor count was written (the dump starts as
    NaN, so a lost contribution cannot pass as a zero), and none past it.
The contributor count of query tile j is n (full mask) or j + 1 (causal), the KV tiles
that see it; ranks are the table's order of those contributions (the schedules of the
paper's section 3). The release build's fused arithmetic is checked by the tolerance
tests; this test pins the ordering, the turn-passing, the accumulator addressing and
the bf16 cast.
"""
import math
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gpu_helpers import make_case, to_device  # noqa: E402
from scheduling_fa_attn_amd import dash, inputs  # noqa: E402
from scheduling_fa_attn_amd.build import REPLAY_LIB_PATH  # noqa: E402

pytestmark = pytest.mark.gpu

# (B, H, Hkv, N, d, causal): 64-row tiles (N < 512) and 128-row tiles, a ragged N, GQA.
CASES = [
    (1, 2, 2, 256, 64, False),
    (1, 2, 2, 256, 64, True),
    (1, 2, 2, 360, 128, True),  # ragged: 6 tiles of 64, rows 360..383 past N
    (1, 4, 2, 512, 128, True),
    (2, 2, 1, 512, 64, False),
]
SCHEDULES = {False: ("naive", "descending", "shift"), True: ("naive", "descending", "sym_shift")}


def _block_rows_cols():
    """Row and column within a 32x32 block of each of its 1024 accumulator floats."""
    f = np.arange(1024)
    i, rem = f // 256, f % 256
    lane, e = rem // 4, rem % 4
    rows = 16 * (i // 2) + 2 * (i % 2) + lane // 32 + 4 * e
    cols = lane % 32
    return rows, cols


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(REPLAY_LIB_PATH):
        pytest.fail(f"replay library {REPLAY_LIB_PATH} is not built (build(replay=True))")
    return dash.open_library(REPLAY_LIB_PATH)


@pytest.mark.parametrize("case_args", CASES, ids=[f"B{c[0]}H{c[1]}Hkv{c[2]}N{c[3]}d{c[4]}-{'causal' if c[5] else 'full'}"
                                                 for c in CASES])
def test_ordered_replay_bitwise(lib, case_args):
    B, H, Hkv, N, d, causal = case_args
    case = make_case(B, H, Hkv, N, d, causal, seed=7)
    dev = to_device(case)
    tile = lib.dash_tile_size(N)
    R = -(-N // tile) * tile
    n_kv = R // tile
    steps = R // 64
    nblk = 2 * (d // 32)
    rows_in, cols_in = _block_rows_cols()
    n_tiles = -(-N // tile)
    for sched in SCHEDULES[causal]:
        if sched == "sym_shift" and n_tiles % 2:
            continue
        print(f"[replay] {case_args} schedule={sched}", flush=True)
        dump_floats = B * H * steps * nblk * n_kv * 1024
        dump = torch.full((dump_floats,), float("nan"), dtype=torch.float32, device="cuda")
        assert lib.dash_replay_attach(dump.data_ptr(), dump_floats * 4) == 0
        ws = torch.zeros(lib.dash_attn_bwd_workspace_size(B, H, Hkv, N, d), dtype=torch.uint8, device="cuda")
        dq = torch.empty_like(dev["q"])
        dk = torch.empty_like(dev["k"])
        dv = torch.empty_like(dev["v"])
        st = dash.dash_attn_bwd(dev["q"], dev["k"], dev["v"], dev["o"], dev["do"], dev["lse"], dq, dk, dv,
                                case["scale"], "causal" if causal else "full", sched, 1, ws, lib=lib)
        assert st == 0, dash.dash_status_string(st)
        torch.cuda.synchronize()
        assert dash.dash_last_kernel_error(lib=lib) == 0
        lib.dash_replay_attach(None, 0)
        d_np = dump.cpu().numpy().reshape(B * H, steps, nblk, n_kv, 1024)
        acc = ws[: B * H * R * d * 4].cpu().numpy().view(np.float32).reshape(B * H, steps, nblk, 1024)
        dq_bits = dq.view(torch.int16).cpu().numpy().view(np.uint16).reshape(B * H, N, d)
        for bh in range(B * H):
            for stp in range(steps):
                j = (stp * 64) // tile  # query tile of this 64-row step
                k = j + 1 if causal else n_kv
                # Slots up to the contributor count were all written, the rest untouched.
                assert not np.isnan(d_np[bh, stp, :, :k]).any(), (sched, bh, stp)
                assert np.isnan(d_np[bh, stp, :, k:]).all(), (sched, bh, stp)
                for blk in range(nblk):
                    s = np.zeros(1024, dtype=np.float32)
                    for r in range(k):
                        s = (s + d_np[bh, stp, blk, r]).astype(np.float32)
                    assert np.array_equal(s.view(np.uint32), acc[bh, stp, blk].view(np.uint32)), (sched, bh, stp, blk)
                    qb, db = blk // (d // 32), blk % (d // 32)
                    rows = stp * 64 + 32 * qb + rows_in
                    cols = 32 * db + cols_in
                    ok = rows < N
                    want = inputs.bf16_round_bits((s * np.float32(case["scale"])).astype(np.float32))
                    got = dq_bits[bh, rows[ok], cols[ok]]
                    assert np.array_equal(got, want[ok]), (sched, bh, stp, blk)


# 128-row tiles: both main kernels, selected explicitly (1: one wave per SIMD, 2: two
# waves per SIMD, the default there).
PAIR_CASES = [
    (1, 4, 2, 512, 128, True),
    (1, 2, 2, 700, 128, False),  # ragged: rows 700..767 past N
    (1, 2, 2, 640, 128, True),   # 5 tiles
    (1, 4, 2, 1000, 64, True),   # d = 64: the A waves reduce all four dQ blocks of a step
    (2, 2, 1, 512, 64, False),
]


@pytest.mark.parametrize("kernel", [2, 1], ids=["two_waves", "one_wave"])
@pytest.mark.parametrize("case_args", PAIR_CASES,
                         ids=[f"B{c[0]}H{c[1]}Hkv{c[2]}N{c[3]}d{c[4]}-{'causal' if c[5] else 'full'}"
                              for c in PAIR_CASES])
def test_ordered_replay_bitwise_d128_kernels(lib, case_args, kernel):
    assert lib.dash_set_kernel(kernel) == 0
    try:
        test_ordered_replay_bitwise(lib, case_args)
    finally:
        lib.dash_set_kernel(0)


def test_replay_dump_too_small_is_rejected(lib):
    B, H, Hkv, N, d = 1, 2, 2, 256, 64
    case = make_case(B, H, Hkv, N, d, False, seed=7)
    dev = to_device(case)
    dump = torch.zeros(16, dtype=torch.float32, device="cuda")
    assert lib.dash_replay_attach(dump.data_ptr(), 64) == 0
    ws = torch.zeros(lib.dash_attn_bwd_workspace_size(B, H, Hkv, N, d), dtype=torch.uint8, device="cuda")
    dq, dk, dv = torch.empty_like(dev["q"]), torch.empty_like(dev["k"]), torch.empty_like(dev["v"])
    st = dash.dash_attn_bwd(dev["q"], dev["k"], dev["v"], dev["o"], dev["do"], dev["lse"], dq, dk, dv,
                            1.0 / math.sqrt(d), "full", "shift", 1, ws, lib=lib)
    lib.dash_replay_attach(None, 0)
    assert st == dash.DASH_ERR_WORKSPACE


# Spread placement (the paper's n-SM layout): groups whose lanes fill whole XCDs (64 or
# 128 lanes on 32-CU XCDs) span XCDs, so consecutive contributors of a dQ tile sit on
# different L2 domains and the chain runs on device-scope loads, stores and flags (the
# one-wave kernel). 64 tiles of 128 rows: 64 lanes for naive, descending and shift;
# 128 tiles: 64 lanes for the symmetric shift, 128 for naive and descending.
SPREAD_CASES = [
    (1, 1, 1, 8192, 64, False),
    (1, 1, 1, 16384, 64, True),
]


@pytest.mark.parametrize("case_args", SPREAD_CASES,
                         ids=[f"B{c[0]}H{c[1]}Hkv{c[2]}N{c[3]}d{c[4]}-{'causal' if c[5] else 'full'}"
                              for c in SPREAD_CASES])
def test_ordered_replay_bitwise_across_xcds(lib, case_args):
    B, H, Hkv, N, d, causal = case_args
    assert lib.dash_set_placement(1) == 0
    assert dash.dash_set_placement("spread") == 0
    try:
        for sched in SCHEDULES[causal]:
            _, local = dash.dash_schedule_table(B, H, Hkv, N, "causal" if causal else "full", sched, 8, 32)
            assert not local, sched  # some dQ chain crosses an XCD
        test_ordered_replay_bitwise(lib, case_args)
    finally:
        lib.dash_set_placement(0)
        dash.dash_set_placement("aggregate")
