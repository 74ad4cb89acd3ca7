"""GPU parity of variable-length batches (dash_attn_bwd_varlen) against the fp64 oracle.

The padded layout holds batch b in rows [0, seqlens[b]) of every tensor. Each batch's
gradients must equal the oracle backward of its own truncated sequence (the textbook
attention gradient, DASH paper section 2.1; causal masks top-left aligned within the
batch), to max |GPU - oracle| / max |oracle| <= 1e-2 per tensor and batch. The padded
input rows are NaN, so that any read of them as data would poison the result; the padded
output rows must come back exactly as they were (a sentinel). Deterministic runs (the ordered
reduction and the two-pass variant) repeat bit for bit.
"""
import math

import numpy as np
import pytest

from oracle import attention as oa
from scheduling_fa_attn_amd import dash, inputs

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

TOL = 1e-2
NAN16 = np.uint16(0x7FC0)       # bf16 quiet NaN
SENTINEL = np.uint16(0x4049)    # bf16 3.140625

CASES = [
    # (B, H, Hkv, N, d, seqlens)
    (3, 4, 2, 1024, 128, (1024, 700, 513)),  # GQA, ragged lengths, odd tile counts (8, 6, 5)
    (2, 2, 2, 768, 64, (300, 768)),          # a batch shorter than one 512-row block
    (2, 2, 1, 1024, 128, (1024, 512)),       # even tile counts (8, 4): symmetric shift allowed
    # More batches than CUs per XCD (the shared layout), lengths 1 .. 512 (single tiles too).
    (34, 1, 1, 512, 64, tuple(int(x) for x in np.random.default_rng(5).integers(1, 513, 34))),
    # Padded length below 512: 64-row tiles (the one-wave kernel), ragged and single-tile batches.
    (3, 2, 1, 448, 128, (448, 130, 64)),
    (2, 2, 2, 320, 64, (1, 320)),
]


def _case(B, H, Hkv, N, d, lens, causal, seed):
    bits = inputs.make_qkvdo(B, H, Hkv, N, d, seed)
    scale = 1.0 / math.sqrt(d)
    o = np.full((B, H, N, d), NAN16, dtype=np.uint16)
    lse = np.full((B, H, N), np.nan, dtype=np.float32)
    ref = []
    for b, nb in enumerate(lens):
        f = {k: inputs.bf16_bits_to_f32(v[b:b + 1, :, :nb]).astype(np.float64) for k, v in bits.items()}
        ob, lb = oa.forward(f["q"], f["k"], f["v"], causal, scale)
        o[b, :, :nb] = inputs.bf16_round_bits(ob[0].astype(np.float32))
        lse[b, :, :nb] = lb[0].astype(np.float32)
        of = inputs.bf16_bits_to_f32(o[b:b + 1, :, :nb]).astype(np.float64)
        ref.append(oa.backward(f["q"], f["k"], f["v"], of, f["do"], lse[b:b + 1, :, :nb].astype(np.float64),
                               causal, scale))
    for k in ("q", "k", "v", "do"):
        for b, nb in enumerate(lens):
            bits[k][b, :, nb:] = NAN16
    bits["o"] = o
    return bits, lse, scale, ref


def _dev(bits, lse):
    dev = {k: torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).cuda() for k, v in bits.items()}
    dev["lse"] = torch.from_numpy(lse).cuda()
    return dev


def _run(dev, lens, scale, mask, schedule, det, ws=None):
    B, H, N, d = dev["q"].shape
    Hkv = dev["k"].shape[1]
    outs = []
    for t in (dev["q"], dev["k"], dev["v"]):
        x = torch.empty_like(t)
        x.view(torch.int16).fill_(int(SENTINEL))
        outs.append(x)
    if ws is None:
        ws = torch.empty(dash.dash_attn_bwd_varlen_workspace_size(B, H, Hkv, N, d), dtype=torch.uint8, device="cuda")
    st = dash.dash_attn_bwd_varlen(dev["q"], dev["k"], dev["v"], dev["o"], dev["do"], dev["lse"], *outs, lens, scale,
                                   mask, schedule, det, ws)
    assert st == dash.DASH_OK, dash.dash_status_string(st)
    torch.cuda.synchronize()
    assert dash.dash_last_kernel_error() == dash.DASH_OK
    return outs, ws


def _check(outs, ref, lens):
    for b, nb in enumerate(lens):
        floor = 1e-3 * max(float(np.abs(r).max()) for r in ref[b])
        for t, r in zip(outs, ref[b]):
            g = t[b:b + 1, :, :nb].float().cpu().numpy().astype(np.float64)
            err = float(np.abs(g - r).max() / max(np.abs(r).max(), floor))
            assert err <= TOL, (b, err)
            pad = t[b, :, nb:].view(torch.int16).cpu().numpy().view(np.uint16)
            assert (pad == SENTINEL).all(), ("padded rows written", b)


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}H{c[1]}Hkv{c[2]}N{c[3]}d{c[4]}" for c in CASES])
def test_varlen_parity(case, causal):
    B, H, Hkv, N, d, lens = case
    bits, lse, scale, ref = _case(B, H, Hkv, N, d, lens, causal, seed=3000 + N + d)
    dev = _dev(bits, lse)
    mask = "causal" if causal else "full"
    tile = dash.dash_tile_size(N)
    even = all(-(-nb // tile) % 2 == 0 for nb in lens)
    scheds = ["auto", "naive", "descending"] + (["sym_shift"] if causal and even else []) + \
        ([] if causal else ["shift"])
    for sched in scheds:
        for det in (1, 0, 2):
            print(f"varlen {case} causal={causal} schedule={sched} det={det}", flush=True)
            outs, _ = _run(dev, lens, scale, mask, sched, det)
            _check(outs, ref, lens)


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_varlen_bitwise_repeatable(causal):
    B, H, Hkv, N, d, lens = CASES[0]
    bits, lse, scale, _ = _case(B, H, Hkv, N, d, lens, causal, seed=31)
    dev = _dev(bits, lse)
    mask = "causal" if causal else "full"
    for det in (1, 2):
        ref, ws = _run(dev, lens, scale, mask, "auto", det)
        ref_bytes = [t.view(torch.int16).cpu().numpy().tobytes() for t in ref]
        for rep in range(9):
            out, ws = _run(dev, lens, scale, mask, "auto", det, ws)
            assert [t.view(torch.int16).cpu().numpy().tobytes() for t in out] == ref_bytes, (det, rep)


def test_varlen_argument_errors():
    B, H, Hkv, N, d = 2, 2, 2, 512, 64
    dev = {k: torch.zeros(B, h, N, d, dtype=torch.bfloat16, device="cuda")
           for k, h in (("q", H), ("k", Hkv), ("v", Hkv), ("o", H), ("do", H))}
    dev["lse"] = torch.zeros(B, H, N, device="cuda")
    outs = [torch.empty_like(dev[k]) for k in ("q", "k", "v")]
    ws = torch.empty(dash.dash_attn_bwd_varlen_workspace_size(B, H, Hkv, N, d), dtype=torch.uint8, device="cuda")

    def call(lens, det=1, sched="auto", w=ws):
        return dash.dash_attn_bwd_varlen(dev["q"], dev["k"], dev["v"], dev["o"], dev["do"], dev["lse"], *outs, lens,
                                         0.125, "causal", sched, det, w)

    # The base workspace has no room for the call's table.
    base = torch.empty(dash.dash_attn_bwd_workspace_size(B, H, Hkv, N, d), dtype=torch.uint8, device="cuda")
    assert call((512, 512), w=base) == dash.DASH_ERR_WORKSPACE

    assert call((0, 512)) == dash.DASH_ERR_INVALID_ARG
    assert call((513, 512)) == dash.DASH_ERR_INVALID_ARG
    assert call((512, 512), det=5) == dash.DASH_ERR_INVALID_ARG
    assert call((512, 512), det=3) == dash.DASH_ERR_UNSUPPORTED  # per-tile partials: one length only
    assert call((512, 384), sched="sym_shift") == dash.DASH_ERR_UNSUPPORTED  # 3 tiles

    small = {k: t[:, :, :256].contiguous() for k, t in dev.items()}
    outs_s = [torch.empty_like(small[k]) for k in ("q", "k", "v")]
    st = dash.dash_attn_bwd_varlen(small["q"], small["k"], small["v"], small["o"], small["do"], small["lse"], *outs_s,
                                   (256, 192), 0.125, "causal", "sym_shift", 1, ws)
    assert st == dash.DASH_ERR_UNSUPPORTED  # 3 tiles of 64 rows in batch 1


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_varlen_one_wave_kernel(causal):
    """The one-wave kernel with per-batch lengths at 128-row tiles (chosen with
    dash_set_kernel; it is also the kernel of chains that cross XCDs): parity and bitwise
    repeats."""
    B, H, Hkv, N, d, lens = CASES[0]
    bits, lse, scale, ref = _case(B, H, Hkv, N, d, lens, causal, seed=77)
    dev = _dev(bits, lse)
    mask = "causal" if causal else "full"
    assert dash.dash_set_kernel("one_wave") == dash.DASH_OK
    try:
        for sched in ("auto", "descending", "naive"):
            for det in (1, 0):
                print(f"varlen one_wave causal={causal} schedule={sched} det={det}", flush=True)
                outs, ws = _run(dev, lens, scale, mask, sched, det)
                _check(outs, ref, lens)
                if det == 1:
                    again, _ = _run(dev, lens, scale, mask, sched, det, ws)
                    assert [t.view(torch.int16).cpu().numpy().tobytes() for t in again] == \
                        [t.view(torch.int16).cpu().numpy().tobytes() for t in outs]
    finally:
        dash.dash_set_kernel("auto")


def test_varlen_distinct_lengths_bounded_memory():
    """100 calls, each with a length vector not seen before: the tables go into the
    caller's workspace through the library's pinned staging ring, so the device memory
    the library holds does not grow with the number of distinct vectors, and the results
    keep matching the oracle (checked on the first and the last call)."""
    B, H, Hkv, N, d = 3, 2, 1, 1024, 64
    rng = np.random.default_rng(5)
    vectors = []
    seen = set()
    while len(vectors) < 100:
        lens = tuple(int(x) for x in rng.integers(1, N + 1, size=B))
        if lens not in seen:
            seen.add(lens)
            vectors.append(lens)
    bits, lse, scale, _ = _case(B, H, Hkv, N, d, vectors[0], True, seed=808)
    dev = _dev(bits, lse)
    ws = torch.empty(dash.dash_attn_bwd_varlen_workspace_size(B, H, Hkv, N, d), dtype=torch.uint8, device="cuda")
    outs, _ = _run(dev, vectors[0], scale, "causal", "auto", 1, ws)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for i, lens in enumerate(vectors[1:]):
        st = dash.dash_attn_bwd_varlen(dev["q"], dev["k"], dev["v"], dev["o"], dev["do"], dev["lse"], *outs, lens,
                                       scale, "causal", "auto", 1, ws)
        assert st == dash.DASH_OK, (i, dash.dash_status_string(st))
    torch.cuda.synchronize()
    assert dash.dash_last_kernel_error() == dash.DASH_OK
    free1, _ = torch.cuda.mem_get_info()
    print(f"device memory free before {free0}, after {free1} bytes", flush=True)
    assert free0 - free1 <= 4 << 20, (free0, free1)
    for lens in (vectors[0], vectors[-1]):
        bits, lse, scale, ref = _case(B, H, Hkv, N, d, lens, True, seed=808)
        outs, _ = _run(_dev(bits, lse), lens, scale, "causal", "auto", 1, ws)
        _check(outs, ref, lens)
