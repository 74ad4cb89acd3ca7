"""dash_attn_bwd_noalloc: the backward for callers that cannot allocate device memory.

Its workspace and schedule table live in the library's static device scratch array. Two
calls in a row, the second with a smaller input (fewer heads, shorter sequence, smaller
head dimension, other mask), must give what dash_attn_bwd gives with a workspace of its
own: bit for bit for the deterministic modes (same kernels, same table), and for the
atomic variant the oracle tolerance (max |GPU - oracle| / max |oracle| <= 1e-2), which
every mode must also meet. Shapes beyond the array's capacity are rejected before
anything is enqueued.
"""
import ctypes

import pytest

from gpu_helpers import bf16_bytes, make_case, oracle_grads, rel_errs, run, to_device

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

TOL = 1e-2

# (B, H, Hkv, N, d, causal, schedule), each call smaller than the one before: the full
# mask at 128-row tiles (the main kernel writes dQ itself there), the causal mask with a
# ragged last tile, then 64-row tiles on the one-wave kernel.
CALLS = [(2, 4, 2, 1024, 128, False, "shift"), (2, 4, 2, 700, 128, True, "sym_shift"),
         (1, 2, 2, 256, 64, False, "shift")]


def _noalloc(case, dev, schedule, det):
    from scheduling_fa_attn_amd import dash
    outs = [torch.empty_like(dev[k]) for k in ("q", "k", "v")]
    st = dash.dash_attn_bwd_noalloc(dev["q"], dev["k"], dev["v"], dev["o"], dev["do"], dev["lse"], *outs,
                                    case["scale"], "causal" if case["causal"] else "full", schedule, det)
    assert st == dash.DASH_OK, dash.dash_status_string(st)
    torch.cuda.synchronize()
    assert dash.dash_last_kernel_error() == dash.DASH_OK
    return outs


@pytest.mark.parametrize("det", [1, 2, 0], ids=["ordered", "two_pass", "atomic"])
def test_noalloc_matches_the_workspace_call(det):
    for B, H, Hkv, N, d, causal, sched in CALLS:
        print(f"noalloc det={det} B={B} H={H} Hkv={Hkv} N={N} d={d} causal={causal} schedule={sched}", flush=True)
        case = make_case(B, H, Hkv, N, d, causal, seed=600 + N)
        dev = to_device(case)
        ref = oracle_grads(case)
        got = _noalloc(case, dev, sched, det)
        errs = rel_errs(got, ref)
        assert max(errs) <= TOL, errs
        if det:
            want, _ = run(case, dev, sched, det)
            assert [bf16_bytes(t) for t in got] == [bf16_bytes(t) for t in want]


def test_noalloc_rejects_shapes_beyond_the_scratch():
    """B=8, H=16, N=2048, d=128 needs a 129 MiB workspace (the array has 56 MiB for it);
    the per-tile partials and variable-length batches are not offered. Checked before any
    pointer is used (the pointers below are never dereferenced)."""
    from scheduling_fa_attn_amd import dash
    lib = dash.load()
    p = ctypes.c_void_p(1 << 12)

    def call(B, H, Hkv, N, d, det=1):
        return lib.dash_attn_bwd_noalloc(p, p, p, p, p, p, p, p, p, B, H, Hkv, N, d, 0.125, 0, 2, det, None)

    assert call(8, 16, 16, 2048, 128) == dash.DASH_ERR_WORKSPACE
    assert call(1, 2, 2, 256, 64, det=3) == dash.DASH_ERR_UNSUPPORTED
    assert call(1, 2, 2, 256, 96) == dash.DASH_ERR_UNSUPPORTED
