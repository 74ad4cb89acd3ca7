"""The C-ABI library loads, exports every entry point of include/dash.h, and rejects bad
arguments before touching the GPU (these calls return before any HIP call)."""
import ctypes
import os
import re

import pytest

from scheduling_fa_attn_amd import dash

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
HEADER = os.path.join(INCLUDE, "dash.h")
PROF_HEADER = os.path.join(INCLUDE, "dash_profile.h")


def header_functions(path=HEADER):
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dash_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = dash.load()
    names = header_functions()
    assert set(names) == set(dash.EXPORTED)
    for name in names:
        assert hasattr(lib, name), name


def test_profiling_build_exports():
    """The profiling build (-DDASH_PROFILE) exports dash.h plus dash_profile.h; the
    release build exports nothing of dash_profile.h."""
    from scheduling_fa_attn_amd.build import PROF_LIB_PATH

    extra = header_functions(PROF_HEADER)
    assert extra == ["dash_profile_attach"]
    rel = ctypes.CDLL(dash.load()._name)
    for name in extra:
        assert not hasattr(rel, name), name
    if not os.path.exists(PROF_LIB_PATH):
        pytest.skip("profiling library not built")
    prof = ctypes.CDLL(PROF_LIB_PATH)
    for name in header_functions() + extra:
        assert hasattr(prof, name), name


def test_replay_build_exports():
    """The replay build (-DDASH_REPLAY) exports dash.h plus dash_replay.h; the release
    build exports nothing of dash_replay.h."""
    from scheduling_fa_attn_amd.build import REPLAY_LIB_PATH

    extra = header_functions(os.path.join(INCLUDE, "dash_replay.h"))
    assert extra == ["dash_replay_attach"]
    rel = ctypes.CDLL(dash.load()._name)
    for name in extra:
        assert not hasattr(rel, name), name
    if not os.path.exists(REPLAY_LIB_PATH):
        pytest.skip("replay library not built")
    lib = ctypes.CDLL(REPLAY_LIB_PATH)
    for name in header_functions() + extra:
        assert hasattr(lib, name), name


def test_status_strings():
    for code in range(0, -8, -1):
        assert dash.dash_status_string(code) != "unknown status"
    assert dash.dash_status_string(42) == "unknown status"


def test_workspace_size():
    assert dash.dash_attn_bwd_workspace_size(1, 2, 2, 256, 64) >= 1 * 2 * 256 * 64 * 4
    # Per-tile partials: (tile / 64) * n^2 slots of 64 x d floats per head (n (n + 1) / 2
    # causal); 64-row tiles below N = 512, 128-row tiles from there.
    base = dash.dash_attn_bwd_workspace_size(1, 2, 2, 256, 64) - 1 * 2 * 256 * 64 * 4
    assert dash.dash_attn_bwd_partials_workspace_size(1, 2, 2, 256, 64, "full") == base + 2 * 16 * 64 * 64 * 4
    assert dash.dash_attn_bwd_partials_workspace_size(1, 2, 2, 256, 64, "causal") == base + 2 * 10 * 64 * 64 * 4
    base = dash.dash_attn_bwd_workspace_size(8, 16, 16, 2048, 128) - 8 * 16 * 2048 * 128 * 4
    assert dash.dash_attn_bwd_partials_workspace_size(8, 16, 16, 2048, 128, "full") == \
        base + 8 * 16 * 2 * 256 * 64 * 128 * 4
    assert dash.dash_attn_bwd_partials_workspace_size(1, 2, 2, 256, 64, 2) == 0
    assert dash.dash_attn_bwd_partials_workspace_size(1, 2, 2, 256, 96, "full") == 0
    assert dash.dash_attn_bwd_workspace_size(1, 2, 2, 256, 96) == 0
    assert dash.dash_attn_bwd_workspace_size(1, 3, 2, 256, 64) == 0
    assert dash.dash_attn_bwd_varlen_workspace_size(1, 3, 2, 256, 64) == 0


@pytest.mark.parametrize("B,H,Hkv,N", [(3, 4, 2, 1024), (34, 1, 1, 512), (2, 2, 2, 320), (1, 16, 16, 16384)])
def test_varlen_workspace_holds_the_table(B, H, Hkv, N):
    """The variable-length workspace adds a table region at least as large as the step
    records (16 bytes per 64-row step) plus the task records (16 bytes per task) of the
    largest table any length vector gives (every batch at the padded length, full mask)."""
    d = 64
    base = dash.dash_attn_bwd_workspace_size(B, H, Hkv, N, d)
    extra = dash.dash_attn_bwd_varlen_workspace_size(B, H, Hkv, N, d) - base
    tile = dash.dash_tile_size(N)
    rec, _ = dash.dash_schedule_table_varlen(B, H, Hkv, N, [N] * B, "full", "auto", 8, 32)
    tasks = len(rec)
    assert tasks == B * H * (-(-N // tile)) ** 2
    assert extra >= 16 * tasks * (tile // 64 + 1) + 16 * B * Hkv * (-(-N // tile)), (extra, tasks)


def _call(**kw):
    lib = dash.load()
    args = dict(q=1 << 12, k=1 << 12, v=1 << 12, o=1 << 12, dO=1 << 12, lse=1 << 12, dq=1 << 12, dk=1 << 12,
                dv=1 << 12, B=1, H=2, Hkv=2, N=256, d=64, scale=0.125, mask=0, schedule=0, det=1,
                ws=1 << 12, ws_bytes=0, stream=None)
    args.update(kw)
    vp = ctypes.c_void_p
    return lib.dash_attn_bwd(*(vp(args[k]) for k in ("q", "k", "v", "o", "dO", "lse", "dq", "dk", "dv")),
                             args["B"], args["H"], args["Hkv"], args["N"], args["d"], args["scale"],
                             args["mask"], args["schedule"], args["det"], vp(args["ws"]), args["ws_bytes"],
                             vp(args["stream"]))


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), dash.DASH_ERR_UNSUPPORTED),
    (dict(H=3), dash.DASH_ERR_INVALID_ARG),
    (dict(Hkv=0), dash.DASH_ERR_INVALID_ARG),
    (dict(mask=2), dash.DASH_ERR_INVALID_ARG),
    (dict(schedule=5), dash.DASH_ERR_INVALID_ARG),
    (dict(mask=1, schedule=2), dash.DASH_ERR_UNSUPPORTED),
    (dict(mask=0, schedule=3), dash.DASH_ERR_UNSUPPORTED),
    (dict(det=5), dash.DASH_ERR_INVALID_ARG),
    (dict(det=-1), dash.DASH_ERR_INVALID_ARG),
    (dict(scale=0.0), dash.DASH_ERR_INVALID_ARG),
    (dict(scale=float("inf")), dash.DASH_ERR_INVALID_ARG),
    (dict(q=None), dash.DASH_ERR_INVALID_ARG),
    (dict(dq=(1 << 12) + 2), dash.DASH_ERR_INVALID_ARG),
    (dict(ws=None), dash.DASH_ERR_INVALID_ARG),
    (dict(ws_bytes=16), dash.DASH_ERR_WORKSPACE),
])
def test_argument_errors_before_any_launch(kw, status):
    assert _call(**kw) == status


def _call_fwd(**kw):
    lib = dash.load()
    args = dict(q=1 << 12, k=1 << 12, v=1 << 12, o=1 << 12, lse=1 << 12, B=1, H=2, Hkv=2, N=256, d=64,
                scale=0.125, mask=0, stream=None)
    args.update(kw)
    vp = ctypes.c_void_p
    return lib.dash_attn_fwd(*(vp(args[k]) for k in ("q", "k", "v", "o", "lse")), args["B"], args["H"],
                             args["Hkv"], args["N"], args["d"], args["scale"], args["mask"], vp(args["stream"]))


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), dash.DASH_ERR_UNSUPPORTED),
    (dict(H=3), dash.DASH_ERR_INVALID_ARG),
    (dict(Hkv=0), dash.DASH_ERR_INVALID_ARG),
    (dict(mask=2), dash.DASH_ERR_INVALID_ARG),
    (dict(scale=-1.0), dash.DASH_ERR_INVALID_ARG),
    (dict(q=None), dash.DASH_ERR_INVALID_ARG),
    (dict(o=(1 << 12) + 8), dash.DASH_ERR_INVALID_ARG),
    (dict(lse=(1 << 12) + 2), dash.DASH_ERR_INVALID_ARG),
    (dict(B=0, q=None, o=None), dash.DASH_OK),
])
def test_forward_argument_errors_before_any_launch(kw, status):
    assert _call_fwd(**kw) == status


def test_empty_inputs_are_a_no_op():
    assert _call(B=0, q=None, ws=None) == dash.DASH_OK
    assert _call(N=0, q=None, ws=None) == dash.DASH_OK


def test_kernel_selection_arguments():
    """dash_set_kernel accepts the three documented values and rejects others; the
    setting is library-wide and is restored here to the default."""
    try:
        for k in ("one_wave", "two_waves", "auto"):
            assert dash.dash_set_kernel(k) == dash.DASH_OK
        for bad in (-1, 3, 99):
            assert dash.dash_set_kernel(bad) == dash.DASH_ERR_INVALID_ARG
    finally:
        dash.dash_set_kernel("auto")


def test_wait_timeout_arguments():
    """dash_set_wait_timeout accepts 0 .. 3.6e9 microseconds and rejects values outside;
    restored here to the default (5 s)."""
    try:
        for us in (0, 1, 5_000_000, 3_600_000_000):
            assert dash.dash_set_wait_timeout(us) == dash.DASH_OK
        for bad in (-1, 3_600_000_001, -(1 << 40)):
            assert dash.dash_set_wait_timeout(bad) == dash.DASH_ERR_INVALID_ARG
    finally:
        assert dash.dash_set_wait_timeout(5_000_000) == dash.DASH_OK


def test_schedule_model_arguments():
    """The host-only model calls check their arguments like the table export."""
    assert dash.dash_schedule_resolve(1, 2, 2, 256, 64, "full", "shift", 1, 4) == 2
    assert dash.dash_schedule_resolve(1, 3, 2, 256, 64, "full", "auto", 1, 4) == dash.DASH_ERR_INVALID_ARG
    assert dash.dash_schedule_resolve(1, 2, 2, 256, 64, "causal", "shift", 1, 4) == dash.DASH_ERR_UNSUPPORTED
    assert dash.dash_schedule_resolve(1, 2, 2, 256, 64, "full", "auto", 1, 0) == dash.DASH_ERR_INVALID_ARG
    lib = dash.load()
    import ctypes
    out = ctypes.c_double(0.0)
    assert lib.dash_schedule_makespan(1, 2, 2, 256, 0, 2, 1, 4, 1.0, 0.0, 0.0, None) == dash.DASH_ERR_INVALID_ARG
    assert lib.dash_schedule_makespan(1, 2, 2, 256, 0, 2, 1, 4, 1.0, 0.0, -1.0, ctypes.byref(out)) == \
        dash.DASH_ERR_INVALID_ARG
    assert lib.dash_schedule_makespan(1, 2, 2, 256, 0, 2, 1, 4, 1.0, 0.0, 0.0, ctypes.byref(out)) == dash.DASH_OK
    assert out.value == 2 * 4 * 1.0  # shift: m n (c + r) with m = 2 heads on n = 4 lanes, r = 0
