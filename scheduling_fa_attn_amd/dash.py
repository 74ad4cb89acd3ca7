"""ctypes binding of the C ABI in include/dash.h (argument marshalling only).

Every function here has the name of the C entry point it calls. The HIP library
must be built (scheduling_fa_attn_amd/build.py); loading fails loudly when it is
missing. PyTorch is used only to hand device pointers and the current stream to
the library.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import LIB_PATH

DASH_OK = 0
DASH_ERR_INVALID_ARG = -1
DASH_ERR_UNSUPPORTED = -2
DASH_ERR_WORKSPACE = -3
DASH_ERR_NOT_CORESIDENT = -4
DASH_ERR_HIP = -5
DASH_ERR_TIMEOUT = -6
DASH_ERR_PLACEMENT = -7

MASKS = {"full": 0, "causal": 1}
SCHEDULES = {"naive": 0, "descending": 1, "shift": 2, "sym_shift": 3, "auto": 4}

EXPORTED = (
    "dash_attn_bwd_workspace_size",
    "dash_attn_bwd_varlen_workspace_size",
    "dash_attn_bwd_partials_workspace_size",
    "dash_attn_bwd",
    "dash_attn_bwd_timed",
    "dash_attn_bwd_noalloc",
    "dash_attn_bwd_varlen",
    "dash_last_kernel_error",
    "dash_status_string",
    "dash_tile_size",
    "dash_schedule_table",
    "dash_schedule_table_varlen",
    "dash_schedule_makespan",
    "dash_schedule_resolve",
    "dash_deterministic_resolve",
    "dash_set_placement",
    "dash_set_kernel",
    "dash_set_wait_timeout",
    "dash_attn_fwd",
)

_lib = None


class DashError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        super().__init__(f"{what}: {dash_status_string(status)} ({status})" if what else dash_status_string(status))
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = open_library(path)
    return _lib


def open_library(path: str) -> ctypes.CDLL:
    """Load a build of the library at `path` (the release build, or the profiling or
    replay build beside it) with the C signatures declared; independent of load()."""
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library {path} is not built; run python scheduling_fa_attn_amd/build.py")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.dash_attn_bwd_workspace_size.argtypes = [i, i, i, i, i]
    lib.dash_attn_bwd_workspace_size.restype = sz
    lib.dash_attn_bwd_varlen_workspace_size.argtypes = [i, i, i, i, i]
    lib.dash_attn_bwd_varlen_workspace_size.restype = sz
    lib.dash_attn_bwd_partials_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.dash_attn_bwd_partials_workspace_size.restype = sz
    common = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp, sz, vp]
    lib.dash_attn_bwd.argtypes = common
    lib.dash_attn_bwd.restype = i
    lib.dash_attn_bwd_timed.argtypes = common + [vp, vp]
    lib.dash_attn_bwd_timed.restype = i
    lib.dash_attn_bwd_noalloc.argtypes = common[:18] + [vp]
    lib.dash_attn_bwd_noalloc.restype = i
    lib.dash_attn_bwd_varlen.argtypes = common[:14] + [ctypes.POINTER(ctypes.c_int)] + common[14:]
    lib.dash_attn_bwd_varlen.restype = i
    lib.dash_last_kernel_error.argtypes = [vp]
    lib.dash_last_kernel_error.restype = i
    lib.dash_status_string.argtypes = [i]
    lib.dash_status_string.restype = ctypes.c_char_p
    lib.dash_tile_size.argtypes = [i]
    lib.dash_tile_size.restype = i
    lib.dash_schedule_table.argtypes = [i, i, i, i, i, i, i, i, ctypes.POINTER(ctypes.c_int), ctypes.c_longlong,
                                        ctypes.POINTER(ctypes.c_longlong), ctypes.POINTER(ctypes.c_int)]
    lib.dash_schedule_table.restype = i
    lib.dash_schedule_table_varlen.argtypes = [i, i, i, i, ctypes.POINTER(ctypes.c_int), i, i, i, i,
                                               ctypes.POINTER(ctypes.c_int), ctypes.c_longlong,
                                               ctypes.POINTER(ctypes.c_longlong), ctypes.POINTER(ctypes.c_int)]
    lib.dash_schedule_table_varlen.restype = i
    lib.dash_schedule_makespan.argtypes = [i, i, i, i, i, i, i, i, ctypes.c_double, ctypes.c_double,
                                           ctypes.c_double, ctypes.POINTER(ctypes.c_double)]
    lib.dash_schedule_makespan.restype = i
    lib.dash_schedule_resolve.argtypes = [i, i, i, i, i, i, i, i, i]
    lib.dash_schedule_resolve.restype = i
    lib.dash_deterministic_resolve.argtypes = [i, i, i, i, i, i, i]
    lib.dash_deterministic_resolve.restype = i
    lib.dash_set_placement.argtypes = [i]
    lib.dash_set_placement.restype = i
    lib.dash_set_kernel.argtypes = [i]
    lib.dash_set_kernel.restype = i
    lib.dash_set_wait_timeout.argtypes = [ctypes.c_longlong]
    lib.dash_set_wait_timeout.restype = i
    lib.dash_attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.dash_attn_fwd.restype = i
    if hasattr(lib, "dash_profile_attach"):
        lib.dash_profile_attach.argtypes = [vp]
        lib.dash_profile_attach.restype = i
    if hasattr(lib, "dash_replay_attach"):
        lib.dash_replay_attach.argtypes = [vp, sz]
        lib.dash_replay_attach.restype = i
    return lib


def dash_status_string(status: int) -> str:
    return load().dash_status_string(int(status)).decode()


def dash_attn_bwd_workspace_size(B: int, H: int, Hkv: int, N: int, d: int) -> int:
    return int(load().dash_attn_bwd_workspace_size(B, H, Hkv, N, d))


def dash_tile_size(N: int) -> int:
    return int(load().dash_tile_size(N))


def dash_attn_bwd_varlen_workspace_size(B: int, H: int, Hkv: int, N: int, d: int) -> int:
    return int(load().dash_attn_bwd_varlen_workspace_size(B, H, Hkv, N, d))


def dash_attn_bwd_partials_workspace_size(B: int, H: int, Hkv: int, N: int, d: int, mask) -> int:
    return int(load().dash_attn_bwd_partials_workspace_size(B, H, Hkv, N, d, MASKS.get(mask, mask)))


def dash_last_kernel_error(stream=None, lib=None) -> int:
    """Kernel-side status of the last backward call enqueued on `stream` (default: torch's
    current stream); synchronizes that stream."""
    if stream is None:
        import torch

        stream = torch.cuda.current_stream().cuda_stream
    return int((lib or load()).dash_last_kernel_error(ctypes.c_void_p(stream)))


PLACEMENTS = {"aggregate": 0, "spread": 1}


def dash_set_placement(placement, lib=None) -> int:
    """Placement of CU groups larger than one XCD for later calls: "aggregate" (default)
    or "spread" (the paper's n-SM layout; chains cross XCDs)."""
    return int((lib or load()).dash_set_placement(PLACEMENTS.get(placement, placement)))


KERNELS = {"auto": 0, "one_wave": 1, "two_waves": 2}


def dash_set_kernel(kernel, lib=None) -> int:
    """Main backward kernel of later calls: "auto" (default), "one_wave" (one wave per
    SIMD, every configuration) or "two_waves" (two waves per SIMD, 128-row tiles with the
    ordered or atomic reduction; other calls keep the one-wave kernel)."""
    return int((lib or load()).dash_set_kernel(KERNELS.get(kernel, kernel)))


def dash_set_wait_timeout(microseconds, lib=None) -> int:
    """Bound of every in-kernel wait of later calls, in microseconds (default 5 s)."""
    return int((lib or load()).dash_set_wait_timeout(int(microseconds)))


def dash_schedule_makespan(B, H, Hkv, N, mask, schedule, num_xcd, cus_per_xcd, c, r_local, r_remote, lib=None):
    """Makespan of the schedule table's DAG under task cost c and reduction costs
    r_local / r_remote (host only). Raises DashError on an error status."""
    out = ctypes.c_double(0.0)
    st = (lib or load()).dash_schedule_makespan(B, H, Hkv, N, MASKS.get(mask, mask), SCHEDULES.get(schedule, schedule),
                                                num_xcd, cus_per_xcd, float(c), float(r_local), float(r_remote),
                                                ctypes.byref(out))
    if st != DASH_OK:
        raise DashError(st, "dash_schedule_makespan")
    return out.value


def dash_schedule_resolve(B, H, Hkv, N, d, mask, schedule, num_xcd, cus_per_xcd, lib=None) -> int:
    """The schedule dash_attn_bwd runs for `schedule` ("auto" resolved by the cost model);
    a negative value is an error status."""
    return int((lib or load()).dash_schedule_resolve(B, H, Hkv, N, d, MASKS.get(mask, mask),
                                                     SCHEDULES.get(schedule, schedule), num_xcd, cus_per_xcd))


def dash_deterministic_resolve(B, H, Hkv, N, d, mask, deterministic, lib=None) -> int:
    """The mode dash_attn_bwd runs for `deterministic` (4 = the faster reproducible mode for
    the shape); a negative value is an error status."""
    return int((lib or load()).dash_deterministic_resolve(B, H, Hkv, N, d, MASKS.get(mask, mask), int(deterministic)))


def dash_schedule_table(B, H, Hkv, N, mask, schedule, num_xcd, cus_per_xcd):
    """Host-only table export: returns (records [T, 7] int32, xcd_local)."""
    lib = load()
    m = MASKS.get(mask, mask)
    s = SCHEDULES.get(schedule, schedule)
    count = ctypes.c_longlong(0)
    local = ctypes.c_int(0)
    st = lib.dash_schedule_table(B, H, Hkv, N, m, s, num_xcd, cus_per_xcd, None, 0, ctypes.byref(count),
                                 ctypes.byref(local))
    if st not in (DASH_OK, DASH_ERR_WORKSPACE):
        raise DashError(st, "dash_schedule_table")
    rec = np.zeros((max(count.value, 1), 7), dtype=np.int32)
    st = lib.dash_schedule_table(B, H, Hkv, N, m, s, num_xcd, cus_per_xcd,
                                 rec.ctypes.data_as(ctypes.POINTER(ctypes.c_int)), count.value,
                                 ctypes.byref(count), ctypes.byref(local))
    if st != DASH_OK:
        raise DashError(st, "dash_schedule_table")
    return rec[: count.value], bool(local.value)


def dash_schedule_table_varlen(B, H, Hkv, N, seqlens, mask, schedule, num_xcd, cus_per_xcd):
    """Host-only export of a variable-length table: returns (records [T, 7] int32, xcd_local)."""
    lib = load()
    m = MASKS.get(mask, mask)
    s = SCHEDULES.get(schedule, schedule)
    lens = (ctypes.c_int * max(len(seqlens), 1))(*[int(x) for x in seqlens])
    count = ctypes.c_longlong(0)
    local = ctypes.c_int(0)
    st = lib.dash_schedule_table_varlen(B, H, Hkv, N, lens, m, s, num_xcd, cus_per_xcd, None, 0, ctypes.byref(count),
                                        ctypes.byref(local))
    if st not in (DASH_OK, DASH_ERR_WORKSPACE):
        raise DashError(st, "dash_schedule_table_varlen")
    rec = np.zeros((max(count.value, 1), 7), dtype=np.int32)
    st = lib.dash_schedule_table_varlen(B, H, Hkv, N, lens, m, s, num_xcd, cus_per_xcd,
                                        rec.ctypes.data_as(ctypes.POINTER(ctypes.c_int)), count.value,
                                        ctypes.byref(count), ctypes.byref(local))
    if st != DASH_OK:
        raise DashError(st, "dash_schedule_table_varlen")
    return rec[: count.value], bool(local.value)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def dash_attn_fwd(q, k, v, o, lse, softmax_scale, mask, stream=None, lib=None) -> int:
    """Call dash_attn_fwd on torch device tensors: q [B, H, N, d], k, v [B, Hkv, N, d] bf16
    (read); o [B, H, N, d] bf16 and lse [B, H, N] fp32 (written). Returns the status code."""
    import torch

    lib = lib or load()
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    return int(lib.dash_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, N, d,
                                 float(softmax_scale), MASKS.get(mask, mask), ctypes.c_void_p(stream)))


def dash_attn_bwd(q, k, v, o, dO, lse, dq, dk, dv, softmax_scale, mask, schedule, deterministic, workspace,
                  stream=None, main_start=None, main_stop=None, lib=None) -> int:
    """Call dash_attn_bwd (or dash_attn_bwd_timed when events are given) on torch device tensors.

    q, o, dO, dq: [B, H, N, d] bf16; k, v, dk, dv: [B, Hkv, N, d] bf16; lse: [B, H, N] fp32;
    workspace: a uint8 device tensor of at least dash_attn_bwd_workspace_size bytes.
    Returns the status code (0 = success); nothing is checked here beyond marshalling.
    `lib`: another build opened with open_library (default: the release build).
    """
    import torch

    lib = lib or load()
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
            B, H, Hkv, N, d, float(softmax_scale), MASKS.get(mask, mask), SCHEDULES.get(schedule, schedule),
            int(deterministic), _ptr(workspace), workspace.numel() * workspace.element_size(),
            ctypes.c_void_p(stream)]
    if main_start is not None or main_stop is not None:
        return int(lib.dash_attn_bwd_timed(*args, ctypes.c_void_p(main_start or 0),
                                           ctypes.c_void_p(main_stop or 0)))
    return int(lib.dash_attn_bwd(*args))


def dash_attn_bwd_noalloc(q, k, v, o, dO, lse, dq, dk, dv, softmax_scale, mask, schedule, deterministic,
                          stream=None, lib=None) -> int:
    """Call dash_attn_bwd_noalloc (no workspace: the library's static device scratch) on
    torch device tensors laid out as for dash_attn_bwd. Returns the status code."""
    import torch

    lib = lib or load()
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    return int(lib.dash_attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse), _ptr(dq), _ptr(dk),
                                         _ptr(dv), B, H, Hkv, N, d, float(softmax_scale), MASKS.get(mask, mask),
                                         SCHEDULES.get(schedule, schedule), int(deterministic),
                                         ctypes.c_void_p(stream)))


def dash_attn_bwd_varlen(q, k, v, o, dO, lse, dq, dk, dv, seqlens, softmax_scale, mask, schedule, deterministic,
                         workspace, stream=None, lib=None) -> int:
    """Call dash_attn_bwd_varlen on torch device tensors in the padded layout ([B, H, N, d]
    etc., N the padded length); seqlens: B host ints, batch b's rows. Returns the status."""
    import torch

    lib = lib or load()
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    lens = (ctypes.c_int * max(len(seqlens), 1))(*[int(x) for x in seqlens])
    return int(lib.dash_attn_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse), _ptr(dq), _ptr(dk),
                                        _ptr(dv), B, H, Hkv, N, d, lens, float(softmax_scale), MASKS.get(mask, mask),
                                        SCHEDULES.get(schedule, schedule), int(deterministic), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), ctypes.c_void_p(stream)))
