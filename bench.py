"""Benchmark of the deterministic attention backward on one MI355X.

One step = one dash_attn_bwd call (preprocess + persistent backward kernel with the
ordered dQ reduction + dQ cast of the final fp32 sums) over one batch of
synthetic bf16 inputs resident in HBM. The headline workload is the full-mask
configuration the metric is quoted on (B=8, H=Hkv=16, N=2048, d=128, 16 384
tokens, hidden 2048) with the shift schedule; the naive ordered schedule and the
atomic (non-deterministic) variant are timed beside it for the det/non-det ratio.
The three causal configurations (d=64 N=4096, d=128 N=16384, GQA d=128 N=8192)
are timed the same way and reported under "other_workloads" (--only skips them).

Prints ONE JSON line on stdout (details on stderr).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "deterministic attn-bwd TFLOPS (full/causal, d=64/128) + det/non-det ratio"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA peak
PEAK_CLOCK_MHZ = 2400.0  # the clock the MI355X dense peaks are quoted at

WORKLOADS = {
    # name: (B, H, Hkv, N, d, causal, best deterministic schedule, other schedules, config index)
    "full-d128-N2048": (8, 16, 16, 2048, 128, False, "shift", ("naive",), 1),
    "causal-d64-N4096": (4, 32, 32, 4096, 64, True, "sym_shift", ("descending", "naive"), 2),
    "causal-d128-N16384": (1, 16, 16, 16384, 128, True, "sym_shift", ("descending", "naive"), 3),
    "gqa-causal-d128-N8192": (1, 32, 8, 8192, 128, True, "sym_shift", ("descending", "naive"), 4),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def flops_bwd(B, H, N, d, causal):
    f = 2.5 * 4.0 * N * N * d * B * H
    return f / 2.0 if causal else f


def flops_fwd(B, H, N, d, causal):
    f = 4.0 * N * N * d * B * H
    return f / 2.0 if causal else f


def time_forward(dev, d, causal, steps, warmup):
    """dash_attn_fwd on the workload's Q, K, V (outputs to scratch tensors): ms per call."""
    import torch

    from scheduling_fa_attn_amd import dash

    o = torch.empty_like(dev["q"])
    lse = torch.empty(dev["q"].shape[:3], dtype=torch.float32, device="cuda")
    mask = "causal" if causal else "full"

    def call():
        st = dash.dash_attn_fwd(dev["q"], dev["k"], dev["v"], o, lse, 1.0 / math.sqrt(d), mask)
        if st != dash.DASH_OK:
            raise dash.DashError(st, "dash_attn_fwd")

    preroll(call)
    for _ in range(warmup):
        call()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(steps):
        call()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def make_inputs(B, H, Hkv, N, d, causal, seed):
    """Seeded bf16 Q, K, V, dO in HBM; O and LSE from the library's forward (dash_attn_fwd)."""
    import numpy as np
    import torch

    from scheduling_fa_attn_amd import dash, inputs

    bits = inputs.make_qkvdo(B, H, Hkv, N, d, seed)
    dev = {k: torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).cuda() for k, v in bits.items()}
    dev["o"] = torch.empty_like(dev["q"])
    dev["lse"] = torch.empty(B, H, N, dtype=torch.float32, device="cuda")
    st = dash.dash_attn_fwd(dev["q"], dev["k"], dev["v"], dev["o"], dev["lse"], 1.0 / math.sqrt(d),
                            "causal" if causal else "full")
    if st != dash.DASH_OK:
        raise dash.DashError(st, "dash_attn_fwd")
    torch.cuda.synchronize()
    return dev


# Back-to-back calls before every timed block, whatever --warmup says: the GPU clock needs
# tens of milliseconds of load to settle after the host has been busy (input generation,
# the previous workload's set-up), and a short warm-up leaves the first block timed
# slower than the ones after it.
PREROLL_MS = 150.0


def preroll(call, min_ms=PREROLL_MS):
    """Calls `call` until at least min_ms of wall time has passed; returns the call count."""
    import torch

    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(4):
            call()
            n += 1
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= min_ms:
            return n


def time_schedule(dev, shape, causal, schedule, deterministic, steps, warmup, workspace):
    """Returns (ms per step over the timed block, mean main-kernel ms from events, outputs)."""
    import torch

    from scheduling_fa_attn_amd import dash

    B, H, Hkv, N, d = shape
    dq = torch.empty_like(dev["q"])
    dk = torch.empty_like(dev["k"])
    dv = torch.empty_like(dev["v"])
    scale = 1.0 / math.sqrt(d)
    mask = "causal" if causal else "full"
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:  # materialise the HIP events
        a.record()
        b.record()

    def call(i=None):
        st = dash.dash_attn_bwd(dev["q"], dev["k"], dev["v"], dev["o"], dev["do"], dev["lse"], dq, dk, dv,
                                scale, mask, schedule, deterministic, workspace, stream=stream.cuda_stream,
                                main_start=None if i is None else ev[i][0].cuda_event,
                                main_stop=None if i is None else ev[i][1].cuda_event)
        if st != dash.DASH_OK:
            raise dash.DashError(st, "dash_attn_bwd")

    preroll(call)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    err = dash.dash_last_kernel_error()
    if err != dash.DASH_OK:
        raise dash.DashError(err, "kernel")
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(steps):
        call(i)
    t_stop.record()
    torch.cuda.synchronize()
    err = dash.dash_last_kernel_error()
    if err != dash.DASH_OK:
        raise dash.DashError(err, "kernel")
    total_ms = t_start.elapsed_time(t_stop)
    main_ms = sum(a.elapsed_time(b) for a, b in ev) / steps
    return total_ms / steps, main_ms, (dq, dk, dv)


def time_cold(dev, shape, causal, schedule, steps, warmup, workspace, flush_mib=512):
    """Whole-call timings (preprocess + main kernel) with the L2 and the memory-side cache
    flushed before every call by writing a flush_mib MiB buffer: per-call HIP events on the
    call's stream, returns (median ms, min ms, median main-kernel ms)."""
    import torch

    from scheduling_fa_attn_amd import dash

    B, H, Hkv, N, d = shape
    dq = torch.empty_like(dev["q"])
    dk = torch.empty_like(dev["k"])
    dv = torch.empty_like(dev["v"])
    scale = 1.0 / math.sqrt(d)
    mask = "causal" if causal else "full"
    stream = torch.cuda.current_stream()
    flush = torch.empty(flush_mib * (1 << 20) // 4, dtype=torch.float32, device="cuda")
    calls = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(4)) for _ in range(steps)]
    for evs in calls:  # materialise the HIP events (the library records the main-kernel pair)
        for e in evs:
            e.record()

    def call(evs=None):
        st = dash.dash_attn_bwd(dev["q"], dev["k"], dev["v"], dev["o"], dev["do"], dev["lse"], dq, dk, dv,
                                scale, mask, schedule, 1, workspace, stream=stream.cuda_stream,
                                main_start=None if evs is None else evs[2].cuda_event,
                                main_stop=None if evs is None else evs[3].cuda_event)
        if st != dash.DASH_OK:
            raise dash.DashError(st, "dash_attn_bwd")

    def flushed_call():
        flush.fill_(1.0)
        call()

    preroll(flushed_call)
    for _ in range(warmup):
        flushed_call()
    torch.cuda.synchronize()
    for evs in calls:
        flush.fill_(1.0)
        evs[0].record()
        call(evs)
        evs[1].record()
    torch.cuda.synchronize()
    err = dash.dash_last_kernel_error()
    if err != dash.DASH_OK:
        raise dash.DashError(err, "kernel")
    whole = sorted(e[0].elapsed_time(e[1]) for e in calls)
    main = sorted(e[2].elapsed_time(e[3]) for e in calls)
    del flush
    return whole[len(whole) // 2], whole[0], main[len(main) // 2]


def run_to_run_deviation(dev, shape, causal, schedule, deterministic, workspace, runs=10):
    """The DASH paper's Table 1 measure: `runs` identical backward passes; for each tensor,
    the mean over runs 2..runs of max |g_r - g_1| (elementwise, in fp32 on the GPU)."""
    import torch

    from scheduling_fa_attn_amd import dash

    B, H, Hkv, N, d = shape
    outs = [torch.empty_like(dev[k]) for k in ("q", "k", "v")]
    first = None
    dev_max = {"dq": [], "dk": [], "dv": []}
    for r in range(runs):
        st = dash.dash_attn_bwd(dev["q"], dev["k"], dev["v"], dev["o"], dev["do"], dev["lse"], *outs,
                                1.0 / math.sqrt(d), "causal" if causal else "full", schedule, deterministic,
                                workspace)
        if st != dash.DASH_OK:
            raise dash.DashError(st, "dash_attn_bwd")
        if r == 0:
            first = [t.clone() for t in outs]
            continue
        for name, a, b in zip(("dq", "dk", "dv"), outs, first):
            dev_max[name].append(float((a.float() - b.float()).abs().max()))
    err = dash.dash_last_kernel_error()
    if err != dash.DASH_OK:
        raise dash.DashError(err, "kernel")
    return {k: sum(v) / len(v) for k, v in dev_max.items()}


def _smi_numbers(obj, path=()):
    """(key path, number) pairs of a parsed amd-smi JSON document."""
    if isinstance(obj, dict):
        for k, v in obj.items():
            yield from _smi_numbers(v, path + (str(k).lower(),))
    elif isinstance(obj, list):
        for i, v in enumerate(obj):
            yield from _smi_numbers(v, path + (str(i),))
    elif isinstance(obj, (int, float)) and not isinstance(obj, bool):
        yield path, float(obj)


def smi_sample():
    """One reading of the GPU's graphics clocks (MHz) and socket power (W) from
    `amd-smi metric` (None where the tool or the field is not available)."""
    import subprocess

    try:
        res = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "-p", "--json"], capture_output=True,
                             text=True, timeout=20)
        doc = json.loads(res.stdout)
    except Exception as e:  # noqa: BLE001
        return {"error": f"{type(e).__name__}: {e}"[:200]}
    return parse_smi(doc)


def parse_smi(doc):
    """GFX clock per XCD (MHz) and socket power (W) from a parsed `amd-smi metric -c -p
    --json` document: .../clock/gfx_<XCD>/clk/value and .../power/socket_power/value."""
    gfx, power = [], []
    for path, val in _smi_numbers(doc):
        if len(path) >= 3 and path[-1] == "value" and path[-2] == "clk" and path[-3].startswith("gfx"):
            gfx.append(val)
        elif len(path) >= 2 and path[-1] == "value" and path[-2] == "socket_power":
            power.append(val)
    return {"gfx_clk_mhz": gfx, "power_w": power}


def sustained_clock(call, seconds=1.5, samples=3, settle=0.5):
    """Runs `call` back to back for `settle` seconds, then for `seconds` more while
    amd-smi reads the clocks `samples` times from another thread; returns the readings.
    (The settle period keeps a reading of the idle board, or telemetry not yet updated
    since the load began, out of the samples.)"""
    import threading

    import torch

    readings = []
    stop = threading.Event()
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < settle:
        for _ in range(8):
            call()
        torch.cuda.synchronize()

    def sampler():
        for _ in range(samples):
            if stop.wait(seconds / (samples + 1)):
                return
            readings.append(smi_sample())

    t = threading.Thread(target=sampler)
    t0 = time.perf_counter()
    t.start()
    n = 0
    while time.perf_counter() - t0 < seconds or t.is_alive():
        for _ in range(8):
            call()
            n += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 > seconds + 30:
            break
    stop.set()
    t.join()
    return {"calls": n, "seconds": round(time.perf_counter() - t0, 2), "readings": readings,
            "source": "amd-smi metric -c -p during back-to-back calls of the headline step"}


def clock_summary(readings, achieved_tflops):
    """The dense peak is quoted at 2.4 GHz; under this load the board's power limit holds
    the clock lower. Mean of the XCD clocks over the readings, the bf16 peak at that clock
    and the main kernel's fraction of it. Readings at less than half the highest socket
    power are idle snapshots and are left out of the mean."""
    pw = [max(r.get("power_w") or [0.0]) for r in readings]
    used = [r for r, w in zip(readings, pw) if w >= 0.5 * max(pw + [0.0])]
    out = {"readings_in_mean": len(used)}
    clks = [c for r in used for c in (r.get("gfx_clk_mhz") or [])]
    if clks:
        mhz = sum(clks) / len(clks)
        peak_at = PEAK_BF16_TFLOPS * mhz / PEAK_CLOCK_MHZ
        out["mean_gfx_mhz"] = round(mhz, 1)
        out["bf16_peak_at_mean_clock_tflops"] = round(peak_at, 1)
        out["main_kernel_frac_at_mean_clock"] = round(achieved_tflops / peak_at, 4)
    return out


def cpu_baseline(shape, causal, seed, budget_s):
    """The fp64 oracle backward on the host cores, on whole heads of the same workload."""
    import numpy as np

    from oracle import attention as oa
    from scheduling_fa_attn_amd import inputs

    B, H, Hkv, N, d = shape
    blas = []
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max((x.get("num_threads", 0) for x in info), default=0) or os.cpu_count()
        blas = [{k: x.get(k) for k in ("internal_api", "version", "num_threads", "threading_layer")}
                for x in info if x.get("user_api") == "blas"]
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    try:
        import subprocess
        nproc = int(subprocess.run(["nproc"], capture_output=True, text=True, timeout=10).stdout.strip())
    except Exception:  # pragma: no cover
        nproc = None
    G = H // Hkv
    scale = 1.0 / math.sqrt(d)
    heads = 0
    elapsed = 0.0
    group = 0
    # Whole KV-head groups (one KV head and its G query heads) of seeded inputs of the
    # workload's shape, until the time budget is spent.
    while heads < B * H and (heads == 0 or elapsed < budget_s):
        bits = inputs.make_qkvdo(1, G, 1, N, d, seed * 1000 + group)
        f = {k: inputs.bf16_bits_to_f32(v).astype(np.float64) for k, v in bits.items()}
        o, lse = oa.forward(f["q"], f["k"], f["v"], causal, scale)
        t0 = time.perf_counter()
        oa.backward(f["q"], f["k"], f["v"], o, f["do"], lse, causal, scale)
        elapsed += time.perf_counter() - t0
        heads += G
        group += 1
    fl = flops_bwd(1, heads, N, d, causal)
    return {"value": fl / elapsed / 1e12, "unit": "TFLOPS", "cores": int(threads), "kind": "oracle",
            "os_cpu_count": os.cpu_count(), "nproc": nproc, "blas": blas,
            "sample": f"{heads} of {B * H} (batch, query head) units at full N={N}, d={d}, seeded inputs of "
                      f"the workload's shape; fp64 numpy backward only, {elapsed:.1f} s"}


def measure_workload(name, schedule, steps, warmup, compare):
    """Times one workload: the chosen (or best) deterministic schedule, and with `compare`
    the other deterministic schedules and the atomic variant of the chosen one."""
    import torch

    from scheduling_fa_attn_amd import dash

    B, H, Hkv, N, d, causal, best, others, cfg_index = WORKLOADS[name]
    schedule = schedule or best
    shape = (B, H, Hkv, N, d)
    seed = 1000 + cfg_index
    log(f"workload {name}: B={B} H={H} Hkv={Hkv} N={N} d={d} causal={causal} seed={seed}")
    dev = make_inputs(B, H, Hkv, N, d, causal, seed)
    ws = torch.empty(dash.dash_attn_bwd_workspace_size(B, H, Hkv, N, d), dtype=torch.uint8, device="cuda")
    fl = flops_bwd(B, H, N, d, causal)
    ms, main_ms, _ = time_schedule(dev, shape, causal, schedule, 1, steps, warmup, ws)
    tflops = fl / (ms * 1e-3) / 1e12
    log(f"  {schedule} det: {ms:.3f} ms/step ({tflops:.1f} TFLOPS), main kernel {main_ms:.3f} ms")
    extra = {schedule: round(tflops, 2)}
    deviation = {}
    ratio = None
    if compare:
        for s in others:
            ms_s, _, _ = time_schedule(dev, shape, causal, s, 1, steps, warmup, ws)
            extra[s] = round(fl / (ms_s * 1e-3) / 1e12, 2)
            log(f"  {s} det: {ms_s:.3f} ms/step ({extra[s]:.1f} TFLOPS)")
        lanes = (-(-N // 128)) // (2 if schedule == "sym_shift" else 1)
        if lanes > 32:
            # Groups larger than one XCD: the paper's n-SM layout (chains across XCDs) beside
            # the default aggregation on one XCD.
            dash.dash_set_placement("spread")
            try:
                ms_sp, _, _ = time_schedule(dev, shape, causal, schedule, 1, steps, warmup, ws)
            finally:
                dash.dash_set_placement("aggregate")
            extra[schedule + "_spread"] = round(fl / (ms_sp * 1e-3) / 1e12, 2)
            log(f"  {schedule} det, spread placement: {ms_sp:.3f} ms/step ({extra[schedule + '_spread']:.1f} TFLOPS)")
        ms_t, _, _ = time_schedule(dev, shape, causal, schedule, 2, steps, warmup, ws)
        extra["two_pass_" + schedule] = round(fl / (ms_t * 1e-3) / 1e12, 2)
        log(f"  {schedule} two-pass (dK/dV pass + separate dQ pass): {ms_t:.3f} ms/step "
            f"({extra['two_pass_' + schedule]:.1f} TFLOPS)")
        # Both automatic choices: the schedule (host cost model) and the reproducible mode
        # (ordered reduction or two-pass) for this shape.
        mode = dash.dash_deterministic_resolve(B, H, Hkv, N, d, "causal" if causal else "full", 4)
        ms_aa, _, _ = time_schedule(dev, shape, causal, "auto", 4, steps, warmup, ws)
        extra["auto_schedule_auto_mode"] = round(fl / (ms_aa * 1e-3) / 1e12, 2)
        log(f"  schedule auto, deterministic auto (mode {mode}): {ms_aa:.3f} ms/step "
            f"({extra['auto_schedule_auto_mode']:.1f} TFLOPS)")
        ws3 = torch.empty(dash.dash_attn_bwd_partials_workspace_size(B, H, Hkv, N, d, "causal" if causal else "full"),
                          dtype=torch.uint8, device="cuda")
        ms_p, _, _ = time_schedule(dev, shape, causal, schedule, 3, steps, warmup, ws3)
        extra["partials_" + schedule] = round(fl / (ms_p * 1e-3) / 1e12, 2)
        log(f"  {schedule} per-tile partials ({ws3.numel() / 2**30:.2f} GiB of slots + consolidation kernel): "
            f"{ms_p:.3f} ms/step ({extra['partials_' + schedule]:.1f} TFLOPS)")
        ms_a, _, _ = time_schedule(dev, shape, causal, schedule, 0, steps, warmup, ws)
        extra["atomic_" + schedule] = round(fl / (ms_a * 1e-3) / 1e12, 2)
        ratio = ms_a / ms
        log(f"  {schedule} atomic: {ms_a:.3f} ms/step ({extra['atomic_' + schedule]:.1f} TFLOPS); "
            f"det/non-det throughput ratio {ratio:.3f}")
        # Table 1 analogue: run-to-run deviation over 10 identical calls per mode.
        for s, det in [(schedule, 0), (schedule, 1)] + [(x, 1) for x in others] + [(schedule, 2), (schedule, 3)]:
            key = {0: "atomic_", 1: "", 2: "two_pass_", 3: "partials_"}[det] + s
            m_r = run_to_run_deviation(dev, shape, causal, s, det, ws3 if det == 3 else ws)
            deviation[key] = {k: float(f"{v:.3e}") for k, v in m_r.items()}
            log(f"  run-to-run max deviation over 10 runs, {key}: {deviation[key]}")
        del ws3
    ms_f = time_forward(dev, d, causal, steps, warmup)
    fl_f = flops_fwd(B, H, N, d, causal)
    fwd = {"ms": round(ms_f, 4), "tflops": round(fl_f / (ms_f * 1e-3) / 1e12, 2),
           "roofline_frac": round(fl_f / (ms_f * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    log(f"  forward (dash_attn_fwd): {ms_f:.3f} ms ({fwd['tflops']:.1f} TFLOPS)")
    del dev, ws
    torch.cuda.empty_cache()
    return {"schedule": schedule, "tflops": round(tflops, 2), "ms_per_step": round(ms, 4),
            "main_kernel_ms": round(main_ms, 4), "det_nondet_ratio": None if ratio is None else round(ratio, 4),
            "schedules_tflops": extra, "run_to_run_max_dev": deviation or None,
            "roofline_frac": round(fl / (main_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4), "forward": fwd}


# The DASH paper's benchmark grid (section 4.1): 16 384 tokens in total and hidden size
# 2048, so B = 16384 / N and H = Hkv = 2048 / d, for each sequence length, head size and
# mask.
SWEEP_N = (512, 1024, 2048, 4096, 8192, 16384)
SWEEP_SCHEDULES = {False: ("naive", "descending", "shift"), True: ("naive", "descending", "sym_shift")}


def sweep(steps, warmup):
    """Every deterministic schedule and the atomic variant (of the best schedule) over the
    paper's grid; returns one record per (N, d, mask)."""
    import torch

    from scheduling_fa_attn_amd import dash

    out = []
    idx = 0
    for d in (64, 128):
        for causal in (False, True):
            for N in SWEEP_N:
                B, H = 16384 // N, 2048 // d
                shape = (B, H, H, N, d)
                seed = 2000 + idx
                idx += 1
                dev = make_inputs(B, H, H, N, d, causal, seed)
                ws = torch.empty(dash.dash_attn_bwd_workspace_size(B, H, H, N, d), dtype=torch.uint8, device="cuda")
                fl = flops_bwd(B, H, N, d, causal)
                rec = {"N": N, "d": d, "B": B, "H": H, "mask": "causal" if causal else "full", "seed": seed,
                       "tflops": {}}
                best = SWEEP_SCHEDULES[causal][-1]
                for s in SWEEP_SCHEDULES[causal]:
                    ms, main_ms, _ = time_schedule(dev, shape, causal, s, 1, steps, warmup, ws)
                    rec["tflops"][s] = round(fl / (ms * 1e-3) / 1e12, 1)
                    if s == best:
                        rec["main_kernel_frac"] = round(fl / (main_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
                ms_t, _, _ = time_schedule(dev, shape, causal, best, 2, steps, warmup, ws)
                rec["tflops"]["two_pass_" + best] = round(fl / (ms_t * 1e-3) / 1e12, 1)
                ws3 = torch.empty(dash.dash_attn_bwd_partials_workspace_size(B, H, H, N, d,
                                                                             "causal" if causal else "full"),
                                  dtype=torch.uint8, device="cuda")
                ms_p, _, _ = time_schedule(dev, shape, causal, best, 3, steps, warmup, ws3)
                rec["tflops"]["partials_" + best] = round(fl / (ms_p * 1e-3) / 1e12, 1)
                del ws3
                ms_a, _, _ = time_schedule(dev, shape, causal, best, 0, steps, warmup, ws)
                rec["tflops"]["atomic_" + best] = round(fl / (ms_a * 1e-3) / 1e12, 1)
                log(f"sweep N={N} d={d} {rec['mask']}: " + ", ".join(f"{k} {v}" for k, v in rec["tflops"].items()))
                out.append(rec)
                del dev, ws
                torch.cuda.empty_cache()
    return out


# Per-wave phase counters of the profiling build (include/dash_profile.h): slot numbers.
PROF_SLOTS = 20
PHASES = {0: "rest_of_step", 1: "step_barrier", 2: "turn_bookkeeping", 3: "turn_wait", 4: "ack_and_signal",
          5: "handoff", 8: "phase_S_or_dP", 9: "phase_softmax_or_dq_stores", 10: "phase_dS", 12: "phase_dV_or_dK",
          13: "phase_loads", 16: "item_prologue", 17: "item_flush", 18: "item_epilogue"}
# Per-task costs (us) the host schedule model uses (measured_costs in csrc/dash_api.cpp).
MODEL_COSTS = {64: (3.2, 0.45, 2.5), 128: (5.6, 0.9, 2.5)}


def phases(workload, schedules, steps, warmup):
    """Pipeline bubbles of each schedule, measured and predicted (DASH paper, section 3.1:
    the DAG's idle time; section 4.2: synchronisation latency). Runs the profiling build
    (per-wave phase cycle counters) and returns one record per schedule:
      - measured: cycles per wave, the share of all wave-cycles spent waiting for a dQ turn
        (turn_wait_frac), the share of steps whose turn had not come when polled, and the
        idle share of the whole launch (1 - busy wave-cycles / (waves x longest wave),
        busy = total minus turn waits: the tail of early finishers counts as idle);
      - predicted: the same idle share of the host DAG model (dash_schedule_makespan with
        the library's per-task costs): 1 - tasks (c + r) / (CUs x makespan)."""
    import numpy as np
    import torch

    from scheduling_fa_attn_amd import dash
    from scheduling_fa_attn_amd.build import PROF_LIB_PATH

    lib = dash.load(PROF_LIB_PATH)
    if not hasattr(lib, "dash_profile_attach"):
        raise SystemExit("--phases needs the profiling build (build(profile=True)) loaded first")
    B, H, Hkv, N, d, causal, best, others, cfg_index = WORKLOADS[workload]
    mask = "causal" if causal else "full"
    shape = (B, H, Hkv, N, d)
    dev = make_inputs(B, H, Hkv, N, d, causal, 1000 + cfg_index)
    ws = torch.empty(dash.dash_attn_bwd_workspace_size(B, H, Hkv, N, d), dtype=torch.uint8, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    buf = torch.zeros(cus * 8 * PROF_SLOTS, dtype=torch.int64, device="cuda")
    c, r, r_remote = MODEL_COSTS[d]
    out = []
    for sched in schedules:
        ms, main_ms, _ = time_schedule(dev, shape, causal, sched, 1, steps, warmup, ws)
        buf.zero_()
        assert lib.dash_profile_attach(buf.data_ptr()) == 0
        try:
            time_schedule(dev, shape, causal, sched, 1, 1, 0, ws)
        finally:
            lib.dash_profile_attach(None)
        a = buf.cpu().numpy().reshape(cus, 8, PROF_SLOTS).astype(np.float64)
        active = a[:, :, 7] > 0
        tot = a[:, :, 7][active]
        wait = a[:, :, 3][active]
        span = float(tot.max())
        nsteps = float(a[:, :, 6][active].sum())
        waves = int(active.sum())
        # The kernel's waves per CU (4 or 8): CUs with no work still count as idle.
        per_cu = int(active.sum(axis=1).max())
        idle = 1.0 - float((tot - wait).sum()) / (cus * per_cu * span)
        rec, _ = dash.dash_schedule_table(B, H, Hkv, N, mask, sched, 8, cus // 8)
        span_model = dash.dash_schedule_makespan(B, H, Hkv, N, mask, sched, 8, cus // 8, c, r, r_remote)
        pred = 1.0 - len(rec) * (c + r) / (cus * span_model)
        res = {"schedule": sched, "ms_per_call": round(ms, 4), "main_kernel_ms": round(main_ms, 4),
               "waves": waves, "longest_wave_cycles": span,
               "cycles_per_wave_step": {PHASES[k]: round(float(a[:, :, k][active].sum()) / nsteps * per_cu, 1)
                                        for k in PHASES if a[:, :, k][active].sum() > 0},
               "turn_wait_frac": round(float(wait.sum() / tot.sum()), 4),
               "late_turn_step_frac": round(float(a[:, :, 14][active].sum()) / nsteps, 4),
               "measured_idle_frac": round(idle, 4),
               "model_makespan_us": round(span_model, 1), "model_idle_frac": round(pred, 4)}
        log(f"  phases {workload} {sched}: " + json.dumps(res))
        out.append(res)
    return {"workload": workload, "phases": out, "costs_us": {"c": c, "r_local": r, "r_remote": r_remote}}


# Sources of the main kernel: the HBM-traffic figures in profiles/ hold for the kernel
# these hashed to when the counters were taken.
COMMON_SOURCES = ("scheduling_fa_attn_amd/csrc/device_common.h", "scheduling_fa_attn_amd/csrc/kernels.h",
                  "scheduling_fa_attn_amd/build.py")
KERNEL_SOURCES = {"bwd_main": ("scheduling_fa_attn_amd/csrc/bwd_main.hip",) + COMMON_SOURCES,
                  "bwd_pair": ("scheduling_fa_attn_amd/csrc/bwd_pair.hip",) + COMMON_SOURCES}


def main_kernel_name(N, d, kernel_choice, causal):
    """The main kernel dash_attn_bwd launches (deterministic = 1, one XCD per chain); the
    two-waves kernel writes bf16 dQ itself under the full mask (last template argument)."""
    if N >= 512 and kernel_choice != "one_wave":
        return f"bwd_pair_kernel<{d}, true, false, {'false' if causal else 'true'}>"
    return f"bwd_main_kernel<{d}, {4 if N >= 512 else 2}, true, false, false, false>"


def kernel_source_hash(kernel="bwd_pair_kernel<128, true, false, true>"):
    import hashlib

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel.split("<")[0].replace("_kernel", "")]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_bytes(workload, kernel):
    """HBM bytes per launch of the main kernel (FETCH + WRITE, calibrated), from the
    counter summary in profiles/, or None when there is none for this kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic__{workload}.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel") != kernel or t.get("source_hash") != kernel_source_hash(kernel):
        return None
    return int(t["fetch_bytes"] + t["write_bytes"])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30,
                    help="untimed steps before each timed block (the clock needs ~30 ms of load to settle)")
    ap.add_argument("--workload", default="full-d128-N2048", choices=list(WORKLOADS))
    ap.add_argument("--schedule", default=None)
    ap.add_argument("--no-compare", action="store_true", help="skip the other schedules and the atomic variant")
    ap.add_argument("--only", action="store_true", help="measure only --workload (not the other configurations)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache timing (L2 and memory-side cache flushed before every call)")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the clock and power readings (amd-smi) during back-to-back headline calls")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--kernel", default="auto", choices=["auto", "one_wave", "two_waves"],
                    help="main backward kernel (dash_set_kernel); two_waves applies to 128-row tiles (N >= 512)")
    ap.add_argument("--sweep", action="store_true",
                    help="only time every schedule and the atomic variant over the paper's grid (16 384 tokens, "
                         "hidden 2048, N = 512 .. 16384, d = 64 and 128, both masks) and print one JSON line")
    ap.add_argument("--phases", action="store_true",
                    help="only measure pipeline bubbles per deterministic schedule of --workload with the profiling "
                         "build (per-wave phase cycles, turn waits) beside the DAG model's prediction; one JSON line")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (the reference for the "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE scale factor) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}); "
              "the backward of independent (batch, KV head) units would shard over GPUs with no exchange.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy:
        torch.cuda.set_device(0)
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n * 4, "repeats": 3}), flush=True)
        return

    torch.cuda.set_device(0)
    from scheduling_fa_attn_amd import dash
    if args.phases:
        wl = WORKLOADS[args.workload]
        scheds = [args.schedule] if args.schedule else [wl[6]] + list(wl[7])
        res = phases(args.workload, scheds, args.steps, args.warmup)
        print(json.dumps(res), flush=True)
        return
    if dash.dash_set_kernel(args.kernel) != dash.DASH_OK:
        raise SystemExit(f"dash_set_kernel({args.kernel}) failed")
    if args.sweep:
        print(json.dumps({"sweep": sweep(args.steps, args.warmup), "unit": "TFLOPS", "steps": args.steps,
                          "warmup": args.warmup, "data": "synthetic"}), flush=True)
        return
    main_res = measure_workload(args.workload, args.schedule, args.steps, args.warmup, not args.no_compare)
    B, H, Hkv, N, d, causal, _, _, cfg_index = WORKLOADS[args.workload]
    others = {}
    if not args.only:
        for name in WORKLOADS:
            if name != args.workload:
                r = measure_workload(name, None, args.steps, args.warmup, not args.no_compare)
                others[name] = {k: r[k] for k in ("schedule", "tflops", "ms_per_step", "main_kernel_ms",
                                                  "det_nondet_ratio", "schedules_tflops", "roofline_frac",
                                                  "run_to_run_max_dev", "forward")}
    fl = flops_bwd(B, H, N, d, causal)
    main_ms = main_res["main_kernel_ms"]
    achieved = fl / (main_ms * 1e-3) / 1e12
    kernel = main_kernel_name(N, d, args.kernel, causal)
    result = {
        "metric": METRIC,
        "value": round(main_res["tflops"], 3),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "H": H, "Hkv": Hkv, "N": N, "d": d,
                   "mask": "causal" if causal else "full", "schedule": main_res["schedule"],
                   "deterministic": True, "seed": 1000 + cfg_index},
        "det_nondet_ratio": main_res["det_nondet_ratio"],
        "schedules_tflops": main_res["schedules_tflops"],
        "run_to_run_max_dev": main_res["run_to_run_max_dev"],
        "preroll_ms": PREROLL_MS,
        "forward": main_res["forward"],
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_bytes(args.workload, kernel),
                     "kernel": kernel, "main_kernel_ms": round(main_ms, 4)},
    }
    if not args.no_cold or not args.no_clock:
        import torch

        from scheduling_fa_attn_amd import dash

        dev = make_inputs(B, H, Hkv, N, d, causal, 1000 + cfg_index)
        ws = torch.empty(dash.dash_attn_bwd_workspace_size(B, H, Hkv, N, d), dtype=torch.uint8, device="cuda")
    if not args.no_clock:
        outs = [torch.empty_like(dev[k]) for k in ("q", "k", "v")]

        def headline_call():
            st = dash.dash_attn_bwd(dev["q"], dev["k"], dev["v"], dev["o"], dev["do"], dev["lse"], *outs,
                                    1.0 / math.sqrt(d), "causal" if causal else "full", main_res["schedule"], 1, ws)
            if st != dash.DASH_OK:
                raise dash.DashError(st, "dash_attn_bwd")

        result["clock"] = sustained_clock(headline_call)
        result["clock"].update(clock_summary(result["clock"]["readings"], achieved))
        log(f"  clock during back-to-back calls: {result['clock']['readings']}")
        del outs
    if not args.no_cold:
        med, mn, main_med = time_cold(dev, (B, H, Hkv, N, d), causal, main_res["schedule"], args.steps,
                                      min(args.warmup, 5), ws)
        result["cold_cache"] = {"flush": "512 MiB written before every call", "median_ms": round(med, 4),
                                "min_ms": round(mn, 4), "main_kernel_median_ms": round(main_med, 4),
                                "tflops_median": round(fl / (med * 1e-3) / 1e12, 2)}
        log(f"  cold cache: median {med:.3f} ms (min {mn:.3f}), main kernel median {main_med:.3f} ms")
        del dev, ws
    if others:
        result["other_workloads"] = others
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline((B, H, Hkv, N, d), causal, 1000 + cfg_index, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
