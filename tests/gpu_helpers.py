"""Helpers shared by the GPU tests: seeded inputs, oracle references, library calls."""
import math

import numpy as np

from oracle import attention as oa
from scheduling_fa_attn_amd import dash, inputs


def make_case(B, H, Hkv, N, d, causal, seed, q_scale=1.0):
    """Seeded bf16 inputs plus O (bf16) and LSE (fp32) from the fp64 oracle forward.
    q_scale multiplies Q before its bf16 rounding (sharp attention: scores far from 0)."""
    bits = inputs.make_qkvdo(B, H, Hkv, N, d, seed)
    if q_scale != 1.0:
        bits["q"] = inputs.bf16_round_bits(inputs.bf16_bits_to_f32(bits["q"]) * np.float32(q_scale))
    f64 = {k: inputs.bf16_bits_to_f32(v).astype(np.float64) for k, v in bits.items()}
    scale = 1.0 / math.sqrt(d)
    o, lse = oa.forward(f64["q"], f64["k"], f64["v"], causal, scale)
    bits["o"] = inputs.bf16_round_bits(o.astype(np.float32))
    lse32 = lse.astype(np.float32)
    case = {"bits": bits, "lse": lse32, "scale": scale, "causal": causal,
            "shape": (B, H, Hkv, N, d)}
    return case


def oracle_grads(case):
    """fp64 oracle backward on exactly the bytes the GPU receives."""
    b = case["bits"]
    f = {k: inputs.bf16_bits_to_f32(v).astype(np.float64) for k, v in b.items()}
    return oa.backward(f["q"], f["k"], f["v"], f["o"], f["do"], case["lse"].astype(np.float64),
                       case["causal"], case["scale"])


def to_device(case):
    import torch
    dev = {}
    for k, v in case["bits"].items():
        dev[k] = torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).cuda()
    dev["lse"] = torch.from_numpy(case["lse"]).cuda()
    return dev


def workspace_bytes(shape, causal, deterministic):
    """Workspace dash_attn_bwd needs for the mode (the per-tile partials have their own size)."""
    B, H, Hkv, N, d = shape
    if deterministic == 3:
        return dash.dash_attn_bwd_partials_workspace_size(B, H, Hkv, N, d, "causal" if causal else "full")
    return dash.dash_attn_bwd_workspace_size(B, H, Hkv, N, d)


def run(case, dev, schedule, deterministic, workspace=None):
    """One dash_attn_bwd call; returns (dq, dk, dv) torch tensors and the workspace used."""
    import torch
    B, H, Hkv, N, d = case["shape"]
    dq = torch.empty_like(dev["q"])
    dk = torch.empty_like(dev["k"])
    dv = torch.empty_like(dev["v"])
    if workspace is None:
        workspace = torch.empty(max(workspace_bytes(case["shape"], case["causal"], deterministic), 256),
                                dtype=torch.uint8, device="cuda")
    st = dash.dash_attn_bwd(dev["q"], dev["k"], dev["v"], dev["o"], dev["do"], dev["lse"], dq, dk, dv,
                            case["scale"], "causal" if case["causal"] else "full", schedule, deterministic,
                            workspace)
    if st != dash.DASH_OK:
        raise dash.DashError(st, "dash_attn_bwd")
    torch.cuda.synchronize()
    err = dash.dash_last_kernel_error()
    if err != dash.DASH_OK:
        raise dash.DashError(err, "kernel")
    return (dq, dk, dv), workspace


def rel_err(got, ref, floor=0.0):
    """max |got - ref| / max(max |ref|, floor) over the whole tensor."""
    g = got.float().cpu().numpy().astype(np.float64)
    return float(np.abs(g - ref).max() / max(np.abs(ref).max(), floor, 1e-30))


def rel_errs(outs, refs):
    """rel_err of (dq, dk, dv). A tensor whose oracle value is exactly zero (a closed-form
    zero, e.g. dQ and dK at N = 1) is measured against 1e-3 of the largest oracle
    gradient magnitude of the call instead of against zero."""
    floor = 1e-3 * max(float(np.abs(r).max()) for r in refs)
    return tuple(rel_err(g, r, floor) for g, r in zip(outs, refs))


def bf16_bytes(t):
    return t.view(dtype=__import__("torch").int16).cpu().numpy().tobytes()
