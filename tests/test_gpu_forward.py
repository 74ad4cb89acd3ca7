"""GPU parity of the forward kernel (dash_attn_fwd) against the fp64 oracle forward.

The forward is the textbook definition ("Writing an Attention Kernel", Step 1), computed
on the GPU tile by tile with an online softmax (Step 2). O is compared with the rule the
backward uses (max |GPU - oracle| / max |oracle| <= 1e-2 per tensor); the LSE, an fp32
output accumulated in fp32 from exact bf16 products, to 1e-3 absolute. Cases: both masks,
64- and 128-wide heads, ragged N (partial last Q and KV tiles), N = 1, GQA; the four
benchmark shapes on sampled heads (causal: a row prefix, which depends only on the keys
before it); bitwise repeatability; and the GPU forward's O and LSE feeding the backward.
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gpu_helpers import make_case, oracle_grads, rel_err, rel_errs, to_device  # noqa: E402
from oracle import attention as oa  # noqa: E402
from scheduling_fa_attn_amd import dash, inputs  # noqa: E402

pytestmark = pytest.mark.gpu

TOL = 1e-2
LSE_TOL = 1e-3

# (B, H, Hkv, N, d)
SMALL = [
    (1, 2, 2, 256, 64),
    (2, 4, 2, 700, 128),   # ragged: 6 Q tiles of 128 with 60 rows; KV tiles of 64 with 60 rows
    (1, 3, 1, 1000, 64),   # GQA 3:1, ragged
    (1, 2, 1, 33, 128),
    (1, 1, 1, 1, 64),
]


def _fwd(dev, d, causal):
    o = torch.empty_like(dev["q"])
    B, H, N, _ = dev["q"].shape
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    st = dash.dash_attn_fwd(dev["q"], dev["k"], dev["v"], o, lse, 1.0 / math.sqrt(d), "causal" if causal else "full")
    assert st == dash.DASH_OK, dash.dash_status_string(st)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("shape", SMALL, ids=[f"B{s[0]}H{s[1]}Hkv{s[2]}N{s[3]}d{s[4]}" for s in SMALL])
def test_forward_parity(shape, causal):
    B, H, Hkv, N, d = shape
    print(f"[fwd] {shape} causal={causal}", flush=True)
    case = make_case(B, H, Hkv, N, d, causal, seed=11)
    dev = to_device(case)
    o_ref, lse_ref = oa.forward(*(inputs.bf16_bits_to_f32(case["bits"][x]).astype(np.float64) for x in "qkv"),
                                causal, case["scale"])
    o, lse = _fwd(dev, d, causal)
    assert rel_err(o, o_ref) <= TOL
    assert float(np.abs(lse.cpu().numpy().astype(np.float64) - lse_ref).max()) <= LSE_TOL


def test_forward_bitwise_repeatable():
    case = make_case(2, 4, 2, 700, 128, True, seed=12)
    dev = to_device(case)
    o1, l1 = _fwd(dev, 128, True)
    for _ in range(5):
        o2, l2 = _fwd(dev, 128, True)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


def test_forward_feeds_backward():
    """The GPU forward's O and LSE as the backward's inputs: gradients within the
    tolerance of the oracle backward computed from the oracle forward."""
    B, H, Hkv, N, d = 1, 4, 2, 512, 64
    for causal, sched in ((False, "shift"), (True, "sym_shift")):
        case = make_case(B, H, Hkv, N, d, causal, seed=13)
        dev = to_device(case)
        dev["o"], dev["lse"] = _fwd(dev, d, causal)
        dq, dk, dv = (torch.empty_like(dev[x]) for x in ("q", "k", "v"))
        ws = torch.empty(dash.dash_attn_bwd_workspace_size(B, H, Hkv, N, d), dtype=torch.uint8, device="cuda")
        st = dash.dash_attn_bwd(dev["q"], dev["k"], dev["v"], dev["o"], dev["do"], dev["lse"], dq, dk, dv,
                                case["scale"], "causal" if causal else "full", sched, 1, ws)
        assert st == dash.DASH_OK
        torch.cuda.synchronize()
        assert dash.dash_last_kernel_error() == dash.DASH_OK
        assert max(rel_errs((dq, dk, dv), oracle_grads(case))) <= TOL


# The benchmark shapes: (name, B, H, Hkv, N, d, causal, sampled (b, h), causal row prefix)
FULL = [
    ("full-d128-N2048", 8, 16, 16, 2048, 128, False, [(0, 0), (7, 15)], None),
    ("causal-d64-N4096", 4, 32, 32, 4096, 64, True, [(0, 0), (3, 31)], 1024),
    ("causal-d128-N16384", 1, 16, 16, 16384, 128, True, [(0, 5)], 1024),
    ("gqa-causal-d128-N8192", 1, 32, 8, 8192, 128, True, [(0, 0), (0, 31)], 1024),
]


@pytest.mark.parametrize("cfg", FULL, ids=[c[0] for c in FULL])
def test_forward_full_configs_sampled(cfg):
    name, B, H, Hkv, N, d, causal, heads, prefix = cfg
    print(f"[fwd] {name}", flush=True)
    bits = inputs.make_qkvdo(B, H, Hkv, N, d, 1000 + [c[0] for c in FULL].index(name) + 1)
    dev = {x: torch.from_numpy(bits[x].view(np.int16)).view(torch.bfloat16).cuda() for x in "qkv"}
    o, lse = _fwd(dev, d, causal)
    o_h = o.float().cpu().numpy()
    lse_h = lse.cpu().numpy()
    G = H // Hkv
    for b, h in heads:
        rows = N if prefix is None else prefix
        f = {x: inputs.bf16_bits_to_f32(bits[x]).astype(np.float64) for x in "qkv"}
        q1 = f["q"][b:b + 1, h:h + 1, :rows]
        k1 = f["k"][b:b + 1, h // G:h // G + 1, :rows if causal else N]
        v1 = f["v"][b:b + 1, h // G:h // G + 1, :rows if causal else N]
        if not causal:
            # Full mask: every row sees every key; the oracle takes all N keys.
            o_ref, lse_ref = oa.forward(q1, k1, v1, False, 1.0 / math.sqrt(d))
        else:
            # Causal: rows 0 .. rows - 1 see only keys 0 .. rows - 1.
            o_ref, lse_ref = oa.forward(q1, k1, v1, True, 1.0 / math.sqrt(d))
        got = o_h[b, h, :rows]
        assert np.abs(got - o_ref[0, 0]).max() / np.abs(o_ref).max() <= TOL, (b, h)
        assert np.abs(lse_h[b, h, :rows].astype(np.float64) - lse_ref[0, 0]).max() <= LSE_TOL, (b, h)
