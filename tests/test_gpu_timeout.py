"""The error path of the kernels' bounded waits, forced from the host.

With the wait bound set to zero (dash_set_wait_timeout(0): a wait gives up after a few
dozen polls), a deterministic call whose dQ chains must wait (naive schedule, 32 KV tiles
per head: the last contributor of a Q tile waits for 31 reductions) records
DASH_ERR_TIMEOUT in its workspace's error word; every kernel still drains (each wait in
the kernels is bounded by the same timeout or ends when another wave has reported an
error). The error word belongs to the call: the next call clears it in stream order, so
a later call with the default bound is correct even when nobody read the error of the
failed one, and reports no error of its own.
"""
import pytest

from gpu_helpers import make_case, oracle_grads, rel_errs, run, to_device

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

TOL = 1e-2
DEFAULT_US = 5_000_000


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("mask", ["full", "causal"])
@pytest.mark.parametrize("kernel", ["two_waves", "one_wave"])
def test_timeout_is_reported_and_the_next_call_is_correct(kernel, mask, d):
    """Full mask, two-waves kernel: the main kernel writes dQ itself and a one-thread kernel
    copies the status word; the other cases end with the dQ cast, which copies it. At
    d = 64 the two-waves kernel's A waves own the dQ blocks (and their waits)."""
    from scheduling_fa_attn_amd import dash
    case = make_case(1, 2, 2, 4096, d, mask == "causal", seed=97)
    dev = to_device(case)
    ref = oracle_grads(case)
    assert dash.dash_set_kernel(kernel) == dash.DASH_OK
    try:
        assert dash.dash_last_kernel_error() == dash.DASH_OK
        print(f"kernel={kernel} mask={mask} d={d}: wait bound 0, naive schedule", flush=True)
        assert dash.dash_set_wait_timeout(0) == dash.DASH_OK
        try:
            with pytest.raises(dash.DashError) as e:
                run(case, dev, "naive", 1)
            assert e.value.status == dash.DASH_ERR_TIMEOUT
            # A second failing call whose error nobody reads.
            B, H, Hkv, N, d = case["shape"]
            ws = torch.empty(dash.dash_attn_bwd_workspace_size(B, H, Hkv, N, d), dtype=torch.uint8, device="cuda")
            outs = [torch.empty_like(dev[k]) for k in ("q", "k", "v")]
            st = dash.dash_attn_bwd(dev["q"], dev["k"], dev["v"], dev["o"], dev["do"], dev["lse"], *outs,
                                    case["scale"], mask, "naive", 1, ws)
            assert st == dash.DASH_OK
        finally:
            assert dash.dash_set_wait_timeout(DEFAULT_US) == dash.DASH_OK
        print(f"kernel={kernel}: default bound, same workspace, error of the failed call never read", flush=True)
        st = dash.dash_attn_bwd(dev["q"], dev["k"], dev["v"], dev["o"], dev["do"], dev["lse"], *outs,
                                case["scale"], mask, "naive", 1, ws)
        assert st == dash.DASH_OK
        torch.cuda.synchronize()
        errs = rel_errs(outs, ref)
        assert max(errs) <= TOL, errs
        assert dash.dash_last_kernel_error() == dash.DASH_OK
        print(f"kernel={kernel}: default bound, fresh workspace", flush=True)
        out, _ = run(case, dev, "naive", 1)
        assert dash.dash_last_kernel_error() == dash.DASH_OK
        errs = rel_errs(out, ref)
        assert max(errs) <= TOL, errs
    finally:
        dash.dash_set_kernel("auto")
        dash.dash_set_wait_timeout(DEFAULT_US)
