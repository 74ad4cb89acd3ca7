"""The error path of the kernels' bounded waits, forced from the host.

With the wait bound set to zero (dash_set_wait_timeout(0): a wait gives up after a few
dozen polls), a deterministic call whose dQ chains must wait (naive schedule, 32 KV tiles
per head: the last contributor of a Q tile waits for 31 reductions) records
DASH_ERR_TIMEOUT; every kernel still drains (each wait in the kernels is bounded by the
same timeout or ends when another wave has reported an error). The next call with the
default bound reports no error and matches the fp64 oracle.
"""
import pytest

from gpu_helpers import make_case, oracle_grads, rel_errs, run, to_device

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

TOL = 1e-2
DEFAULT_US = 5_000_000


@pytest.mark.parametrize("kernel", ["two_waves", "one_wave"])
def test_timeout_is_reported_and_the_next_call_is_correct(kernel):
    from scheduling_fa_attn_amd import dash
    case = make_case(1, 2, 2, 4096, 128, False, seed=97)
    dev = to_device(case)
    assert dash.dash_set_kernel(kernel) == dash.DASH_OK
    try:
        assert dash.dash_last_kernel_error() == dash.DASH_OK
        print(f"kernel={kernel}: wait bound 0, naive schedule", flush=True)
        assert dash.dash_set_wait_timeout(0) == dash.DASH_OK
        try:
            with pytest.raises(dash.DashError) as e:
                run(case, dev, "naive", 1)
            assert e.value.status == dash.DASH_ERR_TIMEOUT
        finally:
            assert dash.dash_set_wait_timeout(DEFAULT_US) == dash.DASH_OK
        print(f"kernel={kernel}: default bound", flush=True)
        out, _ = run(case, dev, "naive", 1)
        assert dash.dash_last_kernel_error() == dash.DASH_OK
        errs = rel_errs(out, oracle_grads(case))
        assert max(errs) <= TOL, errs
    finally:
        dash.dash_set_kernel("auto")
        dash.dash_set_wait_timeout(DEFAULT_US)
