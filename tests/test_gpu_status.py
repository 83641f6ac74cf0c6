"""GPU: the status word of a segmented scan (ss_scan_status).

A wait between segments of L cannot deadlock, so a real timeout cannot be
provoked; the test plan instead makes every wait poll a word nothing sets,
with a short poll limit, so each wait gives up at once and every kernel still
runs to its end.  The call must then report SS_ERR_TIMEOUT (and NaN outputs
after the first segment), and the next ordinary call must report SS_OK.
"""
import pytest
import torch

import workloads
from tests.test_gpu_parity import BF16, DEV, F32, plan, say, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def ss():
    import selective_state_space_softplus_amd as ss

    return ss


def _scan(ss, g, **kw):
    return ss.scan_fwd(g["u"], g["delta"], g["A_log"], g["B"], g["C"], g["D"], g["z"], g["delta_bias"], True,
                       return_last_state=True, **kw)


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_forced_timeout_is_reported_then_cleared(ss, dtype):
    say(f"forced segment-wait timeout, forward {dtype}")
    g = to_dev(workloads.random_scan_inputs(2, 1000, 100, 16, dtype, seed=5, gated=True, bias=True))
    ws = torch.empty(ss.scan_fwd_workspace_bytes(2, 1000, 100, 16, 1 if dtype == BF16 else 0), dtype=torch.uint8,
                     device=DEV)
    y_ok, _ = _scan(ss, g, workspace=ws)
    assert ss.scan_status(ws) == 0
    with plan(segments=4):
        y_seg, _ = _scan(ss, g, workspace=ws)
        assert ss.scan_status(ws) == 0
        assert torch.equal(y_seg, y_ok)          # exact hand-off: segments change nothing
    with ss.test_plan(segments=4, spin_limit=20, wait_never=1):
        y_bad, last_bad = _scan(ss, g, workspace=ws)
        assert ss.scan_status(ws) == ss.SS_ERR_TIMEOUT
        with pytest.raises(ss.SSError) as e:
            _scan(ss, g, workspace=ws, check=True)
        assert e.value.code == ss.SS_ERR_TIMEOUT
    torch.cuda.synchronize()
    assert torch.isnan(last_bad).all()
    first = y_bad[:, :250].float()
    assert torch.isfinite(first).all()           # the first segment never waits
    assert torch.isnan(y_bad[:, -1].float()).all()
    y_again, _ = _scan(ss, g, workspace=ws, check=True)   # cleared by the next call
    assert ss.scan_status(ws) == 0
    assert torch.equal(y_again, y_ok)


def test_forced_timeout_backward_and_cross(ss):
    say("forced segment-wait timeout, backward and cross scan")
    g = to_dev(workloads.random_scan_inputs(2, 640, 64, 4, F32, seed=6, gated=True, bias=True))
    dy = torch.randn_like(g["u"])
    ok = ss.scan_bwd(g["u"], g["delta"], g["A_log"], g["B"], g["C"], g["D"], dy, g["z"], g["delta_bias"], True,
                     check=True)
    with ss.test_plan(segments=3, spin_limit=20, wait_never=1):
        with pytest.raises(ss.SSError) as e:
            ss.scan_bwd(g["u"], g["delta"], g["A_log"], g["B"], g["C"], g["D"], dy, g["z"], g["delta_bias"], True,
                        check=True)
        assert e.value.code == ss.SS_ERR_TIMEOUT
    again = ss.scan_bwd(g["u"], g["delta"], g["A_log"], g["B"], g["C"], g["D"], dy, g["z"], g["delta_bias"], True,
                        check=True)
    for k in ok:
        assert torch.equal(ok[k], again[k]), k

    c = to_dev(workloads.cross_scan_inputs(3, seed=9))
    args = (c["x"][:2].contiguous(), c["delta"][:2].contiguous(), c["A_log"], c["B"][:2].contiguous(),
            c["C"][:2].contiguous(), c["D"], c["delta_bias"], True)
    y_ok = ss.cross_scan_fwd(*args, check=True)
    with ss.test_plan(segments=4, spin_limit=20, wait_never=1):
        with pytest.raises(ss.SSError) as e:
            ss.cross_scan_fwd(*args, check=True)
        assert e.value.code == ss.SS_ERR_TIMEOUT
    assert torch.equal(ss.cross_scan_fwd(*args, check=True), y_ok)


def test_one_pass_cross_clears_a_stale_status(ss):
    """The one-pass cross scan waits on nothing, so it clears the status words a timed-out call left."""
    say("one-pass cross scan after a forced timeout in the same workspace")
    c = to_dev(workloads.cross_scan_inputs(3, seed=9))
    args = (c["x"][:2].contiguous(), c["delta"][:2].contiguous(), c["A_log"], c["B"][:2].contiguous(),
            c["C"][:2].contiguous(), c["D"], c["delta_bias"], True)
    maps, H, W, d_in = args[0].shape
    ws = torch.empty(ss.lib.ss_cross_scan_fwd_ex_workspace_bytes(maps, H, W, d_in, 1, 0, 2), dtype=torch.uint8,
                     device=DEV)
    with ss.test_plan(segments=4, spin_limit=20, wait_never=1):
        ss.cross_scan_fwd(*args, workspace=ws, form="two_pass")
        assert ss.scan_status(ws) == ss.SS_ERR_TIMEOUT
    y1 = ss.cross_scan_fwd(*args, workspace=ws, form="one_pass", check=True)
    assert ss.scan_status(ws) == 0
    assert torch.equal(y1, ss.cross_scan_fwd(*args, form="one_pass"))
