"""GPU: the scan and its gradient captured in HIP graphs.

Both calls cut L into segments here (forced), so a replay runs the kernel that
clears the segment flags, the workgroups' ticket counter and the state (or
adjoint) hand-off between segments -- all in kernels, with no memset node in
the graph.  Between replays the program runs other eager work on the same
library; every replay must reproduce the eager results bit for bit (the
kernels are deterministic).
"""
import pytest
import torch

import workloads
from tests.test_gpu_parity import BF16, DEV, plan, say, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def ss():
    import selective_state_space_softplus_amd as ss

    return ss


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                                     # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = fn()
    return graph, out


@pytest.mark.parametrize("zoh", [False, True])
def test_scan_fwd_graph_replays(ss, zoh):
    say(f"scan_fwd in a HIP graph, zoh={zoh}")
    g = to_dev(workloads.random_scan_inputs(2, 3000, 256, 16, BF16, seed=31, gated=True, bias=True))
    other = to_dev(workloads.random_scan_inputs(1, 500, 128, 16, BF16, seed=32, gated=True, bias=True))
    args = (g["u"], g["delta"], g["A_log"], g["B"], g["C"], g["D"], g["z"], g["delta_bias"], True)
    with plan(segments=4):
        y_e, last_e = ss.scan_fwd(*args, return_last_state=True, zoh=zoh)
        y_g, last_g = torch.empty_like(y_e), torch.empty_like(last_e)
        ws = torch.empty(ss.scan_fwd_workspace_bytes(2, 3000, 256, 16, 1), dtype=torch.uint8, device=DEV)
        graph, _ = _capture(lambda: ss.scan_fwd(*args, return_last_state=True, out=y_g, last_state=last_g,
                                                workspace=ws, zoh=zoh))
        for rep in range(3):
            y_g.zero_()
            last_g.zero_()
            ss.scan_fwd(other["u"], other["delta"], other["A_log"], other["B"], other["C"], other["D"], other["z"],
                        other["delta_bias"], True, zoh=zoh)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(y_g, y_e) and torch.equal(last_g, last_e), f"replay {rep}"


@pytest.mark.parametrize("zoh", [False, True])
def test_scan_bwd_graph_replays(ss, zoh):
    say(f"scan_bwd in a HIP graph, zoh={zoh}")
    g = to_dev(workloads.random_scan_inputs(2, 2000, 192, 16, BF16, seed=33, gated=True, bias=True))
    dy = torch.randn(2, 2000, 192, device=DEV, generator=torch.Generator(device=DEV).manual_seed(34)).to(BF16)
    args = (g["u"], g["delta"], g["A_log"], g["B"], g["C"], g["D"], dy, g["z"], g["delta_bias"], True)
    with plan(segments=3):
        ref = ss.scan_bwd(*args, zoh=zoh)
        ws = torch.empty(ss.lib.ss_scan_bwd_workspace_bytes(2, 2000, 192, 16, 1), dtype=torch.uint8, device=DEV)
        graph, got = _capture(lambda: ss.scan_bwd(*args, workspace=ws, zoh=zoh))
        for rep in range(3):
            for v in got.values():
                v.zero_()
            ss.scan_bwd(*args[:6], dy.flip(1).contiguous(), *args[7:], zoh=zoh)    # other eager work
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for k in ref:
                assert torch.equal(got[k], ref[k]), f"{k}, replay {rep}"


@pytest.mark.parametrize("form", ["two_pass", "one_pass"])
def test_cross_scan_graph_replays(ss, form):
    say(f"cross scan in a HIP graph, form={form}")
    c = to_dev(workloads.cross_scan_inputs(3, seed=41))
    args = (c["x"][:3].contiguous(), c["delta"][:3].contiguous(), c["A_log"], c["B"][:3].contiguous(),
            c["C"][:3].contiguous(), c["D"], c["delta_bias"], True)
    other = (c["x"][3:5].contiguous(), c["delta"][3:5].contiguous(), c["A_log"], c["B"][3:5].contiguous(),
             c["C"][3:5].contiguous(), c["D"], c["delta_bias"], True)
    maps, H, W, d_in = args[0].shape
    with plan(segments=3):
        y_e, last_e = ss.cross_scan_fwd(*args, return_last_state=True, form=form)
        y_g, last_g = torch.empty_like(y_e), torch.empty_like(last_e)
        code = {"two_pass": 2, "one_pass": 1}[form]
        ws = torch.empty(ss.lib.ss_cross_scan_fwd_ex_workspace_bytes(maps, H, W, d_in, 1, 0, code),
                         dtype=torch.uint8, device=DEV)
        graph, _ = _capture(lambda: ss.cross_scan_fwd(*args, return_last_state=True, out=y_g, last_state=last_g,
                                                      workspace=ws, form=form))
        for rep in range(3):
            y_g.zero_()
            last_g.zero_()
            ss.cross_scan_fwd(*other, form=form)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(y_g, y_e) and torch.equal(last_g, last_e), f"replay {rep}"
