"""GPU: the convolution step of a decode step (ss_conv_update) against the oracle.

The step is Mamba.step's "Conv step" on the jiafeimiao.top page: the window of
the last W inputs per channel moves by one, the new input enters last, and the
output is silu(window . weight + bias).  The window is data movement only, so
it must equal the oracle's bit for bit; the output is compared at the parity
tolerances (max relative error 1e-4 for fp32 inputs, 2e-2 for bf16).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity import assert_close, to_f64
from tests.test_gpu_parity import BF16, DEV, F32, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def ss():
    import selective_state_space_softplus_amd as ss

    return ss


def shifted(t):
    """The same values one element further on: breaks 8- and 16-byte alignment."""
    buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
    v = buf[1:].view(t.shape)
    v.copy_(t)
    return v


def conv_inputs(b, d_in, W, dtype, seed, bias=True):
    r = torch.Generator().manual_seed(seed)
    return dict(state=torch.randn(b, d_in, W, generator=r).to(dtype), weight=torch.randn(d_in, W, generator=r) * 0.5,
                bias=torch.randn(d_in, generator=r) * 0.1 if bias else None)


@pytest.mark.parametrize("W", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("aligned", [True, False])
def test_conv_steps(ss, W, dtype, aligned):
    say(f"conv W={W} {dtype} aligned={aligned}")
    b, d_in, steps = 3, 70, 6
    inp = conv_inputs(b, d_in, W, dtype, seed=W * 10 + (dtype == BF16))
    xs = torch.randn(steps, b, d_in, generator=torch.Generator().manual_seed(5)).to(dtype)
    st = inp["state"].to(DEV)
    if not aligned:
        st = shifted(st)
    wd, bd = inp["weight"].to(DEV), inp["bias"].to(DEV)
    ref_state = inp["state"]
    for s in range(steps):
        silu = s % 2 == 0
        out = ss.conv_update(st, xs[s].to(DEV), wd, bd, silu=silu)
        torch.cuda.synchronize()
        ref_state, ref = oracle.conv_update(ref_state, xs[s], inp["weight"], inp["bias"], silu)
        assert np.array_equal(to_f64(st), ref_state), f"window after step {s}"
        assert_close(out, ref, dtype, f"conv out step {s}")


def test_conv_without_bias(ss):
    say("conv without bias")
    inp = conv_inputs(2, 33, 4, F32, seed=3, bias=False)
    x = torch.randn(2, 33)
    st = inp["state"].to(DEV)
    out = ss.conv_update(st, x.to(DEV), inp["weight"].to(DEV), None, silu=True)
    torch.cuda.synchronize()
    ref_state, ref = oracle.conv_update(inp["state"], x, inp["weight"], None, True)
    assert np.array_equal(to_f64(st), ref_state)
    assert_close(out, ref, F32, "conv out without bias")


def test_conv_decode_workload(ss):
    """The decode workload's shape (b=256, d_in=5120, W=4, bf16): every window exact, sampled outputs."""
    cfg = workloads.CONFIGS[4]
    say(f"conv step at {cfg.name} size")
    b, d_in, W = cfg.b, cfg.d_in, 4
    inp = conv_inputs(b, d_in, W, BF16, seed=11)
    x = torch.randn(b, d_in, generator=torch.Generator().manual_seed(12)).to(BF16)
    st = inp["state"].to(DEV)
    out = ss.conv_update(st, x.to(DEV), inp["weight"].to(DEV), inp["bias"].to(DEV), silu=True)
    torch.cuda.synchronize()
    want = torch.cat([inp["state"][:, :, 1:], x[:, :, None]], dim=2)
    assert torch.equal(st.cpu(), want), "rolled windows"
    rows = [0, 1, 100, 255]
    _, ref = oracle.conv_update(inp["state"][rows], x[rows], inp["weight"], inp["bias"], True)
    assert_close(out[rows], ref, BF16, "conv out (sampled rows)")


def test_decode_step_graph_replays(ss):
    """A decode step -- the conv step, then the SSM step on its output -- captured in a HIP graph.

    Between replays the program resets the states with its own eager copies;
    every replay must reproduce the eager results bit for bit.  (dt, B and C
    stand in for the projections of the conv output a full block computes.)
    """
    say("decode step in a HIP graph")
    b, d_in, n, W = 8, 96, 16, 4
    r = torch.Generator().manual_seed(21)
    rn = lambda *s: torch.randn(*s, generator=r).to(DEV)  # noqa: E731
    cs0, x = rn(b, d_in, W).to(BF16), rn(b, d_in).to(BF16)
    cw, cb = rn(d_in, W) * 0.5, rn(d_in) * 0.1
    s0 = rn(b, d_in, n) * 0.5
    dt, z = (rn(b, d_in) - 1).to(BF16), rn(b, d_in).to(BF16)
    Bm, Cm = rn(b, n).to(BF16), rn(b, n).to(BF16)
    A_log, D, dtb = torch.rand(d_in, n, generator=r).to(DEV), rn(d_in), rn(d_in) * 0.1

    def step(cs, s, xc, y):
        ss.conv_update(cs, x, cw, cb, silu=True, out=xc)
        ss.state_update(s, xc, dt, A_log, Bm, Cm, D, z, dtb, True, out=y)

    cs_e, s_e = cs0.clone(), s0.clone()
    xc_e, y_e = torch.empty_like(x), torch.empty_like(x)
    step(cs_e, s_e, xc_e, y_e)
    torch.cuda.synchronize()

    cs_g, s_g = cs0.clone(), s0.clone()
    xc_g, y_g = torch.empty_like(x), torch.empty_like(x)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(cs_g, s_g, xc_g, y_g)                     # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(cs_g, s_g, xc_g, y_g)
    for rep in range(3):
        cs_g.copy_(cs0)
        s_g.copy_(s0)
        y_g.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(cs_g, cs_e) and torch.equal(xc_g, xc_e), f"conv step, replay {rep}"
        assert torch.equal(s_g, s_e) and torch.equal(y_g, y_e), f"SSM step, replay {rep}"
