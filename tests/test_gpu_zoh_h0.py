"""GPU: the zero-order-hold input term and the scan's initial state, against the oracle.

The zero-order hold weights the input by (exp(delta' A) - 1) / A instead of
delta' (mhpn.cn selective_scan walk-through, section 6); the scan may start
from a given state h0 instead of zero (section 4 starts it from zeros).  Both
go through ss_scan_fwd_ex / ss_state_update_ex.  Tolerances are those of the
other parity tests: max relative error 1e-4 for fp32 inputs, 2e-2 for bf16.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity import assert_close, rel_err
from tests.test_gpu_parity import BF16, DEV, F32, plan, say, small_inputs, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def ss():
    import selective_state_space_softplus_amd as ss

    return ss


def gpu_scan(ss, g, h0=None, zoh=False, last=True):
    return ss.scan_fwd(g["u"], g["delta"], g["A_log"], g["B"], g["C"], g["D"], g["z"], g["delta_bias"],
                       g["delta_softplus"], return_last_state=last, initial_state=h0, zoh=zoh)


def oracle_scan(inp, h0=None, zoh=False):
    return oracle.scan(inp["u"], inp["delta"], inp["A_log"], inp["B"], inp["C"], inp["D"], inp["z"],
                       inp["delta_bias"], inp["delta_softplus"], h0=h0, zoh=zoh)


def initial_state(b, d_in, n, seed):
    return torch.randn(b, d_in, n, generator=torch.Generator().manual_seed(seed)) * 0.5


def check(ss, inp, h0, zoh, what):
    g = to_dev(inp)
    y, last = gpu_scan(ss, g, None if h0 is None else h0.to(DEV), zoh)
    torch.cuda.synchronize()
    yr, lr = oracle_scan(inp, h0, zoh)
    e1 = assert_close(y, yr, inp["dtype"], f"{what} y")
    e2 = assert_close(last, lr, inp["dtype"], f"{what} last_state")
    return e1, e2


CASES = [
    # b, L, d_in, n, dtype, gated, bias, softplus
    (2, 300, 130, 16, F32, True, True, True),
    (2, 300, 130, 16, BF16, True, True, True),
    (1, 1, 1, 16, F32, True, True, True),
    (1, 97, 65, 16, F32, True, True, False),
    (2, 200, 40, 1, F32, False, False, True),
    (1, 129, 70, 2, BF16, True, True, True),
    (2, 90, 24, 3, F32, True, True, True),
    (1, 70, 66, 8, BF16, False, True, True),
    (1, 70, 66, 17, F32, True, True, True),
    (2, 61, 42, 40, F32, True, False, True),
    (1, 70, 40, 64, BF16, True, True, True),
]


def _id(c):
    return "b{}_L{}_d{}_n{}_{}_{}{}{}".format(c[0], c[1], c[2], c[3], "f32" if c[4] == F32 else "bf16",
                                               "g" if c[5] else "", "b" if c[6] else "", "s" if c[7] else "")


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
@pytest.mark.parametrize("mode", ["zoh", "h0", "zoh+h0"])
def test_scan_small(ss, case, mode):
    say(f"scan {mode} {case}")
    inp = small_inputs(*case, seed=sum(case[:4]) + 1)
    h0 = initial_state(case[0], case[2], case[3], seed=sum(case[:4])) if "h0" in mode else None
    check(ss, inp, h0, "zoh" in mode, f"{mode} {case}")


@pytest.mark.parametrize("segments,n,L", [(3, 16, 300), (16, 16, 1000), (5, 1, 700), (7, 64, 450)])
@pytest.mark.parametrize("zoh", [False, True])
def test_scan_segments(ss, segments, n, L, zoh):
    """Pieces of the sequence run by different workgroups hand the state on; h0 enters the first."""
    say(f"segments={segments} n={n} L={L} zoh={zoh}")
    inp = workloads.random_scan_inputs(2, L, 100, n, F32, seed=70 + n + L, gated=True, bias=True)
    h0 = initial_state(2, 100, n, seed=n + L)
    with plan(segments=segments):
        check(ss, inp, h0, zoh, f"segments={segments} zoh={zoh}")


@pytest.mark.parametrize("n,dtype", [(16, F32), (16, BF16), (1, F32), (40, F32)])
@pytest.mark.parametrize("zoh", [False, True])
def test_split_scan_in_place_equals_whole(ss, n, dtype, zoh):
    """Scanning the first part, then the rest from its last_state (in place), gives the whole scan."""
    say(f"split scan n={n} {dtype} zoh={zoh}")
    L, L1 = 500, 173
    g = to_dev(workloads.random_scan_inputs(2, L, 90, n, dtype, seed=11 + n, gated=True, bias=True))
    y, last = gpu_scan(ss, g, zoh=zoh)
    part = lambda t0, t1: {k: (v[:, t0:t1].contiguous() if isinstance(v, torch.Tensor) and v.dim() == 3 else v)  # noqa: E731
                           for k, v in g.items()}
    y1, st = gpu_scan(ss, part(0, L1), zoh=zoh)
    p2 = part(L1, L)
    y2 = ss.scan_fwd(p2["u"], p2["delta"], p2["A_log"], p2["B"], p2["C"], p2["D"], p2["z"], p2["delta_bias"], True,
                     return_last_state=True, last_state=st, initial_state=st, zoh=zoh)[0]
    torch.cuda.synchronize()
    tol = 1e-5 if dtype == F32 else 1e-2
    assert rel_err(y1, y[:, :L1]) == 0.0
    assert rel_err(y2, y[:, L1:]) <= tol
    assert rel_err(st, last) <= 1e-5


@pytest.mark.parametrize("b,d_in,n,dtype,gated,bias", [
    (3, 33, 16, F32, True, True), (3, 33, 16, BF16, True, True), (1, 1, 1, F32, False, False),
    (2, 10, 3, F32, True, True), (2, 10, 8, F32, False, True), (2, 10, 64, BF16, True, True),
    (2, 10, 48, F32, True, True),
])
def test_step_zoh(ss, b, d_in, n, dtype, gated, bias):
    say(f"step zoh b={b} d_in={d_in} n={n} {dtype}")
    r = torch.Generator().manual_seed(b * 1000 + d_in * 10 + n + 5)
    rn = lambda *s: torch.randn(*s, generator=r)  # noqa: E731
    state = rn(b, d_in, n) * 0.5
    x, dt, z = rn(b, d_in).to(dtype), (rn(b, d_in) - 1).to(dtype), rn(b, d_in).to(dtype)
    Bm, Cm = rn(b, n).to(dtype), rn(b, n).to(dtype)
    A_log, D = torch.rand(d_in, n) * 4 - 2, rn(d_in)
    bb = (torch.rand(d_in) - 0.5) if bias else None
    zz = z if gated else None
    sg = state.to(DEV)
    dev = lambda t: None if t is None else t.to(DEV)  # noqa: E731
    y = ss.state_update(sg, dev(x), dev(dt), dev(A_log), dev(Bm), dev(Cm), dev(D), dev(zz), dev(bb), True, zoh=True)
    torch.cuda.synchronize()
    sr, yr = oracle.state_update(state, x, dt, A_log, Bm, Cm, D, zz, bb, True, zoh=True)
    assert_close(y, yr, dtype, "zoh step y")
    assert_close(sg, sr, dtype, "zoh step state")


def test_scan_L1_from_h0_equals_step(ss):
    """One ZOH scan step from h0 is one ZOH decode step on that state."""
    say("scan L=1 from h0 vs zoh step")
    g = to_dev(workloads.random_scan_inputs(3, 1, 70, 16, F32, seed=13, gated=True, bias=True))
    h0 = initial_state(3, 70, 16, seed=14).to(DEV)
    y, last = gpu_scan(ss, g, h0=h0, zoh=True)
    state = h0.clone()
    ys = ss.state_update(state, g["u"][:, 0], g["delta"][:, 0], g["A_log"], g["B"][:, 0], g["C"][:, 0], g["D"],
                         g["z"][:, 0], g["delta_bias"], True, zoh=True)
    assert rel_err(ys, y[:, 0]) < 1e-6
    assert rel_err(state, last) < 1e-6


def test_zoh_weight_across_its_two_forms(ss):
    """Step sizes and decay rates chosen so that delta' A sweeps from -1e-6 to -60.

    The kernels take the weight from a series where |delta' A| log2(e) < 1/2
    and from (exp(delta' A) - 1) / A elsewhere; the sweep crosses that border and
    reaches exp(delta' A) far below fp32's smallest normal number.  A single
    state with u = B = C = 1, D = 0 and a zero initial state makes the first
    output the weight itself.
    """
    say("zoh weight sweep")
    x = torch.cat([-torch.logspace(-6, np.log10(60.0), 400, dtype=torch.float64),
                   torch.tensor([-0.34657359, -0.3465736, -0.34657361, -0.5, -87.0, -88.0, -104.0, -120.0],
                                dtype=torch.float64)])
    m = x.numel()
    dl = torch.full((m,), 0.5, dtype=torch.float64)
    A = x / dl                                           # A = delta' A / delta'
    A_log = torch.log(-A).float()
    u = torch.ones(1, 1, m)
    y = ss.scan_fwd(u.to(DEV), dl.float().view(1, 1, m).to(DEV), A_log.view(m, 1).to(DEV),
                    torch.ones(1, 1, 1, device=DEV), torch.ones(1, 1, 1, device=DEV), torch.zeros(m, device=DEV),
                    None, None, False, zoh=True)
    got = y.double().cpu().numpy()[0, 0]
    A32 = -np.exp(A_log.double().numpy())                # the A the kernel sees, from the fp32 A_log
    ref = np.expm1(0.5 * A32) / A32
    rel = np.max(np.abs(got - ref) / np.abs(ref))
    assert rel < 2e-6, f"zoh weight max rel err {rel:.3g}"


@pytest.mark.parametrize("index", [1, 2])
def test_workload_zoh_and_h0_full(ss, index):
    """The mid and long workloads with the zero-order hold and an initial state: every element."""
    cfg = workloads.CONFIGS[index]
    say(f"{cfg.name} full size, zoh + h0, every element")
    inp = workloads.scan_inputs(index)
    inp["h0"] = initial_state(cfg.b, cfg.d_in, cfg.n, seed=index)
    g = to_dev(inp)
    y, last = gpu_scan(ss, g, h0=g["h0"], zoh=True)
    torch.cuda.synchronize()
    y, last = y.cpu(), last.cpu()
    del g
    yr, lr = oracle.scan(inp["u"], inp["delta"], inp["A_log"], inp["B"], inp["C"], inp["D"], inp["z"],
                         inp["delta_bias"], True, lib=oracle.load_parallel(), h0=inp["h0"], zoh=True)
    e1 = assert_close(y, yr, cfg.dtype, f"{cfg.name} zoh y")
    e2 = assert_close(last, lr, cfg.dtype, f"{cfg.name} zoh last_state")
    print(f"{cfg.name} zoh+h0: y err {e1:.3g}, last_state err {e2:.3g} over all {y.numel()} outputs")


def test_empty_scan_keeps_initial_state(ss):
    say("empty scan with h0")
    u = torch.zeros(2, 0, 5, device=DEV)
    h0 = torch.randn(2, 5, 3, device=DEV)
    y, last = ss.scan_fwd(u, u, torch.zeros(5, 3, device=DEV), torch.zeros(2, 0, 3, device=DEV),
                          torch.zeros(2, 0, 3, device=DEV), torch.zeros(5, device=DEV), return_last_state=True,
                          initial_state=h0)
    assert torch.equal(last, h0)
