"""GPU: a seeded sweep of random shapes and options against the oracle.

Each case draws its sizes (b, L, d_in, n; the map sizes of the cross scan),
the input type and the options (gate, bias, softplus, zero-order hold,
initial state, final-state gradient, forced L segments) from its own seed, so
a failure names a case that can be run again as it is.  Sizes stay small enough for the oracle to finish at once;
they are chosen around the tile edges (chunks of 8 and 16 steps, groups of 64
channels, 2, 4 and 8 states per recurrence wave).  Tolerances as everywhere:
max relative error 1e-4 for fp32 inputs, 2e-2 for bf16 inputs.
"""
import random

import pytest
import torch

import oracle
from tests.parity import assert_close
from tests.test_gpu_bwd import compare, grads_gpu, grads_oracle
from tests.test_gpu_cross import check as cross_check, cross_inputs
from tests.test_gpu_parity import BF16, DEV, F32, plan, say, small_inputs, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

LENGTHS = [1, 2, 7, 8, 9, 15, 16, 17, 33, 64, 100, 129, 250]
CHANNELS = [1, 3, 31, 63, 64, 65, 96, 130, 200]
STATES = [1, 2, 3, 5, 8, 9, 15, 16, 17, 24, 32, 33, 48, 64]


@pytest.fixture(scope="module")
def ss():
    import selective_state_space_softplus_amd as ss

    return ss


def draw(seed):
    r = random.Random(seed)
    return dict(b=r.randint(1, 3), L=r.choice(LENGTHS), d_in=r.choice(CHANNELS), n=r.choice(STATES),
                dtype=r.choice([F32, BF16]), gated=r.random() < 0.6, bias=r.random() < 0.6,
                softplus=r.random() < 0.8, zoh=r.random() < 0.3, h0=r.random() < 0.3, dlast=r.random() < 0.3,
                segments=r.choice([None, None, 1, 2, 3, 5]))


def inputs(c, seed):
    inp = small_inputs(c["b"], c["L"], c["d_in"], c["n"], c["dtype"], c["gated"], c["bias"], c["softplus"], seed)
    g = torch.Generator().manual_seed(seed + 1)
    h0 = torch.randn(c["b"], c["d_in"], c["n"], generator=g) * 0.5 if c["h0"] else None
    return inp, h0


def dev(t):
    return None if t is None else t.to(DEV)


@pytest.mark.parametrize("seed", range(3000, 3400))
def test_scan_sweep(ss, seed):
    c = draw(seed)
    say(f"scan sweep seed={seed} {c}")
    inp, h0 = inputs(c, seed)
    g = to_dev(inp)
    with plan(segments=c["segments"]):
        y, last = ss.scan_fwd(g["u"], g["delta"], g["A_log"], g["B"], g["C"], g["D"], g["z"], g["delta_bias"],
                              g["delta_softplus"], return_last_state=True, initial_state=dev(h0), zoh=c["zoh"])
        torch.cuda.synchronize()
    yr, lr = oracle.scan(inp["u"], inp["delta"], inp["A_log"], inp["B"], inp["C"], inp["D"], inp["z"],
                         inp["delta_bias"], inp["delta_softplus"], h0=h0, zoh=c["zoh"])
    assert_close(y, yr, c["dtype"], f"seed {seed} y")
    assert_close(last, lr, c["dtype"], f"seed {seed} last_state")


@pytest.mark.parametrize("seed", range(4000, 4400))
def test_bwd_sweep(ss, seed):
    c = draw(seed)
    say(f"bwd sweep seed={seed} {c}")
    inp, h0 = inputs(c, seed)
    g = torch.Generator().manual_seed(seed + 2)
    dy = torch.randn(c["b"], c["L"], c["d_in"], generator=g).to(c["dtype"])
    dl = torch.randn(c["b"], c["d_in"], c["n"], generator=g) if c["dlast"] else None
    with plan(segments=c["segments"]):
        got = grads_gpu(ss, to_dev(inp), dy.to(DEV), dev(h0), dev(dl), zoh=c["zoh"])
    ref = grads_oracle(inp, dy, h0, dl, zoh=c["zoh"])
    compare(got, ref, c["dtype"], f"seed {seed}")


@pytest.mark.parametrize("seed", range(5000, 5060))
def test_step_sweep(ss, seed):
    r = random.Random(seed)
    b, d_in, n = r.randint(1, 70), r.choice(CHANNELS), r.choice(STATES)
    dtype, gated, bias, zoh = r.choice([F32, BF16]), r.random() < 0.6, r.random() < 0.6, r.random() < 0.3
    say(f"step sweep seed={seed} b={b} d_in={d_in} n={n} {dtype} gated={gated} bias={bias} zoh={zoh}")
    g = torch.Generator().manual_seed(seed)
    rn = lambda *s: torch.randn(*s, generator=g)  # noqa: E731
    state = rn(b, d_in, n) * 0.5
    x, dt, z = rn(b, d_in).to(dtype), (rn(b, d_in) - 1).to(dtype), rn(b, d_in).to(dtype)
    Bm, Cm = rn(b, n).to(dtype), rn(b, n).to(dtype)
    A_log, D = torch.rand(d_in, n, generator=g) * 2 - 1, rn(d_in)
    bb = (torch.rand(d_in, generator=g) - 0.5) if bias else None
    zz = z if gated else None
    sg = state.to(DEV)
    y = ss.state_update(sg, dev(x), dev(dt), dev(A_log), dev(Bm), dev(Cm), dev(D), dev(zz), dev(bb), True, zoh=zoh)
    torch.cuda.synchronize()
    sr, yr = oracle.state_update(state, x, dt, A_log, Bm, Cm, D, zz, bb, True, zoh=zoh)
    assert_close(y, yr, dtype, f"seed {seed} step y")
    assert_close(sg, sr, dtype, f"seed {seed} step state")


@pytest.mark.parametrize("seed", range(6000, 6060))
def test_cross_sweep(ss, seed):
    r = random.Random(seed)
    maps = r.randint(1, 3)
    # Mostly small maps; one case in four up to 70 x 70, beyond what the one-kernel form holds in LDS.
    H, W = (r.randint(1, 70), r.randint(1, 70)) if r.random() < 0.25 else (r.randint(1, 12), r.randint(1, 12))
    n = r.choice([1, 1, 2, 3, 4] + STATES[:8])
    d_in = r.choice(CHANNELS) if H * W * n < 2000 else r.choice(CHANNELS[:5])
    dtype, bias, form = r.choice([F32, BF16]), r.random() < 0.6, r.choice(["auto", "one_pass", "one_pass"])
    say(f"cross sweep seed={seed} maps={maps} {H}x{W} d_in={d_in} n={n} {dtype} bias={bias} form={form}")
    cross_check(ss, cross_inputs(maps, H, W, d_in, n, dtype, seed, bias=bias), f"seed {seed}", form=form)
