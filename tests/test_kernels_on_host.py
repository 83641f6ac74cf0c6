"""CPU: the library's own HIP sources run on the host (tests/host_kernels.py).

Every entry point here goes through the real C ABI code (validation, launch
planning, segments) and the real kernel source, compiled for the CPU against
a stand-in of the HIP device API with AddressSanitizer and
UndefinedBehaviorSanitizer: each tensor is an allocation of exactly its
size, and the bytes of LDS past a launch's dynamic size are poisoned, so a
load, store or direct-to-LDS copy outside its tensor or outside the
workgroup's LDS -- including one through a clamped index or a ring slot --
ends the run with a report.  Outputs are compared with the oracle at the
usual tolerances.  The cases cover every launch shape of the forward
(1x2, 4x2, 8x2, 4x4, 8x4, 8x8 states), both load forms (16-byte and element),
ragged L and d_in, segments along L, the zero-order hold, an initial state,
the backward pass, the decode step and the cross scan; among them is the
case (b=1, L=77, d_in=20, n=3, fp32, gated) that a one-wave shape of the
forward, no longer built, once faulted on.
"""
import shutil

import pytest
import torch

import oracle
import workloads
from tests import host_kernels as hk
from tests.parity import TOL, assert_close

F32, BF16 = torch.float32, torch.bfloat16

pytestmark = pytest.mark.skipif(not shutil.which(hk.CLANG) and not __import__("os").path.exists(hk.CLANG),
                                reason="needs the ROCm host clang")


def _code(dt):
    return 1 if dt == BF16 else 0


def fwd_case(b, L, d, n, dt, gated=True, bias=True, softplus=True, zoh=False, h0=False, segments=0, waves=0,
             seed=0, misalign=False, mode="fwd"):
    inp = workloads.random_scan_inputs(b, L, d, n, dt, seed=seed, gated=gated, bias=bias)
    if not softplus:
        # Without softplus the step size is delta + bias itself, so keep it positive.
        inp["delta"] = (inp["delta"].float().abs() * 0.1 + 0.01).to(dt)
        if inp["delta_bias"] is not None:
            inp["delta_bias"] = inp["delta_bias"].abs() * 0.01
    h = torch.randn(b, d, n, generator=torch.Generator().manual_seed(seed + 1)) * 0.5 if h0 else None
    t = dict(u=inp["u"], delta=inp["delta"], A_log=inp["A_log"], B=inp["B"], C=inp["C"], D=inp["D"], z=inp["z"],
             delta_bias=inp["delta_bias"], h0=h)
    args = dict(b=b, L=L, d_in=d, n=n, dtype=_code(dt), softplus=int(softplus), zoh=int(zoh), segments=segments,
                waves=waves)
    got = hk.run(mode, t, args, dict(y=((b, L, d), dt), last_state=((b, d, n), F32)))
    yr, lr = oracle.scan(inp["u"], inp["delta"], inp["A_log"], inp["B"], inp["C"], inp["D"], inp["z"],
                         inp["delta_bias"], softplus, h0=h, zoh=zoh)
    assert_close(got["y"], yr, dt, "host y")
    assert_close(got["last_state"], lr, dt, "host last_state")


FWD = [
    # b, L, d_in, n, dtype, options
    (1, 77, 20, 3, F32, {}),                            # the case the removed one-wave shape faulted on
    (2, 90, 24, 3, F32, {}),
    (1, 77, 20, 4, BF16, {}),
    (2, 61, 66, 8, BF16, dict(gated=False)),
    (2, 130, 96, 16, BF16, dict(segments=3)),           # 8 x 2 states, 16-byte loads, whole and ragged chunks
    (1, 100, 130, 16, F32, dict(segments=2, h0=True)),
    (2, 97, 64, 16, BF16, dict(waves=4)),               # 4 x 4 states
    (1, 70, 41, 16, BF16, {}),                          # element loads (d_in * 2 not a multiple of 16)
    (1, 70, 40, 32, F32, dict(zoh=True)),               # 8 x 4 states, zero-order hold
    (1, 64, 96, 32, F32, dict(zoh=True, segments=2)),
    (1, 45, 40, 64, BF16, {}),                          # 8 x 8 states
    (2, 33, 10, 1, F32, dict(softplus=False)),          # 1 x 2 states
    (1, 129, 70, 2, BF16, dict(h0=True, zoh=True)),
]


@pytest.mark.parametrize("case", FWD, ids=lambda c: f"b{c[0]}L{c[1]}d{c[2]}n{c[3]}{'bf16' if c[4] == BF16 else 'f32'}"
                         + "".join(f"-{k}{v}" for k, v in c[5].items()) if isinstance(c, tuple) else str(c))
def test_forward_on_host(case):
    b, L, d, n, dt, opt = case
    fwd_case(b, L, d, n, dt, seed=b + L + d + n, **opt)


def test_noalloc_on_host():
    fwd_case(2, 150, 70, 16, BF16, segments=4, seed=5, mode="noalloc")


# n above 16 is taken in slices of 16 states (n = 40: slices of 16, 16, 8).
@pytest.mark.parametrize("case", [(1, 64, 96, 32, F32, True), (2, 50, 70, 16, BF16, False), (1, 40, 64, 64, F32, False),
                                  (2, 37, 33, 40, BF16, True)],
                         ids=["n32-f32-zoh", "n16-bf16", "n64-f32", "n40-bf16-zoh"])
def test_backward_on_host(case):
    b, L, d, n, dt, zoh = case
    inp = workloads.random_scan_inputs(b, L, d, n, dt, seed=11, gated=True, bias=True)
    g = torch.Generator().manual_seed(12)
    dy = torch.randn(b, L, d, generator=g).to(dt)
    t = dict(u=inp["u"], delta=inp["delta"], A_log=inp["A_log"], B=inp["B"], C=inp["C"], D=inp["D"], z=inp["z"],
             delta_bias=inp["delta_bias"], dy=dy)
    args = dict(b=b, L=L, d_in=d, n=n, dtype=_code(dt), softplus=1, zoh=int(zoh), segments=2)
    outs = dict(du=((b, L, d), dt), ddelta=((b, L, d), dt), dA_log=((d, n), F32), dB=((b, L, n), dt),
                dC=((b, L, n), dt), dD=((d,), F32), dz=((b, L, d), dt), ddelta_bias=((d,), F32))
    got = hk.run("bwd", t, args, outs)
    ref = oracle.scan_bwd(inp["u"], inp["delta"], inp["A_log"], inp["B"], inp["C"], inp["D"], inp["z"],
                          inp["delta_bias"], True, None, dy, None, zoh=zoh)
    for k in outs:
        assert_close(got[k], ref[k], dt, f"host {k}")


# The training pair: the saving forward's outputs (y, last state, the state
# after every 8 steps, the readout before the gate) and the backward from them.
@pytest.mark.parametrize("case", [(2, 50, 70, 16, BF16, False, True), (1, 37, 33, 40, F32, True, True),
                                  (2, 21, 64, 8, F32, False, False)],
                         ids=["n16-bf16-gated", "n40-f32-zoh-gated", "n8-f32-ungated"])
def test_training_pair_on_host(case):
    b, L, d, n, dt, zoh, gated = case
    inp = workloads.random_scan_inputs(b, L, d, n, dt, seed=21, gated=gated, bias=True)
    g = torch.Generator().manual_seed(22)
    dy = torch.randn(b, L, d, generator=g).to(dt)
    z = inp["z"] if gated else None
    t = dict(u=inp["u"], delta=inp["delta"], A_log=inp["A_log"], B=inp["B"], C=inp["C"], D=inp["D"], z=z,
             delta_bias=inp["delta_bias"], dy=dy)
    args = dict(b=b, L=L, d_in=d, n=n, dtype=_code(dt), softplus=1, zoh=int(zoh), segments=2)
    nck = (L - 1) // 8
    grads = dict(du=((b, L, d), dt), ddelta=((b, L, d), dt), dA_log=((d, n), F32), dB=((b, L, n), dt),
                 dC=((b, L, n), dt), dD=((d,), F32), ddelta_bias=((d,), F32))
    if gated:
        grads["dz"] = ((b, L, d), dt)
    outs = dict(y=((b, L, d), dt), last_state=((b, d, n), F32), checkpoints=((b, nck, n, d), F32),
                y_pre=((b, L, d), dt), **grads)
    got = hk.run("train", t, args, outs)
    y, last = oracle.scan(inp["u"], inp["delta"], inp["A_log"], inp["B"], inp["C"], inp["D"], z, inp["delta_bias"],
                          True, zoh=zoh)
    assert_close(got["y"], y, dt, "host y")
    assert_close(got["last_state"], last, dt, "host last_state")
    if gated:
        # The readout before the gate is the ungated scan's output.
        y_pre, _ = oracle.scan(inp["u"], inp["delta"], inp["A_log"], inp["B"], inp["C"], inp["D"], None,
                               inp["delta_bias"], True, zoh=zoh)
        assert_close(got["y_pre"], y_pre, dt, "host y_pre")
    else:
        assert "y_pre" not in got
    for i in range(nck):
        # Checkpoint i is the state after step 8 (i + 1): the last state of the scan cut there.
        s = slice(0, 8 * (i + 1))
        _, h = oracle.scan(inp["u"][:, s], inp["delta"][:, s], inp["A_log"], inp["B"][:, s], inp["C"][:, s],
                           inp["D"], None, inp["delta_bias"], True, zoh=zoh)
        assert_close(got["checkpoints"][:, i].transpose(1, 2), h, dt, f"host checkpoint {i}")
    ref = oracle.scan_bwd(inp["u"], inp["delta"], inp["A_log"], inp["B"], inp["C"], inp["D"], z,
                          inp["delta_bias"], True, None, dy, None, zoh=zoh)
    for k in grads:
        assert_close(got[k], ref[k], dt, f"host {k}")


# n = 4 LPC runs the vector kernel (LPC lanes per channel, LPC batch rows per
# workgroup) for LPC = 1, 2, 4, 8, 16; n = 5 and n = 3 run the any-n kernel.  Batch
# sizes leave a partial row group and channel counts a partial tile.
@pytest.mark.parametrize("b,d,n,dt,zoh", [(3, 70, 16, BF16, 0), (5, 70, 4, F32, 0), (3, 130, 8, BF16, 1),
                                          (9, 40, 32, F32, 0), (17, 20, 64, BF16, 1), (2, 33, 5, F32, 1),
                                          (4, 9, 3, F32, 0)])
def test_step_on_host(b, d, n, dt, zoh):
    dec = workloads.decode_inputs(4, steps=1, b=b)
    g = torch.Generator().manual_seed(b + d)
    state = torch.randn(b, d, n, generator=g) * 0.1
    x, dtv, z = (torch.randn(b, d, generator=g).to(dt) for _ in range(3))
    B, C = (torch.randn(b, n, generator=g).to(dt) for _ in range(2))
    A_log = workloads.s4d_real_A_log(d, n)
    D, bias = torch.randn(d, generator=g), dec["dt_bias"][:d].contiguous()
    t = dict(state=state, x=x, dt=dtv, A_log=A_log, B=B, C=C, D=D, z=z, dt_bias=bias)
    got = hk.run("step", t, dict(b=b, d_in=d, n=n, dtype=_code(dt), softplus=1, zoh=zoh),
                 dict(y=((b, d), dt), state=((b, d, n), F32)))
    sr, yr = oracle.state_update(state, x, dtv, A_log, B, C, D, z, bias, True, zoh=bool(zoh))
    assert_close(got["y"], yr, dt, "host step y")
    assert_close(got["state"], sr, dt, "host step state")


CROSS = [
    # maps, H, W, d_in, n, dtype, bias, two_pass (else the one-pass form)
    (2, 5, 7, 24, 1, F32, False, True),      # the two-pass form (workspace outputs + merge), two segments
    (2, 5, 7, 24, 1, F32, True, False),      # one pass, L = 35: a single ragged chunk
    (1, 9, 15, 20, 1, F32, True, False),     # L = 135: three chunks, the last ragged; d_in not a multiple of 8
    (1, 1, 70, 8, 2, BF16, True, False),     # H = 1: the column-major order is the row-major one
    (1, 66, 1, 12, 3, F32, False, False),    # W = 1, n = 3 in four state slots
    (2, 8, 16, 16, 4, BF16, True, False),    # L = 128: two whole chunks, n = 4
]


@pytest.mark.parametrize("maps,H,W,d,n,dt,bias,two_pass", CROSS)
def test_cross_on_host(maps, H, W, d, n, dt, bias, two_pass):
    g = torch.Generator().manual_seed(3 + H + W + n)
    L = H * W
    x = torch.randn(maps, H, W, d, generator=g).to(dt)
    delta = (torch.randn(maps, 4, L, d, generator=g) - 2).to(dt)
    B, C = (torch.randn(maps, 4, L, n, generator=g).to(dt) for _ in range(2))
    A_log = torch.rand(4, d, n, generator=g) * 2 - 1
    D = torch.randn(4, d, generator=g)
    db = (torch.rand(4, d, generator=g) - 0.5) if bias else None
    t = dict(x=x, delta=delta, A_log=A_log, B=B, C=C, D=D, delta_bias=db)
    got = hk.run("cross", t, dict(maps=maps, H=H, W=W, d_in=d, n=n, dtype=_code(dt), softplus=1,
                                  segments=2 if two_pass else 0, form=2 if two_pass else 1),
                 dict(y=((maps, H, W, d), F32), last_state=((maps, 4, d, n), F32)))
    yr, lr = oracle.cross_scan(x, delta, A_log, B, C, D, db, True)
    assert_close(got["y"], yr, F32, "host cross y")
    assert_close(got["last_state"], lr, F32, "host cross last_state")
