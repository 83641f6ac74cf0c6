"""GPU: the fused VMamba cross scan (ss_cross_scan_fwd) against the oracle.

Each feature map is scanned in four traversal orders (row-major, column-major,
both backwards) and the four outputs are added back at their positions
(githubissues.com VMamba issue 206: CrossScan / CrossMerge only arrange the
sequence).  The output map is fp32 whatever the input dtype, and the oracle
sees the same (bf16-exact) inputs, so every case is held to the fp32 bound,
max relative error 1e-4; last states likewise.  Both forms of the call are
covered: the two-pass form (per-direction outputs in the workspace, then a
merge; the default) and the one-pass form (one kernel that adds the
directions into an LDS sum; n <= 4 and maps of up to 4084..4265 positions,
beyond which it returns SS_ERR_UNSUPPORTED).  The two-pass form is identical
bit for bit to the unfused path on the GPU (torch-made traversal copies,
ss_scan_fwd, torch merge).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity import assert_close
from tests.test_gpu_parity import BF16, DEV, F32, plan, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def ss():
    import selective_state_space_softplus_amd as ss

    return ss


def cross_inputs(maps, H, W, d_in, n, dtype, seed, bias=True, shared_params=False):
    g = torch.Generator().manual_seed(seed)
    r = lambda *s: torch.randn(*s, generator=g)  # noqa: E731
    L = H * W
    A_log = torch.rand(4, d_in, n, generator=g) * 2 - 1
    D = r(4, d_in)
    db = (torch.rand(4, d_in, generator=g) - 0.5) if bias else None
    if shared_params:
        A_log, D = A_log[:1].expand(4, -1, -1).contiguous(), D[:1].expand(4, -1).contiguous()
        db = None if db is None else db[:1].expand(4, -1).contiguous()
    return dict(x=r(maps, H, W, d_in).to(dtype), delta=(r(maps, 4, L, d_in) - 2).to(dtype), A_log=A_log,
                B=r(maps, 4, L, n).to(dtype), C=r(maps, 4, L, n).to(dtype), D=D, delta_bias=db)


# Largest map (positions) the one-pass form takes, by state size: its LDS sum
# (8.5 words a position), staging and B, C areas within 160 KB.
ONE_PASS_MAX_L = {1: 4265, 2: 4205, 3: 4084, 4: 4084}


def one_pass_fits(H, W, n):
    return n in ONE_PASS_MAX_L and H * W <= ONE_PASS_MAX_L[n]


def run_gpu(ss, c, softplus=True, form="auto"):
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in c.items()}
    y, last = ss.cross_scan_fwd(g["x"], g["delta"], g["A_log"], g["B"], g["C"], g["D"], g["delta_bias"], softplus,
                                return_last_state=True, form=form)
    torch.cuda.synchronize()
    return y, last


def check(ss, c, what, softplus=True, form="auto"):
    maps, H, W, _ = c["x"].shape
    n = c["A_log"].shape[2]
    if form == "one_pass" and not one_pass_fits(H, W, n):
        with pytest.raises(ss.SSError) as e:
            run_gpu(ss, c, softplus, form)
        assert ss.STATUS[e.value.code] == "SS_ERR_UNSUPPORTED"
        return 0.0, 0.0
    y, last = run_gpu(ss, c, softplus, form)
    yr, lr = oracle.cross_scan(c["x"], c["delta"], c["A_log"], c["B"], c["C"], c["D"], c["delta_bias"], softplus)
    e1 = assert_close(y, yr, F32, f"{what} y")
    e2 = assert_close(last, lr, F32, f"{what} last_state")
    return e1, e2


SMALL = [
    (2, 7, 5, 40, 1, F32), (1, 9, 6, 64, 1, F32), (2, 4, 13, 70, 2, BF16), (1, 5, 8, 64, 16, BF16),
    (2, 6, 3, 33, 5, F32), (1, 1, 17, 20, 1, F32), (1, 11, 1, 20, 3, F32), (1, 1, 1, 8, 1, F32),
    (1, 6, 7, 24, 40, F32), (2, 8, 8, 128, 16, F32), (1, 12, 11, 9, 4, BF16), (3, 17, 19, 24, 2, F32),
    (1, 1, 300, 16, 1, BF16), (1, 128, 1, 8, 3, F32), (2, 64, 64, 16, 1, F32), (1, 64, 64, 8, 4, F32),
    (1, 65, 66, 8, 1, F32),
]


@pytest.mark.parametrize("form", ["auto", "one_pass"])
@pytest.mark.parametrize("maps,H,W,d_in,n,dtype", SMALL)
def test_cross_small(ss, maps, H, W, d_in, n, dtype, form):
    say(f"cross maps={maps} {H}x{W} d_in={d_in} n={n} {dtype} form={form}")
    check(ss, cross_inputs(maps, H, W, d_in, n, dtype, seed=maps + H * 7 + W * 11 + n), f"{H}x{W} n={n}",
          form=form)


@pytest.mark.parametrize("form", ["auto", "one_pass"])
def test_cross_without_softplus_or_bias(ss, form):
    say(f"cross without softplus or bias, form={form}")
    c = cross_inputs(2, 6, 5, 40, 1, F32, seed=3, bias=False)
    c["delta"] = c["delta"].abs() * 0.1 + 0.01
    check(ss, c, "no softplus", softplus=False, form=form)


def test_cross_rejects_an_unknown_form(ss):
    c = cross_inputs(1, 4, 4, 8, 1, F32, seed=1)
    with pytest.raises(ValueError):
        run_gpu(ss, c, form="three_pass")


@pytest.mark.parametrize("segments,n", [(3, 1), (5, 16)])
def test_cross_segments(ss, segments, n):
    """The two-pass form with L cut into segments."""
    say(f"cross with {segments} segments n={n}")
    c = cross_inputs(1, 20, 30, 64, n, F32, seed=9 + n)
    with plan(segments=segments):
        check(ss, c, f"segments={segments}", form="two_pass")


@pytest.mark.parametrize("form", ["two_pass", "one_pass"])
def test_cross_vmamba_workload_full(ss, form):
    """The scan-vmamba workload (16 maps of 56 x 56 x 384, n = 1, fp32), compared in full."""
    cfg = workloads.CONFIGS[3]
    say(f"cross scan at {cfg.name} size, full compare, form={form}")
    c = workloads.cross_scan_inputs(3)
    e1, e2 = check(ss, c, cfg.name, form=form)
    print(f"{cfg.name} cross scan ({form}): y err {e1:.3g}, last_state err {e2:.3g}")


def test_cross_equals_unrolled_scan_and_merge(ss):
    """Unrolled on the GPU with torch, scanned by ss_scan_fwd, merged with torch: the same map as the
    two-pass form, and the one-kernel form within the fp32 bound of both."""
    say("fused cross scan vs unrolled scan + merge")
    maps, H, W, d_in, n = 3, 12, 9, 96, 1
    c = cross_inputs(maps, H, W, d_in, n, F32, seed=17, shared_params=True)
    y1, last1 = run_gpu(ss, c, form="one_pass")
    y, last = run_gpu(ss, c)
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in c.items()}
    L = H * W
    u = workloads.vmamba_unroll(g["x"])                                       # (maps*4, L, d_in)
    yd, ld = ss.scan_fwd(u, g["delta"].reshape(maps * 4, L, d_in), g["A_log"][0], g["B"].reshape(maps * 4, L, n),
                         g["C"].reshape(maps * 4, L, n), g["D"][0], None, g["delta_bias"][0], True,
                         return_last_state=True)
    yd = yd.reshape(maps, 4, L, d_in)
    merged = (yd[:, 0].reshape(maps, H, W, d_in) + yd[:, 1].reshape(maps, W, H, d_in).transpose(1, 2)
              + yd[:, 2].flip(1).reshape(maps, H, W, d_in) + yd[:, 3].flip(1).reshape(maps, W, H, d_in).transpose(1, 2))
    torch.cuda.synchronize()
    # Same per-direction arithmetic and the same order of the four additions: bit for bit.
    assert torch.equal(y, merged), "two-pass vs unrolled"
    assert torch.equal(last, ld.reshape(maps, 4, d_in, n))
    assert_close(y1, merged, F32, "one kernel vs unrolled")
    assert_close(last1, last, F32, "one kernel vs unrolled, last_state")


@pytest.mark.parametrize("n,dtype,form", [(16, BF16, "auto"), (1, F32, "auto"), (1, F32, "one_pass"),
                                          (2, BF16, "one_pass"), (4, F32, "one_pass")])
def test_cross_is_deterministic(ss, n, dtype, form):
    say(f"cross scan run-to-run determinism n={n} form={form}")
    c = cross_inputs(2, 40, 39, 72, n, dtype, seed=23)
    y1, l1 = run_gpu(ss, c, form=form)
    for _ in range(3):
        y2, l2 = run_gpu(ss, c, form=form)
        assert torch.equal(y1, y2) and torch.equal(l1, l2)


def test_cross_vmamba_workload_bf16_one_pass(ss):
    """The scan-vmamba maps with bf16 inputs through the one-pass form, compared in full (the oracle sees the same
    bf16 values; the output is fp32, so the fp32 bound holds)."""
    say("cross scan at scan-vmamba size, bf16 inputs, one pass")
    c = workloads.cross_scan_inputs(3)
    for key in ("x", "delta", "B", "C"):
        c[key] = c[key].to(BF16)
    e1, e2 = check(ss, c, "scan-vmamba bf16", form="one_pass")
    print(f"scan-vmamba bf16 one pass: y err {e1:.3g}, last_state err {e2:.3g}")


@pytest.mark.parametrize("n,form", [(2, "one_pass"), (4, "one_pass"), (4, "auto")])
def test_cross_mid_maps(ss, n, form):
    """8 maps of 40 x 40 x 256 (25 chunks of 64 steps, none ragged) with n = 2 and 4."""
    say(f"cross 8 maps 40x40x256 n={n} form={form}")
    check(ss, cross_inputs(8, 40, 40, 256, n, F32, seed=77 + n), f"40x40 n={n}", form=form)
