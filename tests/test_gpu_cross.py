"""GPU: the fused VMamba cross scan (ss_cross_scan_fwd) against the oracle.

Each feature map is scanned in four traversal orders (row-major, column-major,
both backwards) and the four outputs are added back at their positions
(githubissues.com VMamba issue 206: CrossScan / CrossMerge only arrange the
sequence).  The output map is fp32 whatever the input dtype, and the oracle
sees the same (bf16-exact) inputs, so every case is held to the fp32 bound,
max relative error 1e-4; last states likewise.  Against the unfused path on
the GPU (torch-made traversal copies, ss_scan_fwd, torch merge) the result is
identical bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity import assert_close
from tests.test_gpu_parity import BF16, DEV, F32, env, say

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


def run_gpu(ss, c, softplus=True):
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in c.items()}
    y, last = ss.cross_scan_fwd(g["x"], g["delta"], g["A_log"], g["B"], g["C"], g["D"], g["delta_bias"], softplus,
                                return_last_state=True)
    torch.cuda.synchronize()
    return y, last


def check(ss, c, what, softplus=True):
    y, last = run_gpu(ss, c, softplus)
    yr, lr = oracle.cross_scan(c["x"], c["delta"], c["A_log"], c["B"], c["C"], c["D"], c["delta_bias"], softplus)
    e1 = assert_close(y, yr, F32, f"{what} y")
    e2 = assert_close(last, lr, F32, f"{what} last_state")
    return e1, e2


@pytest.mark.parametrize("maps,H,W,d_in,n,dtype", [
    (2, 7, 5, 40, 1, F32), (1, 9, 6, 64, 1, F32), (2, 4, 13, 70, 2, BF16), (1, 5, 8, 64, 16, BF16),
    (2, 6, 3, 33, 5, F32), (1, 1, 17, 20, 1, F32), (1, 11, 1, 20, 3, F32), (1, 1, 1, 8, 1, F32),
    (1, 6, 7, 24, 40, F32), (2, 8, 8, 128, 16, F32),
])
def test_cross_small(ss, maps, H, W, d_in, n, dtype):
    say(f"cross maps={maps} {H}x{W} d_in={d_in} n={n} {dtype}")
    check(ss, cross_inputs(maps, H, W, d_in, n, dtype, seed=maps + H * 7 + W * 11 + n), f"{H}x{W} n={n}")


def test_cross_without_softplus_or_bias(ss):
    say("cross without softplus or bias")
    c = cross_inputs(2, 6, 5, 40, 1, F32, seed=3, bias=False)
    c["delta"] = c["delta"].abs() * 0.1 + 0.01
    check(ss, c, "no softplus", softplus=False)


@pytest.mark.parametrize("segments,n", [(3, 1), (5, 16)])
def test_cross_segments(ss, segments, n):
    say(f"cross with {segments} segments n={n}")
    c = cross_inputs(1, 20, 30, 64, n, F32, seed=9 + n)
    with env(SS_SCAN_SEGMENTS=segments):
        check(ss, c, f"segments={segments}")


def test_cross_vmamba_workload_full(ss):
    """The scan-vmamba workload (16 maps of 56 x 56 x 384, n = 1, fp32), compared in full."""
    cfg = workloads.CONFIGS[3]
    say(f"cross scan at {cfg.name} size, full compare")
    c = workloads.cross_scan_inputs(3)
    e1, e2 = check(ss, c, cfg.name)
    print(f"{cfg.name} fused cross scan: y err {e1:.3g}, last_state err {e2:.3g}")


def test_cross_equals_unrolled_scan_and_merge(ss):
    """Unrolled on the GPU with torch, scanned by ss_scan_fwd, merged with torch: the same map."""
    say("fused cross scan vs unrolled scan + merge")
    maps, H, W, d_in, n = 3, 12, 9, 96, 1
    c = cross_inputs(maps, H, W, d_in, n, F32, seed=17, shared_params=True)
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
    assert torch.equal(y, merged), "fused vs unrolled"
    assert torch.equal(last, ld.reshape(maps, 4, d_in, n))


def test_cross_is_deterministic(ss):
    say("cross scan run-to-run determinism")
    c = cross_inputs(2, 10, 9, 72, 16, BF16, seed=23)
    y1, l1 = run_gpu(ss, c)
    y2, l2 = run_gpu(ss, c)
    assert torch.equal(y1, y2) and torch.equal(l1, l2)
