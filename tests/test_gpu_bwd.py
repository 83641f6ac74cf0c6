"""GPU: the gradient of the scan (ss_scan_bwd, and ss_scan_bwd_ex with the
zero-order-hold input term) against the oracle's gradient.

The oracle's backward is pinned to torch autograd and to finite differences of
its forward (tests/oracle_pins.py).  Every gradient is compared element by
element at the parity tolerances: max relative error 1e-4 for fp32 inputs,
2e-2 for bf16 inputs (whose per-element gradients are rounded to bf16).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity import TOL, assert_close
from tests.test_gpu_parity import BF16, DEV, F32, plan, say, small_inputs, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

GRADS = ("du", "ddelta", "dA_log", "dB", "dC", "dD", "dz", "ddelta_bias", "dinitial_state")
ORACLE_NAME = {"dinitial_state": "dh0"}


@pytest.fixture(scope="module")
def ss():
    import selective_state_space_softplus_amd as ss

    return ss


def grads_gpu(ss, g, dy, h0=None, dlast=None, zoh=False):
    out = ss.scan_bwd(g["u"], g["delta"], g["A_log"], g["B"], g["C"], g["D"], dy, g["z"], g["delta_bias"],
                      g["delta_softplus"], initial_state=h0, dlast_state=dlast, zoh=zoh)
    torch.cuda.synchronize()
    return out


def grads_oracle(inp, dy, h0=None, dlast=None, zoh=False):
    return oracle.scan_bwd(inp["u"], inp["delta"], inp["A_log"], inp["B"], inp["C"], inp["D"], inp["z"],
                           inp["delta_bias"], inp["delta_softplus"], h0, dy, dlast, zoh=zoh)


def compare(got, ref, dtype, what):
    errs = {}
    for k in GRADS:
        if k in got:
            errs[k] = assert_close(got[k], ref[ORACLE_NAME.get(k, k)], dtype, f"{what} {k}")
    return errs


def extras(b, L, d_in, n, dtype, seed, h0, dlast):
    r = torch.Generator().manual_seed(seed)
    dy = torch.randn(b, L, d_in, generator=r).to(dtype)
    h = torch.randn(b, d_in, n, generator=r) * 0.5 if h0 else None
    dl = torch.randn(b, d_in, n, generator=r) if dlast else None
    return dy, h, dl


CASES = [
    # b, L, d_in, n, dtype, gated, bias, softplus
    (2, 300, 130, 16, F32, True, True, True),
    (2, 300, 130, 16, BF16, True, True, True),
    (1, 1, 1, 16, F32, True, True, True),
    (1, 7, 3, 16, F32, False, False, True),
    (1, 97, 65, 16, F32, True, True, False),
    (2, 200, 40, 1, F32, False, False, True),
    (1, 129, 70, 2, BF16, True, True, True),
    (2, 90, 24, 3, F32, True, True, True),
    (1, 70, 66, 8, BF16, False, True, True),
    (1, 70, 66, 17, F32, True, True, True),
    (2, 61, 42, 32, F32, True, False, True),
    (1, 64, 128, 32, BF16, True, True, True),
    (1, 70, 66, 40, F32, True, True, True),
    (2, 61, 42, 64, F32, True, False, True),
    (1, 64, 128, 64, BF16, True, True, True),
]


def _id(c):
    return "b{}_L{}_d{}_n{}_{}_{}{}{}".format(c[0], c[1], c[2], c[3], "f32" if c[4] == F32 else "bf16",
                                               "g" if c[5] else "", "b" if c[6] else "", "s" if c[7] else "")


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
@pytest.mark.parametrize("h0,dlast", [(False, False), (True, True)])
def test_bwd_small(ss, case, h0, dlast):
    say(f"bwd {case} h0={h0} dlast={dlast}")
    b, L, d_in, n, dtype = case[:5]
    inp = small_inputs(*case, seed=sum(case[:4]) + 3)
    dy, hh, dl = extras(b, L, d_in, n, dtype, seed=b + L + d_in + n, h0=h0, dlast=dlast)
    g = to_dev(inp)
    got = grads_gpu(ss, g, dy.to(DEV), None if hh is None else hh.to(DEV), None if dl is None else dl.to(DEV))
    ref = grads_oracle(inp, dy, hh, dl)
    compare(got, ref, dtype, f"{case}")


def test_bwd_mid_workload_full(ss):
    """The scan-mid workload (b=8, L=2048, d_in=1536, n=16, bf16), every gradient compared in full."""
    cfg = workloads.CONFIGS[1]
    say(f"bwd at {cfg.name} size, full compare")
    inp = workloads.scan_inputs(1)
    dy, _, _ = extras(cfg.b, cfg.L, cfg.d_in, cfg.n, cfg.dtype, seed=77, h0=False, dlast=False)
    got = grads_gpu(ss, to_dev(inp), dy.to(DEV))
    ref = grads_oracle(inp, dy)
    errs = compare(got, ref, cfg.dtype, cfg.name)
    print(f"{cfg.name} bwd errors: " + ", ".join(f"{k} {v:.3g}" for k, v in errs.items()))


def long_channels(d_in):
    """One channel in every 64-channel group (a different lane in each) and the last: every (channel group,
    L segment, batch row) piece of the backward kernel is covered, since each channel spans them all."""
    return sorted({g * 64 + (g * 37) % 64 for g in range(d_in // 64)} | {d_in - 1})


def test_bwd_long_workload_sampled(ss):
    """scan-long (b=4, L=8192, d_in=5120, n=16, bf16): per-channel gradients on one channel of every channel
    group, and dA_log, dD, dbias of those channels (sums over the batch rows) -- everything but dB, dC, which
    sum over all channels and are compared in full at the mid size."""
    cfg = workloads.CONFIGS[2]
    say(f"bwd at {cfg.name} size, sampled channels")
    inp = workloads.scan_inputs(2)
    dy, _, _ = extras(cfg.b, cfg.L, cfg.d_in, cfg.n, cfg.dtype, seed=78, h0=False, dlast=False)
    got = grads_gpu(ss, to_dev(inp), dy.to(DEV))
    for d in long_channels(cfg.d_in):
        sl = lambda t: t[:, :, d:d + 1].contiguous()  # noqa: E731
        ref = oracle.scan_bwd(sl(inp["u"]), sl(inp["delta"]), inp["A_log"][d:d + 1], inp["B"], inp["C"],
                              inp["D"][d:d + 1], sl(inp["z"]), inp["delta_bias"][d:d + 1], True, None, sl(dy), None)
        for k in ("du", "ddelta", "dz"):
            assert_close(got[k][:, :, d:d + 1], ref[k], cfg.dtype, f"{cfg.name} {k} channel {d}")
        assert_close(got["dA_log"][d:d + 1], ref["dA_log"], cfg.dtype, f"{cfg.name} dA_log channel {d}")
        assert_close(got["dD"][d:d + 1], ref["dD"], cfg.dtype, f"{cfg.name} dD channel {d}")
        assert_close(got["ddelta_bias"][d:d + 1], ref["ddelta_bias"], cfg.dtype, f"{cfg.name} dbias channel {d}")


@pytest.mark.parametrize("segments,n,dtype", [(4, 16, BF16), (7, 1, F32), (3, 32, F32), (5, 64, F32)])
def test_bwd_with_segments(ss, segments, n, dtype):
    """The forward pass inside the backward cut into segments: each piece saves only its own states."""
    say(f"bwd with {segments} forward segments n={n}")
    inp = workloads.random_scan_inputs(2, 1000, 100, n, dtype, seed=60 + n, gated=True, bias=True)
    dy, hh, dl = extras(2, 1000, 100, n, dtype, seed=61, h0=True, dlast=True)
    with plan(segments=segments):
        got = grads_gpu(ss, to_dev(inp), dy.to(DEV), hh.to(DEV), dl.to(DEV))
    compare(got, grads_oracle(inp, dy, hh, dl), dtype, f"segments={segments}")


def test_bwd_is_deterministic(ss):
    say("bwd run-to-run determinism")
    inp = to_dev(workloads.random_scan_inputs(2, 500, 200, 16, BF16, seed=5, gated=True, bias=True))
    dy = torch.randn(2, 500, 200, device=DEV).to(BF16)
    a = grads_gpu(ss, inp, dy)
    b = grads_gpu(ss, inp, dy)
    for k in a:
        assert torch.equal(a[k], b[k]), k


def _shifted(t):
    """The same values in a view that starts one element into a larger buffer: element-aligned, but not aligned
    to two elements, so the backward takes its one-channel-at-a-time element mapping instead of channel pairs."""
    buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
    v = buf[1:].view(t.shape)
    v.copy_(t)
    return v


@pytest.mark.parametrize("dtype,zoh,n", [(BF16, False, 16), (F32, False, 16), (BF16, True, 8), (F32, False, 40)])
def test_bwd_channel_pairs_match_single_channels(ss, dtype, zoh, n):
    """With d_in even and aligned tensors the element threads take adjacent channel pairs; shifted by one element
    they take channels one at a time.  Both give the same gradients bit for bit, from recomputation and from
    saved states."""
    say(f"bwd channel pairs vs single channels dtype={dtype} zoh={zoh} n={n}")
    inp = to_dev(workloads.random_scan_inputs(2, 300, 130, n, dtype, seed=80 + n, gated=True, bias=True))
    dy = torch.randn(2, 300, 130, generator=torch.Generator().manual_seed(81)).to(dtype).to(DEV)
    sh = dict(inp)
    for k in ("u", "delta", "z"):
        sh[k] = _shifted(inp[k])
    dys = _shifted(dy)
    a = grads_gpu(ss, inp, dy, zoh=zoh)
    b = grads_gpu(ss, sh, dys, zoh=zoh)
    for k in a:
        if a[k] is not None:
            assert torch.equal(a[k], b[k]), k
    args = lambda g: (g["u"], g["delta"], g["A_log"], g["B"], g["C"], g["D"])  # noqa: E731
    for g, d in ((inp, dy), (sh, dys)):
        g["saved"] = ss.scan_fwd_save(*args(g), g["z"], g["delta_bias"], True, zoh=zoh)
    sa = ss.scan_bwd(*args(inp), dy, inp["z"], inp["delta_bias"], True, zoh=zoh, saved=inp["saved"])
    sb = ss.scan_bwd(*args(sh), dys, sh["z"], sh["delta_bias"], True, zoh=zoh, saved=sh["saved"])
    torch.cuda.synchronize()
    for k in sa:
        if sa[k] is not None:
            assert torch.equal(sa[k], sb[k]), f"saved {k}"


def test_autograd_function(ss):
    """selective_scan under torch autograd: y.backward(dy) gives scan_bwd's gradients."""
    say("autograd function")
    inp = to_dev(workloads.random_scan_inputs(2, 100, 64, 16, F32, seed=9, gated=True, bias=True))
    leaves = {k: inp[k].clone().requires_grad_(True) for k in ("u", "delta", "A_log", "B", "C", "D", "z",
                                                                  "delta_bias")}
    h0 = (torch.randn(2, 64, 16, device=DEV) * 0.5).requires_grad_(True)
    y = ss.selective_scan(leaves["u"], leaves["delta"], leaves["A_log"], leaves["B"], leaves["C"], leaves["D"],
                          leaves["z"], leaves["delta_bias"], True, initial_state=h0)
    dy = torch.randn_like(y)
    y.backward(dy)
    ref = ss.scan_bwd(inp["u"], inp["delta"], inp["A_log"], inp["B"], inp["C"], inp["D"], dy, inp["z"],
                      inp["delta_bias"], True, initial_state=h0.detach())
    names = dict(u="du", delta="ddelta", A_log="dA_log", B="dB", C="dC", D="dD", z="dz", delta_bias="ddelta_bias")
    for k, v in leaves.items():
        assert torch.equal(v.grad, ref[names[k]]), k
    assert torch.equal(h0.grad, ref["dinitial_state"])


# ---- zero-order-hold input term (ss_scan_bwd_ex)

ZOH_CASES = [c for c in CASES if c[:4] in ((2, 300, 130, 16), (1, 1, 1, 16), (1, 97, 65, 16), (2, 200, 40, 1),
                                          (1, 129, 70, 2), (2, 90, 24, 3), (1, 70, 66, 8), (2, 61, 42, 32),
                                          (1, 64, 128, 32), (1, 70, 66, 40), (2, 61, 42, 64))]


@pytest.mark.parametrize("case", ZOH_CASES, ids=[_id(c) for c in ZOH_CASES])
@pytest.mark.parametrize("h0,dlast", [(False, False), (True, True)])
def test_bwd_zoh_small(ss, case, h0, dlast):
    say(f"bwd zoh {case} h0={h0} dlast={dlast}")
    b, L, d_in, n, dtype = case[:5]
    inp = small_inputs(*case, seed=sum(case[:4]) + 5)
    dy, hh, dl = extras(b, L, d_in, n, dtype, seed=b + L + d_in + n + 1, h0=h0, dlast=dlast)
    got = grads_gpu(ss, to_dev(inp), dy.to(DEV), None if hh is None else hh.to(DEV), None if dl is None else dl.to(DEV),
                    zoh=True)
    compare(got, grads_oracle(inp, dy, hh, dl, zoh=True), dtype, f"zoh {case}")


@pytest.mark.parametrize("segments,n,dtype", [(4, 16, BF16), (3, 5, F32)])
def test_bwd_zoh_with_segments(ss, segments, n, dtype):
    say(f"bwd zoh with {segments} segments n={n}")
    inp = workloads.random_scan_inputs(2, 1000, 100, n, dtype, seed=80 + n, gated=True, bias=True)
    dy, hh, dl = extras(2, 1000, 100, n, dtype, seed=81, h0=True, dlast=True)
    with plan(segments=segments):
        got = grads_gpu(ss, to_dev(inp), dy.to(DEV), hh.to(DEV), dl.to(DEV), zoh=True)
    compare(got, grads_oracle(inp, dy, hh, dl, zoh=True), dtype, f"zoh segments={segments}")


def test_bwd_zoh_mid_workload_full(ss):
    """The scan-mid workload with the zero-order hold, every gradient compared in full."""
    cfg = workloads.CONFIGS[1]
    say(f"bwd zoh at {cfg.name} size, full compare")
    inp = workloads.scan_inputs(1)
    dy, _, _ = extras(cfg.b, cfg.L, cfg.d_in, cfg.n, cfg.dtype, seed=79, h0=False, dlast=False)
    got = grads_gpu(ss, to_dev(inp), dy.to(DEV), zoh=True)
    errs = compare(got, grads_oracle(inp, dy, zoh=True), cfg.dtype, f"zoh {cfg.name}")
    print(f"{cfg.name} zoh bwd errors: " + ", ".join(f"{k} {v:.3g}" for k, v in errs.items()))


def test_bwd_zoh_long_workload_sampled(ss):
    """scan-long with the zero-order hold: per-channel gradients on one channel of every group (as for Euler)."""
    cfg = workloads.CONFIGS[2]
    say(f"bwd zoh at {cfg.name} size, sampled channels")
    inp = workloads.scan_inputs(2)
    dy, _, _ = extras(cfg.b, cfg.L, cfg.d_in, cfg.n, cfg.dtype, seed=82, h0=False, dlast=False)
    got = grads_gpu(ss, to_dev(inp), dy.to(DEV), zoh=True)
    for d in long_channels(cfg.d_in):
        sl = lambda t: t[:, :, d:d + 1].contiguous()  # noqa: E731
        ref = oracle.scan_bwd(sl(inp["u"]), sl(inp["delta"]), inp["A_log"][d:d + 1], inp["B"], inp["C"],
                              inp["D"][d:d + 1], sl(inp["z"]), inp["delta_bias"][d:d + 1], True, None, sl(dy), None,
                              zoh=True)
        for k in ("du", "ddelta", "dz"):
            assert_close(got[k][:, :, d:d + 1], ref[k], cfg.dtype, f"zoh {cfg.name} {k} channel {d}")
        for k in ("dA_log", "dD", "ddelta_bias"):
            assert_close(got[k][d:d + 1], ref[k], cfg.dtype, f"zoh {cfg.name} {k} channel {d}")


def test_bwd_zoh_is_deterministic(ss):
    say("bwd zoh run-to-run determinism")
    inp = to_dev(workloads.random_scan_inputs(2, 500, 200, 16, BF16, seed=6, gated=True, bias=True))
    dy = torch.randn(2, 500, 200, device=DEV).to(BF16)
    a = grads_gpu(ss, inp, dy, zoh=True)
    b = grads_gpu(ss, inp, dy, zoh=True)
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_autograd_function_zoh(ss):
    """selective_scan(..., zoh=True) under torch autograd: y.backward(dy) gives scan_bwd's hold gradients,
    and y is the hold forward's."""
    say("autograd function, zero-order hold")
    inp = to_dev(workloads.random_scan_inputs(2, 100, 64, 16, F32, seed=10, gated=True, bias=True))
    leaves = {k: inp[k].clone().requires_grad_(True) for k in ("u", "delta", "A_log", "B", "C", "D", "z",
                                                                  "delta_bias")}
    y = ss.selective_scan(leaves["u"], leaves["delta"], leaves["A_log"], leaves["B"], leaves["C"], leaves["D"],
                          leaves["z"], leaves["delta_bias"], True, zoh=True)
    y_fwd = ss.scan_fwd(inp["u"], inp["delta"], inp["A_log"], inp["B"], inp["C"], inp["D"], inp["z"],
                        inp["delta_bias"], True, zoh=True)
    assert torch.equal(y.detach(), y_fwd)
    dy = torch.randn_like(y)
    y.backward(dy)
    ref = ss.scan_bwd(inp["u"], inp["delta"], inp["A_log"], inp["B"], inp["C"], inp["D"], dy, inp["z"],
                      inp["delta_bias"], True, zoh=True)
    names = dict(u="du", delta="ddelta", A_log="dA_log", B="dB", C="dC", D="dD", z="dz", delta_bias="ddelta_bias")
    for k, v in leaves.items():
        assert torch.equal(v.grad, ref[names[k]]), k
