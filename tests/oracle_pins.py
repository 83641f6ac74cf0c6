"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Every ``pin_*`` function takes a loaded oracle library (the real one or a
deliberately broken build of it) and raises AssertionError when the oracle
disagrees with:
  - values worked out by hand (tests/golden/hand_worked.json);
  - library routines in float64 (numpy.logaddexp for softplus, torch silu);
  - the brute-force unrolled solution of the recurrence,
        y_t = sum_n C_t,n sum_{s<=t} exp(A_n * sum_{r=s+1..t} Delta_r) Delta_s B_s,n u_s + D u_t,
    which never runs the recurrence step by step;
  - closed forms (the geometric sum for constant inputs at n = 1) and the
    limits A -> 0 (a running sum) and A -> -inf (no memory);
  - invariants: linearity in u, causality, a scan of length 1 equals one
    step, a chain of steps equals the scan, prefill then decode equals the
    longer scan, B = 0 leaves only the D skip.
The definition they pin is that of the mhpn.cn selective_scan walk-through
(sections 2-5 and 7) and of Mamba.step on the jiafeimiao.top page, whose
convolution step is pinned to torch's depthwise conv1d and a delay line.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_worked.json")


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, rtol=1e-12, atol=1e-13, what=""):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = np.max(np.abs(a - b) / (atol + rtol * np.abs(b))) if a.size else 0.0
    assert err <= 1.0, f"{what}: mismatch (scaled error {err:.3g})\n{a}\nvs\n{b}"


def _exact(a, b, what=""):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape and np.array_equal(a, b), f"{what}: not identical\n{a}\nvs\n{b}"


def random_case(seed, b=2, L=9, d_in=3, n=4, gated=True, bias=True, softplus=True):
    r = _rng(seed)
    case = dict(
        u=r.standard_normal((b, L, d_in)),
        delta=r.standard_normal((b, L, d_in)) - 1.0,
        A_log=r.uniform(-1.5, 1.5, (d_in, n)),
        B=r.standard_normal((b, L, n)),
        C=r.standard_normal((b, L, n)),
        D=r.standard_normal(d_in),
        z=r.standard_normal((b, L, d_in)) if gated else None,
        delta_bias=r.uniform(-1.0, 0.5, d_in) if bias else None,
        delta_softplus=softplus,
    )
    return case


def brute_force(case):
    """Unrolled closed-form solution of the recurrence (O(L^2), float64).

    With case["h0"] the initial state enters as exp(A * sum_{r<=t} Delta_r) h0;
    with case["zoh"] each input carries the zero-order-hold weight
    expm1(Delta_s A) / A instead of Delta_s.
    """
    u, A_log, B, C, D = case["u"], case["A_log"], case["B"], case["C"], case["D"]
    x = case["delta"] + (0.0 if case["delta_bias"] is None else case["delta_bias"])
    Delta = np.logaddexp(0.0, x) if case["delta_softplus"] else x
    A = -np.exp(A_log)                                   # (d_in, n)
    h0 = case.get("h0")
    zoh = case.get("zoh", False)
    b, L, d_in = u.shape
    y = np.zeros((b, L, d_in))
    last = np.zeros((b, d_in, A.shape[1]))
    for bi in range(b):
        for d in range(d_in):
            S = np.concatenate([[0.0], np.cumsum(Delta[bi, :, d])])   # S[t+1] = sum_{r<=t} Delta_r
            for t in range(L):
                acc = 0.0 if h0 is None else np.exp(A[d] * S[t + 1]) * h0[bi, d]
                for s in range(t + 1):
                    decay = np.exp(A[d] * (S[t + 1] - S[s + 1]))      # prod_{r=s+1..t} exp(Delta_r A)
                    w = np.expm1(Delta[bi, s, d] * A[d]) / A[d] if zoh else Delta[bi, s, d]
                    acc = acc + decay * w * B[bi, s] * u[bi, s, d]
                y[bi, t, d] = np.dot(C[bi, t], acc) + D[d] * u[bi, t, d]
                if t == L - 1:
                    last[bi, d] = acc
    if case["z"] is not None:
        z = case["z"]
        y = y * z / (1.0 + np.exp(-z))
    return y, last


def run(case, lib):
    return oracle.scan(case["u"], case["delta"], case["A_log"], case["B"], case["C"], case["D"], case["z"],
                       case["delta_bias"], case["delta_softplus"], lib=lib, h0=case.get("h0"),
                       zoh=case.get("zoh", False))


# ----------------------------------------------------------------------------- pins

def pin_softplus_silu(lib):
    import torch

    xs = np.concatenate([np.linspace(-60, 60, 241), [-745.0, -30.5, -1e-9, 0.0, 1e-9, 33.3, 700.0]])
    for x in xs:
        _close(oracle.softplus(x, lib), np.logaddexp(0.0, x), rtol=4e-16, atol=1e-300, what=f"softplus({x})")
    zs = torch.linspace(-40, 40, 161, dtype=torch.float64)
    ref = torch.nn.functional.silu(zs).numpy()
    got = np.array([oracle.silu(float(z), lib) for z in zs])
    _close(got, ref, rtol=4e-16, atol=1e-300, what="silu")


def pin_hand_worked(lib):
    g = json.load(open(GOLDEN))
    Dl = math.log(2.0)
    val = lambda pairs: np.array([c0 + c1 * Dl for c0, c1 in pairs])  # noqa: E731
    s = g["scan"]
    A_log = np.log(np.array(s["A_log_exp"]))[None, :]
    u = np.array(s["u"])[None, :, None]
    B = np.array(s["B"])[None]
    C = np.array(s["C"])[None]
    D = np.array([s["D"]])
    for delta, bias in ((s["delta"], None), (g["scan_bias"]["delta"], np.array([g["scan_bias"]["delta_bias"]]))):
        y, last = oracle.scan(u, np.array(delta)[None, :, None], A_log, B, C, D, None, bias, True, lib=lib)
        _close(y[0, :, 0], val(s["y"]), what="hand-worked scan y")
        _close(last[0, 0], val(s["last_state"]), what="hand-worked last_state")
    st = g["step"]
    new, y = oracle.state_update(np.array(st["state"])[None, None], np.array([[st["x"]]]), np.array([[st["dt"]]]),
                                 np.log(np.array(st["A_log_exp"]))[None], np.array(st["B"])[None],
                                 np.array(st["C"])[None], np.array([st["D"]]), lib=lib)
    _close(new[0, 0], val(st["new_state"]), what="hand-worked step state")
    _close(y[0, 0], val([st["y"]])[0], what="hand-worked step y")


def pin_brute_force(lib):
    for seed, kw in enumerate([dict(), dict(gated=False), dict(bias=False), dict(softplus=False, bias=False),
                               dict(b=1, L=12, d_in=2, n=1), dict(b=2, L=5, d_in=3, n=7, bias=False)]):
        case = random_case(100 + seed, **kw)
        if not case["delta_softplus"]:
            case["delta"] = np.abs(case["delta"]) + 0.05     # Delta must stay positive without softplus
        y, last = run(case, lib)
        yb, lb = brute_force(case)
        _close(y, yb, rtol=1e-11, atol=1e-12, what=f"brute force y {kw}")
        _close(last, lb, rtol=1e-11, atol=1e-12, what=f"brute force last_state {kw}")


def pin_geometric_closed_form(lib):
    """n = 1, constant Delta, B and u: h_t = Delta B u (1 - a^t) / (1 - a), a = exp(Delta A), t = 1..L."""
    L = 40
    r = _rng(7)
    for A_exp, delta, softplus in ((3.0, 0.37, False), (0.5, -0.8, True), (1.0, 1.9, True)):
        Delta = math.log1p(math.exp(delta)) if softplus else delta
        Bv, uv = 0.8, -1.3
        C = r.standard_normal((1, L, 1))
        D = np.array([0.25])
        y, last = oracle.scan(np.full((1, L, 1), uv), np.full((1, L, 1), delta), np.array([[math.log(A_exp)]]),
                              np.full((1, L, 1), Bv), C, D, None, None, softplus, lib=lib)
        a = math.exp(-A_exp * Delta)                       # A = -exp(log A_exp) = -A_exp
        t = np.arange(1, L + 1)
        h = Delta * Bv * uv * (1 - a ** t) / (1 - a)
        _close(y[0, :, 0], C[0, :, 0] * h + D[0] * uv, rtol=1e-12, atol=1e-14, what="geometric y")
        _close(last[0, 0, 0], h[-1], what="geometric last_state")


def pin_limits(lib):
    """A -> 0: h is the running sum of Delta B u.  A -> -inf: y = Delta u sum_n B C + D u."""
    case = random_case(11, b=1, L=15, d_in=2, n=3, gated=False, bias=False)
    x = case["delta"]
    Delta = np.logaddexp(0.0, x)
    case["A_log"] = np.full((2, 3), -40.0)                 # |A| ~ 4e-18: exp(Delta A) == 1 in double
    y, last = run(case, lib)
    h = np.cumsum(Delta[..., None] * case["B"][:, :, None, :] * case["u"][..., None], axis=1)  # (b, L, d, n)
    _close(y, np.einsum("btdn,btn->btd", h, case["C"]) + case["D"] * case["u"], rtol=1e-12, atol=1e-13, what="A->0 y")
    _close(last, h[:, -1], what="A->0 last")
    case["A_log"] = np.full((2, 3), 10.0)                  # A = -22026: exp(Delta A) < 1e-95 for Delta >= 0.01
    case["delta"] = np.maximum(case["delta"], -4.0)
    Delta = np.logaddexp(0.0, case["delta"])
    y, last = run(case, lib)
    mem0 = Delta * case["u"] * np.einsum("btn,btn->bt", case["B"], case["C"])[..., None] + case["D"] * case["u"]
    _close(y, mem0, rtol=1e-12, atol=1e-13, what="A->-inf y")


def pin_skip_and_gate(lib):
    case = random_case(12, b=2, L=6, d_in=3, n=4)
    case["B"] = np.zeros_like(case["B"])
    y, last = run(case, lib)
    z = case["z"]
    _close(y, case["D"] * case["u"] * z / (1 + np.exp(-z)), what="B=0 -> gated skip")
    _close(last, np.zeros_like(last), what="B=0 -> zero state")


def pin_linearity_causality(lib):
    case = random_case(13, b=1, L=10, d_in=2, n=5, gated=False)
    u1 = case["u"].copy()
    u2 = _rng(14).standard_normal(u1.shape)
    case["u"] = u1
    y1, _ = run(case, lib)
    case["u"] = u2
    y2, _ = run(case, lib)
    case["u"] = 2.5 * u1 - 0.75 * u2
    y12, _ = run(case, lib)
    _close(y12, 2.5 * y1 - 0.75 * y2, rtol=1e-12, atol=1e-12, what="linearity in u")
    # Causality: changing every input at t0 onwards leaves y before t0 bit-identical.
    case = random_case(15, b=1, L=10, d_in=2, n=5)
    y, _ = run(case, lib)
    t0 = 6
    for k in ("u", "delta", "B", "C", "z"):
        case[k] = case[k].copy()
        case[k][:, t0:] += 1.0
    y2, _ = run(case, lib)
    assert np.array_equal(y[:, :t0], y2[:, :t0]), "causality"
    assert not np.allclose(y[:, t0:], y2[:, t0:]), "later outputs must change"


def pin_step_matches_scan(lib):
    """L = 1 scan == one step from zero; L steps == scan; prefill + decode == longer scan."""
    case = random_case(16, b=2, L=11, d_in=3, n=4)
    y, last = run(case, lib)
    b, L, d_in = case["u"].shape
    n = case["A_log"].shape[1]
    state = np.zeros((b, d_in, n))
    for t in range(L):
        state, yt = oracle.state_update(state, case["u"][:, t], case["delta"][:, t], case["A_log"], case["B"][:, t],
                                        case["C"][:, t], case["D"], case["z"][:, t], case["delta_bias"], True, lib=lib)
        _close(yt, y[:, t], rtol=1e-12, atol=1e-13, what=f"chain of steps y[{t}]")
    _close(state, last, rtol=1e-12, atol=1e-13, what="chain of steps state")
    # prefill on the first L1 steps, then decode the rest from its last_state
    L1 = 7
    pre = {k: (v[:, :L1] if isinstance(v, np.ndarray) and v.ndim == 3 else v) for k, v in case.items()}
    _, st = run(pre, lib)
    for t in range(L1, L):
        st, yt = oracle.state_update(st, case["u"][:, t], case["delta"][:, t], case["A_log"], case["B"][:, t],
                                     case["C"][:, t], case["D"], case["z"][:, t], case["delta_bias"], True, lib=lib)
        _close(yt, y[:, t], rtol=1e-12, atol=1e-13, what=f"prefill->decode y[{t}]")


def pin_bias_placement(lib):
    """softplus(delta + bias): scanning (delta, bias) equals scanning (delta + bias, no bias)."""
    case = random_case(17, b=1, L=8, d_in=3, n=2)
    y1, l1 = run(case, lib)
    c2 = dict(case, delta=case["delta"] + case["delta_bias"], delta_bias=None)
    y2, l2 = run(c2, lib)
    _close(y1, y2, rtol=1e-13, atol=1e-14, what="bias inside softplus")
    _close(l1, l2, rtol=1e-13, atol=1e-14, what="bias inside softplus (state)")


def pin_initial_state(lib):
    """An initial state h0: zero h0 is no h0; closed form at n = 1; brute force; a split scan is the whole scan."""
    case = random_case(18, b=2, L=9, d_in=3, n=4)
    y, last = run(case, lib)
    c0 = dict(case, h0=np.zeros((2, 3, 4)))
    y0, l0 = run(c0, lib)
    assert np.array_equal(y, y0) and np.array_equal(last, l0), "zero h0 must equal no h0"
    # n = 1, constant Delta, B, u: h_t = a^t h0 + Delta B u (1 - a^t) / (1 - a).
    L = 30
    A_exp, Delta, Bv, uv, h0v = 1.7, 0.45, -0.6, 1.1, 2.5
    Cc = _rng(19).standard_normal((1, L, 1))
    y1, l1 = oracle.scan(np.full((1, L, 1), uv), np.full((1, L, 1), Delta), np.array([[math.log(A_exp)]]),
                         np.full((1, L, 1), Bv), Cc, np.array([0.0]), None, None, False, lib=lib,
                         h0=np.array([[[h0v]]]))
    a = math.exp(-A_exp * Delta)
    t = np.arange(1, L + 1)
    h = a ** t * h0v + Delta * Bv * uv * (1 - a ** t) / (1 - a)
    _close(y1[0, :, 0], Cc[0, :, 0] * h, rtol=1e-12, atol=1e-14, what="h0 closed form")
    _close(l1[0, 0, 0], h[-1], what="h0 closed form last")
    for seed, kw in enumerate([dict(), dict(n=1, gated=False), dict(bias=False, n=6)]):
        c = random_case(200 + seed, **kw)
        c["h0"] = _rng(300 + seed).standard_normal((c["u"].shape[0], c["u"].shape[2], c["A_log"].shape[1]))
        yb, lb = brute_force(c)
        yo, lo = run(c, lib)
        _close(yo, yb, rtol=1e-11, atol=1e-12, what=f"h0 brute force y {kw}")
        _close(lo, lb, rtol=1e-11, atol=1e-12, what=f"h0 brute force last {kw}")
    # The second part of a split scan, started from the first part's state, equals the whole scan.
    L1 = 4
    first = {k: (v[:, :L1] if isinstance(v, np.ndarray) and v.ndim == 3 and k not in ("h0",) else v)
             for k, v in case.items()}
    rest = {k: (v[:, L1:] if isinstance(v, np.ndarray) and v.ndim == 3 and k not in ("h0",) else v)
            for k, v in case.items()}
    _, s1 = run(first, lib)
    rest["h0"] = s1
    y2, l2 = run(rest, lib)
    _close(y2, y[:, L1:], rtol=1e-12, atol=1e-13, what="split scan y")
    _close(l2, last, rtol=1e-12, atol=1e-13, what="split scan last")


def pin_zoh(lib):
    """Zero-order-hold input weight: closed form at n = 1, brute force, the A -> 0 limit (Euler), step == scan."""
    L = 30
    for A_exp, Delta, h0v in ((1.7, 0.45, 0.0), (0.2, 1.3, -0.7), (12.0, 0.02, 3.0)):
        Bv, uv = -0.6, 1.1
        Cc = _rng(20).standard_normal((1, L, 1))
        y, last = oracle.scan(np.full((1, L, 1), uv), np.full((1, L, 1), Delta), np.array([[math.log(A_exp)]]),
                              np.full((1, L, 1), Bv), Cc, np.array([0.0]), None, None, False, lib=lib,
                              h0=np.array([[[h0v]]]), zoh=True)
        A = -A_exp
        a = math.exp(A * Delta)
        t = np.arange(1, L + 1)
        h = a ** t * h0v - Bv * uv / A * (1 - a ** t)      # weight (a - 1)/A: the geometric sum telescopes
        _close(y[0, :, 0], Cc[0, :, 0] * h, rtol=1e-12, atol=1e-14, what=f"zoh closed form A={A}")
        _close(last[0, 0, 0], h[-1], rtol=1e-12, atol=1e-14, what=f"zoh closed form last A={A}")
    for seed, kw in enumerate([dict(), dict(n=1, gated=False), dict(bias=False, n=5, softplus=False)]):
        c = random_case(400 + seed, **kw)
        if not c["delta_softplus"]:
            c["delta"] = np.abs(c["delta"]) + 0.05
        c["zoh"] = True
        yb, lb = brute_force(c)
        yo, lo = run(c, lib)
        _close(yo, yb, rtol=1e-11, atol=1e-12, what=f"zoh brute force y {kw}")
        _close(lo, lb, rtol=1e-11, atol=1e-12, what=f"zoh brute force last {kw}")
    # A -> 0: expm1(Delta A) / A -> Delta, so ZOH equals Euler.
    c = random_case(21, b=1, L=12, d_in=2, n=3)
    c["A_log"] = np.full((2, 3), -40.0)
    ye, le = run(c, lib)
    yz, lz = run(dict(c, zoh=True), lib)
    _close(yz, ye, rtol=1e-12, atol=1e-13, what="zoh -> Euler as A -> 0")
    # ZOH steps chained from zero equal the ZOH scan.
    c = random_case(22, b=2, L=7, d_in=3, n=4)
    y, last = run(dict(c, zoh=True), lib)
    state = np.zeros((2, 3, 4))
    for t in range(7):
        state, yt = oracle.state_update(state, c["u"][:, t], c["delta"][:, t], c["A_log"], c["B"][:, t], c["C"][:, t],
                                        c["D"], c["z"][:, t], c["delta_bias"], True, lib=lib, zoh=True)
        _close(yt, y[:, t], rtol=1e-12, atol=1e-13, what=f"zoh chain y[{t}]")
    _close(state, last, rtol=1e-12, atol=1e-13, what="zoh chain state")


def pin_conv_update(lib):
    """The convolution step before the SSM step in Mamba.step (jiafeimiao.top page, "Conv step").

    - Chained over a sequence from a zero window, the steps equal torch's
      depthwise conv1d with W - 1 zeros of left padding (a causal filter,
      out_t = sum_w weight[w] x_(t-W+1+w)), plus the bias, then silu -- for
      W = 1 .. 4;
    - with a one-hot weight at index j (no bias, no silu) the output is the
      input W-1-j steps back: a delay line;
    - after each step the window holds the last W inputs, oldest first;
    - a case worked by hand.
    """
    import torch

    r = _rng(23)
    b, d_in, L = 2, 3, 11
    for W in (1, 2, 3, 4):
        xs = r.standard_normal((L, b, d_in))
        weight = r.standard_normal((d_in, W))
        bias = r.standard_normal(d_in)
        st = np.zeros((b, d_in, W))
        outs = []
        for t in range(L):
            st, o = oracle.conv_update(st, xs[t], weight, bias, True, lib=lib)
            outs.append(o)
            want = np.stack([xs[t - W + 1 + w] if t - W + 1 + w >= 0 else np.zeros((b, d_in)) for w in range(W)], -1)
            _exact(st, want, what=f"conv window W={W} t={t}")
        xt = torch.from_numpy(np.ascontiguousarray(xs.transpose(1, 2, 0)))           # (b, d_in, L)
        ref = torch.nn.functional.conv1d(xt, torch.from_numpy(weight)[:, None, :], torch.from_numpy(bias),
                                         padding=W - 1, groups=d_in)[..., :L]
        ref = torch.nn.functional.silu(ref).numpy().transpose(2, 0, 1)              # (L, b, d_in)
        _close(np.stack(outs), ref, rtol=1e-12, atol=1e-13, what=f"conv chain vs conv1d W={W}")
    W = 4
    xs = r.standard_normal((L, b, d_in))
    for j in range(W):
        weight = np.zeros((d_in, W))
        weight[:, j] = 1.0
        st = np.zeros((b, d_in, W))
        for t in range(L):
            st, o = oracle.conv_update(st, xs[t], weight, None, False, lib=lib)
            lag = W - 1 - j
            _exact(o, xs[t - lag] if t >= lag else np.zeros((b, d_in)), what=f"delay j={j} t={t}")
    st, o = oracle.conv_update(np.array([[[1.0, 2.0, 3.0, 4.0]]]), np.array([[5.0]]), np.array([[1.0, 0.0, -1.0, 2.0]]),
                               np.array([0.5]), True, lib=lib)
    # window [2, 3, 4, 5]; 2*1 + 3*0 + 4*(-1) + 5*2 + 0.5 = 8.5; silu(8.5) = 8.5 / (1 + e^-8.5)
    _exact(st, [[[2.0, 3.0, 4.0, 5.0]]], what="hand-worked window")
    _close(o, [[8.5 / (1.0 + math.exp(-8.5))]], what="hand-worked output")


def _cross_case(seed, maps=2, H=3, W=5, d_in=3, n=2):
    r = _rng(seed)
    L = H * W
    return dict(x=r.standard_normal((maps, H, W, d_in)), delta=r.standard_normal((maps, 4, L, d_in)) - 1.0,
                A_log=r.uniform(-1.5, 1.5, (4, d_in, n)), B=r.standard_normal((maps, 4, L, n)),
                C=r.standard_normal((maps, 4, L, n)), D=r.standard_normal((4, d_in)),
                delta_bias=r.uniform(-1.0, 0.5, (4, d_in)))


def pin_cross_scan(lib):
    """VMamba's cross scan and merge (githubissues.com VMamba issue 206: they only arrange the sequence).

    - The four sequences arranged with torch (reshape, transpose, flip) rather than
      index arithmetic, each scanned with the plain scan, and merged back through the
      inverse arrangement, give the same y and last states;
    - B = 0: every direction returns D_k u, so y = (sum_k D_k) x everywhere;
    - transposing the map swaps the row- and column-major directions: the cross
      scan of x^T with directions (1, 0, 3, 2) is the transposed cross scan of x.
    """
    import torch

    for (H, W, n) in ((3, 5, 2), (4, 1, 1), (1, 6, 3), (5, 5, 1)):
        c = _cross_case(31 + H * W, H=H, W=W, n=n)
        y, last = oracle.cross_scan(c["x"], c["delta"], c["A_log"], c["B"], c["C"], c["D"], c["delta_bias"], True, lib=lib)
        x = torch.from_numpy(c["x"])
        maps, d_in, L = x.shape[0], x.shape[3], H * W
        row = x.reshape(maps, L, d_in)
        col = x.transpose(1, 2).reshape(maps, L, d_in)
        seqs = [row, col, row.flip(1), col.flip(1)]
        ys = []
        for k in range(4):
            yk, lk = oracle.scan(seqs[k].numpy(), c["delta"][:, k], c["A_log"][k], c["B"][:, k], c["C"][:, k], c["D"][k],
                                 None, c["delta_bias"][k], True, lib=lib)
            _close(last[:, k], lk, rtol=1e-13, atol=1e-14, what=f"cross last state k={k} {H}x{W}")
            ys.append(torch.from_numpy(yk))
        want = (ys[0].reshape(maps, H, W, d_in) + ys[1].reshape(maps, W, H, d_in).transpose(1, 2)
                + ys[2].flip(1).reshape(maps, H, W, d_in) + ys[3].flip(1).reshape(maps, W, H, d_in).transpose(1, 2))
        _close(y, want.numpy(), rtol=1e-12, atol=1e-13, what=f"cross scan vs torch arrangement {H}x{W}")
        sw = [1, 0, 3, 2]
        yT, lT = oracle.cross_scan(np.ascontiguousarray(c["x"].transpose(0, 2, 1, 3)), c["delta"][:, sw], c["A_log"][sw],
                                   c["B"][:, sw], c["C"][:, sw], c["D"][sw], c["delta_bias"][sw], True, lib=lib)
        _close(yT, y.transpose(0, 2, 1, 3), rtol=1e-12, atol=1e-13, what=f"cross scan transposed {H}x{W}")
        _close(lT, last[:, sw], rtol=1e-13, atol=1e-14, what=f"cross last transposed {H}x{W}")
    c = _cross_case(41)
    y, _ = oracle.cross_scan(c["x"], c["delta"], c["A_log"], np.zeros_like(c["B"]), c["C"], c["D"], c["delta_bias"], True,
                             lib=lib)
    _close(y, c["x"] * c["D"].sum(0), rtol=1e-13, atol=1e-14, what="cross scan with B = 0")


def _torch_scan_loss(c, dy, dlast, softplus=True, zoh=False):
    """The scan written with torch float64 operations, and <y, dy> + <last state, dlast>; zoh: the input
    weight (exp(delta A) - 1)/A of the zero-order hold in place of Euler's delta."""
    import torch

    u, delta, A_log, B, C, D = (c[k] for k in ("u", "delta", "A_log", "B", "C", "D"))
    b, L, d_in = u.shape
    A = -torch.exp(A_log)
    h = c["h0"] if c.get("h0") is not None else torch.zeros(b, d_in, A.shape[1], dtype=torch.float64)
    loss = 0.0
    for t in range(L):
        x = delta[:, t] + (c["delta_bias"] if c.get("delta_bias") is not None else 0.0)
        dl = torch.nn.functional.softplus(x) if softplus else x
        if zoh:
            h = torch.exp(dl[..., None] * A) * h + torch.expm1(dl[..., None] * A) / A * (u[:, t, :, None] * B[:, t, None, :])
        else:
            h = torch.exp(dl[..., None] * A) * h + (dl * u[:, t])[..., None] * B[:, t, None, :]
        y = (h * C[:, t, None, :]).sum(-1) + D * u[:, t]
        if c.get("z") is not None:
            y = y * torch.nn.functional.silu(c["z"][:, t])
        loss = loss + (y * dy[:, t]).sum()
    if dlast is not None:
        loss = loss + (h * dlast).sum()
    return loss


def pin_scan_bwd(lib):
    """Gradients of the scan (Euler and zero-order-hold input terms): torch autograd of the scan written
    with torch ops, and central finite differences of the oracle's own forward along random directions."""
    import torch

    names = ("u", "delta", "A_log", "B", "C", "D", "z", "delta_bias", "h0")
    grad_of = dict(u="du", delta="ddelta", A_log="dA_log", B="dB", C="dC", D="dD", z="dz", delta_bias="ddelta_bias",
                   h0="dh0")
    for seed, kw, with_h0, with_dlast, sp, zoh in ((50, dict(), True, True, True, False),
                                                   (51, dict(n=1, gated=False), False, True, True, False),
                                                   (52, dict(bias=False, n=3), True, False, True, False),
                                                   (53, dict(softplus=False, L=6), False, False, False, False),
                                                   (54, dict(), True, True, True, True),
                                                   (55, dict(n=2, gated=False, bias=False), False, True, True, True),
                                                   (56, dict(softplus=False, L=7), True, False, False, True)):
        c = random_case(seed, **kw)
        if not sp:
            c["delta"] = np.abs(c["delta"]) * 0.3 + 0.05
        r = _rng(seed + 100)
        b, L, d_in = c["u"].shape
        n = c["A_log"].shape[1]
        c["h0"] = r.standard_normal((b, d_in, n)) if with_h0 else None
        dy = r.standard_normal((b, L, d_in))
        dlast = r.standard_normal((b, d_in, n)) if with_dlast else None
        got = oracle.scan_bwd(c["u"], c["delta"], c["A_log"], c["B"], c["C"], c["D"], c["z"], c["delta_bias"], sp,
                              c["h0"], dy, dlast, lib=lib, zoh=zoh)
        tc = {k: (None if c.get(k) is None else torch.tensor(c[k], dtype=torch.float64, requires_grad=True))
              for k in names}
        loss = _torch_scan_loss(tc, torch.tensor(dy), None if dlast is None else torch.tensor(dlast), sp, zoh)
        loss.backward()
        for k in names:
            if tc[k] is not None:
                _close(got[grad_of[k]], tc[k].grad.numpy(), rtol=1e-10, atol=1e-11, what=f"d{k} vs autograd {kw} zoh={zoh}")
        # finite differences: <grad, v> = (L(x + e v) - L(x - e v)) / 2e
        def loss_at(cc):
            y, last = oracle.scan(cc["u"], cc["delta"], cc["A_log"], cc["B"], cc["C"], cc["D"], cc["z"],
                                  cc["delta_bias"], sp, lib=lib, h0=cc["h0"], zoh=zoh)
            return float((y * dy).sum() + ((last * dlast).sum() if dlast is not None else 0.0))
        for j in range(3):
            v = {k: (None if c.get(k) is None else r.standard_normal(np.shape(c[k]))) for k in names}
            eps = 1e-6
            plus = {k: (None if c.get(k) is None else c[k] + eps * v[k]) for k in names}
            minus = {k: (None if c.get(k) is None else c[k] - eps * v[k]) for k in names}
            fd = (loss_at(plus) - loss_at(minus)) / (2 * eps)
            an = sum(float((got[grad_of[k]] * v[k]).sum()) for k in names if c.get(k) is not None)
            assert abs(fd - an) <= 1e-6 * (1 + abs(an)), f"finite differences {kw} zoh={zoh}: {fd} vs {an}"


def pin_segment_sum_closed_form(lib):
    """A second formulation with no recurrence at all, in numpy float64: since A is constant in time, the product
    of the decays exp(delta'_r A) over r = s+1..t is exp(A (S_t - S_s)) with S the cumulative sum of delta' along
    the sequence, so h_t = sum_{s<=t} exp(A (S_t - S_s)) delta'_s B_s u_s (a lower-triangular matrix of those
    factors applied to the inputs), and y_t = sum_k C_t,k h_t,k + D u_t, gated.  The oracle's sequential loop
    (update, then read out) must agree with it, and its last state with h_(L-1)."""
    for seed, kw in enumerate([dict(), dict(n=1, gated=False, bias=False), dict(b=3, L=11, d_in=5, n=6),
                               dict(L=40, softplus=False)]):
        c = random_case(900 + seed, **kw)
        if not c["delta_softplus"]:
            # Without the softplus the step size is delta + bias itself: keep it positive.
            c["delta"] = np.abs(c["delta"]) * 0.1 + 0.01
            if c["delta_bias"] is not None:
                c["delta_bias"] = np.abs(c["delta_bias"]) * 0.01
        x = c["delta"] + (c["delta_bias"] if c["delta_bias"] is not None else 0.0)
        dl = np.logaddexp(0.0, x) if c["delta_softplus"] else x                   # (b, L, d)
        A = -np.exp(c["A_log"])                                                   # (d, n)
        S = np.cumsum(dl, axis=1)                                                 # (b, L, d)
        L = dl.shape[1]
        tri = np.tril(np.ones((L, L), bool))                                      # s <= t
        # E[b, t, s, d, k] = exp(A[d, k] (S[b, t, d] - S[b, s, d])) for s <= t, else 0
        diff = S[:, :, None, :] - S[:, None, :, :]                                 # (b, t, s, d)
        E = np.where(tri[None, :, :, None, None], np.exp(diff[..., None] * A[None, None, None]), 0.0)
        inp = (dl * c["u"])[:, :, :, None] * c["B"][:, :, None, :]                 # (b, s, d, k)
        h = np.einsum("btsdk,bsdk->btdk", E, inp)                                 # (b, t, d, k)
        y = np.einsum("btdk,btk->btd", h, c["C"]) + c["D"] * c["u"]
        if c["z"] is not None:
            y = y * c["z"] / (1.0 + np.exp(-c["z"]))
        yo, lo = run(c, lib)
        _close(yo, y, rtol=1e-11, atol=1e-12, what=f"segment-sum closed form y {kw}")
        _close(lo, h[:, -1], rtol=1e-11, atol=1e-12, what=f"segment-sum closed form last state {kw}")


ALL_PINS = [pin_softplus_silu, pin_hand_worked, pin_brute_force, pin_geometric_closed_form, pin_limits,
            pin_skip_and_gate, pin_linearity_causality, pin_step_matches_scan, pin_bias_placement,
            pin_initial_state, pin_zoh, pin_conv_update, pin_cross_scan, pin_scan_bwd, pin_segment_sum_closed_form]
