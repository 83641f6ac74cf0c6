"""CPU: the C ABI of libss_scan.so -- it loads, exports every declared entry
point, and rejects bad arguments with the documented status before it touches
the GPU (no compute call is made here; the pointers are fake addresses that
are never dereferenced because validation fails first)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ss_scan.h")

OK, NULL, SHAPE, DTYPE, UNSUP, WS, HIP, ALIAS, ALIGN, MODE, TIMEOUT = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10


@pytest.fixture(scope="module")
def ss():
    import selective_state_space_softplus_amd as ss

    return ss


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ss_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(["ss_conv_update", "ss_cross_scan_fwd", "ss_cross_scan_fwd_workspace_bytes",
                                           "ss_cross_scan_fwd_ex", "ss_cross_scan_fwd_ex_workspace_bytes",
                                           "ss_scan_bwd", "ss_scan_bwd_ex", "ss_scan_bwd_workspace_bytes", "ss_scan_fwd",
                                           "ss_scan_fwd_ex", "ss_scan_fwd_noalloc", "ss_scan_status",
                                           "ss_scan_fwd_workspace_bytes", "ss_set_test_plan", "ss_state_update",
                                           "ss_state_update_ex", "ss_status_string", "ss_scan_checkpoint_bytes",
                                           "ss_scan_fwd_save", "ss_scan_bwd_saved",
                                           "ss_scan_bwd_saved_workspace_bytes"])


def test_library_exports_every_declared_symbol(ss):
    lib = ctypes.CDLL(ss.LIBRARY)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(ss.EXPORTS)


def test_status_strings(ss):
    for code in (OK, NULL, SHAPE, DTYPE, UNSUP, WS, HIP, ALIAS, ALIGN, MODE, TIMEOUT):
        s = ss.status_string(code)
        assert s and s != "unknown status"
    assert ss.status_string(12345) == "unknown status"


def test_status_codes_match_header(ss):
    text = open(HEADER).read()
    for name, code in (("SS_OK", OK), ("SS_ERR_NULL", NULL), ("SS_ERR_SHAPE", SHAPE), ("SS_ERR_DTYPE", DTYPE),
                       ("SS_ERR_UNSUPPORTED", UNSUP), ("SS_ERR_WORKSPACE", WS), ("SS_ERR_HIP", HIP),
                       ("SS_ERR_ALIAS", ALIAS), ("SS_ERR_ALIGN", ALIGN), ("SS_ERR_MODE", MODE),
                       ("SS_ERR_TIMEOUT", TIMEOUT)):
        assert re.search(rf"\b{name}\s*=\s*{code}\b", text), name
        assert ss.STATUS[code] == name
    for name, code in (("SS_DISC_EULER", ss.SS_DISC_EULER), ("SS_DISC_ZOH", ss.SS_DISC_ZOH)):
        assert re.search(rf"\b{name}\s*=\s*{code}\b", text), name


def test_workspace_query(ss):
    q = ss.scan_fwd_workspace_bytes
    assert q(4, 8192, 5120, 16, 1) > 0
    assert q(4, 8192, 5120, 16, 1) == q(4, 8192, 5120, 16, 0)       # independent of the element type
    assert q(4, 8192, 5120, 16, 1) == q(4, 100, 5120, 16, 1)        # and of L
    assert q(4, 8192, 5120, 16, 1) >= 15 * 4 * 80 * 16 * 64 * 4     # room for 15 published states per group
    for bad in ((0, 1, 1, 1, 0), (1, 0, 1, 1, 0), (1, 1, -1, 1, 0), (1, 1, 1, 0, 0), (1, 1, 1, 65, 0),
                (1, 1, 1, 1, 2), (1 << 30, 1 << 30, 1, 1, 0)):
        assert q(*bad) == 0, bad


# fake, well-separated, aligned "device" addresses: validation never dereferences them
BASE = 1 << 40


def addr(i):
    return BASE + i * (1 << 32)


def scan_args(**over):
    a = dict(u=addr(1), delta=addr(2), A_log=addr(3), B=addr(4), C=addr(5), D=addr(6), z=addr(7), bias=addr(8),
             softplus=1, y=addr(9), last=addr(10), b=2, L=64, d_in=32, n=16, dtype=0, ws=addr(11),
             ws_bytes=1 << 30, stream=None)
    a.update(over)
    return a


def call_scan(ss, a):
    return ss.lib.ss_scan_fwd(a["u"], a["delta"], a["A_log"], a["B"], a["C"], a["D"], a["z"], a["bias"],
                              a["softplus"], a["y"], a["last"], a["b"], a["L"], a["d_in"], a["n"], a["dtype"],
                              a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(u=None), NULL), (dict(delta=None), NULL), (dict(A_log=None), NULL), (dict(B=None), NULL),
    (dict(C=None), NULL), (dict(D=None), NULL), (dict(y=None), NULL),
    (dict(b=0), SHAPE), (dict(L=0), SHAPE), (dict(d_in=-3), SHAPE), (dict(n=0), SHAPE),
    (dict(b=1 << 24, L=1 << 24, d_in=1 << 24), SHAPE),
    (dict(dtype=2), DTYPE), (dict(dtype=-1), DTYPE),
    (dict(n=65), UNSUP), (dict(n=1000), UNSUP),
    (dict(ws=None), WS), (dict(ws_bytes=100), WS),
    (dict(u=addr(1) + 2), ALIGN), (dict(dtype=1, u=addr(1) + 1), ALIGN), (dict(A_log=addr(3) + 2), ALIGN),
    (dict(last=addr(10) + 1), ALIGN),
    (dict(y=addr(1) + 64), ALIAS), (dict(last=addr(4)), ALIAS), (dict(y=addr(10)), ALIAS),
    (dict(ws=addr(9)), ALIAS), (dict(ws=addr(1)), ALIAS), (dict(last=addr(8) + 4), ALIAS),
    (dict(ws=addr(11) + 4), ALIGN), (dict(ws=addr(11) + 128), ALIGN),
])
def test_scan_rejects(ss, over, code):
    assert call_scan(ss, scan_args(**over)) == code


def call_scan_noalloc(ss, a, h0=None, disc=0):
    return ss.lib.ss_scan_fwd_noalloc(a["u"], a["delta"], a["A_log"], a["B"], a["C"], a["D"], a["z"], a["bias"],
                                      a["softplus"], h0, disc, a["y"], a["last"], a["b"], a["L"], a["d_in"], a["n"],
                                      a["dtype"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(u=None), NULL), (dict(y=None), NULL), (dict(b=0), SHAPE), (dict(dtype=2), DTYPE), (dict(n=65), UNSUP),
    (dict(u=addr(1) + 2), ALIGN), (dict(y=addr(1) + 64), ALIAS), (dict(last=addr(4)), ALIAS),
])
def test_scan_noalloc_rejects_before_touching_the_device(ss, over, code):
    # The static scratch is looked up only after validation, so these run without a GPU.
    assert call_scan_noalloc(ss, scan_args(**over)) == code
    assert call_scan_noalloc(ss, scan_args(), disc=7) == MODE


def test_scan_status_rejects(ss):
    out = ctypes.c_void_p(addr(20))
    assert ss.lib.ss_scan_status(addr(11), 1 << 20, None, None) == NULL
    assert ss.lib.ss_scan_status(addr(11), 100, out, None) == WS
    assert ss.lib.ss_scan_status(addr(11) + 4, 1 << 20, out, None) == ALIGN
    assert ss.lib.ss_scan_status(addr(11), 1 << 20, ctypes.c_void_p(addr(20) + 2), None) == ALIGN


def test_test_plan_validates_and_resets(ss):
    bad = ((-1, 0, 0, 0, 0), (17, 0, 0, 0, 0), (0, 2, 0, 0, 0), (0, 0, 2, 0, 0), (0, 0, 0, -5, 0), (0, 0, 0, 0, 3))
    for args in bad:
        assert ss.lib.ss_set_test_plan(*args) == SHAPE, args
    assert ss.lib.ss_set_test_plan(4, 4, 1, 100, 1) == OK
    assert ss.lib.ss_set_test_plan(0, 0, 0, 0, 0) == OK
    with ss.test_plan(segments=3):
        pass
    with pytest.raises(ss.SSError):
        with ss.test_plan(segments=99):
            pass


def test_scan_optional_pointers_may_be_null(ss):
    # z, bias and last_state are optional: with them NULL and a bad dtype the
    # dtype error (not a NULL error) is what comes back.
    assert call_scan(ss, scan_args(z=None, bias=None, last=None, dtype=9)) == DTYPE


def step_args(**over):
    a = dict(state=addr(1), x=addr(2), dt=addr(3), A_log=addr(4), B=addr(5), C=addr(6), D=addr(7), z=addr(8),
             bias=addr(9), softplus=1, y=addr(10), b=256, d_in=5120, n=16, dtype=1, stream=None)
    a.update(over)
    return a


def call_step(ss, a):
    return ss.lib.ss_state_update(a["state"], a["x"], a["dt"], a["A_log"], a["B"], a["C"], a["D"], a["z"], a["bias"],
                                  a["softplus"], a["y"], a["b"], a["d_in"], a["n"], a["dtype"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(state=None), NULL), (dict(x=None), NULL), (dict(dt=None), NULL), (dict(A_log=None), NULL),
    (dict(B=None), NULL), (dict(C=None), NULL), (dict(D=None), NULL), (dict(y=None), NULL),
    (dict(b=0), SHAPE), (dict(d_in=0), SHAPE), (dict(n=-1), SHAPE), (dict(dtype=3), DTYPE), (dict(n=65), UNSUP),
    (dict(state=addr(1) + 2), ALIGN), (dict(x=addr(2) + 1), ALIGN),
    (dict(y=addr(2)), ALIAS), (dict(state=addr(9)), ALIAS), (dict(y=addr(1) + 8), ALIAS),
])
def test_step_rejects(ss, over, code):
    assert call_step(ss, step_args(**over)) == code


def test_python_binding_checks_tensors(ss):
    import torch

    u = torch.zeros(2, 8, 4)
    with pytest.raises((TypeError, ValueError)):
        ss.scan_fwd(u, u, torch.zeros(4, 16), torch.zeros(2, 8, 16), torch.zeros(2, 8, 16),
                    torch.zeros(4, dtype=torch.float64))
    with pytest.raises((TypeError, ValueError)):
        ss.scan_fwd(u, u[:, :4], torch.zeros(4, 16), torch.zeros(2, 8, 16), torch.zeros(2, 8, 16), torch.zeros(4))


def call_scan_ex(ss, a, h0=None, disc=0):
    return ss.lib.ss_scan_fwd_ex(a["u"], a["delta"], a["A_log"], a["B"], a["C"], a["D"], a["z"], a["bias"],
                                 a["softplus"], h0, disc, a["y"], a["last"], a["b"], a["L"], a["d_in"], a["n"],
                                 a["dtype"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,h0,disc,code", [
    ({}, None, 2, MODE), ({}, None, -1, MODE), ({}, addr(12), 7, MODE),
    ({}, addr(12) + 2, 0, ALIGN),
    ({}, addr(9), 1, ALIAS),                      # initial state on top of y
    ({}, addr(10) + 4, 0, ALIAS),                 # initial state partly over last_state
    ({}, addr(11) + 64, 1, ALIAS),                # initial state inside the workspace
    (dict(ws_bytes=100), addr(10), 1, WS),        # in place (== last_state) passes the alias check
    (dict(ws_bytes=100), addr(12), 1, WS),
    (dict(n=0), addr(12), 1, SHAPE), (dict(u=None), addr(12), 1, NULL),
])
def test_scan_ex_rejects(ss, over, h0, disc, code):
    assert call_scan_ex(ss, scan_args(**over), h0, disc) == code


def test_scan_ex_is_scan_with_defaults(ss):
    # With no initial state and Euler weights, every rejection matches ss_scan_fwd's.
    for over in (dict(u=None), dict(b=0), dict(dtype=2), dict(n=65), dict(ws=None), dict(u=addr(1) + 2),
                 dict(y=addr(10)), dict(ws_bytes=100)):
        a = scan_args(**over)
        assert call_scan_ex(ss, a) == call_scan(ss, a), over


def test_step_ex_rejects(ss):
    a = step_args()
    args = lambda a, disc: (a["state"], a["x"], a["dt"], a["A_log"], a["B"], a["C"], a["D"], a["z"],  # noqa: E731
                            a["bias"], a["softplus"], disc, a["y"], a["b"], a["d_in"], a["n"], a["dtype"], a["stream"])
    assert ss.lib.ss_state_update_ex(*args(a, 2)) == MODE
    assert ss.lib.ss_state_update_ex(*args(a, -3)) == MODE
    for over, code in ((dict(x=None), NULL), (dict(n=65), UNSUP), (dict(y=addr(2)), ALIAS)):
        assert ss.lib.ss_state_update_ex(*args(step_args(**over), 1)) == code, over


def test_python_binding_checks_initial_state(ss):
    import torch

    u = torch.zeros(2, 8, 4)
    with pytest.raises((TypeError, ValueError)):
        ss.scan_fwd(u, u, torch.zeros(4, 16), torch.zeros(2, 8, 16), torch.zeros(2, 8, 16), torch.zeros(4),
                    initial_state=torch.zeros(2, 4, 15))


def conv_args(**over):
    a = dict(state=addr(1), x=addr(2), weight=addr(3), bias=addr(4), silu=1, out=addr(5), b=256, d_in=5120, W=4,
             dtype=1, stream=None)
    a.update(over)
    return a


def call_conv(ss, a):
    return ss.lib.ss_conv_update(a["state"], a["x"], a["weight"], a["bias"], a["silu"], a["out"], a["b"], a["d_in"],
                                 a["W"], a["dtype"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(state=None), NULL), (dict(x=None), NULL), (dict(weight=None), NULL), (dict(out=None), NULL),
    (dict(b=0), SHAPE), (dict(d_in=-1), SHAPE), (dict(W=0), SHAPE), (dict(b=1 << 20, d_in=1 << 10), SHAPE),
    (dict(dtype=2), DTYPE), (dict(W=9), UNSUP),
    (dict(state=addr(1) + 1), ALIGN), (dict(dtype=0, x=addr(2) + 2), ALIGN), (dict(weight=addr(3) + 2), ALIGN),
    (dict(out=addr(1) + 8), ALIAS), (dict(out=addr(2)), ALIAS), (dict(state=addr(3)), ALIAS),
    (dict(state=addr(4) - 8), ALIAS), (dict(out=addr(4)), ALIAS),
])
def test_conv_rejects(ss, over, code):
    assert call_conv(ss, conv_args(**over)) == code


def test_conv_bias_is_optional(ss):
    assert call_conv(ss, conv_args(bias=None, dtype=7)) == DTYPE


def cross_args(**over):
    a = dict(x=addr(1), delta=addr(2), A_log=addr(3), B=addr(4), C=addr(5), D=addr(6), bias=addr(7), softplus=1,
             y=addr(8), last=addr(9), maps=16, H=56, W=56, d_in=384, n=1, dtype=0, form=0, ws=addr(10),
             ws_bytes=1 << 30, stream=None)
    a.update(over)
    return a


def call_cross(ss, a):
    return ss.lib.ss_cross_scan_fwd_ex(a["x"], a["delta"], a["A_log"], a["B"], a["C"], a["D"], a["bias"],
                                       a["softplus"], a["y"], a["last"], a["maps"], a["H"], a["W"], a["d_in"], a["n"],
                                       a["dtype"], a["form"], a["ws"], a["ws_bytes"], a["stream"])


TWO_PASS_WS = 16 * 16 * 3136 * 384


@pytest.mark.parametrize("over,code", [
    (dict(x=None), NULL), (dict(delta=None), NULL), (dict(A_log=None), NULL), (dict(B=None), NULL),
    (dict(C=None), NULL), (dict(D=None), NULL), (dict(y=None), NULL),
    (dict(maps=0), SHAPE), (dict(H=0), SHAPE), (dict(W=-2), SHAPE), (dict(d_in=0), SHAPE), (dict(n=0), SHAPE),
    (dict(H=1 << 16, W=1 << 16), SHAPE), (dict(maps=1 << 45), SHAPE),
    (dict(dtype=3), DTYPE), (dict(n=65), UNSUP), (dict(form=3), MODE), (dict(form=-1), MODE),
    (dict(form=1, n=5), UNSUP), (dict(form=1, H=64, W=67), UNSUP), (dict(form=1, H=64, W=64, n=3), UNSUP),
    (dict(ws=None), WS), (dict(ws_bytes=10), WS), (dict(ws_bytes=TWO_PASS_WS - 1), WS),
    (dict(form=2, ws_bytes=TWO_PASS_WS - 1), WS), (dict(form=1, ws_bytes=255), WS),
    (dict(x=addr(1) + 2), ALIGN), (dict(y=addr(8) + 2), ALIGN), (dict(last=addr(9) + 1), ALIGN),
    (dict(ws=addr(10) + 16), ALIGN), (dict(form=1, ws=addr(10) + 16), ALIGN),
    (dict(y=addr(1)), ALIAS), (dict(last=addr(3)), ALIAS), (dict(y=addr(9)), ALIAS), (dict(ws=addr(8)), ALIAS),
    (dict(bias=addr(9) + 8), ALIAS), (dict(form=1, y=addr(1)), ALIAS),
])
def test_cross_rejects(ss, over, code):
    assert call_cross(ss, cross_args(**over)) == code


def test_cross_plain_entry_is_the_auto_form(ss):
    a = cross_args(ws_bytes=TWO_PASS_WS - 1)
    assert ss.lib.ss_cross_scan_fwd(a["x"], a["delta"], a["A_log"], a["B"], a["C"], a["D"], a["bias"], a["softplus"],
                                    a["y"], a["last"], a["maps"], a["H"], a["W"], a["d_in"], a["n"], a["dtype"],
                                    a["ws"], a["ws_bytes"], a["stream"]) == WS


def test_cross_optional_pointers_may_be_null(ss):
    assert call_cross(ss, cross_args(bias=None, last=None, dtype=5)) == DTYPE


def test_cross_workspace_query(ss):
    q = ss.lib.ss_cross_scan_fwd_workspace_bytes
    qx = ss.lib.ss_cross_scan_fwd_ex_workspace_bytes
    full = q(16, 56, 56, 384, 1, 0)
    assert full >= TWO_PASS_WS + ss.scan_fwd_workspace_bytes(64, 3136, 384, 1, 0)
    assert full == q(16, 56, 56, 384, 1, 1) == qx(16, 56, 56, 384, 1, 0, 0) == qx(16, 56, 56, 384, 1, 0, 2)
    # One pass: the status words only, where the map's sum fits in LDS (n <= 4).
    assert qx(16, 56, 56, 384, 1, 0, 1) == 256 == qx(16, 56, 56, 384, 4, 1, 1) == qx(3, 64, 65, 8, 2, 0, 1)
    assert qx(1, 4265, 1, 8, 1, 0, 1) == 256 and qx(1, 4266, 1, 8, 1, 0, 1) == 0
    assert qx(1, 4205, 1, 8, 2, 0, 1) == 256 and qx(1, 4206, 1, 8, 2, 0, 1) == 0
    assert qx(1, 4084, 1, 8, 3, 0, 1) == 256 and qx(1, 4085, 1, 8, 4, 0, 1) == 0
    assert qx(1, 5, 5, 8, 5, 0, 1) == 0
    for bad in ((0, 5, 5, 8, 1, 0), (1, 0, 5, 8, 1, 0), (1, 5, 5, 8, 65, 0), (1, 5, 5, 8, 1, 2)):
        assert q(*bad) == 0, bad
        assert qx(*bad, 1) == 0, bad
    assert qx(1, 5, 5, 8, 1, 0, 7) == 0


def bwd_args(**over):
    a = dict(u=addr(1), delta=addr(2), A_log=addr(3), B=addr(4), C=addr(5), D=addr(6), z=addr(7), bias=addr(8),
             softplus=1, h0=addr(9), dy=addr(10), dlast=addr(11), du=addr(12), ddelta=addr(13), dA=addr(14),
             dB=addr(15), dC=addr(16), dD=addr(17), dz=addr(18), dbias=addr(19), dh0=addr(20), b=2, L=64, d_in=32,
             n=16, dtype=1, ws=addr(21), ws_bytes=1 << 30, stream=None)
    a.update(over)
    return a


def call_bwd(ss, a):
    k = ("u", "delta", "A_log", "B", "C", "D", "z", "bias", "softplus", "h0", "dy", "dlast", "du", "ddelta", "dA",
         "dB", "dC", "dD", "dz", "dbias", "dh0", "b", "L", "d_in", "n", "dtype", "ws", "ws_bytes", "stream")
    return ss.lib.ss_scan_bwd(*[a[x] for x in k])


@pytest.mark.parametrize("over,code", [
    (dict(u=None), NULL), (dict(dy=None), NULL), (dict(du=None), NULL), (dict(dA=None), NULL), (dict(dC=None), NULL),
    (dict(dz=None), NULL), (dict(b=0), SHAPE), (dict(L=-1), SHAPE), (dict(n=0), SHAPE), (dict(dtype=2), DTYPE),
    (dict(n=65), UNSUP), (dict(ws=None), WS), (dict(ws_bytes=100), WS), (dict(ws=addr(21) + 128), ALIGN),
    (dict(du=addr(12) + 1), ALIGN), (dict(dA=addr(14) + 2), ALIGN), (dict(dh0=addr(20) + 1), ALIGN),
    (dict(du=addr(1)), ALIAS), (dict(dB=addr(12)), ALIAS), (dict(dA=addr(3)), ALIAS), (dict(dh0=addr(9)), ALIAS),
    (dict(ws=addr(12)), ALIAS), (dict(dD=addr(19) - 8), ALIAS), (dict(dz=addr(21)), ALIAS),
])
def test_bwd_rejects(ss, over, code):
    assert call_bwd(ss, bwd_args(**over)) == code


def call_bwd_ex(ss, a, mode):
    k1 = ("u", "delta", "A_log", "B", "C", "D", "z", "bias", "softplus", "h0")
    k2 = ("dy", "dlast", "du", "ddelta", "dA", "dB", "dC", "dD", "dz", "dbias", "dh0", "b", "L", "d_in", "n", "dtype",
          "ws", "ws_bytes", "stream")
    return ss.lib.ss_scan_bwd_ex(*[a[x] for x in k1], mode, *[a[x] for x in k2])


@pytest.mark.parametrize("over,code", [
    (dict(u=None), NULL), (dict(dz=None), NULL), (dict(b=0), SHAPE), (dict(dtype=2), DTYPE), (dict(n=65), UNSUP),
    (dict(ws_bytes=100), WS), (dict(du=addr(12) + 1), ALIGN), (dict(du=addr(1)), ALIAS),
])
@pytest.mark.parametrize("mode", [0, 1])
def test_bwd_ex_rejects(ss, over, code, mode):
    assert call_bwd_ex(ss, bwd_args(**over), mode) == code


@pytest.mark.parametrize("mode", [-1, 2, 7])
def test_bwd_ex_rejects_unknown_discretization(ss, mode):
    assert call_bwd_ex(ss, bwd_args(), mode) == MODE


def test_bwd_optional_pointers_may_be_null(ss):
    # No gate (then dz may be NULL), no bias, no h0, no dlast, no dh0: only the dtype error remains.
    assert call_bwd(ss, bwd_args(z=None, dz=None, bias=None, dbias=None, h0=None, dlast=None, dh0=None, dtype=7)) == DTYPE


def test_bwd_workspace_query(ss):
    q = ss.lib.ss_scan_bwd_workspace_bytes
    assert q(4, 8192, 5120, 16, 1) > 4 * 1023 * 16 * 5120 * 4
    assert q(4, 8192, 5120, 65, 1) == 0 and q(0, 1, 1, 1, 0) == 0 and q(1, 1, 1, 1, 3) == 0


# ---- the training pair: ss_scan_fwd_save and ss_scan_bwd_saved


def call_fwd_save(ss, a, ck=addr(12), ypre=addr(13), disc=0):
    return ss.lib.ss_scan_fwd_save(a["u"], a["delta"], a["A_log"], a["B"], a["C"], a["D"], a["z"], a["bias"],
                                   a["softplus"], None, disc, a["y"], a["last"], ck, ypre, a["b"], a["L"], a["d_in"],
                                   a["n"], a["dtype"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,ck,ypre,code", [
    (dict(), None, addr(13), NULL),                       # no checkpoint buffer
    (dict(), addr(12), None, NULL),                       # gated without y_pre
    (dict(u=None), addr(12), addr(13), NULL),
    (dict(n=65), addr(12), addr(13), UNSUP),
    (dict(b=0), addr(12), addr(13), SHAPE),
    (dict(), addr(12) + 2, addr(13), ALIGN),
    (dict(), addr(12), addr(13) + 2, ALIGN),
    (dict(), addr(1), addr(13), ALIAS),                   # checkpoints over u
    (dict(), addr(12), addr(9), ALIAS),                   # y_pre over y
    (dict(), addr(12), addr(12) + 64, ALIAS),             # y_pre over the checkpoints
    (dict(), addr(11) + 256, addr(13), ALIAS),            # checkpoints in the workspace
    (dict(ws_bytes=100), addr(12), addr(13), WS),
])
def test_fwd_save_rejects(ss, over, ck, ypre, code):
    assert call_fwd_save(ss, scan_args(**over), ck, ypre) == code


def test_fwd_save_without_gate_needs_no_y_pre(ss):
    # Ungated: y_pre may be NULL; only the dtype error remains.
    assert call_fwd_save(ss, scan_args(z=None, dtype=5), addr(12), None) == DTYPE


def call_bwd_saved(ss, a, ck=addr(22), ypre=addr(23), mode=0):
    k1 = ("u", "delta", "A_log", "B", "C", "D", "z", "bias", "softplus", "h0")
    k2 = ("dy", "dlast", "du", "ddelta", "dA", "dB", "dC", "dD", "dz", "dbias", "dh0", "b", "L", "d_in", "n", "dtype",
          "ws", "ws_bytes", "stream")
    return ss.lib.ss_scan_bwd_saved(*[a[x] for x in k1], mode, ck, ypre, *[a[x] for x in k2])


@pytest.mark.parametrize("over,ck,ypre,code", [
    (dict(), None, addr(23), NULL), (dict(), addr(22), None, NULL), (dict(u=None), addr(22), addr(23), NULL),
    (dict(n=65), addr(22), addr(23), UNSUP), (dict(ws_bytes=100), addr(22), addr(23), WS),
    (dict(), addr(22) + 2, addr(23), ALIGN), (dict(), addr(22), addr(23) + 1, ALIGN),
    (dict(), addr(12), addr(23), ALIAS),                  # checkpoints over du
    (dict(), addr(22), addr(18), ALIAS),                  # y_pre over dz
    (dict(), addr(21) + 256, addr(23), ALIAS),            # checkpoints in the workspace
])
def test_bwd_saved_rejects(ss, over, ck, ypre, code):
    assert call_bwd_saved(ss, bwd_args(**over), ck, ypre) == code


def test_bwd_saved_without_gate_needs_no_y_pre(ss):
    assert call_bwd_saved(ss, bwd_args(z=None, dz=None, dtype=7), addr(22), None) == DTYPE


def test_training_pair_queries(ss):
    lib = ss.lib
    b, L, d, n = 4, 8192, 5120, 16
    assert lib.ss_scan_checkpoint_bytes(b, L, d, n) == b * ((L - 1) // 8) * n * d * 4
    assert lib.ss_scan_checkpoint_bytes(2, 8, 32, 16) == 0            # no checkpoint before step 8 < L
    assert lib.ss_scan_checkpoint_bytes(2, 9, 32, 16) == 2 * 1 * 16 * 32 * 4
    saved = lib.ss_scan_bwd_saved_workspace_bytes(b, L, d, n, 1)
    full = lib.ss_scan_bwd_workspace_bytes(b, L, d, n, 1)
    # The saved backward needs neither the forward pass's room nor checkpoints of its own.
    assert 0 < saved <= full - lib.ss_scan_checkpoint_bytes(b, L, d, n)
    for bad in ((0, 1, 1, 1), (1, 1, 1, 65), (1, 0, 1, 1)):
        assert lib.ss_scan_checkpoint_bytes(*bad) == 0, bad
        assert lib.ss_scan_bwd_saved_workspace_bytes(*bad, 0) == 0, bad
