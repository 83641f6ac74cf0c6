"""MI355X (gfx950) selective scan with a softplus step size, and its decode step.

A thin ctypes binding over ``libss_scan.so`` (built from ``csrc/`` by
``build.py``).  Every arithmetic step runs in the library's HIP kernels; this
module only checks tensor properties, allocates outputs and workspace with
PyTorch, and passes raw device pointers and the current HIP stream.  If the
library is missing, importing this package raises.

Entry points mirror the C ABI (``include/ss_scan.h``):

  scan_fwd(u, delta, A_log, B, C, D, z=None, delta_bias=None, delta_softplus=True,
           return_last_state=False, initial_state=None, zoh=False)
                                             -> y  or  (y, last_state)
  state_update(state, x, dt, A_log, B, C, D, z=None, dt_bias=None, dt_softplus=True,
               zoh=False)                    -> y  (state is updated in place)
  scan_bwd(u, delta, A_log, B, C, D, dy, z=None, delta_bias=None, delta_softplus=True,
           initial_state=None, dlast_state=None, zoh=False)  -> dict of gradients
  selective_scan(u, delta, A_log, B, C, D, z=None, delta_bias=None, delta_softplus=True,
                 initial_state=None, zoh=False) -> y, differentiable (torch.autograd.Function
                                                 calling scan_fwd / scan_bwd)
  cross_scan_fwd(x, delta, A_log, B, C, D, delta_bias=None, delta_softplus=True,
                 return_last_state=False, form="auto")
                                             -> y (maps, H, W, d_in) fp32  or  (y, last_state)
  conv_update(conv_state, x, weight, bias=None, silu=True)
                                             -> out (b, d_in)  (conv_state is updated in place)
  scan_fwd_workspace_bytes(b, L, d_in, n, dtype) -> int
  scan_status(workspace) -> int    (SS_OK, or SS_ERR_TIMEOUT if a segment wait gave up)
  status_string(code) -> str
  test_plan(segments=0, waves=0, time_parallel=0, spin_limit=0, wait_never=0)
                                             context manager over ss_set_test_plan (tests, tuning)

scan_fwd, cross_scan_fwd and scan_bwd take ``check=True`` to synchronise and
raise SSError(SS_ERR_TIMEOUT) when the call's status says a wait between
segments gave up (its outputs then hold NaN).  ``scan_fwd(noalloc=True)`` runs
ss_scan_fwd_noalloc, which works in the library's static scratch instead of a
workspace.

Shapes follow the mhpn.cn selective_scan walk-through (section 2): u, delta
(b, L, d_in); A_log (d_in, n) with A = -exp(A_log); B, C (b, L, n); D (d_in).
The step follows jiafeimiao.top's Mamba.step / selective_state_update call:
state (b, d_in, n) fp32 updated in place; x, dt, z (b, d_in); B, C (b, n).
``initial_state`` (b, d_in, n) fp32 starts the scan from a given state and
``zoh=True`` selects the zero-order-hold input term (mhpn.cn, section 6); calls
that use either go through ``ss_scan_fwd_ex`` / ``ss_state_update_ex`` (``ss_scan_bwd_ex`` for the
gradient of a zero-order-hold scan).
``cross_scan_fwd`` is VMamba's CrossScan + scan + CrossMerge in one pass (githubissues.com
VMamba #206): x (maps, H, W, d_in); delta (maps, 4, H*W, d_in); B, C (maps, 4, H*W, n);
A_log (4, d_in, n); D, delta_bias (4, d_in); directions 0 row-major, 1 column-major,
2 and 3 those reversed; y is the fp32 sum of the four directions at each position.
``conv_update`` is the convolution step of Mamba.step (jiafeimiao.top): conv_state
(b, d_in, W) in the dtype of x, weight (d_in, W) and bias (d_in) fp32.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_HERE, "libss_scan.so")

SS_F32 = 0
SS_BF16 = 1
SS_MAX_STATE = 64
SS_MAX_CONV_WIDTH = 8
SS_MAX_BWD_STATE = 64
SS_DISC_EULER = 0
SS_DISC_ZOH = 1
SS_ERR_TIMEOUT = -10
SS_NOALLOC_SCRATCH_BYTES = 8 << 20
STATUS = {0: "SS_OK", -1: "SS_ERR_NULL", -2: "SS_ERR_SHAPE", -3: "SS_ERR_DTYPE", -4: "SS_ERR_UNSUPPORTED",
          -5: "SS_ERR_WORKSPACE", -6: "SS_ERR_HIP", -7: "SS_ERR_ALIAS", -8: "SS_ERR_ALIGN", -9: "SS_ERR_MODE",
          -10: "SS_ERR_TIMEOUT"}
EXPORTS = ("ss_scan_fwd_workspace_bytes", "ss_scan_fwd", "ss_scan_fwd_ex", "ss_scan_fwd_noalloc", "ss_scan_status",
           "ss_state_update", "ss_state_update_ex", "ss_scan_bwd", "ss_scan_bwd_ex", "ss_scan_bwd_workspace_bytes",
           "ss_cross_scan_fwd", "ss_cross_scan_fwd_workspace_bytes", "ss_cross_scan_fwd_ex",
           "ss_cross_scan_fwd_ex_workspace_bytes", "ss_conv_update", "ss_status_string",
           "ss_set_test_plan", "ss_scan_checkpoint_bytes", "ss_scan_fwd_save", "ss_scan_bwd_saved",
           "ss_scan_bwd_saved_workspace_bytes")


class SSError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {STATUS.get(code, code)} ({status_string(code)})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIBRARY):
        raise ImportError(f"{LIBRARY} is not built; run `python selective_state_space_softplus_amd/build.py` "
                          "(or __graft_entry__.build())")
    lib = ctypes.CDLL(LIBRARY)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.ss_scan_fwd_workspace_bytes.restype = ctypes.c_size_t
    lib.ss_scan_fwd_workspace_bytes.argtypes = [I64, I64, I64, I64, I]
    lib.ss_scan_fwd.restype = I
    lib.ss_scan_fwd.argtypes = [P, P, P, P, P, P, P, P, I, P, P, I64, I64, I64, I64, I, P, ctypes.c_size_t, P]
    lib.ss_scan_fwd_ex.restype = I
    lib.ss_scan_fwd_ex.argtypes = [P, P, P, P, P, P, P, P, I, P, I, P, P, I64, I64, I64, I64, I, P, ctypes.c_size_t, P]
    lib.ss_scan_fwd_noalloc.restype = I
    lib.ss_scan_fwd_noalloc.argtypes = [P, P, P, P, P, P, P, P, I, P, I, P, P, I64, I64, I64, I64, I, P]
    lib.ss_scan_status.restype = I
    lib.ss_scan_status.argtypes = [P, ctypes.c_size_t, P, P]
    lib.ss_set_test_plan.restype = I
    lib.ss_set_test_plan.argtypes = [I, I, I, I, I]
    lib.ss_state_update.restype = I
    lib.ss_state_update.argtypes = [P, P, P, P, P, P, P, P, P, I, P, I64, I64, I64, I, P]
    lib.ss_state_update_ex.restype = I
    lib.ss_state_update_ex.argtypes = [P, P, P, P, P, P, P, P, P, I, I, P, I64, I64, I64, I, P]
    lib.ss_scan_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.ss_scan_bwd_workspace_bytes.argtypes = [I64, I64, I64, I64, I]
    lib.ss_scan_bwd.restype = I
    lib.ss_scan_bwd.argtypes = [P] * 8 + [I] + [P] * 12 + [I64, I64, I64, I64, I, P, ctypes.c_size_t, P]
    lib.ss_scan_bwd_ex.restype = I
    lib.ss_scan_bwd_ex.argtypes = [P] * 8 + [I, P, I] + [P] * 11 + [I64, I64, I64, I64, I, P, ctypes.c_size_t, P]
    lib.ss_scan_checkpoint_bytes.restype = ctypes.c_size_t
    lib.ss_scan_checkpoint_bytes.argtypes = [I64, I64, I64, I64]
    lib.ss_scan_bwd_saved_workspace_bytes.restype = ctypes.c_size_t
    lib.ss_scan_bwd_saved_workspace_bytes.argtypes = [I64, I64, I64, I64, I]
    lib.ss_scan_fwd_save.restype = I
    lib.ss_scan_fwd_save.argtypes = [P] * 8 + [I, P, I, P, P, P, P, I64, I64, I64, I64, I, P, ctypes.c_size_t, P]
    lib.ss_scan_bwd_saved.restype = I
    lib.ss_scan_bwd_saved.argtypes = [P] * 8 + [I, P, I] + [P] * 13 + [I64, I64, I64, I64, I, P, ctypes.c_size_t, P]
    lib.ss_cross_scan_fwd_workspace_bytes.restype = ctypes.c_size_t
    lib.ss_cross_scan_fwd_workspace_bytes.argtypes = [I64, I64, I64, I64, I64, I]
    lib.ss_cross_scan_fwd.restype = I
    lib.ss_cross_scan_fwd.argtypes = [P, P, P, P, P, P, P, I, P, P, I64, I64, I64, I64, I64, I, P, ctypes.c_size_t, P]
    lib.ss_cross_scan_fwd_ex_workspace_bytes.restype = ctypes.c_size_t
    lib.ss_cross_scan_fwd_ex_workspace_bytes.argtypes = [I64, I64, I64, I64, I64, I, I]
    lib.ss_cross_scan_fwd_ex.restype = I
    lib.ss_cross_scan_fwd_ex.argtypes = [P, P, P, P, P, P, P, I, P, P, I64, I64, I64, I64, I64, I, I, P,
                                         ctypes.c_size_t, P]
    lib.ss_conv_update.restype = I
    lib.ss_conv_update.argtypes = [P, P, P, P, I, P, I64, I64, I64, I, P]
    lib.ss_status_string.restype = ctypes.c_char_p
    lib.ss_status_string.argtypes = [I]
    return lib


lib = _load()


def status_string(code: int) -> str:
    return lib.ss_status_string(int(code)).decode()


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return SS_F32
    if t == torch.bfloat16:
        return SS_BF16
    raise TypeError(f"inputs must be float32 or bfloat16, got {t}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, shape, dtype, device):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def scan_fwd_workspace_bytes(b: int, L: int, d_in: int, n: int, dtype: int) -> int:
    return int(lib.ss_scan_fwd_workspace_bytes(b, L, d_in, n, dtype))


def scan_status(workspace, device=None) -> int:
    """Status the last scan call with ``workspace`` (None: the static scratch of the last
    noalloc scan on ``device``) left: SS_OK or SS_ERR_TIMEOUT.  Synchronises the stream."""
    dev = workspace.device if workspace is not None else torch.device(device if device is not None else "cuda")
    out = torch.empty(1, dtype=torch.int32, device=dev)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(dev):
        rc = lib.ss_scan_status(_ptr(workspace), nbytes, _ptr(out), _stream(dev))
    if rc != 0:
        raise SSError(rc, "ss_scan_status")
    return int(out.item())


def _raise_on_timeout(workspace, where, device=None):
    code = scan_status(workspace, device)
    if code != 0:
        raise SSError(code, where)


@contextlib.contextmanager
def test_plan(segments=0, waves=0, time_parallel=0, spin_limit=0, wait_never=0):
    """Override how the scans split their work (ss_set_test_plan) inside a with block."""
    rc = lib.ss_set_test_plan(int(segments), int(waves), int(time_parallel), int(spin_limit), int(wait_never))
    if rc != 0:
        raise SSError(rc, "ss_set_test_plan")
    try:
        yield
    finally:
        lib.ss_set_test_plan(0, 0, 0, 0, 0)


_workspaces: dict = {}


def _workspace(device, nbytes: int):
    """A cached uint8 device buffer of at least nbytes for this device (and stream)."""
    if nbytes == 0:
        return None
    key = (device, torch.cuda.current_stream(device).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def scan_fwd(u, delta, A_log, B, C, D, z=None, delta_bias=None, delta_softplus=True, return_last_state=False,
             out=None, last_state=None, workspace=None, initial_state=None, zoh=False, noalloc=False, check=False):
    """Selective scan forward on the GPU; returns y (and last_state if asked).

    ``initial_state`` may be the ``last_state`` buffer itself (carried over in place).
    ``noalloc``: ss_scan_fwd_noalloc (the library's static scratch; no workspace).
    ``check``: synchronise and raise if a wait between segments gave up.
    """
    if u.dim() != 3 or A_log.dim() != 2:
        raise ValueError("u must be (b, L, d_in) and A_log (d_in, n)")
    b, L, d_in = u.shape
    n = A_log.shape[1]
    dev = u.device
    code = _dtype_code(u.dtype)
    _check(u, "u", (b, L, d_in), u.dtype, dev)
    _check(delta, "delta", (b, L, d_in), u.dtype, dev)
    _check(A_log, "A_log", (d_in, n), torch.float32, dev)
    _check(B, "B", (b, L, n), u.dtype, dev)
    _check(C, "C", (b, L, n), u.dtype, dev)
    _check(D, "D", (d_in,), torch.float32, dev)
    _check(z, "z", (b, L, d_in), u.dtype, dev)
    _check(delta_bias, "delta_bias", (d_in,), torch.float32, dev)
    y = torch.empty_like(u) if out is None else out
    _check(y, "out", (b, L, d_in), u.dtype, dev)
    if return_last_state and last_state is None:
        last_state = torch.empty((b, d_in, n), dtype=torch.float32, device=dev)
    _check(last_state, "last_state", (b, d_in, n), torch.float32, dev)
    _check(initial_state, "initial_state", (b, d_in, n), torch.float32, dev)
    if b == 0 or L == 0 or d_in == 0:
        # Nothing to scan: no steps leave the initial state as it is.
        if last_state is not None:
            if initial_state is None:
                last_state.zero_()
            elif initial_state.data_ptr() != last_state.data_ptr():
                last_state.copy_(initial_state)
        return (y, last_state) if return_last_state else y
    if noalloc:
        with torch.cuda.device(dev):
            rc = lib.ss_scan_fwd_noalloc(_ptr(u), _ptr(delta), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                         _ptr(delta_bias), int(bool(delta_softplus)), _ptr(initial_state),
                                         SS_DISC_ZOH if zoh else SS_DISC_EULER, _ptr(y), _ptr(last_state),
                                         b, L, d_in, n, code, _stream(dev))
        if rc != 0:
            raise SSError(rc, "ss_scan_fwd_noalloc")
        if check:
            _raise_on_timeout(None, "ss_scan_fwd_noalloc", dev)
        return (y, last_state) if return_last_state else y
    need = scan_fwd_workspace_bytes(b, L, d_in, n, code)
    if workspace is None:
        workspace = _workspace(dev, need)
    ws_ptr = _ptr(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(dev):
        if initial_state is None and not zoh:
            where = "ss_scan_fwd"
            rc = lib.ss_scan_fwd(_ptr(u), _ptr(delta), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                 _ptr(delta_bias), int(bool(delta_softplus)), _ptr(y), _ptr(last_state),
                                 b, L, d_in, n, code, ws_ptr, ws_bytes, _stream(dev))
        else:
            where = "ss_scan_fwd_ex"
            rc = lib.ss_scan_fwd_ex(_ptr(u), _ptr(delta), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                    _ptr(delta_bias), int(bool(delta_softplus)), _ptr(initial_state),
                                    SS_DISC_ZOH if zoh else SS_DISC_EULER, _ptr(y), _ptr(last_state),
                                    b, L, d_in, n, code, ws_ptr, ws_bytes, _stream(dev))
    if rc != 0:
        raise SSError(rc, where)
    if check:
        _raise_on_timeout(workspace, where)
    return (y, last_state) if return_last_state else y


def scan_fwd_save(u, delta, A_log, B, C, D, z=None, delta_bias=None, delta_softplus=True, initial_state=None,
                  zoh=False, return_last_state=False, workspace=None, check=False):
    """Forward for training (ss_scan_fwd_save): returns a dict with y (and last_state if asked) and what
    scan_bwd(saved=...) starts from: checkpoints (b, (L - 1) // 8, n, d_in) fp32 and, gated, y_pre."""
    if u.dim() != 3 or A_log.dim() != 2:
        raise ValueError("u must be (b, L, d_in) and A_log (d_in, n)")
    b, L, d_in = u.shape
    n = A_log.shape[1]
    dev = u.device
    code = _dtype_code(u.dtype)
    for t, name, shape, dt in ((u, "u", (b, L, d_in), u.dtype), (delta, "delta", (b, L, d_in), u.dtype),
                               (A_log, "A_log", (d_in, n), torch.float32), (B, "B", (b, L, n), u.dtype),
                               (C, "C", (b, L, n), u.dtype), (D, "D", (d_in,), torch.float32),
                               (z, "z", (b, L, d_in), u.dtype), (delta_bias, "delta_bias", (d_in,), torch.float32),
                               (initial_state, "initial_state", (b, d_in, n), torch.float32)):
        _check(t, name, shape, dt, dev)
    out = dict(y=torch.empty_like(u),
               checkpoints=torch.empty((b, max(L - 1, 0) // 8, n, d_in), dtype=torch.float32, device=dev))
    if z is not None:
        out["y_pre"] = torch.empty_like(u)
    if return_last_state:
        out["last_state"] = torch.empty((b, d_in, n), dtype=torch.float32, device=dev)
    if b == 0 or L == 0 or d_in == 0:
        # Nothing to scan: no steps leave the initial state as it is, and nothing is saved.
        if return_last_state:
            if initial_state is None:
                out["last_state"].zero_()
            else:
                out["last_state"].copy_(initial_state)
        return out
    need = scan_fwd_workspace_bytes(b, L, d_in, n, code)
    if workspace is None:
        workspace = _workspace(dev, need)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(dev):
        rc = lib.ss_scan_fwd_save(_ptr(u), _ptr(delta), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                  _ptr(delta_bias), int(bool(delta_softplus)), _ptr(initial_state),
                                  SS_DISC_ZOH if zoh else SS_DISC_EULER, _ptr(out["y"]), _ptr(out.get("last_state")),
                                  _ptr(out["checkpoints"]), _ptr(out.get("y_pre")), b, L, d_in, n, code,
                                  _ptr(workspace), ws_bytes, _stream(dev))
    if rc != 0:
        raise SSError(rc, "ss_scan_fwd_save")
    if check:
        _raise_on_timeout(workspace, "ss_scan_fwd_save")
    return out


def state_update(state, x, dt, A_log, B, C, D, z=None, dt_bias=None, dt_softplus=True, out=None, zoh=False):
    """One decode step; updates ``state`` in place and returns y (b, d_in)."""
    if state.dim() != 3:
        raise ValueError("state must be (b, d_in, n)")
    b, d_in, n = state.shape
    dev = state.device
    code = _dtype_code(x.dtype)
    _check(state, "state", (b, d_in, n), torch.float32, dev)
    _check(x, "x", (b, d_in), x.dtype, dev)
    _check(dt, "dt", (b, d_in), x.dtype, dev)
    _check(A_log, "A_log", (d_in, n), torch.float32, dev)
    _check(B, "B", (b, n), x.dtype, dev)
    _check(C, "C", (b, n), x.dtype, dev)
    _check(D, "D", (d_in,), torch.float32, dev)
    _check(z, "z", (b, d_in), x.dtype, dev)
    _check(dt_bias, "dt_bias", (d_in,), torch.float32, dev)
    y = torch.empty_like(x) if out is None else out
    _check(y, "out", (b, d_in), x.dtype, dev)
    if b == 0 or d_in == 0:
        return y
    with torch.cuda.device(dev):
        if not zoh:
            where = "ss_state_update"
            rc = lib.ss_state_update(_ptr(state), _ptr(x), _ptr(dt), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D),
                                     _ptr(z), _ptr(dt_bias), int(bool(dt_softplus)), _ptr(y), b, d_in, n, code,
                                     _stream(dev))
        else:
            where = "ss_state_update_ex"
            rc = lib.ss_state_update_ex(_ptr(state), _ptr(x), _ptr(dt), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D),
                                        _ptr(z), _ptr(dt_bias), int(bool(dt_softplus)), SS_DISC_ZOH, _ptr(y),
                                        b, d_in, n, code, _stream(dev))
    if rc != 0:
        raise SSError(rc, where)
    return y


def conv_update(conv_state, x, weight, bias=None, silu=True, out=None):
    """One convolution step; updates ``conv_state`` (b, d_in, W) in place and returns out (b, d_in)."""
    if conv_state.dim() != 3:
        raise ValueError("conv_state must be (b, d_in, W)")
    b, d_in, W = conv_state.shape
    dev = conv_state.device
    code = _dtype_code(x.dtype)
    _check(conv_state, "conv_state", (b, d_in, W), x.dtype, dev)
    _check(x, "x", (b, d_in), x.dtype, dev)
    _check(weight, "weight", (d_in, W), torch.float32, dev)
    _check(bias, "bias", (d_in,), torch.float32, dev)
    y = torch.empty_like(x) if out is None else out
    _check(y, "out", (b, d_in), x.dtype, dev)
    if b == 0 or d_in == 0:
        return y
    with torch.cuda.device(dev):
        rc = lib.ss_conv_update(_ptr(conv_state), _ptr(x), _ptr(weight), _ptr(bias), int(bool(silu)), _ptr(y),
                                b, d_in, W, code, _stream(dev))
    if rc != 0:
        raise SSError(rc, "ss_conv_update")
    return y


CROSS_FORMS = {"auto": 0, "one_pass": 1, "two_pass": 2}


def cross_scan_fwd(x, delta, A_log, B, C, D, delta_bias=None, delta_softplus=True, return_last_state=False,
                   out=None, last_state=None, workspace=None, check=False, form="auto"):
    """VMamba cross scan + merge on the GPU; returns y (maps, H, W, d_in) fp32 (and last_state (maps, 4, d_in, n)).

    form: "auto" (the library's choice), "one_pass" (the four directions summed in LDS by one kernel; n <= 4 and
    maps of up to about 4000 positions, else SSError(SS_ERR_UNSUPPORTED)) or "two_pass" (per-direction outputs in
    the workspace, then a merge kernel)."""
    if form not in CROSS_FORMS:
        raise ValueError(f"form must be one of {sorted(CROSS_FORMS)}")
    fcode = CROSS_FORMS[form]
    if x.dim() != 4 or A_log.dim() != 3:
        raise ValueError("x must be (maps, H, W, d_in) and A_log (4, d_in, n)")
    maps, H, W, d_in = x.shape
    n = A_log.shape[2]
    L = H * W
    dev = x.device
    code = _dtype_code(x.dtype)
    _check(x, "x", (maps, H, W, d_in), x.dtype, dev)
    _check(delta, "delta", (maps, 4, L, d_in), x.dtype, dev)
    _check(A_log, "A_log", (4, d_in, n), torch.float32, dev)
    _check(B, "B", (maps, 4, L, n), x.dtype, dev)
    _check(C, "C", (maps, 4, L, n), x.dtype, dev)
    _check(D, "D", (4, d_in), torch.float32, dev)
    _check(delta_bias, "delta_bias", (4, d_in), torch.float32, dev)
    y = torch.empty((maps, H, W, d_in), dtype=torch.float32, device=dev) if out is None else out
    _check(y, "out", (maps, H, W, d_in), torch.float32, dev)
    if return_last_state and last_state is None:
        last_state = torch.empty((maps, 4, d_in, n), dtype=torch.float32, device=dev)
    _check(last_state, "last_state", (maps, 4, d_in, n), torch.float32, dev)
    if maps == 0 or L == 0 or d_in == 0:
        y.zero_()
        if last_state is not None:
            last_state.zero_()
        return (y, last_state) if return_last_state else y
    need = int(lib.ss_cross_scan_fwd_ex_workspace_bytes(maps, H, W, d_in, n, code, fcode))
    if workspace is None:
        workspace = _workspace(dev, need)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(dev):
        rc = lib.ss_cross_scan_fwd_ex(_ptr(x), _ptr(delta), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D),
                                      _ptr(delta_bias), int(bool(delta_softplus)), _ptr(y), _ptr(last_state), maps, H,
                                      W, d_in, n, code, fcode, _ptr(workspace), ws_bytes, _stream(dev))
    if rc != 0:
        raise SSError(rc, "ss_cross_scan_fwd_ex")
    if check:
        _raise_on_timeout(workspace, "ss_cross_scan_fwd")
    return (y, last_state) if return_last_state else y


def scan_bwd(u, delta, A_log, B, C, D, dy, z=None, delta_bias=None, delta_softplus=True, initial_state=None,
             dlast_state=None, workspace=None, zoh=False, check=False, saved=None):
    """Gradients of the scan for output gradients dy (and dlast_state): the delta' B u input term, or
    with zoh=True the zero-order hold's (ss_scan_bwd_ex).  ``saved``: the dict scan_fwd_save returned
    for these inputs; the backward then starts from it (ss_scan_bwd_saved) instead of running the
    forward scan again.

    Returns a dict: du, ddelta, dz (dtype of u; dz only with z), dA_log, dD, ddelta_bias (fp32; only
    with delta_bias), dB, dC (dtype of u), dinitial_state (fp32; only with initial_state).
    """
    if u.dim() != 3 or A_log.dim() != 2:
        raise ValueError("u must be (b, L, d_in) and A_log (d_in, n)")
    b, L, d_in = u.shape
    n = A_log.shape[1]
    dev = u.device
    code = _dtype_code(u.dtype)
    for t, name, shape, dt in ((u, "u", (b, L, d_in), u.dtype), (delta, "delta", (b, L, d_in), u.dtype),
                               (A_log, "A_log", (d_in, n), torch.float32), (B, "B", (b, L, n), u.dtype),
                               (C, "C", (b, L, n), u.dtype), (D, "D", (d_in,), torch.float32),
                               (z, "z", (b, L, d_in), u.dtype), (delta_bias, "delta_bias", (d_in,), torch.float32),
                               (initial_state, "initial_state", (b, d_in, n), torch.float32),
                               (dy, "dy", (b, L, d_in), u.dtype),
                               (dlast_state, "dlast_state", (b, d_in, n), torch.float32)):
        _check(t, name, shape, dt, dev)
    g = dict(du=torch.empty_like(u), ddelta=torch.empty_like(u),
             dA_log=torch.empty((d_in, n), dtype=torch.float32, device=dev),
             dB=torch.empty_like(B), dC=torch.empty_like(C), dD=torch.empty(d_in, dtype=torch.float32, device=dev))
    if z is not None:
        g["dz"] = torch.empty_like(z)
    if delta_bias is not None:
        g["ddelta_bias"] = torch.empty(d_in, dtype=torch.float32, device=dev)
    if initial_state is not None:
        g["dinitial_state"] = torch.empty((b, d_in, n), dtype=torch.float32, device=dev)
    if b == 0 or L == 0 or d_in == 0:
        for k, v in g.items():
            if k == "dinitial_state" and dlast_state is not None:
                v.copy_(dlast_state)
            else:
                v.zero_()
        return g
    if saved is not None:
        _check(saved["checkpoints"], "checkpoints", (b, (L - 1) // 8, n, d_in), torch.float32, dev)
        _check(saved.get("y_pre"), "y_pre", (b, L, d_in), u.dtype, dev)
        need = int(lib.ss_scan_bwd_saved_workspace_bytes(b, L, d_in, n, code))
    else:
        need = int(lib.ss_scan_bwd_workspace_bytes(b, L, d_in, n, code))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(dev):
        head = (_ptr(u), _ptr(delta), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                int(bool(delta_softplus)), _ptr(initial_state))
        tail = (_ptr(dy), _ptr(dlast_state), _ptr(g["du"]), _ptr(g["ddelta"]), _ptr(g["dA_log"]), _ptr(g["dB"]),
                _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g.get("dz")), _ptr(g.get("ddelta_bias")),
                _ptr(g.get("dinitial_state")), b, L, d_in, n, code, _ptr(workspace), ws_bytes, _stream(dev))
        disc = SS_DISC_ZOH if zoh else SS_DISC_EULER
        if saved is not None:
            where = "ss_scan_bwd_saved"
            rc = lib.ss_scan_bwd_saved(*head, disc, _ptr(saved["checkpoints"]), _ptr(saved.get("y_pre")), *tail)
        elif zoh:
            where = "ss_scan_bwd_ex"
            rc = lib.ss_scan_bwd_ex(*head, disc, *tail)
        else:
            where = "ss_scan_bwd"
            rc = lib.ss_scan_bwd(*head, *tail)
    if rc != 0:
        raise SSError(rc, where)
    if check:
        _raise_on_timeout(workspace, where)
    return g


class _SelectiveScan(torch.autograd.Function):
    """The scan as an autograd function: forward ss_scan_fwd_save, backward ss_scan_bwd_saved (from
    the checkpoints and pre-gate readout the forward kept)."""

    @staticmethod
    def forward(ctx, u, delta, A_log, B, C, D, z, delta_bias, delta_softplus, initial_state, zoh):
        out = scan_fwd_save(u, delta, A_log, B, C, D, z, delta_bias, delta_softplus, initial_state=initial_state,
                            zoh=zoh)
        ctx.delta_softplus = delta_softplus
        ctx.zoh = zoh
        ctx.save_for_backward(u, delta, A_log, B, C, D, z, delta_bias, initial_state, out["checkpoints"],
                              out.get("y_pre"))
        return out["y"]

    @staticmethod
    def backward(ctx, dy):
        u, delta, A_log, B, C, D, z, delta_bias, initial_state, ckpt, y_pre = ctx.saved_tensors
        saved = dict(checkpoints=ckpt)
        if y_pre is not None:
            saved["y_pre"] = y_pre
        g = scan_bwd(u, delta, A_log, B, C, D, dy.contiguous(), z, delta_bias, ctx.delta_softplus, initial_state,
                     zoh=ctx.zoh, saved=saved)
        return (g["du"], g["ddelta"], g["dA_log"], g["dB"], g["dC"], g["dD"], g.get("dz"), g.get("ddelta_bias"),
                None, g.get("dinitial_state"), None)


def selective_scan(u, delta, A_log, B, C, D, z=None, delta_bias=None, delta_softplus=True, initial_state=None,
                   zoh=False):
    """y of the scan, differentiable with respect to every tensor argument (torch autograd); zoh selects
    the zero-order-hold input term."""
    return _SelectiveScan.apply(u, delta, A_log, B, C, D, z, delta_bias, delta_softplus, initial_state, bool(zoh))
