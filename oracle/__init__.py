"""Double-precision CPU oracle of the selective scan and its state-update step.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``; never by the library itself.

The arithmetic lives in ``ss_oracle.c`` (plain C, double, sequential loops in
the order the pages define them: the mamba-minimal ``selective_scan`` walk-through
on the mhpn.cn page, sections 2-5 and 7, and ``Mamba.step`` on the
jiafeimiao.top page, including its convolution step).  This module only widens inputs to float64 and calls it
through ctypes.  Parity of every function here is pinned by
``tests/test_oracle_pins.py`` (brute force, closed forms, limits, invariants).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "ss_oracle.c")
LIBRARY = os.path.join(_HERE, "libss_oracle.so")
# The same source with OpenMP over the independent (batch, channel) loops of
# the scan and the step: bit-identical results, all host cores.
LIBRARY_OMP = os.path.join(_HERE, "libss_oracle_omp.so")
CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math"]

_lib = None
_lib_omp = None


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the oracle with gcc (no HIP, no fast-math), serially and with OpenMP.  Returns the serial path."""
    subprocess.run(["gcc", *CFLAGS, "-o", output, source, "-lm"], check=True)
    omp = os.path.join(os.path.dirname(output), os.path.basename(LIBRARY_OMP)) if output != LIBRARY else LIBRARY_OMP
    subprocess.run(["gcc", *CFLAGS, "-fopenmp", "-o", omp, source, "-lm"], check=True)
    return output


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the compiled oracle (building it first if it was never built)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(LIBRARY):
            build()
        _lib = _bind(ctypes.CDLL(LIBRARY))
    return _lib


def load_parallel() -> ctypes.CDLL:
    """The OpenMP build (OMP_NUM_THREADS threads; ``threads(lib)`` says how many)."""
    global _lib_omp
    if _lib_omp is None:
        if not os.path.exists(LIBRARY_OMP):
            build()
        _lib_omp = _bind(ctypes.CDLL(LIBRARY_OMP))
    return _lib_omp


def threads(lib=None) -> int:
    """Threads the (batch, channel) loops of ``lib`` use (1 for the serial build)."""
    return int((lib or load()).ss_oracle_threads())


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.ss_oracle_softplus.restype = ctypes.c_double
    lib.ss_oracle_softplus.argtypes = [ctypes.c_double]
    lib.ss_oracle_silu.restype = ctypes.c_double
    lib.ss_oracle_silu.argtypes = [ctypes.c_double]
    lib.ss_oracle_threads.restype = ctypes.c_int
    lib.ss_oracle_threads.argtypes = []
    lib.ss_oracle_scan.restype = ctypes.c_int
    lib.ss_oracle_scan.argtypes = [P] * 8 + [ctypes.c_int, P, P, I64, I64, I64, I64]
    lib.ss_oracle_state_update.restype = ctypes.c_int
    lib.ss_oracle_state_update.argtypes = [P] * 9 + [ctypes.c_int, P, I64, I64, I64]
    lib.ss_oracle_scan_ex.restype = ctypes.c_int
    lib.ss_oracle_scan_ex.argtypes = [P] * 8 + [ctypes.c_int, P, ctypes.c_int, P, P, I64, I64, I64, I64]
    lib.ss_oracle_state_update_ex.restype = ctypes.c_int
    lib.ss_oracle_state_update_ex.argtypes = [P] * 9 + [ctypes.c_int, ctypes.c_int, P, I64, I64, I64]
    lib.ss_oracle_scan_bwd.restype = ctypes.c_int
    lib.ss_oracle_scan_bwd.argtypes = [P] * 8 + [ctypes.c_int] + [P] * 12 + [I64, I64, I64, I64]
    lib.ss_oracle_scan_bwd_ex.restype = ctypes.c_int
    lib.ss_oracle_scan_bwd_ex.argtypes = [P] * 8 + [ctypes.c_int, P, ctypes.c_int] + [P] * 11 + [I64, I64, I64, I64]
    lib.ss_oracle_cross_scan.restype = ctypes.c_int
    lib.ss_oracle_cross_scan.argtypes = [P] * 7 + [ctypes.c_int, P, P, I64, I64, I64, I64, I64]
    lib.ss_oracle_conv_update.restype = ctypes.c_int
    lib.ss_oracle_conv_update.argtypes = [P] * 4 + [ctypes.c_int, P, I64, I64, I64]
    return lib


def _f64(a):
    """Exact widening of a numpy array or torch tensor (fp32/bf16/fp16/f64) to float64."""
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor (bf16 has no numpy dtype)
        import torch

        a = a.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def softplus(x: float, lib=None) -> float:
    return (lib or load()).ss_oracle_softplus(float(x))


def silu(x: float, lib=None) -> float:
    return (lib or load()).ss_oracle_silu(float(x))


def scan(u, delta, A_log, B, C, D, z=None, delta_bias=None, delta_softplus=True, lib=None, h0=None, zoh=False):
    """y (b, L, d_in) and last_state (b, d_in, n), both float64.

    u, delta, z: (b, L, d_in); A_log: (d_in, n); B, C: (b, L, n); D, delta_bias: (d_in);
    h0: optional initial state (b, d_in, n); zoh: zero-order-hold input weight instead of Euler.
    """
    lib = lib or load()
    u, delta, A_log, B, C, D = map(_f64, (u, delta, A_log, B, C, D))
    z, delta_bias, h0 = _f64(z), _f64(delta_bias), _f64(h0)
    b, L, d_in = u.shape
    n = A_log.shape[1]
    assert delta.shape == u.shape and A_log.shape == (d_in, n)
    assert B.shape == (b, L, n) and C.shape == (b, L, n) and D.shape == (d_in,)
    assert z is None or z.shape == u.shape
    assert delta_bias is None or delta_bias.shape == (d_in,)
    assert h0 is None or h0.shape == (b, d_in, n)
    y = np.empty((b, L, d_in), np.float64)
    last = np.empty((b, d_in, n), np.float64)
    rc = lib.ss_oracle_scan_ex(_ptr(u), _ptr(delta), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                               _ptr(delta_bias), int(bool(delta_softplus)), _ptr(h0), int(bool(zoh)),
                               _ptr(y), _ptr(last), b, L, d_in, n)
    if rc != 0:
        raise ValueError(f"ss_oracle_scan returned {rc}")
    return y, last


def state_update(state, x, dt, A_log, B, C, D, z=None, dt_bias=None, dt_softplus=True, lib=None, zoh=False):
    """One decode step on a copy of ``state``: returns (new_state (b, d_in, n), y (b, d_in))."""
    lib = lib or load()
    st = _f64(state).copy()
    x, dt, A_log, B, C, D = map(_f64, (x, dt, A_log, B, C, D))
    z, dt_bias = _f64(z), _f64(dt_bias)
    b, d_in, n = st.shape
    assert x.shape == (b, d_in) and dt.shape == (b, d_in) and A_log.shape == (d_in, n)
    assert B.shape == (b, n) and C.shape == (b, n) and D.shape == (d_in,)
    y = np.empty((b, d_in), np.float64)
    rc = lib.ss_oracle_state_update_ex(_ptr(st), _ptr(x), _ptr(dt), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D),
                                       _ptr(z), _ptr(dt_bias), int(bool(dt_softplus)), int(bool(zoh)), _ptr(y),
                                       b, d_in, n)
    if rc != 0:
        raise ValueError(f"ss_oracle_state_update returned {rc}")
    return st, y


def scan_channels(inputs: dict, channels, delta_softplus=True, lib=None, zoh=False):
    """Oracle outputs for selected (batch, channel) pairs of a full-size scan.

    Each pair is an independent recurrence, so its slice of the inputs is run
    as a scan with b = 1, d_in = 1.  Returns {(bi, d): (y (L,), last_state (n,))}.
    """
    out = {}
    for bi, d in channels:
        sl = lambda t: None if t is None else t[bi:bi + 1, :, d:d + 1]  # noqa: E731
        z = inputs.get("z")
        bias = inputs.get("delta_bias")
        y, last = scan(sl(inputs["u"]), sl(inputs["delta"]), inputs["A_log"][d:d + 1], inputs["B"][bi:bi + 1],
                       inputs["C"][bi:bi + 1], inputs["D"][d:d + 1], sl(z) if z is not None else None,
                       None if bias is None else bias[d:d + 1], delta_softplus, lib=lib,
                       h0=None if inputs.get("h0") is None else inputs["h0"][bi:bi + 1, d:d + 1], zoh=zoh)
        out[(bi, d)] = (y[0, :, 0], last[0, 0])
    return out


def conv_update(conv_state, x, weight, bias=None, act=True, lib=None):
    """One convolution step on a copy of ``conv_state``: returns (new_state (b, d_in, W), out (b, d_in)).

    conv_state: (b, d_in, W); x: (b, d_in); weight: (d_in, W); bias: (d_in) or None; act: apply silu.
    """
    lib = lib or load()
    st = _f64(conv_state).copy()
    x, weight, bias = _f64(x), _f64(weight), _f64(bias)
    b, d_in, W = st.shape
    assert x.shape == (b, d_in) and weight.shape == (d_in, W)
    assert bias is None or bias.shape == (d_in,)
    out = np.empty((b, d_in), np.float64)
    rc = lib.ss_oracle_conv_update(_ptr(st), _ptr(x), _ptr(weight), _ptr(bias), int(bool(act)), _ptr(out),
                                   b, d_in, W)
    if rc != 0:
        raise ValueError(f"ss_oracle_conv_update returned {rc}")
    return st, out


def cross_scan(x, delta, A_log, B, C, D, delta_bias=None, delta_softplus=True, lib=None):
    """VMamba cross scan + merge: returns (y (maps, H, W, d_in), last_state (maps, 4, d_in, n)), float64.

    x: (maps, H, W, d_in); delta: (maps, 4, H*W, d_in); B, C: (maps, 4, H*W, n);
    A_log: (4, d_in, n); D, delta_bias: (4, d_in).  Directions: 0 row-major,
    1 column-major, 2 and 3 those two backwards.
    """
    lib = lib or load()
    x, delta, A_log, B, C, D = map(_f64, (x, delta, A_log, B, C, D))
    delta_bias = _f64(delta_bias)
    maps, H, W, d_in = x.shape
    n = A_log.shape[2]
    L = H * W
    assert delta.shape == (maps, 4, L, d_in) and A_log.shape == (4, d_in, n)
    assert B.shape == (maps, 4, L, n) and C.shape == (maps, 4, L, n) and D.shape == (4, d_in)
    assert delta_bias is None or delta_bias.shape == (4, d_in)
    y = np.empty((maps, H, W, d_in), np.float64)
    last = np.empty((maps, 4, d_in, n), np.float64)
    rc = lib.ss_oracle_cross_scan(_ptr(x), _ptr(delta), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D), _ptr(delta_bias),
                                  int(bool(delta_softplus)), _ptr(y), _ptr(last), maps, H, W, d_in, n)
    if rc != 0:
        raise ValueError(f"ss_oracle_cross_scan returned {rc}")
    return y, last


def scan_bwd(u, delta, A_log, B, C, D, z=None, delta_bias=None, delta_softplus=True, h0=None, dy=None, dlast=None,
             lib=None, zoh=False):
    """Gradients of the scan for output gradients dy (b, L, d_in) and dlast (b, d_in, n); zoh: the
    zero-order-hold input term instead of Euler.

    Returns a dict of float64 arrays: du, ddelta, dA_log, dB, dC, dD, and dz, ddelta_bias, dh0 when z,
    delta_bias, h0 are given.
    """
    lib = lib or load()
    u, delta, A_log, B, C, D, dy = map(_f64, (u, delta, A_log, B, C, D, dy))
    z, delta_bias, h0, dlast = _f64(z), _f64(delta_bias), _f64(h0), _f64(dlast)
    b, L, d_in = u.shape
    n = A_log.shape[1]
    assert dy.shape == u.shape and (dlast is None or dlast.shape == (b, d_in, n))
    out = dict(du=np.empty_like(u), ddelta=np.empty_like(u), dA_log=np.empty((d_in, n)), dB=np.empty((b, L, n)),
               dC=np.empty((b, L, n)), dD=np.empty(d_in))
    if z is not None:
        out["dz"] = np.empty_like(u)
    if delta_bias is not None:
        out["ddelta_bias"] = np.empty(d_in)
    if h0 is not None:
        out["dh0"] = np.empty((b, d_in, n))
    rc = lib.ss_oracle_scan_bwd_ex(_ptr(u), _ptr(delta), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                _ptr(delta_bias), int(bool(delta_softplus)), _ptr(h0), int(bool(zoh)), _ptr(dy),
                                _ptr(dlast),
                                _ptr(out["du"]), _ptr(out["ddelta"]), _ptr(out["dA_log"]), _ptr(out["dB"]),
                                _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out.get("dz")), _ptr(out.get("ddelta_bias")),
                                _ptr(out.get("dh0")), b, L, d_in, n)
    if rc != 0:
        raise ValueError(f"ss_oracle_scan_bwd returned {rc}")
    return out
