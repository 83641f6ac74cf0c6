"""Error metric and tolerances for GPU-vs-oracle parity.

The tolerance is a maximum relative error: 1e-4 when the inputs are fp32 and
2e-2 when they are bf16 (the state is fp32 in both cases).  An element-wise
|e| / |r| is meaningless where the readout cancels to almost zero, so the
relative error of element i is taken against max(|r_i|, rms(r)):

    err = max_i |got_i - ref_i| / max(|ref_i|, rms(ref))

computed per output tensor (y, last_state, decode state).
"""
from __future__ import annotations

import numpy as np
import torch

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def to_f64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, np.float64)


def rel_err(got, ref) -> float:
    g = to_f64(got)
    r = to_f64(ref)
    assert g.shape == r.shape, (g.shape, r.shape)
    if r.size == 0:
        return 0.0
    if not np.all(np.isfinite(g)):
        return float("inf")
    rms = float(np.sqrt(np.mean(r * r)))
    den = np.maximum(np.abs(r), rms if rms > 0 else 1e-300)
    return float(np.max(np.abs(g - r) / den))


def assert_close(got, ref, dtype, what="", tol=None):
    tol = TOL[dtype] if tol is None else tol
    e = rel_err(got, ref)
    assert e <= tol, f"{what}: max relative error {e:.3g} > {tol:g}"
    return e
