"""Seeded synthetic inputs for the selective scan and the decode step.

This module only draws random numbers and arranges them into the shapes the
pages use; it holds none of the scan's arithmetic and imports neither the
library nor the oracle, so both sides can share it.

Workloads (shapes and distributions):
  scan-tiny    b=2,  L=64,   d_in=32,   n=16, fp32  -- the usage example of
               Mamba(d_model=16, d_state=16, expand=2) on batch 2, length 64
               (jiafeimiao.top page, usage listing)
  scan-mid     b=8,  L=2048, d_in=1536, n=16, bf16 in/out, fp32 state
  scan-long    b=4,  L=8192, d_in=5120, n=16, bf16 in/out, fp32 state
  scan-vmamba  16 feature maps of 56x56x384 unrolled along 4 traversal orders
               (row-major, column-major, and both reversed) -> b=64, L=3136,
               d_in=384, n=1, fp32, ungated (githubissues.com VMamba #206:
               d_state = 1 and the CrossScan arrangement of four directions)
  decode       b=256, d_in=5120, n=16 fp32 state ~ N(0, 0.1), 64 single-token
               steps with bf16 x, z, B, C and dt
Distributions: u, B, C, z, D ~ N(0,1); delta (before softplus) ~ N(0,1) - 2;
A_log = log(1..n) per channel, the S4D-real initialisation (mhpn.cn page,
section 7); the delta bias, where present, ~ U(log 1e-3, log 1e-1).
Every tensor is drawn in fp32 from a CPU generator seeded with
1000 + workload index, then cast to the workload's dtype.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

BF16 = torch.bfloat16
F32 = torch.float32


@dataclass(frozen=True)
class ScanConfig:
    name: str
    index: int
    b: int
    L: int
    d_in: int
    n: int
    dtype: torch.dtype
    gated: bool = True
    bias: bool = False
    vmamba: bool = False          # build b from 4 traversal orders of 56x56 maps
    maps: int = 0                 # number of feature maps (vmamba only)
    side: int = 0                 # map side (vmamba only)

    @property
    def updates(self) -> int:
        return self.b * self.L * self.d_in * self.n


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    index: int
    b: int
    d_in: int
    n: int
    steps: int
    dtype: torch.dtype = BF16
    state_std: float = 0.1

    @property
    def updates(self) -> int:
        return self.b * self.d_in * self.n * self.steps


CONFIGS = {
    0: ScanConfig("scan-tiny", 0, 2, 64, 32, 16, F32, gated=True, bias=False),
    1: ScanConfig("scan-mid", 1, 8, 2048, 1536, 16, BF16, gated=True, bias=True),
    2: ScanConfig("scan-long", 2, 4, 8192, 5120, 16, BF16, gated=True, bias=True),
    3: ScanConfig("scan-vmamba", 3, 64, 3136, 384, 1, F32, gated=False, bias=False, vmamba=True, maps=16, side=56),
    4: DecodeConfig("decode", 4, 256, 5120, 16, 64),
}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator("cpu")
    g.manual_seed(seed)
    return g


def s4d_real_A_log(d_in: int, n: int) -> torch.Tensor:
    """A_log[d, k] = log(k + 1): the S4D-real initialisation (A = -(k+1))."""
    return torch.log(torch.arange(1, n + 1, dtype=F32)).repeat(d_in, 1).contiguous()


def bias_uniform_log(d_in: int, g: torch.Generator, lo: float = 1e-3, hi: float = 1e-1) -> torch.Tensor:
    return torch.empty(d_in, dtype=F32).uniform_(math.log(lo), math.log(hi), generator=g)


def random_scan_inputs(b: int, L: int, d_in: int, n: int, dtype=F32, seed: int = 0, gated: bool = True,
                       bias: bool = False, delta_shift: float = -2.0, A_log: torch.Tensor | None = None) -> dict:
    """General seeded scan inputs (CPU tensors) in the scan-tiny distributions."""
    g = _gen(seed)
    r = lambda *s: torch.randn(*s, generator=g, dtype=F32)  # noqa: E731
    u = r(b, L, d_in)
    delta = r(b, L, d_in) + delta_shift
    Bm = r(b, L, n)
    Cm = r(b, L, n)
    z = r(b, L, d_in) if gated else None
    D = r(d_in)
    db = bias_uniform_log(d_in, g) if bias else None
    A = s4d_real_A_log(d_in, n) if A_log is None else A_log.to(F32).contiguous()
    cast = lambda t: None if t is None else t.to(dtype).contiguous()  # noqa: E731
    return {"u": cast(u), "delta": cast(delta), "A_log": A, "B": cast(Bm), "C": cast(Cm), "D": D.contiguous(),
            "z": cast(z), "delta_bias": db, "delta_softplus": True, "dtype": dtype}


def vmamba_unroll(fmap: torch.Tensor) -> torch.Tensor:
    """(maps, H, W, C) -> (maps*4, H*W, C): row-major, column-major, and both reversed.

    Batch index = map * 4 + direction.  This is the CrossScan arrangement of
    the VMamba issue thread, done on the host as input preparation.
    """
    m, H, W, Cc = fmap.shape
    row = fmap.reshape(m, H * W, Cc)
    col = fmap.permute(0, 2, 1, 3).reshape(m, H * W, Cc)
    dirs = torch.stack([row, col, row.flip(1), col.flip(1)], dim=1)  # (m, 4, L, C)
    return dirs.reshape(m * 4, H * W, Cc).contiguous()


def scan_inputs(cfg: ScanConfig | int, seed: int | None = None) -> dict:
    """Inputs of a named scan workload as CPU tensors in the workload dtype."""
    if isinstance(cfg, int):
        cfg = CONFIGS[cfg]
    seed = 1000 + cfg.index if seed is None else seed
    if not cfg.vmamba:
        return random_scan_inputs(cfg.b, cfg.L, cfg.d_in, cfg.n, cfg.dtype, seed, cfg.gated, cfg.bias)
    g = _gen(seed)
    r = lambda *s: torch.randn(*s, generator=g, dtype=F32)  # noqa: E731
    fmap = r(cfg.maps, cfg.side, cfg.side, cfg.d_in)
    u = vmamba_unroll(fmap)
    assert u.shape == (cfg.b, cfg.L, cfg.d_in)
    delta = r(cfg.b, cfg.L, cfg.d_in) - 2.0       # each direction draws its own delta
    Bm = r(cfg.b, cfg.L, cfg.n)
    Cm = r(cfg.b, cfg.L, cfg.n)
    D = r(cfg.d_in)
    A_log = torch.zeros(cfg.d_in, cfg.n, dtype=F32)  # A = -1
    cast = lambda t: t.to(cfg.dtype).contiguous()  # noqa: E731
    return {"u": cast(u), "delta": cast(delta), "A_log": A_log, "B": cast(Bm), "C": cast(Cm), "D": D,
            "z": None, "delta_bias": None, "delta_softplus": True, "dtype": cfg.dtype}


def cross_scan_inputs(cfg: ScanConfig | int = 3, seed: int | None = None) -> dict:
    """A map workload in the layout of the fused cross scan (CPU tensors).

    The same draws as scan_inputs for that workload, kept as the feature map
    x (maps, H, W, d_in) instead of its four unrolled copies; delta, B, C
    become (maps, 4, L, .) and A_log, D one set per direction (the shared
    values repeated), so the fused cross scan of these inputs merges exactly
    the four scans of scan_inputs(cfg).
    """
    if isinstance(cfg, int):
        cfg = CONFIGS[cfg]
    assert cfg.vmamba
    seed = 1000 + cfg.index if seed is None else seed
    g = _gen(seed)
    r = lambda *s: torch.randn(*s, generator=g, dtype=F32)  # noqa: E731
    fmap = r(cfg.maps, cfg.side, cfg.side, cfg.d_in)
    delta = r(cfg.b, cfg.L, cfg.d_in) - 2.0
    Bm = r(cfg.b, cfg.L, cfg.n)
    Cm = r(cfg.b, cfg.L, cfg.n)
    D = r(cfg.d_in)
    m = cfg.maps
    cast = lambda t: t.to(cfg.dtype).contiguous()  # noqa: E731
    return {"x": cast(fmap), "delta": cast(delta.reshape(m, 4, cfg.L, cfg.d_in)),
            "A_log": torch.zeros(4, cfg.d_in, cfg.n, dtype=F32), "B": cast(Bm.reshape(m, 4, cfg.L, cfg.n)),
            "C": cast(Cm.reshape(m, 4, cfg.L, cfg.n)), "D": D.expand(4, cfg.d_in).contiguous(), "delta_bias": None,
            "delta_softplus": True, "dtype": cfg.dtype}


def decode_inputs(cfg: DecodeConfig | int = 4, seed: int | None = None, steps: int | None = None,
                  b: int | None = None) -> dict:
    """Initial state and pre-drawn per-step inputs of the decode workload (CPU tensors).

    x, dt, z: (steps, b, d_in); B, C: (steps, b, n); dt is the value before softplus.
    """
    if isinstance(cfg, int):
        cfg = CONFIGS[cfg]
    seed = 1000 + cfg.index if seed is None else seed
    steps = cfg.steps if steps is None else steps
    b = cfg.b if b is None else b
    g = _gen(seed)
    r = lambda *s: torch.randn(*s, generator=g, dtype=F32)  # noqa: E731
    state = r(b, cfg.d_in, cfg.n) * cfg.state_std
    x = r(steps, b, cfg.d_in)
    z = r(steps, b, cfg.d_in)
    dt = r(steps, b, cfg.d_in) - 2.0
    Bm = r(steps, b, cfg.n)
    Cm = r(steps, b, cfg.n)
    D = r(cfg.d_in)
    dt_bias = bias_uniform_log(cfg.d_in, g)
    cast = lambda t: t.to(cfg.dtype).contiguous()  # noqa: E731
    return {"state": state.contiguous(), "x": cast(x), "dt": cast(dt), "z": cast(z), "B": cast(Bm), "C": cast(Cm),
            "A_log": s4d_real_A_log(cfg.d_in, cfg.n), "D": D, "dt_bias": dt_bias, "dt_softplus": True,
            "dtype": cfg.dtype}
