"""GPU: element indices beyond 32 bits, in the longest segment the library runs.

One batch row of 64 channels and L = 2^25 + 40 steps: u, delta, z, y, dy and the
per-element gradients hold more than 2^31 elements (byte offsets above 2^32);
with n = 64 the forward's B and C rows, and with n = 16 the backward's state
checkpoints (b, L / 8, n, d_in), pass the same marks.  A single 64-channel
group is one piece along the whole sequence, so the per-segment step indices
run up to L as well.

u and dy are zero except in the last W steps, so every state is exactly zero
before them, and with the body's step sizes large (Delta >= 1.8, so the adjoint
underflows to zero within a few hundred steps going backwards) every output
before the last W + M steps is exactly zero: those rows are checked to be zero
on the GPU, and the oracle computes the last W + M steps, from a zero state,
for comparison element by element.  The body of delta, z, B and C is a tiled
seeded block unlike the window's values, so an address that wrapped would read
the wrong data.  The inputs are built on the GPU with torch and their window is
copied to the host for the oracle.
"""
import pytest
import torch

import oracle
import workloads
from tests.parity import assert_close
from tests.test_gpu_parity import BF16, DEV, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

L = (1 << 25) + 40     # (1, L, 64) holds 2^31 + 2560 elements
D_IN = 64
W = 600                # steps at the end with nonzero u (and dy)
M = 256                # steps before them that the oracle also covers
BLOCK = 4096           # rows of the tiled body


@pytest.fixture(scope="module")
def ss():
    import selective_state_space_softplus_amd as ss

    return ss


def _full(body, tail):
    """(1, L, X) device tensor: `body` (1, BLOCK, X) tiled along L, its last W rows replaced by `tail`."""
    x = body.shape[2]
    t = torch.empty((1, L, x), dtype=body.dtype, device=DEV)
    nfull = L // BLOCK
    blk = body[0].to(DEV)
    t[0, :nfull * BLOCK].view(nfull, BLOCK, x).copy_(blk.expand(nfull, BLOCK, x))
    t[0, nfull * BLOCK:].copy_(blk[:L - nfull * BLOCK])
    t[0, L - W:].copy_(tail[0].to(DEV))
    return t


def big_inputs(n, seed):
    tail = workloads.random_scan_inputs(1, W, D_IN, n, dtype=BF16, seed=seed, gated=True, bias=True)
    body = workloads.random_scan_inputs(1, BLOCK, D_IN, n, dtype=BF16, seed=seed + 1, gated=True)
    g = {
        "u": torch.zeros((1, L, D_IN), dtype=BF16, device=DEV),
        "delta": _full((body["delta"].float() + 15.0).to(BF16), tail["delta"]),
        "z": _full(body["z"], tail["z"]),
        "B": _full(body["B"], tail["B"]),
        "C": _full(body["C"], tail["C"]),
        "A_log": tail["A_log"].to(DEV), "D": tail["D"].to(DEV), "delta_bias": tail["delta_bias"].to(DEV),
    }
    g["u"][0, L - W:].copy_(tail["u"][0].to(DEV))
    return g


def window(t):
    """The last W + M rows of a (1, L, X) device tensor, on the host."""
    return t[:, L - W - M:].cpu()


def zero_before_window(t, what):
    nz = int(torch.count_nonzero(t[:, :L - W - M]).item())
    assert nz == 0, f"{what}: {nz} nonzero values before the last {W + M} steps"


@pytest.mark.parametrize("n", [16, 64])
def test_scan_beyond_32_bit_indices(ss, n):
    say(f"scan b=1 L={L} d_in={D_IN} n={n} bf16 gated bias softplus, one piece")
    g = big_inputs(n, seed=81 + n)
    y, last = ss.scan_fwd(g["u"], g["delta"], g["A_log"], g["B"], g["C"], g["D"], g["z"], g["delta_bias"], True,
                          return_last_state=True)
    torch.cuda.synchronize()
    zero_before_window(y, "y")
    yr, lr = oracle.scan(window(g["u"]), window(g["delta"]), g["A_log"].cpu(), window(g["B"]), window(g["C"]),
                         g["D"].cpu(), window(g["z"]), g["delta_bias"].cpu(), True)
    assert_close(window(y), yr, BF16, "y")
    assert_close(last, lr, BF16, "last_state")


def test_scan_bwd_beyond_32_bit_indices(ss):
    n = 16
    say(f"scan_bwd b=1 L={L} d_in={D_IN} n={n} bf16 gated bias softplus, one piece")
    g = big_inputs(n, seed=97)
    dyt = torch.randn(1, W, D_IN, generator=torch.Generator().manual_seed(98)).to(BF16)
    dy = torch.zeros((1, L, D_IN), dtype=BF16, device=DEV)
    dy[0, L - W:].copy_(dyt[0].to(DEV))
    out = ss.scan_bwd(g["u"], g["delta"], g["A_log"], g["B"], g["C"], g["D"], dy, g["z"], g["delta_bias"], True)
    torch.cuda.synchronize()
    for k in ("du", "ddelta", "dz", "dB", "dC"):
        zero_before_window(out[k], k)
    ref = oracle.scan_bwd(window(g["u"]), window(g["delta"]), g["A_log"].cpu(), window(g["B"]), window(g["C"]),
                          g["D"].cpu(), window(g["z"]), g["delta_bias"].cpu(), True, None, window(dy), None)
    for k in ("du", "ddelta", "dz", "dB", "dC"):
        assert_close(window(out[k]), ref[k], BF16, k)
    for k in ("dA_log", "dD", "ddelta_bias"):
        assert_close(out[k], ref[k], BF16, k)
