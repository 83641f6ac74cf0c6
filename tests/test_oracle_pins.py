"""CPU: the oracle against its pins, and the pins against planted mistakes.

The second half builds broken copies of ``oracle/ss_oracle.c`` (one planted
mistake each: a dropped term, a wrong sign, a wrong or shifted index, a
swapped operand, a misplaced bias or gate) and checks that every one of them
fails at least one pin, so the pins are strong enough to catch that class
of error in the real oracle.
"""
import os
import shutil
import subprocess
import sys

import pytest

import oracle
from tests import oracle_pins

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin, oracle_lib):
    pin(oracle_lib)


# A mutant whose wrong index can write outside its buffers runs its pins in a
# child process: a crash there counts as caught.
ISOLATE = "isolate"

# (description, text in ss_oracle.c, replacement[, ISOLATE])
MUTANTS = [
    ("A sign", "A[k] = -exp(A_log[d * n + k]);          /*", "A[k] = exp(A_log[d * n + k]);          /*"),
    ("A without exp", "A[k] = -exp(A_log[d * n + k]);          /*", "A[k] = -A_log[d * n + k];          /*"),
    ("bwd A sign", "A[k] = -exp(A_log[d * n + k]);\n                hs[k]", "A[k] = exp(A_log[d * n + k]);\n                hs[k]"),
    ("nonzero initial state", "h[k] = h0 ? h0[(bi * d_in + d) * n + k] : 0.0;",
     "h[k] = h0 ? h0[(bi * d_in + d) * n + k] : 1e-3;"),
    ("initial state ignored", "h[k] = h0 ? h0[(bi * d_in + d) * n + k] : 0.0;", "h[k] = 0.0;"),
    ("initial state transposed", "h[k] = h0 ? h0[(bi * d_in + d) * n + k] : 0.0;",
     "h[k] = h0 ? h0[(bi * d_in + d) * n + (n - 1 - k)] : 0.0;"),
    ("decay without delta", "double dA = exp(dl * A[k]);", "double dA = exp(A[k]);"),
    ("Euler decay 1 + delta*A", "double dA = exp(dl * A[k]);", "double dA = 1.0 + dl * A[k];"),
    ("input without delta", "if (!zoh)\n        return dl * Bk;", "if (!zoh)\n        return Bk;"),
    ("input uses C", "double dBu = input_weight(dl, A[k], B[r + k], zoh) * u[e];",
     "double dBu = input_weight(dl, A[k], C[r + k], zoh) * u[e];"),
    ("zoh weight uses exp", "return expm1(dl * A) / A * Bk;", "return exp(dl * A) / A * Bk;"),
    ("zoh weight without 1/A", "return expm1(dl * A) / A * Bk;", "return expm1(dl * A) * Bk;"),
    ("zoh weight sign", "return expm1(dl * A) / A * Bk;", "return -expm1(dl * A) / A * Bk;"),
    ("zoh weight is Euler", "return expm1(dl * A) / A * Bk;", "return dl * Bk;"),
    ("dropped decay", "h[k] = dA * h[k] + dBu;", "h[k] = h[k] + dBu;"),
    ("decayed input", "h[k] = dA * h[k] + dBu;", "h[k] = dA * (h[k] + dBu);"),
    ("readout uses B", "yt += C[r + k] * h[k];", "yt += B[r + k] * h[k];"),
    ("readout one state short", "for (int64_t k = 0; k < n; k++)\n                    yt += C[r + k] * h[k];",
     "for (int64_t k = 0; k + 1 < n; k++)\n                    yt += C[r + k] * h[k];"),
    ("B/C one step late", "int64_t r = (bi * L + t) * n;", "int64_t r = (bi * L + (t > 0 ? t - 1 : 0)) * n;"),
    ("mirrored channel", "int64_t e = (bi * L + t) * d_in + d;", "int64_t e = (bi * L + t) * d_in + (d_in - 1 - d);"),
    ("dropped D skip", "yt += D[d] * u[e];", "yt += 0.0 * D[d] * u[e];"),
    ("skip uses delta", "yt += D[d] * u[e];", "yt += D[d] * delta[e];"),
    ("gate without sigmoid", "                    yt *= ss_oracle_silu(z[e]);\n                y[e] = yt;",
     "                    yt *= z[e];\n                y[e] = yt;"),
    ("step gate uses x", "                yt *= ss_oracle_silu(z[e]);\n            y[e] = yt;",
     "                yt *= ss_oracle_silu(x[e]);\n            y[e] = yt;"),
    ("gate before skip", "yt += D[d] * u[e];\n                /* optional gate, applied after the skip */\n                if (z)\n                    yt *= ss_oracle_silu(z[e]);",
     "if (z)\n                    yt *= ss_oracle_silu(z[e]);\n                yt += D[d] * u[e];"),
    ("bias after softplus", "double v = delta + (bias ? bias[d] : 0.0);\n    return softplus ? ss_oracle_softplus(v) : v;",
     "double v = softplus ? ss_oracle_softplus(delta) : delta;\n    return v + (bias ? bias[d] : 0.0);"),
    ("softplus drops x", "return x + log1p(exp(-x));", "return log1p(exp(-x));"),
    ("softplus is exp", "return log1p(exp(x));", "return exp(x);"),
    ("silu sign", "return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    ("last_state wrong slot", "last_state[(bi * d_in + d) * n + k] = h[k];", "last_state[(bi * d_in + d) * n + k] = h[n - 1 - k];"),
    ("step without decay", "*h = *h * dA + x[e] * dB;", "*h = *h + x[e] * dB;"),
    ("step readout before update", "*h = *h * dA + x[e] * dB;               /* in place */\n                yt += C[bi * n + k] * *h;",
     "yt += C[bi * n + k] * *h;\n                *h = *h * dA + x[e] * dB;"),
    ("step B index", "double dB = input_weight(dl, A, B[bi * n + k], zoh);",
     "double dB = input_weight(dl, A, B[k], zoh);"),
    ("step ignores zoh", "double dB = input_weight(dl, A, B[bi * n + k], zoh);",
     "double dB = input_weight(dl, A, B[bi * n + k], 0);"),
    ("step dropped skip", "yt += D[d] * x[e];", "yt += 0.0 * x[e];"),
    ("step A index", "double A = -exp(A_log[d * n + k]);", "double A = -exp(A_log[k]);"),
    ("conv rolls the other way", "for (int64_t w = 0; w + 1 < W; w++)          /* roll by -1 */\n                win[w] = win[w + 1];",
     "for (int64_t w = W - 1; w > 0; w--)\n                win[w] = win[w - 1];"),
    ("conv without roll", "win[w] = win[w + 1];", "(void)0;"),
    ("conv newest input first", "win[W - 1] = x[bi * d_in + d];", "win[0] = x[bi * d_in + d];"),
    ("conv weight reversed", "acc += win[w] * weight[d * W + w];", "acc += win[w] * weight[d * W + (W - 1 - w)];"),
    ("conv weight of channel 0", "acc += win[w] * weight[d * W + w];", "acc += win[w] * weight[w];"),
    ("conv bias after silu", "if (bias)\n                acc += bias[d];\n            out[bi * d_in + d] = act ? ss_oracle_silu(acc) : acc;",
     "out[bi * d_in + d] = (act ? ss_oracle_silu(acc) : acc) + (bias ? bias[d] : 0.0);"),
    ("cross column-major by W", "int64_t w = s / H, h = s % H;", "int64_t w = s / W, h = s % W;", ISOLATE),
    ("cross reversed directions run forwards", "int64_t s = (k >= 2) ? H * W - 1 - t : t;", "int64_t s = t;"),
    ("cross column-major reversed only", "int64_t s = (k >= 2) ? H * W - 1 - t : t;", "int64_t s = (k == 3) ? H * W - 1 - t : t;"),
    ("cross merge overwrites", "y[(m * L + cross_position(k, t, H, W)) * d_in + d] += yk[t * d_in + d];",
     "y[(m * L + cross_position(k, t, H, W)) * d_in + d] = yk[t * d_in + d];"),
    ("cross merge at the step index", "y[(m * L + cross_position(k, t, H, W)) * d_in + d] += yk[t * d_in + d];",
     "y[(m * L + t) * d_in + d] += yk[t * d_in + d];"),
    ("cross parameters of direction 0", "rc = ss_oracle_scan_ex(uk, delta + seq * L * d_in, A_log + k * d_in * n,",
     "rc = ss_oracle_scan_ex(uk, delta + seq * L * d_in, A_log,"),
    ("cross D of direction 0", "B + seq * L * n, C + seq * L * n, D + k * d_in, NULL,", "B + seq * L * n, C + seq * L * n, D, NULL,"),
    ("cross inputs of direction 0", "rc = ss_oracle_scan_ex(uk, delta + seq * L * d_in,", "rc = ss_oracle_scan_ex(uk, delta + m * 4 * L * d_in,"),
    ("bwd adjoint not decayed", "g[k] *= a;                                /* on to h_(t-1) */", "(void)a;"),
    ("bwd adjoint misses the readout", "g[k] += dyp * C[r + k];                   /* dL/dh_tk */", "g[k] += 0.0 * C[r + k];"),
    ("bwd dC from the previous state", "dC[r + k] += dyp * hs[(t + 1) * n + k];", "dC[r + k] += dyp * hs[t * n + k];"),
    ("bwd dB without delta", "dB[r + k] += g[k] * beta * u[e];", "dB[r + k] += g[k] * u[e];"),
    ("bwd du without the input weight", "dut += g[k] * beta * B[r + k];", "dut += g[k] * B[r + k];"),
    ("bwd zoh weight taken as Euler", "double beta = zoh ? expm1(dl * A[k]) / A[k] : dl;", "double beta = dl;"),
    ("bwd zoh dDelta input term without the decay", "double dbeta_ddl = zoh ? a : 1.0;", "double dbeta_ddl = 1.0;"),
    ("bwd zoh dA_log misses the weight's term", "double dbeta_dA = zoh ? (dl * a - beta) / A[k] : 0.0;",
     "double dbeta_dA = 0.0;"),
    ("bwd zoh weight derivative sign", "double dbeta_dA = zoh ? (dl * a - beta) / A[k] : 0.0;",
     "double dbeta_dA = zoh ? (beta - dl * a) / A[k] : 0.0;"),
    ("bwd zoh forward recomputed with Euler", "hs[t * n + k] + input_weight(dl, A[k], B[r + k], zoh) * u[e];",
     "hs[t * n + k] + input_weight(dl, A[k], B[r + k], 0) * u[e];"),
    ("bwd du without the skip", "double dut = dyp * D[d];", "double dut = 0.0;"),
    ("bwd dDelta without the decay term", "ddl += g[k] * (A[k] * a * hprev + dbeta_ddl * B[r + k] * u[e]);",
     "ddl += g[k] * dbeta_ddl * B[r + k] * u[e];"),
    ("bwd dDelta uses the new state", "ddl += g[k] * (A[k] * a * hprev + dbeta_ddl * B[r + k] * u[e]);",
     "ddl += g[k] * (A[k] * a * hs[(t + 1) * n + k] + dbeta_ddl * B[r + k] * u[e]);"),
    ("bwd dA_log without A", "dA_log[d * n + k] += g[k] * (dl * a * hprev + dbeta_dA * B[r + k] * u[e]) * A[k];",
     "dA_log[d * n + k] += g[k] * (dl * a * hprev + dbeta_dA * B[r + k] * u[e]);"),
    ("bwd softplus derivative", "double dd = delta_softplus ? ddl / (1.0 + exp(-x)) : ddl;",
     "double dd = delta_softplus ? ddl / (1.0 + exp(x)) : ddl;"),
    ("bwd dz without y'", "dz[e] = dy[e] * yp * sg * (1.0 + z[e] * (1.0 - sg));", "dz[e] = dy[e] * sg * (1.0 + z[e] * (1.0 - sg));"),
    ("bwd silu derivative", "dz[e] = dy[e] * yp * sg * (1.0 + z[e] * (1.0 - sg));", "dz[e] = dy[e] * yp * sg;"),
    ("bwd gate ignored", "dyp = dy[e] * z[e] * sg;                                /* dy * silu(z) */", "(void)sg;"),
    ("bwd dD uses dy", "dD[d] += dyp * u[e];", "dD[d] += dy[e] * u[e];"),
    ("bwd bias gradient missing", "ddelta_bias[d] += dd;", "ddelta_bias[d] += 0.0;"),
    ("bwd last-state gradient ignored", "g[k] = dlast ? dlast[(bi * d_in + d) * n + k] : 0.0;", "g[k] = 0.0;"),
    ("bwd forward ignores h0", "hs[k] = h0 ? h0[(bi * d_in + d) * n + k] : 0.0;", "hs[k] = 0.0;"),
    ("conv silu ignored", "out[bi * d_in + d] = act ? ss_oracle_silu(acc) : acc;", "out[bi * d_in + d] = acc;"),
]


def failing_pins(lib):
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError, FloatingPointError, OverflowError):
            failed.append(pin.__name__)
    return failed


CHILD = (
    "import sys, warnings\n"
    "warnings.simplefilter('ignore')\n"
    "sys.path.insert(0, sys.argv[2])\n"
    "import oracle\n"
    "from tests.test_oracle_pins import failing_pins\n"
    "print(','.join(failing_pins(oracle.load(sys.argv[1]))))\n"
)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(mutant, tmp_path):
    desc, old, new = mutant[:3]
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation anchor not found exactly once: {old!r}"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    so = str(tmp_path / "libmutant.so")
    subprocess.run(["gcc", *oracle.CFLAGS, "-o", so, str(mutated), "-lm"], check=True)
    if ISOLATE in mutant[3:]:
        root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
        r = subprocess.run([sys.executable, "-c", CHILD, so, root], capture_output=True, text=True, timeout=300)
        failed = r.stdout.strip().split(",") if r.returncode == 0 else [f"crashed ({r.returncode})"]
        failed = [f for f in failed if f]
    else:
        failed = failing_pins(oracle.load(so))
    assert failed, f"planted mistake '{desc}' passed every pin"


def test_openmp_build_is_bit_identical():
    """The OpenMP build of the oracle (the all-cores baseline and the full-size parity reference) only hands
    the independent (batch, channel) recurrences to threads: every output equals the serial build's exactly."""
    import numpy as np
    import torch

    import workloads

    ser, par = oracle.load(), oracle.load_parallel()
    for i, (b, L, d, n, dt, zoh, h0, sp) in enumerate([(3, 97, 70, 16, torch.bfloat16, False, False, True),
                                                       (2, 50, 33, 5, torch.float32, True, True, True),
                                                       (4, 20, 130, 1, torch.float32, False, True, False)]):
        inp = workloads.random_scan_inputs(b, L, d, n, dt, seed=300 + i, gated=i != 2, bias=True)
        if not sp:
            inp["delta"] = inp["delta"].float().abs().to(dt)
            inp["delta_bias"] = inp["delta_bias"].abs()
        hh = torch.randn(b, d, n, generator=torch.Generator().manual_seed(i)) if h0 else None
        args = (inp["u"], inp["delta"], inp["A_log"], inp["B"], inp["C"], inp["D"], inp["z"], inp["delta_bias"], sp)
        y1, l1 = oracle.scan(*args, lib=ser, h0=hh, zoh=zoh)
        y2, l2 = oracle.scan(*args, lib=par, h0=hh, zoh=zoh)
        assert np.array_equal(y1, y2) and np.array_equal(l1, l2), f"scan case {i}"
    dec = workloads.decode_inputs(4, steps=1, b=6)
    st = dec["state"][:, :300].contiguous()
    step = (dec["x"][0][:, :300], dec["dt"][0][:, :300], dec["A_log"][:300], dec["B"][0], dec["C"][0],
            dec["D"][:300], dec["z"][0][:, :300], dec["dt_bias"][:300], True)
    s1, y1 = oracle.state_update(st, *step, lib=ser)
    s2, y2 = oracle.state_update(st, *step, lib=par)
    assert np.array_equal(s1, s2) and np.array_equal(y1, y2)
    assert oracle.threads(ser) == 1
