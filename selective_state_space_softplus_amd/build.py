"""Build libss_scan.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python selective_state_space_softplus_amd/build.py

(run as a script: importing the package loads the library this builds).

Packed-fp32 VALU instructions are switched off for all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libss_scan.so")
SOURCES = [os.path.join(CSRC, "ss_scan.hip")]
ARCH = os.environ.get("SS_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def command(output: str = LIBRARY) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-fvisibility=hidden", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC, "-o", output, *SOURCES]


def build(output: str = LIBRARY, verbose: bool = False) -> str:
    tmp = output + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build(verbose=True))
