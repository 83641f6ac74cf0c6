"""Build libss_scan.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python selective_state_space_softplus_amd/build.py

(run as a script: importing the package loads the library this builds).

Packed-fp32 VALU instructions are switched off for all device code.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libss_scan.so")
# The C ABI and the small kernels, then the scan_seq and scan_bwd launchers
# per input type: separate translation units, compiled in parallel.
SOURCES = [os.path.join(CSRC, name) for name in ("ss_scan.hip", "inst_seq_bf16.hip", "inst_seq_f32.hip",
                                                 "inst_bwd_bf16.hip", "inst_bwd_f32.hip")]
ARCH = os.environ.get("SS_OFFLOAD_ARCH", "gfx950")
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops"]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def compile_command(source: str, obj: str) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", *FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", "-o", obj, source]


def link_command(objects: list[str], output: str) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", output, *objects]


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}: {' '.join(cmd[-3:])}")


def build(output: str = LIBRARY, verbose: bool = False) -> str:
    objdir = tempfile.mkdtemp(prefix="ss_build_")
    try:
        objects = [os.path.join(objdir, os.path.basename(src) + ".o") for src in SOURCES]
        workers = max(1, min(len(SOURCES), os.cpu_count() or 1))
        with concurrent.futures.ThreadPoolExecutor(workers) as pool:
            for f in [pool.submit(_run, compile_command(src, obj), verbose) for src, obj in zip(SOURCES, objects)]:
                f.result()
        tmp = output + ".tmp"
        _run(link_command(objects, tmp), verbose)
        os.replace(tmp, output)
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    return output


if __name__ == "__main__":
    print(build(verbose=True))
