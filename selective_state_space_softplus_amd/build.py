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
# The VALU issue-rate probe that bench.py --valu-probe runs (a measurement aid).
PROBE_SOURCE = os.path.join(CSRC, "valu_probe.hip")
PROBE_LIBRARY = os.path.join(PKG, "libss_probe.so")
# The C ABI and the small kernels in one translation unit; the scan_seq and
# scan_bwd launchers (launch_seq.h, launch_bwd.h) are instantiated once per
# input type and launch shape, each in a small generated unit of its own, so
# that the kernels compile in parallel.
SOURCES = [os.path.join(CSRC, "ss_scan.hip")]
INPUT_TYPES = ("uint16_t", "float")
SEQ_SHAPES = ((1, 2), (4, 2), (4, 4), (8, 2), (8, 4), (8, 8))   # must cover ss_host::seq_shape
BWD_SHAPES = ((1, 2, False), (4, 2, False), (8, 2, False), (8, 2, True))   # must cover ss_host::bwd_shape
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


def instantiation_units(objdir: str) -> list[str]:
    """Write one source per (launcher, input type, shape) into objdir; returns their paths."""
    units = []
    for ty in INPUT_TYPES:
        for header, fn, shapes, sig in (
                ("launch_seq.h", "launch_seq", [(sc, nsw, None) for sc, nsw in SEQ_SHAPES],
                 "ss::ScanParams, SeqMode, void*, size_t, hipStream_t"),
                ("launch_bwd.h", "launch_bwd", BWD_SHAPES, "ss::BwdParams, bool, bool, hipStream_t, int*")):
            for sc, nsw, sl in shapes:
                targs = f"{ty}, {sc}, {nsw}" + ("" if sl is None else f", {'true' if sl else 'false'}")
                tag = f"{sc}x{nsw}" + ("" if not sl else "_sliced")
                path = os.path.join(objdir, f"{fn}_{ty}_{tag}.hip")
                with open(path, "w") as f:
                    f.write(f'#include "{header}"\nnamespace ss_host {{\n'
                            f"template int {fn}<{targs}>({sig});\n}}\n")
                units.append(path)
    return units


def build(output: str = LIBRARY, verbose: bool = False) -> str:
    objdir = tempfile.mkdtemp(prefix="ss_build_")
    try:
        sources = SOURCES + instantiation_units(objdir)
        objects = [os.path.join(objdir, os.path.basename(src) + ".o") for src in sources]
        workers = max(1, min(len(sources), os.cpu_count() or 1))
        with concurrent.futures.ThreadPoolExecutor(workers) as pool:
            # The largest units first, so the pool does not end on one of them.
            order = sorted(range(len(sources)), key=lambda i: "_8x" not in sources[i] and "ss_scan" not in sources[i])
            futures = [pool.submit(_run, compile_command(sources[i], objects[i]), verbose) for i in order]
            for f in futures:
                f.result()
        tmp = output + ".tmp"
        _run(link_command(objects, tmp), verbose)
        os.replace(tmp, output)
        if output == LIBRARY:
            probe_obj = os.path.join(objdir, "valu_probe.hip.o")
            _run(compile_command(PROBE_SOURCE, probe_obj), verbose)
            _run(link_command([probe_obj], PROBE_LIBRARY + ".tmp"), verbose)
            os.replace(PROBE_LIBRARY + ".tmp", PROBE_LIBRARY)
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    return output


if __name__ == "__main__":
    print(build(verbose=True))
