"""The library's HIP sources compiled for the CPU and run there (test infrastructure).

build() copies csrc/ and the generated instantiation units into a cache
directory, turns the kernels' one ``extern __shared__`` declaration into a
pointer to the host LDS buffer (a host compiler has no LDS) and the scalar-
register constraint of an empty asm statement into a host one, and compiles
them with tests/kernel_host/ (a stand-in for the HIP API and the gfx950
builtins the kernels call) into the ``scan_host`` driver, with
AddressSanitizer and UndefinedBehaviorSanitizer.  run() writes a case's
inputs, runs one entry point of the C ABI on them, and reads the outputs.
Work-items are host threads and workgroups run one after another, so this
checks the kernels' indexing, LDS layout, ring protocol and arithmetic, not
their timing.
"""
from __future__ import annotations

import concurrent.futures
import fcntl
import hashlib
import os
import subprocess
import tempfile

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "selective_state_space_softplus_amd", "csrc")
STUB = os.path.join(ROOT, "tests", "kernel_host")
INCLUDE = os.path.join(ROOT, "include")
CLANG = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib", "llvm", "bin", "clang++")
FLAGS = ["-std=c++20", "-O0", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-Wno-unused-command-line-argument",
         "-mllvm", "-asan-globals=0"]   # template constants repeat in every unit; LDS is poisoned by hand
SHARED_DECL = "extern __shared__ __align__(16) float smem[];"
SHARED_HOST = "float* const smem = reinterpret_cast<float*>(emu::lds_base());"
# Register-class constraints of the GPU's inline asm, as the host compiler spells them.
ASM_CONSTRAINTS = (('"+s"(', '"+r"('), ('"+v"(', '"+r"('))


def _sources() -> dict[str, str]:
    out = {}
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".h", ".hip")):
            with open(os.path.join(CSRC, name)) as f:
                text = f.read().replace(SHARED_DECL, SHARED_HOST)
                for a, b in ASM_CONSTRAINTS:
                    text = text.replace(a, b)
                out[name] = text
    for name in ("emu.cpp", os.path.join("hip", "hip_runtime.h")):
        with open(os.path.join(STUB, name)) as f:
            out["stub:" + name] = f.read()
    with open(os.path.join(INCLUDE, "ss_scan.h")) as f:
        out["include:ss_scan.h"] = f.read()
    return out


def build(verbose: bool = False) -> str:
    """Path of the scan_host executable, compiled once per version of the sources."""
    srcs = _sources()
    key = hashlib.sha256(("".join(k + v for k, v in sorted(srcs.items())) + " ".join(FLAGS)).encode()).hexdigest()[:16]
    cache = os.path.join(tempfile.gettempdir(), f"ss_scan_host_{key}")
    exe = os.path.join(cache, "scan_host")
    if os.path.exists(exe):
        return exe
    os.makedirs(cache, exist_ok=True)
    # One builder per cache directory (pytest-xdist workers share it): a
    # source rewritten under a running compiler would break that compile.
    with open(os.path.join(cache, ".lock"), "w") as lock:
        fcntl.flock(lock, fcntl.LOCK_EX)
        if os.path.exists(exe):
            return exe
        return _build_locked(srcs, cache, exe)


def _build_locked(srcs: dict, cache: str, exe: str) -> str:
    import importlib.util

    for name, text in srcs.items():
        if ":" not in name:
            with open(os.path.join(cache, name), "w") as f:
                f.write(text)
    spec = importlib.util.spec_from_file_location(
        "_ss_hip_build", os.path.join(ROOT, "selective_state_space_softplus_amd", "build.py"))
    hb = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(hb)
    units = [os.path.join(cache, "ss_scan.hip")] + hb.instantiation_units(cache) + [os.path.join(STUB, "emu.cpp")]
    objs = [os.path.join(cache, os.path.basename(u) + ".o") for u in units]

    def compile_one(src, obj):
        cmd = [CLANG, *FLAGS, "-I", STUB, "-I", INCLUDE, "-I", cache, "-x", "c++", "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"host build of {os.path.basename(src)} failed:\n{r.stderr[-4000:]}")

    with concurrent.futures.ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as pool:
        for f in [pool.submit(compile_one, s, o) for s, o in zip(units, objs)]:
            f.result()
    tmp = exe + ".tmp"
    r = subprocess.run([CLANG, "-fsanitize=address,undefined", "-pthread", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"host link failed:\n{r.stderr[-4000:]}")
    os.replace(tmp, exe)
    return exe


def _np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).numpy()
    return t.contiguous().numpy()


def run(mode: str, tensors: dict, args: dict, outputs: dict, timeout: float = 600.0) -> dict:
    """Run entry point `mode` on the host.  tensors: name -> CPU tensor (None = absent);
    args: name -> int; outputs: name -> (shape, torch dtype).  Returns name -> tensor."""
    exe = build()
    with tempfile.TemporaryDirectory(prefix="ss_host_case_") as d:
        for k, v in tensors.items():
            if v is not None:
                _np(v).tofile(os.path.join(d, k + ".bin"))
        with open(os.path.join(d, "args.txt"), "w") as f:
            for k, v in args.items():
                f.write(f"{k} {int(v)}\n")
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:detect_odr_violation=0", UBSAN_OPTIONS="print_stacktrace=1")
        r = subprocess.run([exe, mode, d], capture_output=True, text=True, timeout=timeout, env=env)
        if r.returncode != 0:
            raise AssertionError(f"scan_host {mode} failed ({r.returncode}):\n{r.stderr[-6000:]}")
        out = {}
        for k, (shape, dt) in outputs.items():
            path = os.path.join(d, k + ".out.bin")
            if not os.path.exists(path):
                continue
            raw = np.fromfile(path, np.int16 if dt == torch.bfloat16 else np.float32)
            t = torch.from_numpy(raw.copy())
            out[k] = (t.view(torch.bfloat16) if dt == torch.bfloat16 else t).reshape(shape)
        return out
