"""Throughput of the selective scan (and of the decode step) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]

A step is one ss_scan_fwd over the scan-long workload (b=4, L=8192, d_in=5120,
n=16, bf16 inputs/outputs, fp32 state, gated, delta bias, last state
written), with every input already resident in HBM.  The value is achieved
algorithmic HBM bandwidth in GB/s; state updates/s and the fraction of the
8 TB/s HBM peak are reported beside it.  The decode step (b=256, d_in=5120,
n=16, 64 back-to-back single-token steps) and the convolution step that
precedes it in a decode step (same b and d_in, width 4, bf16) are timed in the
same run, and so are the other scan workloads (scan-tiny, scan-mid after a
write that evicts the last-level cache, scan-vmamba as a plain scan).

Algorithmic bytes are what the fused method must move (the (b, L, d_in, n)
intermediates are never stored):
  scan   = s*(3 bLd [u, delta, y] + bLd [z] + 2 bLn [B, C]) + 4*(d n [A_log] + d [D] + d [bias]) + 4 b d n [last state]
  decode = 8 b d n [state read + write] + s*(4 b d [x, dt, z, y] + 2 b n [B, C]) + 4*(d n + 2 d)
  conv   = s*b d (2 W [window read + write] + 2 [x, out]) + 4*(d W + d) [weight, bias]
with s the input element size.

The dominant kernel at n = 16 is bound by VALU issue, not by HBM: each state
update needs 4 fp32 VALU operations plus one v_exp_f32, which issues at half
the fp32 rate, i.e. 6 issue slots per update.  The roofline object therefore
reports bound "alu": achieved = updates/s * 6 slots, peak = 256 CUs * 64 lanes
* 2.4 GHz = 39.3 T slots/s.

The CPU baseline is the double-precision oracle (plain C) timed on the host
on a bounded sample of the same workload (about 15 s of work each): whole
batches of all channels, or the first channels of batch 0, over the full
length -- once with its OpenMP build on all host threads (the value; the
thread count is reported) and once single-threaded.

--copy-probe runs only a plain 1 GiB device copy; its HBM byte counters
calibrate the counters read on the scan kernel.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
VALU_PEAK_TSLOTS = 256 * 64 * 2.4e9 / 1e12      # 39.32 T fp32 VALU lane-slots/s
SLOTS_PER_UPDATE = 6                              # mul, exp (2 slots), mul, fma, fma
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def scan_bytes(b, L, d, n, s, gated=True, bias=True, last=True):
    return (s * (3 * b * L * d + (b * L * d if gated else 0) + 2 * b * L * n)
            + 4 * (d * n + d + (d if bias else 0)) + (4 * b * d * n if last else 0))


def decode_bytes(b, d, n, s, gated=True, bias=True):
    return 8 * b * d * n + s * ((4 if gated else 3) * b * d + 2 * b * n) + 4 * (d * n + d + (d if bias else 0))


def conv_bytes(b, d, W, s, bias=True):
    return s * b * d * (2 * W + 2) + 4 * (d * W + (d if bias else 0))


def cross_bytes(maps, L, d, n, s, bias=False):
    """Fused cross scan: the map once, per-direction delta, B, C, the fp32 output map, parameters."""
    return s * (maps * L * d + 4 * maps * L * d + 8 * maps * L * n) + 4 * maps * L * d + 4 * (4 * d * n + 4 * d * (2 if bias else 1))


# Sources of the forward scan kernel (scan_seq) and its launch: the measured
# traffic in profiles/traffic.json is used only while these are unchanged.
SCAN_KERNEL_SOURCES = ("scan_kernels.h", "ss_device.h", "ss_host.h", "launch_seq.h")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "selective_state_space_softplus_amd", "csrc")
    for name in SCAN_KERNEL_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch from the rocprofv3 counter runs, if they match the current kernel source."""
    try:
        rec = json.load(open(TRAFFIC_FILE))[kernel]
    except (OSError, KeyError, ValueError):
        return None
    return rec.get("bytes_per_launch") if rec.get("source_hash") == kernel_source_hash() else None


def time_scan(ss, torch, g, steps, warmup, last, prewarm_s=0.3):
    """Average step time over `steps` launches after `warmup` untimed ones.

    Before the warm-up steps the scan runs untimed for about `prewarm_s`
    seconds: an idle GPU first raises its clocks, and the first few hundred
    milliseconds of launches run measurably slower than the steady state the
    throughput figure is about.
    """
    args = (g["u"], g["delta"], g["A_log"], g["B"], g["C"], g["D"], g["z"], g["delta_bias"], g["delta_softplus"])
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < prewarm_s:
        for _ in range(10):
            ss.scan_fwd(*args, return_last_state=last)
        torch.cuda.synchronize()
    for _ in range(warmup):
        ss.scan_fwd(*args, return_last_state=last)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_all0.record()
    for e0, e1 in ev:
        e0.record()
        ss.scan_fwd(*args, return_last_state=last)
        e1.record()
    t_all1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    per = [e0.elapsed_time(e1) for e0, e1 in ev]
    return t_all0.elapsed_time(t_all1) / steps, sum(per) / len(per), wall


def other_workloads(ss, torch, workloads, dev, reps=20):
    """The other scan workloads, each timed with HIP events on the launch stream (median of `reps`):
    scan-tiny (launch-bound: 200 back-to-back calls), scan-mid (its 203 MB fit the 256 MB last-level
    cache, so each timed call follows a 512 MB write that evicts it; back-to-back calls reported beside),
    scan-vmamba as a plain scan of the four unrolled directions (b=64, n=1, fp32, ungated)."""
    import statistics

    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    out = {}
    for idx in (0, 1, 3):
        cfg = workloads.CONFIGS[idx]
        inp = workloads.scan_inputs(idx)
        g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
        s = 2 if cfg.dtype == torch.bfloat16 else 4
        gated, bias = g["z"] is not None, g["delta_bias"] is not None
        nbytes = scan_bytes(cfg.b, cfg.L, cfg.d_in, cfg.n, s, gated, bias, True)
        y = torch.empty_like(g["u"])
        last = torch.empty((cfg.b, cfg.d_in, cfg.n), dtype=torch.float32, device=dev)

        def call():
            ss.scan_fwd(g["u"], g["delta"], g["A_log"], g["B"], g["C"], g["D"], g["z"], g["delta_bias"], True,
                        out=y, last_state=last, return_last_state=True)

        for _ in range(20):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        row = {"workload": f"{cfg.name}: b={cfg.b} L={cfg.L} d_in={cfg.d_in} n={cfg.n}, "
                           f"{'bf16' if s == 2 else 'fp32'}{', gated' if gated else ''}"
                           f"{', delta bias' if bias else ''}, softplus, last state written",
               "algorithmic_bytes": nbytes}
        if idx == 0:
            k = 200
            e0.record()
            for _ in range(k):
                call()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / k
            row["note"] = f"{k} back-to-back calls: launch-bound"
        else:
            per = []
            for _ in range(reps):
                if idx == 1:
                    flush.zero_()
                e0.record()
                call()
                e1.record()
                torch.cuda.synchronize()
                per.append(e0.elapsed_time(e1) * 1e3)
            us = statistics.median(per)
            if idx == 1:
                row["note"] = "each call after a 512 MB write that evicts the last-level cache"
                b2b = []
                for _ in range(reps):
                    e0.record()
                    call()
                    e1.record()
                    torch.cuda.synchronize()
                    b2b.append(e0.elapsed_time(e1) * 1e3)
                row["us_back_to_back"] = round(statistics.median(b2b), 2)
        row["us"] = round(us, 2)
        row["GBps"] = round(nbytes / (us * 1e-6) / 1e9, 1)
        row["hbm_frac"] = round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)
        row["updates_per_s"] = float(f"{cfg.updates / (us * 1e-6):.4g}")
        out[cfg.name] = row
        del g, y, last
    return out


def valu_probe(torch, dev, iters=16384, reps=10, settle_s=0.3):
    """Issue rates of fp32 FMA, multiply and exp2 chains (libss_probe.so) at 8, 4 and 2 waves per SIMD.

    Each work-item runs `iters` steps of 8 independent chains; a step is one
    v_fma_f32 (mix 0), one v_mul_f32 (mix 1), one v_exp_f32 plus one
    v_mul_f32 (mix 2) or one v_exp_f32 (mix 3).  The issue cost of
    v_exp_f32, in multiplies, is t3 / t1 alone and t2 / t1 - 1 mixed.  The
    probe first runs untimed for `settle_s` seconds so the clocks settle.
    """
    import ctypes

    lib = ctypes.CDLL(os.path.join(ROOT, "selective_state_space_softplus_amd", "libss_probe.so"))
    lib.ss_probe_valu.restype = ctypes.c_int
    lib.ss_probe_valu.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.empty(cus * 8 * 256, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    run = lambda mix, blocks: lib.ss_probe_valu(mix, blocks, iters, ctypes.c_void_p(out.data_ptr()), stream)  # noqa: E731
    t0 = time.time()
    while time.time() - t0 < settle_s:
        assert run(0, cus * 4) == 0
        torch.cuda.synchronize()
    res = {"metric": "VALU issue rates (probe)", "cus": cus, "iters": iters, "chains_per_work_item": 8}
    for waves_per_simd in (8, 4, 2):
        blocks = cus * waves_per_simd     # 256 work-items = 4 waves a block, one per SIMD
        row = {}
        for mix, name, instr in ((0, "fma", 1), (1, "mul", 1), (2, "exp2+mul", 2), (3, "exp2", 1)):
            assert run(mix, blocks) == 0
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                run(mix, blocks)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            lane_instr = blocks * 256 * iters * 8 * instr
            row[name] = {"ms": round(ms, 4), "lane_instr_per_s_T": round(lane_instr / (ms * 1e-3) / 1e12, 2)}
        row["exp2_cost_in_muls_alone"] = round(row["exp2"]["ms"] / row["mul"]["ms"], 3)
        row["exp2_cost_in_muls_mixed"] = round(row["exp2+mul"]["ms"] / row["mul"]["ms"] - 1.0, 3)
        res[f"{waves_per_simd}_waves_per_simd"] = row
    res["fp32_vector_peak_T"] = round(cus * 4 * 16 * 2.4e9 / 1e12, 2)
    print(json.dumps(res), flush=True)
    return 0


def copy_probe(torch, dev, nbytes=1 << 30, reps=5):
    """A plain device copy of known size: each launch reads and writes nbytes."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "launches": 2 * reps,
                      "ms_per_copy": round(ms, 4), "GBps": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}), flush=True)
    return 0


def shape_sweep(torch, ss, workloads, dev):
    """Forward (and backward) throughput over state sizes, input types and the
    zero-order hold at b=4, L=8192, d_in=5120, plus the b=8, L=2048, d_in=1536
    scan: one JSON line per case, HIP events over 10 launches (5 for the
    backward) after 0.3 s of untimed ones."""
    cases = [(4, 8192, 5120, n, torch.bfloat16, False) for n in (1, 2, 4, 8, 16, 32, 64)]
    cases += [(4, 8192, 5120, 16, torch.float32, False), (4, 8192, 5120, 16, torch.bfloat16, True),
              (8, 2048, 1536, 16, torch.bfloat16, False)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, reps=10, settle_s=0.3):
        # Untimed launches for settle_s seconds first: the GPU idles while the
        # next case's inputs are generated and must raise its clocks again.
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < settle_s:
            fn()
            torch.cuda.synchronize()
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    for b, L, d, n, dt, zoh in cases:
        inp = workloads.random_scan_inputs(b, L, d, n, dtype=dt, seed=7, gated=True, bias=True)
        g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
        del inp
        args = (g["u"], g["delta"], g["A_log"], g["B"], g["C"], g["D"], g["z"], g["delta_bias"], True)
        ms = timed(lambda: ss.scan_fwd(*args, return_last_state=True, zoh=zoh))
        s = 2 if dt == torch.bfloat16 else 4
        upd = b * L * d * n
        row = {"b": b, "L": L, "d_in": d, "n": n, "io_dtype": "bf16" if s == 2 else "f32", "zoh": zoh,
               "fwd_ms": round(ms, 4), "fwd_updates_per_s": float(f"{upd / (ms * 1e-3):.4g}"),
               "fwd_GBps": round(scan_bytes(b, L, d, n, s) / (ms * 1e-3) / 1e9, 1)}
        if n in (1, 16, 64) and not zoh:
            dy = torch.randn_like(g["u"])
            mb = timed(lambda: ss.scan_bwd(*args[:6], dy, g["z"], g["delta_bias"], True), reps=5)
            row.update(bwd_ms=round(mb, 4), bwd_updates_per_s=float(f"{upd / (mb * 1e-3):.4g}"))
            del dy
        print(json.dumps(row), flush=True)
        del g, args
        torch.cuda.empty_cache()
    return 0


def cpu_baseline(cfg, inp, s, budget):
    """The oracle timed on this host on bounded samples of the workload: all threads, then one."""
    import numpy as np
    import torch

    import oracle

    # Inputs widened to float64 once, outside the timed region (the oracle
    # computes in double on float64 arrays).
    f64 = {k: (inp[k].to(torch.float64).numpy() if isinstance(inp[k], torch.Tensor) else inp[k])
           for k in ("u", "delta", "A_log", "B", "C", "D", "z", "delta_bias")}

    def run(lib, nb, k):
        sl = lambda t: None if t is None else np.ascontiguousarray(t[0:nb, :, 0:k])  # noqa: E731
        a = (sl(f64["u"]), sl(f64["delta"]), np.ascontiguousarray(f64["A_log"][:k]), f64["B"][0:nb],
             f64["C"][0:nb], np.ascontiguousarray(f64["D"][:k]), sl(f64["z"]),
             np.ascontiguousarray(f64["delta_bias"][:k]))
        t0 = time.perf_counter()
        oracle.scan(*a, True, lib=lib)
        return time.perf_counter() - t0

    def sample(lib, budget):
        """Whole batch rows (all channels, all steps) if one fits the budget, else the first channels of
        batch 0; returns (batches, channels, seconds)."""
        per_rec = run(lib, 1, 64) / 64
        want = max(1, int(budget / max(per_rec, 1e-9)))
        if want <= cfg.d_in:
            nb, k = 1, min(want, cfg.d_in)
        else:
            nb, k = min(cfg.b, max(1, want // cfg.d_in)), cfg.d_in
        return nb, k, run(lib, nb, k)

    def leg(lib, nb, k, secs, cores):
        cb = scan_bytes(nb, cfg.L, k, cfg.n, s, cfg.gated, cfg.bias, True)
        return {"value": round(cb / secs / 1e9, 4), "unit": "GB/s",
                "updates_per_s": float(f"{nb * cfg.L * k * cfg.n / secs:.4g}"), "cores": cores,
                "kind": "oracle",
                "sample": f"{cfg.name}: batches 0..{nb - 1}, channels 0..{k - 1}, all {cfg.L} steps "
                          f"({nb * k} of {cfg.b * cfg.d_in} recurrences), double precision, "
                          f"{cores} thread{'s' if cores > 1 else ''}, {secs:.1f} s"}

    par = oracle.load_parallel()
    threads = oracle.threads(par)
    nb, k, secs = sample(par, budget)
    out = leg(par, nb, k, secs, threads)
    nb1, k1, secs1 = sample(oracle.load(), budget)
    out["single_core"] = leg(None, nb1, k1, secs1, 1)
    out["note"] = ("the same C oracle built twice: with OpenMP over the independent (batch, channel) "
                   "recurrences on all host threads, and serially")
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--prewarm", type=float, default=0.3, help="seconds of untimed scans before the warm-up steps")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-step measurement")
    ap.add_argument("--no-cross", action="store_true", help="skip the VMamba cross-scan measurement")
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward-pass measurement")
    ap.add_argument("--no-others", action="store_true", help="skip the scan-tiny, scan-mid and scan-vmamba timings")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target duration of the CPU baseline sample")
    ap.add_argument("--valu-probe", action="store_true",
                    help="only time the VALU issue-rate probe (fma, mul, exp2 chains) and print its JSON line")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (calibrates the HBM byte counters)")
    ap.add_argument("--sweep", action="store_true",
                    help="only time the forward and backward over state sizes, input types and shapes")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the scan shards over batch and channels with no communication, "
              f"and no multi-GPU path is built (asked for --gpus {args.gpus})", file=sys.stderr)
        return 2

    import torch

    import selective_state_space_softplus_amd as ss
    import workloads

    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.copy_probe:
        return copy_probe(torch, dev)
    if args.valu_probe:
        return valu_probe(torch, dev)
    if args.sweep:
        return shape_sweep(torch, ss, workloads, dev)
    cfg = workloads.CONFIGS[2]
    inp = workloads.scan_inputs(2)
    g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    s = 2 if cfg.dtype == torch.bfloat16 else 4
    nbytes = scan_bytes(cfg.b, cfg.L, cfg.d_in, cfg.n, s, cfg.gated, cfg.bias, True)
    ms_step, ms_kernel, wall = time_scan(ss, torch, g, args.steps, args.warmup, True, args.prewarm)
    gbps = nbytes / (ms_step * 1e-3) / 1e9
    ups = cfg.updates / (ms_step * 1e-3)
    kernel_gbps = nbytes / (ms_kernel * 1e-3) / 1e9
    kernel_ups = cfg.updates / (ms_kernel * 1e-3)
    achieved_slots = kernel_ups * SLOTS_PER_UPDATE / 1e12

    result = {
        "metric": "selective-scan achieved HBM GB/s (% of MI355X peak) + state updates/s",
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",                           # the arithmetic: state, recurrence and readout in fp32
        "io_dtype": "bf16",                       # u, delta, z, B, C read and y written as bf16
        "data": "synthetic (seeded N(0,1) inputs, delta ~ N(0,1)-2 plus bias ~ U(log 1e-3, log 1e-1), A_log = log(1..16))",
        "config": {"workload": f"{cfg.name}: selective scan fwd b={cfg.b} L={cfg.L} d_in={cfg.d_in} n={cfg.n}, "
                               "bf16, gated, delta bias + softplus, last state written",
                   "global_batch": cfg.b, "seq_len": cfg.L, "d_in": cfg.d_in, "d_state": cfg.n,
                   "parallelism": "single GPU"},
        "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "updates_per_s": float(f"{ups:.4g}"),
        "algorithmic_bytes_per_step": nbytes,
        "roofline": {
            "bound": "alu",
            "kernel": "scan_seq<bf16, 8 recurrence waves x 2 states + 4 element waves + 1 loader wave>",
            "achieved": round(achieved_slots, 2),
            "peak": round(VALU_PEAK_TSLOTS, 2),
            "unit": "Tslot/s",
            "op": "fp32 VALU lane issue slots; 6 per state update (v_exp_f32 counts 2: half rate on gfx950)",
            "frac": round(achieved_slots / VALU_PEAK_TSLOTS, 4),
            "traffic": measured_traffic("scan_seq"),
            "hbm_achieved_GBps": round(kernel_gbps, 1),
            "hbm_peak_GBps": HBM_PEAK_GBPS,
            "kernel_ms": round(ms_kernel, 4),
        },
        "host_wall_s": round(wall, 3),
        "prewarm_s": args.prewarm,
    }

    if not args.no_others:
        result["other_workloads"] = other_workloads(ss, torch, workloads, dev)

    if not args.no_decode:
        dcfg = workloads.CONFIGS[4]
        dinp = workloads.decode_inputs(4)
        d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in dinp.items()}
        state = d["state"].clone()

        def run64():
            for t in range(dcfg.steps):
                ss.state_update(state, d["x"][t], d["dt"][t], d["A_log"], d["B"][t], d["C"][t], d["D"], d["z"][t],
                                d["dt_bias"], True)

        run64()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 3
        e0.record()
        for _ in range(reps):
            run64()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / (reps * dcfg.steps)
        db = decode_bytes(dcfg.b, dcfg.d_in, dcfg.n, 2)
        result["decode"] = {
            "workload": f"{dcfg.name}: b={dcfg.b} d_in={dcfg.d_in} n={dcfg.n}, fp32 state, bf16 x/dt/z/B/C, "
                        f"{dcfg.steps} back-to-back steps (one state of {dcfg.b * dcfg.d_in * dcfg.n * 4 / 1e6:.1f} MB, "
                        "which the 256 MB last-level cache can hold between steps; *_hbm: each step on the next of "
                        "6 states, so the state is read from and written to HBM)",
            "us_per_step": round(ms * 1e3, 2),
            "GBps": round(db / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(db / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "updates_per_s": float(f"{dcfg.b * dcfg.d_in * dcfg.n / (ms * 1e-3):.4g}"),
            "algorithmic_bytes_per_step": db,
        }
        # The convolution step of the same decode step (width 4, bf16 window).
        W = 4
        gen = torch.Generator(device=dev).manual_seed(4)
        cst = torch.randn(dcfg.b, dcfg.d_in, W, device=dev, generator=gen).to(torch.bfloat16)
        cx = torch.randn(dcfg.steps, dcfg.b, dcfg.d_in, device=dev, generator=gen).to(torch.bfloat16)
        cw = torch.randn(dcfg.d_in, W, device=dev, generator=gen) * 0.5
        cb = torch.randn(dcfg.d_in, device=dev, generator=gen) * 0.1
        cout = torch.empty(dcfg.b, dcfg.d_in, device=dev, dtype=torch.bfloat16)

        def conv64():
            for t in range(dcfg.steps):
                ss.conv_update(cst, cx[t], cw, cb, silu=True, out=cout)

        conv64()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            conv64()
        e1.record()
        torch.cuda.synchronize()
        cms = e0.elapsed_time(e1) / (reps * dcfg.steps)
        cbytes = conv_bytes(dcfg.b, dcfg.d_in, W, 2)

        # Both steps again as HIP graphs of 64 launches each: what a decode loop
        # that captures its steps sees, without the per-call host overhead.
        def graphed(fn):
            side = torch.cuda.Stream(device=dev)
            side.wait_stream(torch.cuda.current_stream(dev))
            with torch.cuda.stream(side):
                fn()
            torch.cuda.current_stream(dev).wait_stream(side)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                fn()
            graph.replay()
            torch.cuda.synchronize()
            e0.record()
            for _ in range(reps):
                graph.replay()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / (reps * dcfg.steps)

        ms_g = graphed(run64)
        cms_g = graphed(conv64)

        # The state resident in HBM: the same 64 back-to-back steps, each on the
        # next of 6 state buffers in turn (6 x 84 MB, more than the 256 MB
        # last-level cache holds, so a step finds its state evicted by the
        # other five).  Timing single steps after a cache flush instead would
        # add the launch and event latency (about 15 us) to every step.
        nrot = 6
        rot = [state.clone() for _ in range(nrot)]

        def run64_rot():
            for t in range(dcfg.steps):
                ss.state_update(rot[t % nrot], d["x"][t], d["dt"][t], d["A_log"], d["B"][t], d["C"][t], d["D"],
                                d["z"][t], d["dt_bias"], True)

        run64_rot()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            run64_rot()
        e1.record()
        torch.cuda.synchronize()
        ms_h = e0.elapsed_time(e1) / (reps * dcfg.steps)
        del rot
        # A plain device copy (torch) of one state, rotated over 6 buffer pairs
        # in the same way: what a kernel of this size that reads and writes
        # the state once reaches, beside the step's own rate.
        src = [state.clone() for _ in range(nrot)]
        dst = [torch.empty_like(state) for _ in range(nrot)]

        def copy64():
            for t in range(dcfg.steps):
                dst[t % nrot].copy_(src[t % nrot])

        copy64()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            copy64()
        e1.record()
        torch.cuda.synchronize()
        ms_c = e0.elapsed_time(e1) / (reps * dcfg.steps)
        del src, dst
        copy_gbps = 2 * state.numel() * state.element_size() / (ms_c * 1e-3) / 1e9
        result["decode"]["us_per_step_hbm"] = round(ms_h * 1e3, 2)
        result["decode"]["GBps_hbm"] = round(db / (ms_h * 1e-3) / 1e9, 1)
        result["decode"]["state_copy_GBps"] = round(copy_gbps, 1)
        result["decode"]["hbm_frac_of_state_copy"] = round(db / (ms_h * 1e-3) / 1e9 / copy_gbps, 3)
        result["decode"]["us_per_step_graph"] = round(ms_g * 1e3, 2)
        result["decode"]["GBps_graph"] = round(db / (ms_g * 1e-3) / 1e9, 1)
        result["decode"]["conv_step"] = {
            "workload": f"conv step: b={dcfg.b} d_in={dcfg.d_in} W={W}, bf16 window/x/out, fp32 weight and bias, "
                        f"silu, {dcfg.steps} back-to-back steps",
            "us_per_step": round(cms * 1e3, 2),
            "GBps": round(cbytes / (cms * 1e-3) / 1e9, 1),
            "us_per_step_graph": round(cms_g * 1e3, 2),
            "GBps_graph": round(cbytes / (cms_g * 1e-3) / 1e9, 1),
            "algorithmic_bytes_per_step": cbytes,
        }

    # A plain device copy of 1 GiB (torch's copy kernel): what this machine's HBM
    # delivers to a streaming kernel, the practical ceiling beside the 8 TB/s
    # specification.
    csrc_t = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    cdst_t = torch.empty_like(csrc_t)
    for _ in range(3):
        cdst_t.copy_(csrc_t)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(5):
        cdst_t.copy_(csrc_t)
    c1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * (1 << 30) / (c0.elapsed_time(c1) / 5 * 1e-3) / 1e9
    del csrc_t, cdst_t
    result["copy_GBps"] = round(copy_gbps, 1)
    result["hbm_frac_of_copy"] = round(gbps / copy_gbps, 4)

    if not args.no_bwd:
        # The gradient of the same scan-long scan (ss_scan_bwd: the forward
        # again with state checkpoints every 8 steps, the adjoint pass, the
        # fixed-order sums), for an output gradient dy of y's shape.
        dyb = torch.randn(g["u"].shape, device=dev, generator=torch.Generator(device=dev).manual_seed(5)).to(g["u"].dtype)
        bws = torch.empty(ss.lib.ss_scan_bwd_workspace_bytes(cfg.b, cfg.L, cfg.d_in, cfg.n, 1), dtype=torch.uint8,
                          device=dev)

        def bwd():
            ss.scan_bwd(g["u"], g["delta"], g["A_log"], g["B"], g["C"], g["D"], dyb, g["z"], g["delta_bias"], True,
                        workspace=bws)

        for _ in range(2):
            bwd()
        torch.cuda.synchronize()
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b0.record()
        for _ in range(5):
            bwd()
        b1.record()
        torch.cuda.synchronize()
        bms = b0.elapsed_time(b1) / 5
        result["backward"] = {
            "workload": f"{cfg.name}: gradient of the scan above for a given dy (du, ddelta, dz, dA_log, dB, dC, dD, "
                        "dbias), forward recomputed inside with state checkpoints every 8 steps",
            "ms": round(bms, 4),
            "updates_per_s": float(f"{cfg.updates / (bms * 1e-3):.4g}"),
            "vs_forward": round(bms / ms_step, 2),
        }
        del bws
        # The training pair: a forward that keeps the state every 8 steps and
        # the pre-gate readout (ss_scan_fwd_save), and the backward from them
        # (ss_scan_bwd_saved), each timed on its own and as one training step.
        fws = torch.empty(ss.scan_fwd_workspace_bytes(cfg.b, cfg.L, cfg.d_in, cfg.n, 1), dtype=torch.uint8,
                          device=dev)
        sws = torch.empty(ss.lib.ss_scan_bwd_saved_workspace_bytes(cfg.b, cfg.L, cfg.d_in, cfg.n, 1),
                          dtype=torch.uint8, device=dev)
        saved = {}

        def fwd_save():
            saved.update(ss.scan_fwd_save(g["u"], g["delta"], g["A_log"], g["B"], g["C"], g["D"], g["z"],
                                          g["delta_bias"], True, workspace=fws))

        def bwd_saved():
            ss.scan_bwd(g["u"], g["delta"], g["A_log"], g["B"], g["C"], g["D"], dyb, g["z"], g["delta_bias"], True,
                        workspace=sws, saved=saved)

        def timed(fn, reps=5):
            for _ in range(2):
                fn()
            torch.cuda.synchronize()
            b0.record()
            for _ in range(reps):
                fn()
            b1.record()
            torch.cuda.synchronize()
            return b0.elapsed_time(b1) / reps

        fms = timed(fwd_save)
        sms = timed(bwd_saved)
        result["backward"]["from_saved"] = {
            "workload": f"{cfg.name}: ss_scan_fwd_save (y, plus the state every 8 steps and the readout before the "
                        "gate) and ss_scan_bwd_saved (the same gradients, starting from those)",
            "fwd_save_ms": round(fms, 4),
            "bwd_saved_ms": round(sms, 4),
            "bwd_saved_updates_per_s": float(f"{cfg.updates / (sms * 1e-3):.4g}"),
            "training_step_ms": round(fms + sms, 4),
            "training_step_ms_recomputing": round(ms_step + bms, 4),
        }
        del saved, fws, sws

    if not args.no_cross:
        # VMamba's cross scan on the scan-vmamba maps: the fused kernel against
        # the same work done the unfused way (the four traversal copies made
        # with torch, the plain scan, the merge with torch).
        vcfg = workloads.CONFIGS[3]
        ci = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in workloads.cross_scan_inputs(3).items()}
        maps, H, L, d, n = vcfg.maps, vcfg.side, vcfg.L, vcfg.d_in, vcfg.n
        yout = torch.empty(maps, H, H, d, device=dev)

        def fused(form="auto"):
            ss.cross_scan_fwd(ci["x"], ci["delta"], ci["A_log"], ci["B"], ci["C"], ci["D"], None, True, out=yout,
                              form=form)

        dl2, B2, C2 = ci["delta"].reshape(maps * 4, L, d), ci["B"].reshape(maps * 4, L, n), ci["C"].reshape(maps * 4, L, n)

        def unfused():
            u = workloads.vmamba_unroll(ci["x"])
            yd = ss.scan_fwd(u, dl2, ci["A_log"][0], B2, C2, ci["D"][0], None, None, True).reshape(maps, 4, L, d)
            return (yd[:, 0].reshape(maps, H, H, d) + yd[:, 1].reshape(maps, H, H, d).transpose(1, 2)
                    + yd[:, 2].flip(1).reshape(maps, H, H, d) + yd[:, 3].flip(1).reshape(maps, H, H, d).transpose(1, 2))

        u_pre = workloads.vmamba_unroll(ci["x"])

        def scan_only():
            ss.scan_fwd(u_pre, dl2, ci["A_log"][0], B2, C2, ci["D"][0], None, None, True)

        def timed(fn, reps=10):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record()
            for _ in range(reps):
                fn()
            a1.record()
            torch.cuda.synchronize()
            return a0.elapsed_time(a1) / reps

        ms_f, ms_u, ms_s = timed(fused), timed(unfused), timed(scan_only)
        ms_1 = timed(lambda: fused("one_pass"))
        xb = cross_bytes(maps, L, d, n, 4)
        result["vmamba_cross"] = {
            "workload": f"{vcfg.name}: {maps} maps of {H}x{H}x{d}, 4 traversal orders, n={n}, fp32, softplus, no gate",
            "fused_ms": round(ms_f, 4),
            "fused_GBps": round(xb / (ms_f * 1e-3) / 1e9, 1),
            "algorithmic_bytes": xb,
            "one_pass_ms": round(ms_1, 4),
            "one_pass_GBps": round(xb / (ms_1 * 1e-3) / 1e9, 1),
            "unfused_ms": round(ms_u, 4),
            "unfused_scan_only_ms": round(ms_s, 4),
            "note": "fused = ss_cross_scan_fwd (its default two-pass form: the directions' outputs through a "
                    "workspace, then a merge kernel); one_pass = the four directions summed in LDS by one kernel; "
                    "unfused = four traversal copies made with torch + ss_scan_fwd + torch merge; scan_only = "
                    "ss_scan_fwd on copies made beforehand",
        }

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(cfg, inp, s, args.cpu_seconds)

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
