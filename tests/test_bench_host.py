"""CPU: the benchmark's host-side contract -- the GPU count it accepts and its
algorithmic byte counts, checked against the sizes worked out by hand from
the tensors each step reads and writes."""
import bench


def test_more_than_one_gpu_is_refused():
    assert bench.main(["--gpus", "2"]) == 2
    assert bench.main(["--gpus", "8"]) == 2


def test_scan_long_bytes():
    # b=4, L=8192, d_in=5120, n=16, bf16: u, delta, y and z (4 x 167 772 160 elements) and B, C
    # (2 x 524 288) at 2 bytes; A_log (81 920), D and bias (2 x 5 120) and the last state (327 680) at 4.
    assert bench.scan_bytes(4, 8192, 5120, 16, 2, True, True, True) == (
        2 * (4 * 167_772_160 + 2 * 524_288) + 4 * (81_920 + 2 * 5_120 + 327_680))
    assert bench.scan_bytes(4, 8192, 5120, 16, 2, True, True, True) == 1_345_953_792


def test_decode_step_bytes():
    # b=256, d_in=5120, n=16: the fp32 state read and written (2 x 20 971 520 x 4 bytes); x, dt, z, y
    # (4 x 1 310 720) and B, C (2 x 4 096) in bf16; A_log, D and dt_bias in fp32.
    assert bench.decode_bytes(256, 5120, 16, 2) == (
        2 * 20_971_520 * 4 + 2 * (4 * 1_310_720 + 2 * 4_096) + 4 * (81_920 + 2 * 5_120))
    assert bench.decode_bytes(256, 5120, 16, 2) == 178_642_944


def test_cross_scan_bytes():
    # 16 maps of 56 x 56 (L = 3136) x 384, n = 1, fp32: the map once, four directions' delta, B and C,
    # the fp32 output map, and A_log, D of the four directions (no bias).
    maps, L, d = 16, 3136, 384
    assert bench.cross_bytes(maps, L, d, 1, 4) == (
        4 * (maps * L * d + 4 * maps * L * d + 8 * maps * L) + 4 * maps * L * d + 4 * (4 * d + 4 * d))
    assert bench.cross_bytes(maps, L, d, 1, 4) == 464_039_936


def test_conv_step_bytes():
    # b=256, d_in=5120, window 4, bf16: the window read and written (2 x 4 elements), x in and y out; the
    # fp32 weights (d_in x 4) and bias.
    assert bench.conv_bytes(256, 5120, 4, 2) == 2 * 256 * 5120 * (2 * 4 + 2) + 4 * (5120 * 4 + 5120)
    assert bench.conv_bytes(256, 5120, 4, 2) == 26_316_800


def test_valu_probe_library_loads_and_validates():
    """libss_probe.so (built beside libss_scan.so) exports the probe and rejects bad arguments before any launch."""
    import ctypes
    import os

    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "selective_state_space_softplus_amd", "libss_probe.so")
    lib = ctypes.CDLL(path)
    f = lib.ss_probe_valu
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    buf = ctypes.c_void_p(16)
    for mix, blocks, iters, out in ((4, 1, 1, buf), (-1, 1, 1, buf), (0, 0, 1, buf), (0, 1, 0, buf), (0, 1, 1, None)):
        assert f(mix, blocks, iters, out, None) == -1, (mix, blocks, iters, out)
