"""The seeded input generators (host only, no GEMM arithmetic) and the
benchmark's command line."""
import os
import subprocess
import sys

import numpy as np
import torch

import oracle
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_mxfp8_blocks_follow_the_shared_exponent_rule():
    # OCP MX: X = floor(log2(amax)) - 8 for E4M3 (largest exponent 8), so each
    # block's largest element lands in [256, 512) before rounding, at most 448
    # after it; dequantized values are within E4M3's half-ulp of x
    g = np.random.default_rng(5)
    x = g.standard_normal((6, 128)) * np.exp(g.uniform(-8, 8, size=(6, 1)))
    codes, sc = wl.mx_quantize_e4m3(x)
    vals = oracle.decode("e4m3", np.ascontiguousarray(codes)).reshape(6, 128)
    scale = np.ldexp(1.0, sc.astype(np.int64) - 127)
    blk = np.abs(vals.reshape(6, 4, 32)).max(axis=2)
    assert ((blk >= 256) & (blk <= 448)).all()
    deq = (vals.reshape(6, 4, 32) * scale[:, :, None]).reshape(6, 128)
    ref = torch.from_numpy((x / np.repeat(scale, 32, axis=1)).astype(np.float32)).clamp(-448, 448)
    want = ref.to(torch.float8_e4m3fn).double().numpy() * np.repeat(scale, 32, axis=1)
    assert np.array_equal(deq, want)


def test_fp8_kinds_scale_each_operand_to_its_format():
    for kind, (ta, tb) in (("fp8", ("e4m3", "e4m3")), ("fp8e5m2", ("e5m2", "e5m2")),
                           ("fp8e4e5", ("e4m3", "e5m2")), ("fp8e5e4", ("e5m2", "e4m3"))):
        w = wl.make(kind, 9, 7, 64)
        assert (w.type_a, w.type_b) == (ta, tb)
        top = {"e4m3": 448.0, "e5m2": 57344.0}
        a = np.abs(oracle.decode(ta, np.ascontiguousarray(w.a))).max()
        b = np.abs(oracle.decode(tb, np.ascontiguousarray(w.b))).max()
        assert a <= top[ta] and b <= top[tb]
        assert a >= top[ta] / 2 and b >= top[tb] / 2  # the per-tensor scale fills the range


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_bench_bookkeeping_reproduces_the_profiler_sample():
    # The profiler's sample output on the pages ("Technical Documentation:
    # NVIDIA/cutlass", "Performance Profiling"): an f16 x f16 -> f32 GEMM with
    # M=3456, N=4096, K=4096 and beta = 0 prints FLOPs 115992428544 and Bytes
    # 118489088 (A and B at 2 bytes, D at 4).
    sys.path.insert(0, ROOT)
    import bench

    flops, byts = bench.page_flops_bytes(3456, 4096, 4096, 2, 2, 4)
    assert flops == 115992428544
    assert byts == 118489088


def test_bench_compulsory_bytes_of_the_headline_workload():
    # bf16 8192^3 with C and bias: A, B, C, D at 2 bytes plus an 8192-row bf16 bias
    sys.path.insert(0, ROOT)
    import bench

    w = wl.make("bf16", 64, 48, 32)
    assert bench.compulsory_bytes(w) == 2 * (64 * 32 + 32 * 48 + 64 * 48 + 64 * 48 + 64)
    w4 = wl.make("mxfp4", 64, 48, 64)
    # packed fp4 operands, one scale byte per 32 K-elements per row and column, C and D bf16
    assert bench.compulsory_bytes(w4) == 64 * 32 + 48 * 32 + (64 + 48) * 2 + 2 * 2 * 64 * 48


def test_bench_lists_every_configuration():
    sys.path.insert(0, ROOT)
    import bench

    shapes = {(c[1], c[2], c[3], c[4]) for c in bench.CONFIGS}
    for need in (("fp16", 256, 256, 256), ("bf16", 4096, 4096, 4096), ("bf16", 8192, 8192, 8192),
                 ("int8", 4096, 4096, 4096), ("fp8", 8192, 8192, 8192), ("fp8", 4097, 1000, 2040),
                 ("fp8", 1, 8192, 8192), ("mxfp4", 8192, 8192, 8192)):
        assert need in shapes
    assert bench.HEADLINE == "bf16_8192"


def test_mx_e5m2_blocks_follow_the_shared_exponent_rule():
    # E5M2's largest exponent is 15: each block's largest element lands in
    # [2^15, 57344] after scaling, and mixed kinds give each operand its format
    g = np.random.default_rng(6)
    x = g.standard_normal((4, 96)) * np.exp(g.uniform(-8, 8, size=(4, 1)))
    codes, sc = wl.mx_quantize_fp8(x, "e5m2")
    vals = oracle.decode("e5m2", np.ascontiguousarray(codes)).reshape(4, 96)
    blk = np.abs(vals.reshape(4, 3, 32)).max(axis=2)
    assert ((blk >= 2.0 ** 15) & (blk <= 57344)).all()
    for kind, ta, tb in (("mxfp8e5m2", "e5m2", "e5m2"), ("mxfp8e4e5", "e4m3", "e5m2"), ("mxfp8e5e4", "e5m2", "e4m3")):
        w = wl.make(kind, 5, 7, 64)
        assert (w.type_a, w.type_b) == (ta, tb) and w.sfa is not None and w.sfb is not None
