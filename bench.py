"""Benchmark of the fused-epilogue GEMM on one MI355X.

A step is one pass of the hot path: one thl_gemm call (validation, dispatch,
the tiled MFMA kernel with its fused epilogue) over inputs already resident
in HBM.  The headline workload is the bf16 GEMM at M = N = K = 8192, all
operands column-major (op N/N), with the relu(A.B + C + bias[m]) epilogue
(bf16 out, fp32 accumulate); the fp8 (e4m3 and e5m2, per-tensor scales),
MXFP8 (e4m3 with E8M0 block scales) and MXFP4 (e2m1 with E8M0 block scales,
D = A.B + C)
GEMMs at 8192^3 are timed the same way and reported in the same line, and
so are the single-row fp8 GEMM (M = 1, N = K = 8192), against the HBM peak,
and a batched bf16 GEMM (16 problems of 2048^3 in one launch).

Prints ONE JSON line on stdout (diagnostics go to stderr).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published dense peaks (TFLOP/s, TOP/s for int8) and HBM bandwidth.
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "e4m3": 5033.2, "e5m2": 5033.2, "mxe4m3": 5033.2, "e2m1": 10066.3,
               "i8": 5033.2}
HBM_PEAK_GBS = 8000.0

CSRC = os.path.join(ROOT, "tile_hierarchy_linear_amd", "csrc")
# Summary of the FETCH_SIZE / WRITE_SIZE counter runs over this script.
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gemm_8192_hbm_traffic.md")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def page_flops_bytes(m, n, k, a_bytes, b_bytes, d_bytes, c_bytes=0):
    """The profiler's bookkeeping on the pages: FLOPs = 2MNK + 2MN and
    Bytes = |A| + |B| + |D| (+|C| when beta != 0)."""
    return 2 * m * n * k + 2 * m * n, m * k * a_bytes + k * n * b_bytes + m * n * d_bytes + m * n * c_bytes


def compulsory_bytes(w):
    """Algorithmic HBM bytes of one GEMM: A, B, block scales, C (if read), bias, D."""
    import workloads as wl

    eb = wl.ELEM_BYTES
    total = w.m * w.k * eb[w.type_a] + w.k * w.n * eb[w.type_b] + w.m * w.n * eb[w.type_d]
    if w.beta != 0.0 and w.c is not None:
        total += w.m * w.n * eb[w.type_c]
    if w.bias is not None:
        total += w.m * eb[w.type_bias]
    if w.sfa is not None:
        total += (w.m + w.n) * (w.k // 32)
    return total


def kernel_source_hash():
    """Hash of every source the GEMM kernels and their launch are built from."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.startswith("gemm") or name == "index_maps.hpp":
            h.update(name.encode())
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(variant, m, n, k):
    """HBM bytes per launch (read + written) of `variant` at this shape from the
    committed counter summary, each counter scaled by what it read for a plain
    copy of known size.  None when no summary covers it or the kernel sources
    have changed since the counters were taken."""
    try:
        with open(TRAFFIC_SUMMARY) as f:
            lines = [l.split()[1:] for l in f if l.startswith("traffic ")]
    except OSError:
        return None
    here = kernel_source_hash()
    for fields in lines:
        kv = dict(x.split("=", 1) for x in fields)
        if (kv.get("variant") == variant and kv.get("mnk") == f"{m}x{n}x{k}" and kv.get("sources") == here):
            return int(kv["read_bytes"]) + int(kv["write_bytes"])
    return None


def time_gemm(dp, steps, warmup, stream):
    """Average duration of one thl_gemm launch, with HIP events recorded on
    the stream the kernel runs on."""
    import torch

    for _ in range(warmup):
        st = dp.run(stream=stream.cuda_stream)
        assert st == 0, st
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        dp.run(stream=stream.cuda_stream)
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps  # ms


def quick_parity(w, dp, count=512):
    from oracle import compare

    rows, cols = w.sample(count)
    res = compare.parity_check(w, dp.d_values(rows, cols), rows, cols)
    return "ok" if res["ok"] else f"FAIL({res['n_bad']}/{res['n']})"


def cpu_baseline(w, budget_s):
    """The oracle timed on this host's cores over a bounded sample of D."""
    import numpy as np

    import oracle

    nthreads = oracle.max_threads()
    # Two pilots: the first includes one-time setup and overestimates the
    # per-output cost; the second, sized for about a tenth of the budget,
    # sets the size of the timed sample.
    pilot = 16 * nthreads
    for _ in range(2):
        rows, cols = w.sample(pilot)
        t0 = time.perf_counter()
        oracle.gemm_elements(w.oracle_problem(), rows, cols, nthreads)
        t1 = time.perf_counter() - t0
        per = max(t1, 1e-6) / pilot
        pilot = int(min(max(pilot, 0.1 * budget_s / per), w.m * w.n))
    count = int(min(max(16 * nthreads, budget_s / per), w.m * w.n))
    rows, cols = w.sample(count)
    t0 = time.perf_counter()
    oracle.gemm_elements(w.oracle_problem(), rows, cols, nthreads)
    dt = time.perf_counter() - t0
    flops = 2.0 * w.k * count
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": nthreads, "kind": "oracle",
            "sample": f"{count} seeded outputs of the {w.m}x{w.n}x{w.k} {w.type_a} GEMM "
                      f"({2 * w.k} flops each) in {dt:.1f} s; full D extrapolated "
                      f"{dt * w.m * w.n / count / 3600:.1f} h"}


def copy_calibration(mib):
    """A plain device copy of known size, for scaling HBM byte counters."""
    import torch

    n = mib * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy calibration: {mib} MiB read + {mib} MiB written per copy kernel")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--size", type=int, default=8192)
    ap.add_argument("--only", default="", help="comma list of bf16,e4m3,e5m2,mxe4m3,e2m1,m1,batched (default: all)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0)
    ap.add_argument("--sweep-variants", action="store_true",
                    help="also time every built variant of each dtype (stderr)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the GEMM would shard by "
              "output tiles with no exchange). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import tile_hierarchy_linear_amd as thl
    import workloads as wl
    from workloads.device import DeviceProblem

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    s = args.size
    only = set(x for x in args.only.split(",") if x) or {"bf16", "e4m3", "e5m2", "mxe4m3", "e2m1", "m1", "batched"}

    results = {}
    headline = None
    for key, kind, kw in (("bf16", "bf16", {}), ("e4m3", "fp8", {}), ("e5m2", "fp8e5m2", {}), ("mxe4m3", "mxfp8", {}),
                          ("e2m1", "mxfp4", {})):
        if key not in only:
            continue
        t0 = time.perf_counter()
        w = wl.make(kind, s, s, s, **kw)
        dp = DeviceProblem(w)
        log(f"[{key}] inputs generated and uploaded in {time.perf_counter() - t0:.1f} s")
        ms = time_gemm(dp, args.steps, args.warmup, stream)
        variant = thl.thl_last_variant()
        flops = w.flops()
        tflops = flops / (ms * 1e-3) / 1e12
        byt = compulsory_bytes(w)
        entry = {"tflops": round(tflops, 1), "frac_of_peak": round(tflops / PEAK_TFLOPS[key], 4),
                 "peak_tflops": PEAK_TFLOPS[key], "ms": round(ms, 4), "variant": variant,
                 "op": w.op_a + w.op_b, "epilogue": {"act": w.act, "beta": w.beta, "bias": w.bias is not None},
                 "hbm_gbs_compulsory": round(byt / (ms * 1e-3) / 1e9, 1), "algorithmic_bytes": byt,
                 "traffic": measured_traffic(variant, w.m, w.n, w.k)}
        try:
            entry["parity_sampled"] = quick_parity(w, dp)
        except Exception as e:  # noqa: BLE001 -- reported, not fatal for timing
            entry["parity_sampled"] = f"error: {e}"
        results[key] = entry
        log(f"[{key}] {ms:.3f} ms  {tflops:.1f} TFLOP/s  ({100 * tflops / PEAK_TFLOPS[key]:.1f}% of peak) "
            f"via {variant}; parity {entry['parity_sampled']}")
        if key == "bf16":
            headline = (w, ms, byt, variant)
        if headline is None and key == min(only - {"m1", "batched"}):
            headline = (w, ms, byt, variant)
        if args.sweep_variants:
            fam = key
            ops = (w.op_a + w.op_b).lower()
            for v in thl.variants():
                if not v.startswith(f"{fam}_{ops}_"):
                    continue
                os.environ["THL_FORCE_VARIANT"] = v
                try:
                    vms = time_gemm(dp, max(3, args.steps // 2), 2, stream)
                    log(f"   sweep {v}: {vms:.3f} ms {flops / (vms * 1e-3) / 1e12:.1f} TFLOP/s")
                except AssertionError as e:
                    log(f"   sweep {v}: not applicable ({e})")
                finally:
                    os.environ.pop("THL_FORCE_VARIANT", None)
        del dp
        torch.cuda.empty_cache()

    # The single-row fp8 configuration (M = 1, N = K = s): HBM-bound, so its
    # roofline is bytes per second against the HBM peak.  A launch is about
    # 12 us, so it is timed over ten times as many launches.
    small_m = None
    if "m1" in only:
        w1 = wl.make("fp8", 1, s, s)
        dp1 = DeviceProblem(w1)
        ms1 = time_gemm(dp1, 10 * args.steps, 2 * args.warmup, stream)
        v1 = thl.thl_last_variant()
        byt1 = compulsory_bytes(w1)
        gbs = byt1 / (ms1 * 1e-3) / 1e9
        small_m = {"workload": f"fp8 e4m3 GEMM M=1, N=K={s}, op TN, per-tensor scales, bf16 out",
                   "us": round(ms1 * 1e3, 2), "variant": v1,
                   "tflops": round(w1.flops() / (ms1 * 1e-3) / 1e12, 2),
                   "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes": byt1,
                                "traffic": measured_traffic(v1, w1.m, w1.n, w1.k)}}
        try:
            small_m["parity_sampled"] = quick_parity(w1, dp1)
        except Exception as e:  # noqa: BLE001 -- reported, not fatal for timing
            small_m["parity_sampled"] = f"error: {e}"
        log(f"[m1] {ms1 * 1e3:.2f} us  {gbs:.0f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}% of HBM peak) via {v1}; "
            f"parity {small_m['parity_sampled']}")
        del dp1
        torch.cuda.empty_cache()

    # Batched (L mode): 16 problems of the headline's layout and epilogue at
    # M = N = K = s/4, one thl_gemm_batched launch.
    batched = None
    if "batched" in only:
        from oracle import compare
        from workloads.device import BatchedDeviceProblem

        L, sz = 16, max(256, s // 4)
        t0 = time.perf_counter()
        ws = [wl.make("bf16", sz, sz, sz, seed=1002 + 100 * z) for z in range(L)]
        bp = BatchedDeviceProblem(ws)
        log(f"[batched] {L} problems generated and uploaded in {time.perf_counter() - t0:.1f} s")

        msb = time_gemm(bp, args.steps, args.warmup, stream)
        vb = thl.thl_last_variant()
        tfb = L * ws[0].flops() / (msb * 1e-3) / 1e12
        status = "ok"
        for z in (0, L - 1):
            rows, cols = ws[z].sample(512)
            got = bp.d_all(z)[rows, cols]
            res = compare.parity_check(ws[z], got, rows, cols)
            if not res["ok"]:
                status = f"FAIL(problem {z}: {res['n_bad']}/{res['n']})"
        batched = {"workload": f"bf16 GEMM, {L} problems of M=N=K={sz}, op NN, D = relu(A.B + C + bias[m]), "
                               "bf16 out, one batched launch",
                   "ms": round(msb, 4), "tflops": round(tfb, 1), "frac_of_peak": round(tfb / PEAK_TFLOPS["bf16"], 4),
                   "variant": vb, "parity_sampled": status}
        log(f"[batched] {msb:.3f} ms  {tfb:.1f} TFLOP/s ({100 * tfb / PEAK_TFLOPS['bf16']:.1f}% of peak) via {vb}; "
            f"parity {status}")
        del bp
        torch.cuda.empty_cache()

    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)

    if headline is None:
        print("--only needs one of bf16, e4m3, e5m2, mxe4m3, e2m1 for the headline line", file=sys.stderr)
        sys.exit(2)
    w, ms, byt, variant = headline
    key = w.type_a
    tflops = w.flops() / (ms * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_budget)
    line = {
        "metric": "GEMM TFLOP/s and % of MFMA peak (bf16, fp8, MXFP4 at M=N=K=8192)",
        "value": round(tflops, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.type_a,
        "data": "synthetic (seeded PCG64; U[-1,1] bf16 A, B, C, bias)",
        "config": {"workload": f"{key} GEMM M=N=K={s} op {w.op_a}{w.op_b}, D = relu(A.B + C + bias[m]), "
                               f"fp32 accumulate, {w.type_d} out", "m": w.m, "n": w.n, "k": w.k,
                   "kernel_variant": variant},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_TFLOPS[key], "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_TFLOPS[key], 4),
                     "traffic": measured_traffic(variant, w.m, w.n, w.k),
                     "algorithmic_bytes": byt, "kernel_sources": kernel_source_hash()},
        "dtypes": results,
        "small_m": small_m,
        "batched": batched,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
