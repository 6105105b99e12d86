"""Benchmark of the fused-epilogue GEMM on one MI355X.

A step is one pass of the hot path: one thl_gemm call (validation, dispatch,
the tiled MFMA kernel with its fused epilogue) over inputs already resident
in HBM.  The headline workload is the bf16 GEMM at M = N = K = 8192, all
operands column-major (op N/N), with the relu(A.B + C + bias[m]) epilogue
(bf16 out, fp32 accumulate).

Every configuration of the benchmark set is timed the same way and reported
in the same line under "configs", each with its own bound (MFMA, HBM or
launch latency), fraction of that bound's peak, a parity check against the
oracle (all outputs at 256^3, else a seeded sample of 4096 outputs, plus the
whole last row and column of the ragged shapes) and the oracle's own time
for the outputs it checked:

  fp16 256^3 (T/N, fp32 out), bf16 4096^3 and 8192^3 (N/N, relu(A.B + C +
  bias)), int8 4096^3 (T/N, int32 out, exact), fp8 e4m3 8192^3,
  4097x1000x2040 and 1x8192x8192 (T/N, per-tensor scales, bf16 out), MXFP4
  8192^3 (T/N, D = A.B + C); and, beside them, e5m2 and MXFP8 at 8192^3 and a
  batched bf16 GEMM (16 problems of 2048^3 in one launch).

The timed launches run back to back between two HIP events on the stream
they run on: their mean is the throughput.  A second pass with an event
around each launch gives the median and minimum per-launch times reported
with it.  Each call's arguments are marshalled once, before timing.

Prints ONE JSON line on stdout (diagnostics go to stderr).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published dense peaks (TFLOP/s; TOP/s for int8) and HBM bandwidth.
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "e4m3": 5033.2, "e5m2": 5033.2, "mxe4m3": 5033.2, "e2m1": 10066.3,
               "i8": 5033.2, "e2m3": 10066.3, "e3m2": 10066.3}
HBM_PEAK_GBS = 8000.0

CSRC = os.path.join(ROOT, "tile_hierarchy_linear_amd", "csrc")
# Summary of the FETCH_SIZE / WRITE_SIZE counter runs over this script.
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gemm_8192_hbm_traffic.md")

# Least wall time of each configuration's untimed warm-up (seconds): the
# chip takes about 40 ms of GEMM load to reach its steady clock from idle,
# and it idles between configurations while the oracle checks parity.
WARM_S = 0.1

METRIC = "GEMM TFLOP/s and % of MFMA peak (bf16, fp8, MXFP4 at M=N=K=8192)"

# (key, workload kind, m, n, k, bound, launches per timed step)
CONFIGS = [
    ("fp16_256", "fp16", 256, 256, 256, "latency", 10),
    ("bf16_4096", "bf16", 4096, 4096, 4096, "mfma", 2),
    ("bf16_8192", "bf16", 8192, 8192, 8192, "mfma", 1),
    ("int8_4096", "int8", 4096, 4096, 4096, "mfma", 2),
    ("fp8_8192", "fp8", 8192, 8192, 8192, "mfma", 1),
    ("fp8_4097x1000x2040", "fp8", 4097, 1000, 2040, "mfma", 5),
    ("fp8_1x8192x8192", "fp8", 1, 8192, 8192, "hbm", 10),
    ("mxfp4_8192", "mxfp4", 8192, 8192, 8192, "mfma", 1),
    ("e5m2_8192", "fp8e5m2", 8192, 8192, 8192, "mfma", 1),
    ("mxfp8_8192", "mxfp8", 8192, 8192, 8192, "mfma", 1),
    # through the conversion pass (the timed call includes it)
    ("fp8_nn_8192", "fp8@NN", 8192, 8192, 8192, "mfma", 1),
    ("mxfp6_8192", "narrow:e2m3:e2m3:mx@TN", 8192, 8192, 8192, "mfma", 1),
]
HEADLINE = "bf16_8192"
PEAK_KEY = {"f16": "f16", "bf16": "bf16", "i8": "i8", "e4m3": "e4m3", "e5m2": "e5m2", "e2m1": "e2m1",
            "e2m3": "e2m3", "e3m2": "e3m2"}


def make_workload(kind, m, n, k):
    """A configuration's workload: a kind of workloads.make, optionally with
    "@<opA><opB>" storage, or "narrow:<type A>:<type B>:<mx|dense>@<ops>" for
    workloads.make_narrow."""
    import workloads as wl

    kind, _, ops = kind.partition("@")
    kw = dict(op_a=ops[0], op_b=ops[1]) if ops else {}
    if kind.startswith("narrow:"):
        _, ta, tb, scaled = kind.split(":")
        return wl.make_narrow(ta, tb, m, n, k, mx=scaled == "mx", **kw)
    return wl.make(kind, m, n, k, **kw)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def page_flops_bytes(m, n, k, a_bytes, b_bytes, d_bytes, c_bytes=0):
    """The profiler's bookkeeping on the pages ("Technical Documentation:
    NVIDIA/cutlass", "Performance Profiling", its sample output): FLOPs =
    2MNK + 2MN and Bytes = |A| + |B| + |D| (+|C| when beta != 0), with
    elements of a_bytes, b_bytes, c_bytes, d_bytes bytes."""
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
    return int(total)


def kernel_source_hash():
    """Hash of the device code of the GEMM kernels: the kernel templates, their
    arguments, launch wrappers and instantiations, and the index maps (not
    the host-side dispatch in gemm.hip, which chooses among them)."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if (name.startswith("gemm") and name != "gemm.hip") or name == "index_maps.hpp":
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


def time_launches(run, steps, warmup, stream, min_warm_s=WARM_S):
    """Launch `run` untimed: `warmup` times, and more until at least
    `min_warm_s` seconds have passed (the clock ramp from idle takes some
    40 ms of load).  Then time `steps` launches back to back on `stream` (the
    stream the kernels run on) between two HIP events: the mean per launch.
    A second pass of `steps` launches, each between events of its own, gives
    the median and the minimum (an event between launches adds a few
    microseconds of queue work, so it stays out of the mean).  Returns
    (mean, median, min) per launch in ms."""
    import torch

    t0 = time.perf_counter()
    for _ in range(warmup):
        st = run()
        assert st == 0, st
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < min_warm_s:
        for _ in range(max(1, warmup)):
            run()
        torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        run()
    end.record(stream)
    torch.cuda.synchronize()
    mean = start.elapsed_time(end) / steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        run()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    each = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    return mean, each[len(each) // 2], each[0]


def parity_and_oracle_time(w, dp, full=False, edges=False):
    """Compare D with the oracle (every output when `full`, else the seeded
    4096-output sample; `edges` adds the whole last row and column) and time
    the oracle's evaluation of the outputs it checked (all host threads)."""
    import numpy as np

    import oracle
    from oracle import compare

    if full:
        ii, jj = np.meshgrid(np.arange(w.m), np.arange(w.n), indexing="ij")
        rows, cols = ii.ravel(), jj.ravel()
        kind = f"all {w.m * w.n} outputs"
    else:
        rows, cols = w.sample(4096)
        kind = f"{rows.size} seeded outputs"
        if edges:
            rows = np.concatenate([rows, np.full(w.n, w.m - 1), np.arange(w.m)])
            cols = np.concatenate([cols, np.arange(w.n), np.full(w.m, w.n - 1)])
            kind += f" + last row ({w.n}) and last column ({w.m})"
    t0 = time.perf_counter()
    ref = oracle.gemm_elements(w.oracle_problem(), rows, cols)
    dt = time.perf_counter() - t0
    res = compare.parity_check(w, dp.d_values(rows, cols), rows, cols, ref=ref)
    bar = "bit-exact" if w.type_a == "i8" else "2^-20*K*max|a'|*max|b'| + 1 ulp"
    out = {"ok": bool(res["ok"]), "checked": kind, "n_bad": res["n_bad"], "bar": bar}
    if "max_err" in res:
        out["max_err"] = res["max_err"]
    oracle_t = {"outputs": int(rows.size), "seconds": round(dt, 3), "threads": oracle.max_threads(),
                "extrapolated_full_d_s": round(dt * w.m * w.n / rows.size, 1)}
    return out, oracle_t


def run_config(key, kind, m, n, k, bound, mult, args, stream):
    import torch

    import tile_hierarchy_linear_amd as thl
    import workloads as wl
    from workloads.device import DeviceProblem

    t0 = time.perf_counter()
    w = make_workload(kind, m, n, k)
    dp = DeviceProblem(w)
    log(f"[{key}] inputs generated and uploaded in {time.perf_counter() - t0:.1f} s")
    steps, warmup = args.steps * mult, args.warmup * mult
    call = dp.bind(stream=stream.cuda_stream)  # arguments marshalled once, outside the timed region
    mean, med, mn = time_launches(call, steps, warmup, stream)
    variant = thl.thl_last_variant()
    flops = w.flops()
    peak_key = "mxe4m3" if kind == "mxfp8" else PEAK_KEY[w.type_a]  # fp6: the fp6 MFMA peak
    peak = PEAK_TFLOPS[peak_key]
    tflops = flops / (mean * 1e-3) / 1e12
    byt = compulsory_bytes(w)
    gbs = byt / (mean * 1e-3) / 1e9
    eb = wl.ELEM_BYTES
    pf, pb = page_flops_bytes(m, n, k, eb[w.type_a], eb[w.type_b], eb[w.type_d],
                              eb[w.type_c] if w.beta != 0.0 else 0)
    entry = {
        "workload": describe(w), "variant": variant, "launches": steps,
        "ms_mean": round(mean, 5), "ms_median": round(med, 5), "ms_min": round(mn, 5),
        "tflops": round(tflops, 2), "bound": bound,
        "algorithmic_bytes": byt, "hbm_gbs_algorithmic": round(gbs, 1),
        "page_convention": {"flops": int(pf), "bytes": int(pb)},
        "traffic": measured_traffic(variant, m, n, k),
    }
    if bound == "hbm":
        entry["roofline"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(gbs / HBM_PEAK_GBS, 4)}
    else:
        entry["roofline"] = {"bound": "mfma" if bound == "mfma" else "latency", "achieved": round(tflops, 2),
                             "peak": peak, "unit": "TOP/s" if w.type_a == "i8" else "TFLOP/s",
                             "frac": round(tflops / peak, 4)}
    try:
        entry["parity"], entry["oracle"] = parity_and_oracle_time(w, dp, full=m * n <= 65536,
                                                                  edges=(m % 256 != 0 or n % 256 != 0))
    except Exception as e:  # noqa: BLE001 -- reported in the line, not fatal for timing
        entry["parity"] = {"ok": False, "error": str(e)}
    log(f"[{key}] mean {mean * 1e3:.1f} us (median {med * 1e3:.1f}, min {mn * 1e3:.1f}) {tflops:.1f} TFLOP/s "
        f"frac {entry['roofline']['frac']:.3f} of the {entry['roofline']['bound']} peak via {variant}; "
        f"parity {entry['parity'].get('ok')}")
    if args.sweep_variants:
        ops = (w.op_a + w.op_b).lower()
        fam = variant.split("_")[0]
        for v in thl.variants():
            if not v.startswith(f"{fam}_{ops}_"):
                continue
            os.environ["THL_FORCE_VARIANT"] = v
            try:
                vm, _, _ = time_launches(lambda: dp.run(stream=stream.cuda_stream), max(3, steps // 2), 2, stream)
                log(f"   sweep {v}: {vm * 1e3:.1f} us {flops / (vm * 1e-3) / 1e12:.1f} TFLOP/s")
            except AssertionError as e:
                log(f"   sweep {v}: not applicable ({e})")
            finally:
                os.environ.pop("THL_FORCE_VARIANT", None)
    del dp
    torch.cuda.empty_cache()
    return w, entry


def describe(w):
    epi = []
    if w.beta != 0.0:
        epi.append("C")
    if w.bias is not None:
        epi.append("bias[m]")
    body = "A.B" + "".join(" + " + e for e in epi)
    if w.act != "none":
        body = f"{w.act}({body})"
    scales = ""
    if w.sfa is not None:
        scales = ", E8M0 scale per 32 K-elements"
    elif w.type_a in ("e4m3", "e5m2"):
        scales = ", per-tensor scales"
    fmt = w.type_a if w.type_a == w.type_b else f"{w.type_a} x {w.type_b}"
    return (f"{fmt} GEMM M={w.m} N={w.n} K={w.k}, op {w.op_a}{w.op_b}{scales}, D = {body}, "
            f"{w.type_d} out")


def run_batched(args, stream):
    import torch

    import tile_hierarchy_linear_amd as thl
    import workloads as wl
    from oracle import compare
    from workloads.device import BatchedDeviceProblem

    L, sz = 16, 2048
    t0 = time.perf_counter()
    ws = [wl.make("bf16", sz, sz, sz, seed=1002 + 100 * z) for z in range(L)]
    bp = BatchedDeviceProblem(ws)
    log(f"[batched] {L} problems generated and uploaded in {time.perf_counter() - t0:.1f} s")
    mean, med, mn = time_launches(lambda: bp.run(stream=stream.cuda_stream), args.steps, args.warmup, stream)
    vb = thl.thl_last_variant()
    tfb = L * ws[0].flops() / (mean * 1e-3) / 1e12
    ok = True
    for z in (0, L - 1):
        rows, cols = ws[z].sample(4096)
        got = bp.d_all(z)[rows, cols]
        ok = ok and compare.parity_check(ws[z], got, rows, cols)["ok"]
    out = {"workload": f"bf16 GEMM, {L} problems of M=N=K={sz}, op NN, D = relu(A.B + C + bias[m]), bf16 out, "
                       "one batched launch",
           "variant": vb, "ms_mean": round(mean, 5), "ms_median": round(med, 5), "ms_min": round(mn, 5),
           "tflops": round(tfb, 1),
           "roofline": {"bound": "mfma", "achieved": round(tfb, 1), "peak": PEAK_TFLOPS["bf16"], "unit": "TFLOP/s",
                        "frac": round(tfb / PEAK_TFLOPS["bf16"], 4)},
           "parity": {"ok": bool(ok), "checked": "4096 seeded outputs of problems 0 and 15"}}
    log(f"[batched] {mean:.3f} ms {tfb:.1f} TFLOP/s via {vb}; parity {ok}")
    del bp
    torch.cuda.empty_cache()
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(w, budget_s, budget_1t_s):
    """The oracle timed on this host's cores over a bounded sample of the
    headline D: all OpenMP threads for about budget_s seconds, then one thread
    for about budget_1t_s."""
    import oracle

    def timed(nthreads, budget):
        # Two pilots: the first includes one-time setup and overestimates the
        # per-output cost; the second, sized for about a tenth of the budget,
        # sets the size of the timed sample.
        pilot = 16 * nthreads
        per = 1.0
        for _ in range(2):
            rows, cols = w.sample(pilot)
            t0 = time.perf_counter()
            oracle.gemm_elements(w.oracle_problem(), rows, cols, nthreads)
            per = max(time.perf_counter() - t0, 1e-6) / pilot
            pilot = int(min(max(pilot, 0.1 * budget / per), w.m * w.n))
        count = int(min(max(16 * nthreads, budget / per), w.m * w.n))
        rows, cols = w.sample(count)
        t0 = time.perf_counter()
        oracle.gemm_elements(w.oracle_problem(), rows, cols, nthreads)
        return count, time.perf_counter() - t0

    nthreads = oracle.max_threads()
    count, dt = timed(nthreads, budget_s)
    count1, dt1 = timed(1, budget_1t_s)
    flops = 2.0 * w.k
    return {"value": round(flops * count / dt / 1e12, 6), "unit": "TFLOP/s", "cores": nthreads, "kind": "oracle",
            "sample": f"{count} seeded outputs of the {w.m}x{w.n}x{w.k} {w.type_a} GEMM ({2 * w.k} flops each) "
                      f"in {dt:.1f} s on {nthreads} threads; full D extrapolated "
                      f"{dt * w.m * w.n / count / 3600:.1f} h",
            "one_thread": {"value": round(flops * count1 / dt1 / 1e12, 6), "unit": "TFLOP/s",
                           "sample": f"{count1} seeded outputs in {dt1:.1f} s; full D extrapolated "
                                     f"{dt1 * w.m * w.n / count1 / 3600:.1f} h"},
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}


def mfma_ceiling(stream):
    """The matrix cores alone (csrc/mfma_probe.hip): TFLOP/s of a loop of
    independent MFMAs on every SIMD, at the clock the chip holds under that
    load, for bf16, e4m3 and e2m1 (scaled).  HIP events around 50 launches of
    about 0.9 ms each after 50 warm-up launches (the clock's ramp from idle,
    as for the GEMMs)."""
    import ctypes

    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "tile_hierarchy_linear_amd", "libthl_probe.so"))
    lib.thl_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.thl_probe_mfma.restype = ctypes.c_int
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(cus * 256, dtype=torch.float32, device="cuda")
    res = {}
    for fmt, name, flops_each, iters in ((0, "bf16", 32768, 8000), (1, "e4m3", 131072, 4000),
                                         (2, "e2m1", 131072, 8000)):
        def run():
            return lib.thl_probe_mfma(fmt, iters, cus, ctypes.c_void_p(out.data_ptr()),
                                      ctypes.c_void_p(stream.cuda_stream))
        mean, med, mn = time_launches(run, 50, 50, stream)
        tf = cus * 4 * iters * 8 * flops_each / (mean * 1e-3) / 1e12
        peak = PEAK_TFLOPS[name]
        res[name] = {"tflops": round(tf, 1), "frac_of_peak": round(tf / peak, 4), "ms_per_launch": round(mean, 4),
                     "mfma_per_wave": iters * 8}
        log(f"[mfma only] {name}: {tf:.1f} TFLOP/s, {tf / peak:.3f} of the dense peak")
    return res


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
    # The chip takes about 50 launches of the 8192^3 GEMM (some 40 ms of load)
    # to reach its steady clock from idle: bf16 measured 1,073 TFLOP/s at the
    # 5th launch, 1,305 at the 20th and 1,390-1,400 from the 50th to the
    # 1,000th.  Each configuration's warm-up is W launches (times its
    # multiplier) and at least WARM_S seconds, which covers that ramp also
    # for the short kernels.
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--only", default="",
                    help="comma list of configuration keys (" + ",".join(c[0] for c in CONFIGS) +
                         ",batched); default: all")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work on all threads")
    ap.add_argument("--cpu-budget-1t", type=float, default=4.0, help="seconds of oracle work on one thread")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mfma-ceiling", action="store_true",
                    help="skip the matrix-core-only loop (the ceiling at the chip's loaded clock)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0)
    ap.add_argument("--sweep-variants", action="store_true",
                    help="also time every built variant of each configuration's family (stderr)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the GEMM would shard by "
              "output tiles with no exchange). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    keys = [c[0] for c in CONFIGS] + ["batched"]
    only = [x for x in args.only.split(",") if x] or keys
    unknown = set(only) - set(keys)
    if unknown:
        print(f"unknown configuration keys {sorted(unknown)}", file=sys.stderr)
        sys.exit(2)

    configs = {}
    workloads = {}
    for key, kind, m, n, k, bound, mult in CONFIGS:
        if key in only:
            workloads[key], configs[key] = run_config(key, kind, m, n, k, bound, mult, args, stream)
    if "batched" in only:
        configs["batched"] = run_batched(args, stream)
    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)
    ceiling = None if args.no_mfma_ceiling else mfma_ceiling(stream)

    head = HEADLINE if HEADLINE in configs else next((k for k in configs if k != "batched"), None)
    if head is None:
        print("--only needs one GEMM configuration for the headline line", file=sys.stderr)
        sys.exit(2)
    w, h = workloads[head], configs[head]
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_budget, args.cpu_budget_1t)
    roof = dict(h["roofline"])
    roof.update({"traffic": h["traffic"], "algorithmic_bytes": h["algorithmic_bytes"],
                 "kernel_sources": kernel_source_hash()})
    if ceiling and w.type_a in ceiling:
        c = ceiling[w.type_a]
        roof["mfma_only_ceiling"] = {"achieved": c["tflops"], "frac_of_peak": c["frac_of_peak"],
                                     "gemm_frac_of_ceiling": round(h["tflops"] / c["tflops"], 4)}
    line = {
        "metric": METRIC,
        "value": h["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_min_s": WARM_S,
        "ms_per_step": h["ms_mean"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.type_a,
        "data": "synthetic (seeded PCG64 streams per tensor; see each configuration's workload)",
        "config": {"workload": h["workload"] + ", fp32 accumulate", "m": w.m, "n": w.n, "k": w.k,
                   "kernel_variant": h["variant"], "ms_median": h["ms_median"], "ms_min": h["ms_min"],
                   "parity": h.get("parity")},
        "roofline": roof,
        "configs": configs,
        "mfma_only_ceiling": ceiling,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
