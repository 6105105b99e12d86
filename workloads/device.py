"""Run a Workload on the GPU through the C ABI: upload the stored bits,
call thl_gemm on the current stream, read D back.  Device memory and streams
come from torch; every arithmetic step runs in libthl's kernels."""
from __future__ import annotations

import numpy as np
import torch

import tile_hierarchy_linear_amd as thl

_TORCH_D = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "i32": torch.int32}
# D formats written as MX blocks (element codes plus one E8M0 scale per 32 rows)
MX_D = ("e2m1", "e4m3", "e5m2")


def upload(arr, device="cuda"):
    if arr is None:
        return None
    raw = np.ascontiguousarray(arr).view(np.uint8).reshape(-1)
    return torch.from_numpy(raw.copy()).to(device)


class DeviceProblem:
    """Device copies of a workload's buffers plus its output."""

    def __init__(self, w, device="cuda", d_fill=float("nan"), ldd=None):
        self.w = w
        self.a = upload(w.a, device)
        self.b = upload(w.b, device)
        self.c = upload(w.c, device) if w.c is not None and w.beta != 0.0 else None
        self.bias = upload(w.bias, device)
        self.sfa = upload(w.sfa, device)
        self.sfb = upload(w.sfb, device)
        self.ldd = ldd or w.ldd
        self.sfd, self.ld_sfd = None, 0
        if w.type_d in MX_D:
            # codes as bytes (two a byte for e2m1), the scales beside them; 0xEE marks unwritten bytes
            ld_bytes = self.ldd // 2 if w.type_d == "e2m1" else self.ldd
            self.d = torch.full((max(1, w.n), ld_bytes), 0xEE, dtype=torch.uint8, device=device)
            self.ld_sfd = max(1, (w.m + 31) // 32)
            self.sfd = torch.full((max(1, w.n), self.ld_sfd), 0xEE, dtype=torch.uint8, device=device)
        else:
            self.d = torch.empty((max(1, w.n), self.ldd), dtype=_TORCH_D[w.type_d], device=device)
            if w.type_d == "i32":
                self.d.fill_(-(2 ** 31) + 7)
            else:
                self.d.fill_(d_fill)

    def _structs(self):
        w = self.w
        dt = thl.make_dtypes(w.type_a, w.type_b, w.type_c, w.type_d,
                             w.type_bias if w.bias is not None else "none")
        flags = (thl.THL_EPI_BIAS if w.bias is not None else 0) | \
            {"none": 0, "relu": thl.THL_EPI_RELU, "gelu": thl.THL_EPI_GELU}[w.act]
        epi = thl.thl_epilogue(flags, self.bias.data_ptr() if self.bias is not None else None,
                               self.sfd.data_ptr() if self.sfd is not None else None, self.ld_sfd)
        sc = thl.thl_scales(float(w.a_scale), float(w.b_scale),
                            self.sfa.data_ptr() if self.sfa is not None else None, int(w.ld_sfa),
                            self.sfb.data_ptr() if self.sfb is not None else None, int(w.ld_sfb))
        return dt, epi, sc

    def _args(self, d=None, c=None, ldc=None):
        w = self.w
        dd = self.d if d is None else d
        cc = self.c if c is None else c
        a_ptr = self.a.data_ptr() if self.a is not None and self.a.numel() else None
        b_ptr = self.b.data_ptr() if self.b is not None and self.b.numel() else None
        return (w.m, w.n, w.k, a_ptr, w.lda, w.op_a, b_ptr, w.ldb, w.op_b,
                cc.data_ptr() if cc is not None else None, ldc or w.ldc or max(1, w.m),
                dd.data_ptr(), self.ldd, w.alpha, w.beta)

    def run(self, stream=None, d=None, c=None, ldc=None, entry=None):
        """Run through thl_gemm (or `entry`, an entry point of the same
        arguments, e.g. thl.thl_gemm_noalloc)."""
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        return (entry or thl.thl_gemm)(*self._args(d, c, ldc), *self._structs(), stream)

    def bind(self, stream=None, entry="thl_gemm"):
        """run()'s call with its arguments marshalled once: a callable that
        issues it (for timing loops, where marshalling per call would cost
        more host time than a small kernel runs)."""
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        return thl.bind_thl_gemm(*self._args(), *self._structs(), stream, entry)

    def d_values(self, rows, cols) -> np.ndarray:
        """D at (rows[t], cols[t]) as float64 (int64 for int32 outputs)."""
        host = self.d.cpu()
        r = torch.as_tensor(np.asarray(rows, dtype=np.int64))
        c = torch.as_tensor(np.asarray(cols, dtype=np.int64))
        vals = host[c, r]
        if self.w.type_d == "i32":
            return vals.to(torch.int64).numpy()
        return vals.to(torch.float64).numpy()

    def mx_all(self):
        """MX-format D: (element codes (m, n) uint8, scale codes (ceil(m/32), n) uint8)."""
        w = self.w
        raw = self.d.cpu().numpy()[: w.n]
        if w.type_d == "e2m1":
            codes = np.empty((w.n, raw.shape[1] * 2), np.uint8)
            codes[:, 0::2], codes[:, 1::2] = raw & 0xF, raw >> 4
        else:
            codes = raw
        return codes[:, : w.m].T.copy(), self.sfd.cpu().numpy()[: w.n, : (w.m + 31) // 32].T.copy()

    def d_all(self) -> np.ndarray:
        """All of D as an (m, n) array [i, j]."""
        host = self.d.cpu()[: self.w.n, : self.w.m].T
        if self.w.type_d == "i32":
            return host.to(torch.int64).numpy()
        return host.to(torch.float64).numpy()


class BatchedDeviceProblem:
    """Workloads of one shape and format packed at fixed strides in shared
    device buffers and run with one thl_gemm_batched call.  Each array's
    stride is its largest stored size rounded up to `pad` bytes (0 for an
    array listed in `shared`, which then comes from the first workload).
    The per-tensor fp8 scales, alpha, beta, activation and types are one set
    for the whole batch: the first workload's.  The workloads are updated to
    what runs (shared arrays and the fp8 scales copied from the first), so
    that each can be checked against the oracle as it stands."""

    def __init__(self, ws, device="cuda", shared=(), pad=256, d_fill=float("nan")):
        self.ws = ws
        w0 = ws[0]
        for w in ws[1:]:
            w.a_scale, w.b_scale = w0.a_scale, w0.b_scale
            for name in shared:
                setattr(w, name, getattr(w0, name))
        self.L = len(ws)
        self.strides = {}
        self.bufs = {}
        eb = {"f32": 4, "f16": 2, "bf16": 2, "i8": 1, "i32": 4, "e4m3": 1, "e5m2": 1, "e2m1": 0.5, "e8m0": 1,
              "e2m3": 0.75, "e3m2": 0.75}
        types = {"a": w0.type_a, "b": w0.type_b, "c": w0.type_c, "bias": w0.type_bias, "sfa": "e8m0",
                 "sfb": "e8m0"}
        for name in ("a", "b", "c", "bias", "sfa", "sfb"):
            arrs = [getattr(w, name) for w in ws]
            if arrs[0] is None or (name == "c" and w0.beta == 0.0):
                self.bufs[name], self.strides[name] = None, 0
                continue
            raws = [np.ascontiguousarray(x).view(np.uint8).reshape(-1) for x in arrs]
            if name in shared:
                raws = raws[:1]
            sb = (max(len(r) for r in raws) + pad - 1) // pad * pad
            host = np.zeros(sb * len(raws), np.uint8)
            for z, r in enumerate(raws):
                host[z * sb: z * sb + len(r)] = r
            self.bufs[name] = torch.from_numpy(host).to(device)
            assert (sb / eb[types[name]]).is_integer(), "pad must hold whole elements (768 bytes for fp6)"
            self.strides[name] = 0 if name in shared else int(sb / eb[types[name]])
        es_d = eb[w0.type_d]
        self.stride_d = (w0.ldd * max(1, w0.n) * es_d + pad - 1) // pad * pad // es_d
        self.d = torch.empty((self.L * self.stride_d,), dtype=_TORCH_D[w0.type_d], device=device)
        if w0.type_d == "i32":
            self.d.fill_(-(2 ** 31) + 7)
        else:
            self.d.fill_(d_fill)

    def run(self, stream=None):
        w = self.ws[0]
        b = self.bufs

        def ptr(name):
            t = b[name]
            return t.data_ptr() if t is not None and t.numel() else None

        dt = thl.make_dtypes(w.type_a, w.type_b, w.type_c, w.type_d, w.type_bias if w.bias is not None else "none")
        flags = (thl.THL_EPI_BIAS if w.bias is not None else 0) | \
            {"none": 0, "relu": thl.THL_EPI_RELU, "gelu": thl.THL_EPI_GELU}[w.act]
        epi = thl.thl_epilogue(flags, ptr("bias"))
        sc = thl.thl_scales(float(w.a_scale), float(w.b_scale), ptr("sfa"), int(w.ld_sfa), ptr("sfb"),
                            int(w.ld_sfb))
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        s = self.strides
        return thl.thl_gemm_batched(self.L, w.m, w.n, w.k, ptr("a"), w.lda, s["a"], w.op_a, ptr("b"), w.ldb,
                                    s["b"], w.op_b, ptr("c"), w.ldc or max(1, w.m), s["c"], self.d.data_ptr(),
                                    w.ldd, self.stride_d, w.alpha, w.beta, dt, epi, s["bias"], sc, s["sfa"],
                                    s["sfb"], stream)

    def d_all(self, z) -> np.ndarray:
        """All of problem z's D as an (m, n) array [i, j]."""
        w = self.ws[z]
        host = self.d[z * self.stride_d: z * self.stride_d + w.ldd * w.n].cpu().reshape(w.n, w.ldd)[:, : w.m].T
        if w.type_d == "i32":
            return host.to(torch.int64).numpy()
        return host.to(torch.float64).numpy()


class GroupedDeviceProblem:
    """Workloads of different shapes, one format and one epilogue, each
    uploaded to buffers of its own, run with one thl_gemm_grouped call.  The
    descriptor array is built on the host and copied to the device; the
    per-tensor fp8 scales, alpha, beta, activation and types are the first
    workload's (the others are updated to match, so that each can be checked
    against the oracle as it stands)."""

    def __init__(self, ws, device="cuda", d_fill=float("nan")):
        self.ws = ws
        w0 = ws[0]
        for w in ws[1:]:
            w.a_scale, w.b_scale = w0.a_scale, w0.b_scale
        self.probs = [DeviceProblem(w, device=device, d_fill=d_fill) for w in ws]
        arr = (thl.thl_group_problem * len(ws))()

        def ptr(t):
            return t.data_ptr() if t is not None and t.numel() else None

        for z, (w, dp) in enumerate(zip(ws, self.probs)):
            arr[z] = thl.thl_group_problem(w.m, w.n, w.k, ptr(dp.a), w.lda, ptr(dp.b), w.ldb, ptr(dp.c),
                                           w.ldc or max(1, w.m), dp.d.data_ptr(), dp.ldd, ptr(dp.bias), ptr(dp.sfa),
                                           int(w.ld_sfa), ptr(dp.sfb), int(w.ld_sfb))
        self.host = arr
        raw = np.frombuffer(bytes(arr), dtype=np.uint8).copy() if len(ws) else np.zeros(0, np.uint8)
        self.dev = torch.from_numpy(raw).to(device)

    def run(self, stream=None):
        w = self.ws[0]
        dt = thl.make_dtypes(w.type_a, w.type_b, w.type_c, w.type_d, w.type_bias if w.bias is not None else "none")
        flags = (thl.THL_EPI_BIAS if w.bias is not None else 0) | \
            {"none": 0, "relu": thl.THL_EPI_RELU, "gelu": thl.THL_EPI_GELU}[w.act]
        epi = thl.thl_epilogue(flags, None)
        sc = thl.thl_scales(float(w.a_scale), float(w.b_scale), None, 0, None, 0)
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        return thl.thl_gemm_grouped(len(self.ws), self.host, self.dev.data_ptr() if self.dev.numel() else None,
                                    w.op_a, w.op_b, w.alpha, w.beta, dt, epi, sc, stream)

    def d_all(self, z) -> np.ndarray:
        return self.probs[z].d_all()
