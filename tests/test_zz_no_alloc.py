"""thl_gemm_noalloc: the allocation-free variant of thl_gemm, whose split-K
partial matrices live in the library's static scratch array.  Checked through
the C ABI against thl_gemm on the same inputs, on two calls in a row (the
second smaller), plus the oracle's sample and the scratch limit."""
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run_both(w):
    """D from thl_gemm and from thl_gemm_noalloc on the same inputs, and the
    split count each ran with."""
    import tile_hierarchy_linear_amd as thl
    from workloads.device import DeviceProblem

    dp = DeviceProblem(w)
    outs = []
    for entry in (thl.thl_gemm, thl.thl_gemm_noalloc):
        dp.d.fill_(float("nan"))
        assert dp.run(entry=entry) == 0
        torch.cuda.synchronize()
        outs.append((dp.d.clone(), thl.thl_last_splits()))
    return dp, outs


def _check_oracle(w, dp):
    from oracle import compare

    rows, cols = w.sample(4096)
    res = compare.parity_check(w, dp.d_values(rows, cols), rows, cols)
    assert res["ok"], res


def test_noalloc_matches_thl_gemm_on_two_calls_the_second_smaller():
    _gpu()
    import workloads as wl

    # call 1: 15 tiles, K split 16 ways through the scratch array;
    # call 2: smaller, 4 tiles of a 256x256 output, split again
    for w, want in ((wl.make("fp16", 640, 384, 8192), 16), (wl.make("bf16", 256, 256, 8192), 16)):
        print(f"[noalloc] {w.name} {w.m}x{w.n}x{w.k}", flush=True)
        dp, ((d_ref, s_ref), (d_na, s_na)) = _run_both(w)
        assert s_ref == s_na == want
        # same kernels, same split, same order of the sums: the same bits
        assert torch.equal(d_ref.view(torch.int16 if d_ref.element_size() == 2 else torch.int32),
                           d_na.view(torch.int16 if d_na.element_size() == 2 else torch.int32))
        _check_oracle(w, dp)


def test_noalloc_without_a_split_is_thl_gemm():
    _gpu()
    import workloads as wl

    w = wl.make("fp8", 300, 200, 1024)
    dp, ((d_ref, s_ref), (d_na, s_na)) = _run_both(w)
    assert s_ref == s_na == 1
    assert torch.equal(d_ref.view(torch.int16), d_na.view(torch.int16))
    _check_oracle(w, dp)


def test_noalloc_refuses_a_split_larger_than_its_scratch():
    _gpu()
    import tile_hierarchy_linear_amd as thl
    import workloads as wl
    from workloads.device import DeviceProblem

    # 16 forced splits of a 2048^2 fp32 output need 256 MiB: refused, D untouched
    w = wl.make("fp16", 2048, 2048, 4096)
    dp = DeviceProblem(w)
    os.environ["THL_FORCE_VARIANT"] = "f16_tn_128x128_v16_s4_o2"
    os.environ["THL_FORCE_SPLITS"] = "16"
    try:
        assert dp.run(entry=thl.thl_gemm_noalloc) == thl.THL_ERR_SCRATCH
    finally:
        os.environ.pop("THL_FORCE_VARIANT")
        os.environ.pop("THL_FORCE_SPLITS")
    torch.cuda.synchronize()
    assert torch.isnan(dp.d).all()
    assert "scratch" in thl.thl_status_string(thl.THL_ERR_SCRATCH)
