"""gemm_run_noalloc, the handle-free call that allocates nothing (its split-K partials go
to a static device array), against gemm_run on a handle: two calls in a row, the second
smaller, each bitwise equal to gemm_run (same policy choice, same kernels) and within the
oracle's bound; then its argument errors."""
import numpy as np
import pytest

import gemm_inputs as gi
from gpu_util import compare, empty_c, run_gpu, to_device, to_host

pytestmark = pytest.mark.gpu


def _noalloc(p, data, policy=None):
    import torch
    import dense_blas3_gemm_amd as d
    A = to_device(data["A"], p.in_dtype)
    B = to_device(data["B"], p.in_dtype)
    C = to_device(data["C"], p.c_dtype) if "C" in data else empty_c(p.M, p.N, p.c_dtype)
    d.run_noalloc(A, B, C, transA=p.transA, transB=p.transB, alpha=p.alpha, beta=p.beta, dtype=p.dtype_code,
                  policy=policy)
    torch.cuda.synchronize()
    return to_host(C)


def test_noalloc_matches_gemm_run(gpu):
    import dense_blas3_gemm_amd as d
    cases = [
        # long K on a small output: the shape-driven choice splits K, partials in the array
        gi.Gemm("t", 512, 512, 8192, dist="normal"),
        # then a smaller call (fp32 C, beta != 0) that reuses the array
        gi.Gemm("t", 264, 200, 4096, c_dtype="f32", beta=0.5, c_dist="normal", dist="normal"),
    ]
    assert "+sk" in d.query_policy(512, 512, 8192, handle=gpu.handle)
    for p in cases:
        data = p.make()
        want = run_gpu(gpu, p, data)
        got = _noalloc(p, data)
        assert np.array_equal(got, want), p
        res = compare(p, data, got)
        assert res["ok"], res


def test_noalloc_forced_policy_and_errors(gpu):
    import dense_blas3_gemm_amd as d
    p = gi.Gemm("t", 1024, 768, 2048, dist="normal")
    data = p.make()
    pol = "bf16_dma_m128n128k64_w2x4_mt16_s4+sk4"
    want = run_gpu(gpu, p, data, policy=pol)
    assert np.array_equal(_noalloc(p, data, policy=pol), want)
    # a forced split whose partials (1024 tiles x 16 splits x 64 x 64 floats = 256 MiB) exceed the array
    with pytest.raises(d.GemmError, match="NOT_SUPPORTED"):
        _noalloc(gi.Gemm("t", 2048, 2048, 4096), gi.Gemm("t", 2048, 2048, 4096).make(),
                 policy="bf16_dma_m64n64k64_w2x2_mt16_s4+sk16")
    with pytest.raises(d.GemmError, match="INVALID_VALUE"):
        _noalloc(p, data, policy="no_such_policy")
    assert d.run_noalloc_raw(64, 0, None, 0, 0, 8, 8, 8, 1.0, 16, 8, 16, 8, 0.0, 16, 8, d.BF16_BF16) == 1
    assert d.run_noalloc_raw(-1, 0, None, 0, 0, 8, 8, 8, 1.0, 16, 8, 16, 8, 0.0, 16, 8, d.BF16_BF16) == 1
