"""Split-K through the C-ABI: the K range of each output tile is shared by several
workgroups whose fp32 partials a second kernel adds in split order.  Checked against
the fp64 oracle element by element, bit for bit on integer inputs, for determinism,
and for reuse of the workspace by calls of other shapes."""
import numpy as np
import pytest

import gemm_inputs as gi
import oracle
import tolerance
from gpu_util import compare, run_gpu

pytestmark = pytest.mark.gpu

TRANS = [(0, 0), (0, 1), (1, 0), (1, 1)]
SPLIT_POLICIES = ["bf16_dma_m64n64k64_w2x2_mt16_s4", "bf16_dma_m128n128k64_w2x4_mt16_s4",
                  "bf16_dma_m128n128k64_w2x2_mt32_s3", "bf16_dma_m256n256k64_w2x4_mt16_s2",
                  "bf16_dma_m256n256k64_w2x4_mt32_s2", "bf16_dma_m128n256k64_w2x4_mt16_s3"]


def _assert_ok(res, what):
    assert res["ok"], f"{what}: {res}"


@pytest.mark.parametrize("tA,tB", TRANS)
@pytest.mark.parametrize("splits", [2, 4, 8])
@pytest.mark.parametrize("policy", SPLIT_POLICIES)
def test_splitk_bf16(gpu, policy, splits, tA, tB):
    """K = 1000 is 16 K tiles of 64 with a ragged last one; alpha/beta both visible."""
    for c_dtype in ("bf16", "f32"):
        p = gi.Gemm("t", 328, 296, 1000, transA=tA, transB=tB, c_dtype=c_dtype, alpha=1.5, beta=-0.5,
                    dist="normal", c_dist="normal")
        data = p.make()
        C = run_gpu(gpu, p, data, policy=f"{policy}+sk{splits}")
        _assert_ok(compare(p, data, C), f"{policy}+sk{splits} {tA}{tB} {c_dtype}")


@pytest.mark.parametrize("splits,K", [(2, 1040), (4, 1040), (8, 2000)])
@pytest.mark.parametrize("c_dtype", ["bf16", "f32"])
def test_splitk_integer_inputs_bitwise(gpu, splits, K, c_dtype):
    """Exact partials add exactly: C == RNE(R) bit for bit (K = 1040 is 17 K tiles)."""
    p = gi.Gemm("t", 520, 392, K, c_dtype=c_dtype, dist="int4")
    data = p.make()
    C = run_gpu(gpu, p, data, policy=f"bf16_dma_m64n64k64_w2x2_mt16_s4+sk{splits}")
    R, _ = oracle.gemm_problem(p, data, with_abs=False)
    want = oracle.round_bf16(R) if c_dtype == "bf16" else oracle.round_f32(R)
    assert np.array_equal(C, want)


def test_splitk_beta_zero_never_reads_c(gpu):
    p = gi.Gemm("t", 200, 136, 1024, dist="normal")
    data = p.make()
    nan = gi.f32_to_bf16_bits(np.full((p.M, p.N), np.nan, dtype=np.float32))
    C = run_gpu(gpu, p, data, C_init=nan, policy="bf16_dma_m64n64k64_w2x2_mt16_s4+sk4")
    _assert_ok(compare(p, data, C), "beta 0")


@pytest.mark.parametrize("tA,tB", TRANS)
@pytest.mark.parametrize("splits", [2, 4])
def test_splitk_e4m3_native(gpu, splits, tA, tB):
    p = gi.Gemm("t", 320, 288, 1024, transA=tA, transB=tB, in_dtype="e4m3", c_dtype="f32", dist="e4m3")
    data = p.make()
    C = run_gpu(gpu, p, data, policy=f"e4m3native_dma_m256n256k128_w2x4_mt32_s2+sk{splits}")
    _assert_ok(compare(p, data, C, accumulate="e4m3_native"), f"sk{splits} {tA}{tB}")


def test_splitk_deterministic_and_workspace_reuse(gpu):
    """Same call twice gives the same bits, also with a call of another shape and split
    in between that reuses the workspace."""
    pol = "bf16_dma_m64n64k64_w2x2_mt16_s4+sk8"
    p1 = gi.Gemm("t", 512, 512, 2048, dist="normal")
    p2 = gi.Gemm("t", 960, 704, 1024, dist="normal")
    d1, d2 = p1.make(), p2.make(seeds=(7, 8, 9))
    c1 = run_gpu(gpu, p1, d1, policy=pol)
    c2 = run_gpu(gpu, p2, d2, policy="bf16_dma_m64n64k64_w2x2_mt16_s4+sk4")
    c3 = run_gpu(gpu, p1, d1, policy=pol)
    c4 = run_gpu(gpu, p1, d1)  # auto
    assert np.array_equal(c1, c3)
    _assert_ok(compare(p1, d1, c1), "first")
    _assert_ok(compare(p2, d2, c2), "between")
    _assert_ok(compare(p1, d1, c4), "auto")


def test_splitk_policy_names(gpu):
    import dense_blas3_gemm_amd as d
    # a split the workspace cannot hold, or that leaves a split without two K tiles
    gpu.set_policy("bf16_dma_m64n64k64_w2x2_mt16_s4+sk16")
    try:
        with pytest.raises(d.GemmError, match="NOT_SUPPORTED"):
            gpu.query_policy(4096, 4096, 4096)
        with pytest.raises(d.GemmError, match="NOT_SUPPORTED"):
            gpu.query_policy(512, 512, 1024)
        assert gpu.query_policy(512, 512, 4096) == "bf16_dma_m64n64k64_w2x2_mt16_s4+sk16"
    finally:
        gpu.set_policy(None)
    for bad in ("bf16_dma_m64n64k64_w2x2_mt16_s4+sk3", "bf16_dma_m64n64k64_w2x2_mt16_s4+sk",
                "bf16_m128n128k64_w2x2_mt32_s2+sk2", "+sk2"):
        with pytest.raises(d.GemmError, match="INVALID"):
            gpu.set_policy(bad)
    assert "+sk" in gpu.query_policy(512, 512, 8192)
    assert "+sk" not in gpu.query_policy(4096, 4096, 4096)
