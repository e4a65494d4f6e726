"""GPU parity of stream-K on the ping-pong kernels: the whole-round tiles run one per
workgroup, the rest of the tiles' K loops are shared by the stream-K workgroups, and
partial tiles are handed to each tile's owner.  Forced grids of a few workgroups give
ranges that start and end inside tiles, cover whole tiles in the middle, and tiles shared
by many workgroups."""
import dataclasses

import numpy as np
import pytest

import gemm_inputs as gi
import oracle
from gpu_util import compare, run_gpu

pytestmark = pytest.mark.gpu

PP = "bf16_pp_m256n256k32_w2x4_mt16_s4"
PP64 = "bf16_pp_m256n256k64_w2x4_mt16_s2"
PP192 = "bf16_pp_m192n256k64_w2x4_mt16_s2"
PPE = "e4m3_pp_m256n256k64_w2x4_mt16_s4"


def _ok(res, what):
    assert res["ok"], f"{what}: {res}"


@pytest.mark.parametrize("policy", [PP, PP64])
@pytest.mark.parametrize("grid", ["", "7", "4", "2"])
@pytest.mark.parametrize("tA,tB", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_streamk_forced_grids(gpu, policy, grid, tA, tB):
    """600 x 520 (a 3 x 3 grid of 256 x 256 tiles, ragged) x 1000 (ragged K): with G stream-K
    workgroups the first 9 - 9 % G tiles run whole and the rest are shared (all 9 with one
    workgroup per CU)."""
    p = gi.Gemm("t", 600, 520, 1000, transA=tA, transB=tB, dist="normal")
    data = p.make()
    C = run_gpu(gpu, p, data, policy=f"{policy}+streamk{grid}")
    _ok(compare(p, data, C), f"{policy}+streamk{grid} {tA}{tB}")


@pytest.mark.parametrize("shape", [(1000, 1000, 2048), (2048, 1280, 512), (264, 1800, 4096)])
def test_streamk_one_per_cu(gpu, shape):
    """Fewer tiles than CUs: every tile is shared by several workgroups (up to 16 here)."""
    M, N, K = shape
    p = gi.Gemm("t", M, N, K, dist="normal")
    data = p.make()
    C = run_gpu(gpu, p, data, policy=PP + "+streamk")
    _ok(compare(p, data, C), f"{shape}")


def test_streamk_192_tiles_and_beta(gpu):
    """The 192-row tile, fp32 C with beta: the owner's epilogue reads C once."""
    p = gi.Gemm("t", 700, 904, 1496, c_dtype="f32", beta=0.75, c_dist="normal", dist="normal")
    data = p.make()
    C = run_gpu(gpu, p, data, policy=PP192 + "+streamk5")
    _ok(compare(p, data, C), "192 beta")


@pytest.mark.parametrize("c_dtype", ["bf16", "f32"])
def test_streamk_e4m3(gpu, c_dtype):
    p = gi.Gemm("t", 520, 608, 1536, in_dtype="e4m3", c_dtype=c_dtype, dist="e4m3")
    data = p.make()
    C = run_gpu(gpu, p, data, policy=PPE + "+streamk6")
    _ok(compare(p, data, C), "e4m3 " + c_dtype)


@pytest.mark.parametrize("grid", ["", "7", "5"])
def test_streamk_integer_bitwise(gpu, grid):
    """Integer inputs: every partial sum is exact, so the handed-off partials must add up to
    the oracle's value rounded once, bit for bit (a lost, doubled or misplaced partial
    cannot hide in rounding)."""
    p = gi.Gemm("t", 776, 520, 2000, dist="int4")
    data = p.make()
    C = run_gpu(gpu, p, data, policy=PP + "+streamk" + grid)
    R, _ = oracle.gemm_problem(p, data, with_abs=False)
    assert np.array_equal(C, oracle.round_bf16(R))


def test_streamk_deterministic_and_flags_reset(gpu):
    """Back-to-back calls (each owner clears the flags it waited for): identical bits, and a
    call after one with other inputs is not served stale partials."""
    p = gi.Gemm("t", 1000, 1000, 2048, dist="normal")
    d0, d1 = p.make(), p.make(seeds=(5, 6, 7))
    pol = PP + "+streamk"
    a = run_gpu(gpu, p, d0, policy=pol)
    b = run_gpu(gpu, p, d1, policy=pol)
    c = run_gpu(gpu, p, d0, policy=pol)
    assert np.array_equal(a, c)
    assert (a != b).mean() > 0.99
    _ok(compare(p, d1, b), "second inputs")


def test_streamk_reported_by_query(gpu):
    """A forced stream-K policy is reported with its suffix where it runs stream-K."""
    import dense_blas3_gemm_amd as d
    gpu.set_policy(PP + "+streamk7")
    try:
        assert d.query_policy(600, 520, 1000, handle=gpu.handle) == PP + "+streamk7"  # 9 tiles
        assert d.query_policy(1792, 256, 512, handle=gpu.handle) == PP  # 7 tiles: one whole round
    finally:
        gpu.set_policy(None)


def test_streamk_noalloc_matches_gemm_run(gpu):
    """The handle-free call runs the same stream-K plan from its static array."""
    import torch
    import dense_blas3_gemm_amd as d
    from gpu_util import empty_c, to_device, to_host
    p = gi.Gemm("t", 1000, 1000, 2048, dist="normal")
    data = p.make()
    want = run_gpu(gpu, p, data, policy=PP + "+streamk")
    A, B = to_device(data["A"], "bf16"), to_device(data["B"], "bf16")
    C = empty_c(p.M, p.N, "bf16")
    d.run_noalloc(A, B, C, policy=PP + "+streamk")
    torch.cuda.synchronize()
    assert np.array_equal(to_host(C), want)


def test_streamk_forced_whole_rounds_runs_plain(gpu):
    """A grid that makes whole rounds has no stream-K part: same bits as the plain kernel."""
    p = dataclasses.replace(gi.Gemm("t", 768, 768, 512), dist="normal")  # 9 tiles, G = 3
    data = p.make()
    assert np.array_equal(run_gpu(gpu, p, data, policy=PP + "+streamk3"), run_gpu(gpu, p, data, policy=PP))
