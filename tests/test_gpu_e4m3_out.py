"""E4M3 output (GEMM_E4M3_E4M3 and GEMM_MXE4M3_E4M3) through the C-ABI against the fp64
oracle and its E4M3 rounding (oracle.round_e4m3): every kernel family, the edge
columns of a ragged tile, the beta term read from E4M3 codes, split-K, saturation."""
import numpy as np
import pytest

import gemm_inputs as gi
import oracle
import tolerance

pytestmark = pytest.mark.gpu

POLICIES = [None, "e4m3_m256n256k64_w2x4_mt16_s2", "e4m3_m128n128k64_w2x4_mt16_s2",
            "e4m3native_dma_m256n256k128_w2x4_mt32_s2", "simt_generic"]
NATIVE = {"e4m3native_dma_m256n256k128_w2x4_mt32_s2", "mxe4m3native_dma_m256n256k128_w2x4_mt32_s2"}


def _codes_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.float8_e4m3fn).cuda()


def _c_dev(M, N, ldc, C0=None):
    """E4M3 C [M][N] inside rows of ldc bytes; NaN codes everywhere C0 does not set."""
    import torch
    buf = np.full((M, ldc), 0x7F, dtype=np.uint8)
    if C0 is not None:
        buf[:, :N] = C0
    return torch.from_numpy(buf).view(torch.float8_e4m3fn).cuda()[:, :N]


def _host(C):
    import torch
    return C.cpu().contiguous().view(torch.uint8).numpy()


def _run(gpu, A, B, M, N, K, tA, tB, alpha, beta, C0, ldc, policy):
    import torch
    C = _c_dev(M, N, ldc, C0)
    gpu.set_policy(policy)
    try:
        gpu(_codes_dev(A), _codes_dev(B), C, transA=tA, transB=tB, alpha=alpha, beta=beta)
    finally:
        gpu.set_policy(None)
    torch.cuda.synchronize()
    return _host(C)


def _oracle(A, B, M, N, K, tA, tB, alpha, beta, C0):
    return oracle.gemm(tA, tB, M, N, K, alpha, A, A.shape[1], B, B.shape[1], beta,
                       None if C0 is None else np.ascontiguousarray(C0), N, oracle.IN_E4M3, oracle.C_E4M3)


def _operands(M, N, K, tA, tB, seed, kind="e4m3"):
    ash = (K, M) if tA else (M, K)
    bsh = (N, K) if tB else (K, N)
    if kind == "int8":
        return gi.ints(ash, seed, -8, 8, gi.E4M3), gi.ints(bsh, seed + 1, -8, 8, gi.E4M3)
    return gi.e4m3_normal(ash, seed), gi.e4m3_normal(bsh, seed + 1)


@pytest.mark.parametrize("policy", POLICIES)
@pytest.mark.parametrize("tA,tB,M,N", [(0, 0, 336, 304), (0, 1, 336, 304), (1, 0, 336, 304), (1, 1, 336, 304),
                                       (0, 1, 328, 298)])
def test_e4m3_out_parity(gpu, policy, tA, tB, M, N):
    """M x N x 1008 with ragged tiles (N = 298: the last group of four columns is cut,
    C rows padded to 304 bytes), alpha = 1/8: values spread over the normal and
    subnormal E4M3 range."""
    K = 1008
    A, B = _operands(M, N, K, tA, tB, 11)
    got = _run(gpu, A, B, M, N, K, tA, tB, 0.125, 0.0, None, 304, policy)
    R, S = _oracle(A, B, M, N, K, tA, tB, 0.125, 0.0, None)
    res = tolerance.check_e4m3(got, R, S, K, 0.125, "e4m3_native" if policy in NATIVE else "fp32")
    assert res["ok"], res


@pytest.mark.parametrize("policy", [None, "e4m3_m128n128k64_w2x4_mt16_s2", "simt_generic"])
def test_e4m3_out_integer_bit_exact(gpu, policy):
    """Integer elements in [-8, 8] and alpha = 2^-4: the accumulation and alpha * acc are
    exact in fp32, so the output codes are exactly the oracle's rounding of R, ties
    (odd multiples of half an E4M3 step) included; alpha = 2^3 saturates many.  K = 528,
    a multiple of 16 as the MFMA kernels need for E4M3."""
    M, N, K = 264, 200, 528
    A, B = _operands(M, N, K, 0, 1, 5, kind="int8")
    for alpha in (2.0 ** -4, 8.0):
        got = _run(gpu, A, B, M, N, K, 0, 1, alpha, 0.0, None, 208, policy)
        R, _ = _oracle(A, B, M, N, K, 0, 1, alpha, 0.0, None)
        want = oracle.round_e4m3(R)
        assert np.array_equal(got, want), (alpha, int((got != want).sum()))


@pytest.mark.parametrize("policy", [None, "e4m3_m256n256k64_w2x4_mt16_s2", "simt_generic"])
def test_e4m3_out_beta_reads_codes(gpu, policy):
    """C <- alpha*A*B + beta*C_old with C_old given as E4M3 codes."""
    M, N, K = 300, 282, 512
    A, B = _operands(M, N, K, 0, 1, 21)
    C0 = gi.e4m3_normal((M, N), 23)
    got = _run(gpu, A, B, M, N, K, 0, 1, 0.25, -1.5, C0, 288, policy)
    R, S = _oracle(A, B, M, N, K, 0, 1, 0.25, -1.5, C0)
    res = tolerance.check_e4m3(got, R, S, K, 0.25)
    assert res["ok"], res


@pytest.mark.parametrize("splits", [2, 4])
def test_e4m3_out_split_k(gpu, splits):
    """The split-K reduction runs the same epilogue: E4M3 C with beta."""
    M, N, K = 256, 256, 2048
    A, B = _operands(M, N, K, 0, 0, 31)
    C0 = gi.e4m3_normal((M, N), 33)
    got = _run(gpu, A, B, M, N, K, 0, 0, 0.0625, 0.5, C0, 256, f"e4m3native_dma_m256n256k128_w2x4_mt32_s2+sk{splits}")
    R, S = _oracle(A, B, M, N, K, 0, 0, 0.0625, 0.5, C0)
    res = tolerance.check_e4m3(got, R, S, K, 0.0625, "e4m3_native")
    assert res["ok"], res


@pytest.mark.parametrize("policy", [None, "mxe4m3native_dma_m256n256k128_w2x4_mt32_s2", "simt_generic"])
def test_mx_e4m3_out(gpu, policy):
    """Block-scaled operands with E4M3 C (GEMM_MXE4M3_E4M3): scales 2^-3 .. 2^1 keep the
    outputs in range; alpha folds in a caller scale of 2^-6."""
    import torch
    M, N, K = 328, 296, 1024
    d = gi.mx_operands(M, N, K, seeds=(41, 42, 43, 44))
    d["SA"] = gi.ue8m0_bytes(d["SA"].shape, 45, 124, 128)
    d["SB"] = gi.ue8m0_bytes(d["SB"].shape, 46, 124, 128)
    C = _c_dev(M, N, 304)
    gpu.set_policy(policy)
    try:
        gpu.run_mx(_codes_dev(d["A"]), torch.from_numpy(d["SA"]).cuda(), _codes_dev(d["B"]),
                   torch.from_numpy(d["SB"]).cuda(), C, alpha=2.0 ** -6)
    finally:
        gpu.set_policy(None)
    torch.cuda.synchronize()
    got = _host(C)
    nb = K // 32
    R, S = oracle.gemm_mx(M, N, K, 2.0 ** -6, d["A"], K, d["SA"], nb, d["B"], K, d["SB"], nb, 0.0, None, N,
                          oracle.C_E4M3)
    res = tolerance.check_e4m3(got, R, S, K, 2.0 ** -6, "e4m3_native" if policy in NATIVE else "fp32")
    assert res["ok"], res


def test_e4m3_out_query_and_errors(gpu):
    import ctypes
    import dense_blas3_gemm_amd as d
    lib = d.load_library()
    p = ctypes.c_void_p(0x1000)
    # E4M3 C is allowed with E4M3 inputs; the block-scaled dtype is refused by gemm_run
    assert gpu.query_policy(4096, 4096, 4096, 0, 0, d.E4M3_E4M3) != ""
    assert lib.gemm_run(gpu.handle, 0, 1, 64, 64, 64, 1.0, p, 64, p, 64, 0.0, p, 64, d.MXE4M3_E4M3) == 1
    # ldc below N
    assert lib.gemm_run(gpu.handle, 0, 0, 64, 64, 64, 1.0, p, 64, p, 64, 0.0, p, 32, d.E4M3_E4M3) == 1
