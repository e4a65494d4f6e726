"""The C-ABI library on the host: it loads, exports every symbol include/gemm.h
declares, and rejects bad arguments before touching a device (no GPU needed)."""
import ctypes
import os
import re

import pytest

import dense_blas3_gemm_amd as d

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm.h")

OK, INVALID, NOT_SUPPORTED, NOT_INIT = 0, 1, 2, 3
BF16_BF16 = d.BF16_BF16
A, B, C = 0x1000, 0x2000, 0x3000  # host-side stand-ins; never dereferenced by these calls


def header_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"\b(gemm_[a-z0-9_]+)\s*\(", text)


def test_library_exports_every_declared_symbol():
    lib = d.load_library()
    syms = header_symbols()
    assert set(syms) == set(d.EXPORTS), syms
    for s in syms:
        assert hasattr(lib, s), s


def test_version_and_policy_table():
    assert d.version().startswith("dbgemm ")
    names = d.policies()
    assert names[0] == "simt_generic"
    assert len(names) == len(set(names))
    assert any(n.startswith("bf16_") for n in names) and any(n.startswith("e4m3_") for n in names)
    lib = d.load_library()
    assert lib.gemm_policy_name(-1) is None and lib.gemm_policy_name(len(names)) is None
    assert lib.gemm_status_string(1) == b"GEMM_STATUS_INVALID_VALUE"


def chk(**kw):
    a = dict(transA=0, transB=0, M=64, N=64, K=64, alpha=1.0, A=A, lda=64, B=B, ldb=64, beta=0.0,
             C=C, ldc=64, dtype=BF16_BF16)
    a.update(kw)
    return d.check_args(a["transA"], a["transB"], a["M"], a["N"], a["K"], a["alpha"], a["A"], a["lda"],
                        a["B"], a["ldb"], a["beta"], a["C"], a["ldc"], a["dtype"])


def test_check_args_accepts_valid():
    assert chk() == OK
    assert chk(transA=1, lda=64) == OK
    assert chk(M=0, C=0, A=0, B=0) == OK  # empty output: nothing is touched
    assert chk(K=0, A=0, B=0) == OK       # C = beta*C only
    assert chk(alpha=0.0, A=0, B=0) == OK


@pytest.mark.parametrize("kw", [
    dict(transA=2), dict(transB=-1), dict(dtype=4), dict(dtype=-1),
    dict(M=-1), dict(N=-5), dict(K=-1), dict(M=1 << 31),
    dict(lda=63), dict(ldb=63), dict(ldc=63),
    dict(transA=1, M=100, lda=64), dict(transB=1, K=100, ldb=64),
    dict(C=0), dict(A=0), dict(B=0),
])
def test_check_args_rejects_invalid(kw):
    assert chk(**kw) == INVALID


def test_check_args_non_finite_scalars():
    assert chk(alpha=float("nan")) == NOT_SUPPORTED
    assert chk(beta=float("inf")) == NOT_SUPPORTED


def test_null_handle_is_not_initialized():
    lib = d.load_library()
    st = lib.gemm_run(None, 0, 0, 8, 8, 8, 1.0, ctypes.c_void_p(A), 8, ctypes.c_void_p(B), 8, 0.0,
                      ctypes.c_void_p(C), 8, BF16_BF16)
    assert st == NOT_INIT
    assert lib.gemm_set_stream(None, None) == NOT_INIT
    assert lib.gemm_set_policy(None, b"auto") == NOT_INIT
    assert lib.gemm_destroy(None) == OK
    # a pointer that was never a handle is rejected, not dereferenced
    assert lib.gemm_destroy(ctypes.c_void_p(0x1234)) == NOT_INIT
    assert lib.gemm_run(ctypes.c_void_p(0x1234), 0, 0, 8, 8, 8, 1.0, ctypes.c_void_p(A), 8,
                        ctypes.c_void_p(B), 8, 0.0, ctypes.c_void_p(C), 8, BF16_BF16) == NOT_INIT


def test_noalloc_checks_arguments_before_the_device():
    """gemm_run_noalloc: argument and policy-name errors come first, before any device is
    touched; without a GPU a valid call reports NOT_INITIALIZED."""
    def call(policy=None, M=8, dev=0):
        return d.run_noalloc_raw(dev, 0, policy, 0, 0, M, 8, 8, 1.0, A, 8, B, 8, 0.0, C, 8, BF16_BF16)
    assert call(M=-1) == INVALID
    assert call(policy="no_such_policy") == INVALID
    assert call(policy="bf16_pp_m256n256k32_w2x4_mt16_s4+sk4") == INVALID  # split-K: ring policies only
    assert call(policy="bf16_dma_m64n64k64_w2x2_mt16_s4+streamk") == INVALID  # stream-K: ping-pong only
    for bad in ("+streamk0", "+streamk4097", "+streamkx", "+stream", "+sk3"):
        assert call(policy="bf16_pp_m256n256k32_w2x4_mt16_s4" + bad) == INVALID, bad
    st = call()
    if st != OK:  # no GPU here
        assert st == NOT_INIT
        assert call(policy="auto") == NOT_INIT
        assert call(policy="bf16_pp_m256n256k32_w2x4_mt16_s4+streamk7") == NOT_INIT


def test_create_without_device_or_with_one():
    lib = d.load_library()
    h = ctypes.c_void_p()
    st = lib.gemm_create(ctypes.byref(h), 0)
    if st == OK:  # a GPU is visible
        assert h.value
        assert lib.gemm_destroy(h) == OK
        assert lib.gemm_destroy(h) == NOT_INIT  # already destroyed
    else:
        assert st == NOT_INIT and not h.value
    assert lib.gemm_create(None, 0) == INVALID


def test_policy_selection_is_shape_driven_and_deterministic():
    q = lambda *a, **k: d.query_policy(*a, A_ptr=A, B_ptr=B, C_ptr=C, **k)
    big = q(4096, 4096, 4096)
    assert big.startswith("bf16_") and "m256n256" in big and big == q(4096, 4096, 4096)
    assert q(4096, 4096, 4096, dtype=d.E4M3_BF16).startswith("e4m3_")
    # misaligned pointers or strides fall back to the generic kernel
    assert d.query_policy(4096, 4096, 4096, A_ptr=A + 2, B_ptr=B, C_ptr=C) == "simt_generic"
    assert q(64, 64, 60) == "simt_generic"           # K not a whole number of 16-byte chunks
    assert q(512, 512, 256).startswith("bf16_")
    assert q(5120, 5120, 2048, transA=1).startswith("bf16_")
    small = q(256, 256, 256, dtype=d.BF16_F32)
    assert small.startswith("bf16_") and "m256n256" not in small  # more than one tile for 256^3
    # split-K only where the tiles alone leave most CUs idle
    assert "+sk" in q(512, 512, 8192) and "+sk" not in q(4096, 4096, 4096)
    assert "+sk" not in q(512, 512, 256)  # too few K tiles to share


def test_large_workload_choices():
    """The shape-driven choice for the large workloads: the 256 x 256 ping-pong tile (bf16)
    and its 128-deep E4M3 and block-scaled E4M3 forms, never split and never stream-K
    (stream-K is named only)."""
    q = lambda *a, **k: d.query_policy(*a, A_ptr=A, B_ptr=B, C_ptr=C, **k)
    for M, N, K, tA, tB, dt, prefix in [(4096, 4096, 4096, 0, 0, d.BF16_BF16, "bf16_pp_m256n256k32"),
                                        (2048, 5120, 5120, 0, 0, d.BF16_BF16, "bf16_pp_m256n256k32"),
                                        (5120, 5120, 2048, 1, 0, d.BF16_BF16, "bf16_pp_m256n256k32"),
                                        (16384, 5120, 5120, 0, 0, d.E4M3_BF16, "e4m3_pp_m256n256k128"),
                                        (16384, 5120, 5120, 0, 1, d.MXE4M3_BF16, "mxe4m3_pp_m256n256k128")]:
        name = q(M, N, K, transA=tA, transB=tB, dtype=dt)
        assert name.startswith(prefix) and "+" not in name, (M, N, K, name)


def test_small_k_choices():
    """At 4096^2 the four-slot 32-deep ping-pong tile at every K from 256 (measured against the
    two-slot 64-deep one: 14.8-15.7 against 15.6-16.4 us at K = 256, 20.7-22.6 against
    21.2-22.5 at K = 512, 31.9-33.6 against 32.2-34.5 at K = 1024)."""
    q = lambda *a, **k: d.query_policy(*a, A_ptr=A, B_ptr=B, C_ptr=C, **k)
    for K in (256, 512, 1024, 2048):
        assert q(4096, 4096, K, dtype=d.BF16_BF16) == "bf16_pp_m256n256k32_w2x4_mt16_s4", K


def test_lds_probe_rejects_bad_arguments():
    lib = d.load_library()
    assert lib.gemm_hw_probe(None, 0, 0, 1, 1, None, 0, ctypes.c_void_p(C)) == NOT_INIT
    ok = (ctypes.c_uint32 * 512)(*([0] * 512))
    assert lib.gemm_lds_probe(None, 0, ok, 1, 1) == NOT_INIT
    assert lib.gemm_lds_probe(ctypes.c_void_p(0x1234), 0, ok, 1, 1) == NOT_INIT


def test_query_policy_rejects_bad_arguments():
    lib = d.load_library()
    buf = ctypes.create_string_buffer(64)
    assert lib.gemm_query_policy(None, 3, 0, 8, 8, 8, None, 8, None, 8, None, 8, 1, buf, 64) == INVALID
    assert lib.gemm_query_policy(None, 0, 0, -8, 8, 8, None, 8, None, 8, None, 8, 1, buf, 64) == INVALID
    assert lib.gemm_query_policy(None, 0, 0, 8, 8, 8, None, 8, None, 8, None, 8, 1, None, 0) == INVALID


def test_blas3_calls_reject_a_missing_handle():
    """Every BLAS3 entry point checks the handle before anything else (no device needed)."""
    lib = d.load_library()
    vp = ctypes.c_void_p
    for h in (None, vp(0x1234)):
        assert lib.gemm_syrk(h, 0, 0, 8, 8, 1.0, vp(A), 8, 0.0, vp(C), 8, BF16_BF16) == NOT_INIT
        assert lib.gemm_syr2k(h, 0, 0, 8, 8, 1.0, vp(A), 8, vp(B), 8, 0.0, vp(C), 8, BF16_BF16) == NOT_INIT
        assert lib.gemm_symm(h, 0, 0, 8, 8, 1.0, vp(A), 8, vp(B), 8, 0.0, vp(C), 8, BF16_BF16) == NOT_INIT
        assert lib.gemm_trmm(h, 0, 0, 0, 0, 8, 8, 1.0, vp(A), 8, vp(B), 8, vp(C), 8, BF16_BF16) == NOT_INIT
        assert lib.gemm_trsm(h, 0, 0, 0, 0, 8, 8, 1.0, vp(A), 8, vp(B), 8, BF16_BF16) == NOT_INIT
