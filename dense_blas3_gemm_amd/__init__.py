"""MI355X (gfx950) dense GEMM: C = alpha*op(A)*op(B) + beta*C.

A thin ctypes binding over the C-ABI in ``include/gemm.h``; every step of the
computation runs in the library's HIP kernels.  PyTorch supplies device memory and
the current stream only.  The binding fails loudly when ``libdbgemm.so`` has not
been built (``python -m dense_blas3_gemm_amd.build``): there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
# DBGEMM_LIB selects another build of the same library (the sanitized host-only build the
# CPU tests run under AddressSanitizer)
LIB_PATH = os.environ.get("DBGEMM_LIB") or os.path.join(PKG, "libdbgemm.so")

OP_N, OP_T = 0, 1
BF16_F32, BF16_BF16, E4M3_BF16, E4M3_F32, MXE4M3_BF16, MXE4M3_F32, E4M3_E4M3, MXE4M3_E4M3 = range(8)
STATUS = {0: "SUCCESS", 1: "INVALID_VALUE", 2: "NOT_SUPPORTED", 3: "NOT_INITIALIZED",
          4: "LAUNCH_FAILED", 5: "INTERNAL"}

# The exported C symbols, in the order include/gemm.h declares them.
EXPORTS = ["gemm_create", "gemm_destroy", "gemm_set_stream", "gemm_run", "gemm_run_noalloc", "gemm_run_mx",
           "gemm_quantize_mx", "gemm_check_args", "gemm_query_policy", "gemm_set_policy",
           "gemm_lds_probe", "gemm_hw_probe", "gemm_policy_count", "gemm_policy_name", "gemm_version",
           "gemm_status_string", "gemm_syrk", "gemm_syr2k", "gemm_symm", "gemm_trmm", "gemm_trsm"]

LOWER, UPPER = 0, 1
LEFT, RIGHT = 0, 1
NON_UNIT, UNIT = 0, 1

_lib = None


class GemmError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {STATUS.get(status, status)} ({status})")
        self.status = status


def _hip_runtimes():
    """Distinct libamdhip64 files mapped into this process."""
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    paths.add(os.path.realpath(line.split()[-1]))
    except OSError:
        pass
    return paths


def load_library():
    """Loads libdbgemm.so and declares the C signatures; raises if it is missing.

    PyTorch is imported first so that its HIP runtime is the one already mapped when
    the library's libamdhip64.so.7 dependency is resolved: the process then holds a
    single HIP runtime, and torch's streams and allocations are valid in the
    library's launches.
    """
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m dense_blas3_gemm_amd.build`")
    try:
        import torch  # noqa: F401  (maps torch's HIP runtime before the library's)
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    runtimes = _hip_runtimes()
    if len(runtimes) > 1:
        raise RuntimeError(f"two HIP runtimes are mapped into this process: {sorted(runtimes)}")
    i32, i64, vp, f32 = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
    lib.gemm_create.argtypes = [ctypes.POINTER(vp), i32]
    lib.gemm_destroy.argtypes = [vp]
    lib.gemm_set_stream.argtypes = [vp, vp]
    lib.gemm_run.argtypes = [vp, i32, i32, i64, i64, i64, f32, vp, i64, vp, i64, f32, vp, i64, i32]
    lib.gemm_run_noalloc.argtypes = [i32, vp, ctypes.c_char_p, i32, i32, i64, i64, i64, f32, vp, i64, vp, i64, f32,
                                     vp, i64, i32]
    lib.gemm_check_args.argtypes = [i32, i32, i64, i64, i64, f32, vp, i64, vp, i64, f32, vp, i64, i32]
    lib.gemm_query_policy.argtypes = [vp, i32, i32, i64, i64, i64, vp, i64, vp, i64, vp, i64, i32,
                                      ctypes.c_char_p, ctypes.c_size_t]
    lib.gemm_set_policy.argtypes = [vp, ctypes.c_char_p]
    lib.gemm_lds_probe.argtypes = [vp, i32, ctypes.POINTER(ctypes.c_uint32), i32, i32]
    lib.gemm_hw_probe.argtypes = [vp, i32, i32, i32, i32, vp, i64, vp]
    lib.gemm_run_mx.argtypes = [vp, i64, i64, i64, f32, vp, i64, vp, i64, vp, i64, vp, i64, f32, vp, i64, i32]
    lib.gemm_quantize_mx.argtypes = [vp, i64, i64, vp, i64, vp, i64, vp, i64]
    lib.gemm_policy_count.argtypes = []
    lib.gemm_policy_name.argtypes = [i32]
    lib.gemm_policy_name.restype = ctypes.c_char_p
    lib.gemm_version.argtypes = []
    lib.gemm_version.restype = ctypes.c_char_p
    lib.gemm_status_string.argtypes = [i32]
    lib.gemm_status_string.restype = ctypes.c_char_p
    lib.gemm_syrk.argtypes = [vp, i32, i32, i64, i64, f32, vp, i64, f32, vp, i64, i32]
    lib.gemm_syr2k.argtypes = [vp, i32, i32, i64, i64, f32, vp, i64, vp, i64, f32, vp, i64, i32]
    lib.gemm_symm.argtypes = [vp, i32, i32, i64, i64, f32, vp, i64, vp, i64, f32, vp, i64, i32]
    lib.gemm_trmm.argtypes = [vp, i32, i32, i32, i32, i64, i64, f32, vp, i64, vp, i64, vp, i64, i32]
    lib.gemm_trsm.argtypes = [vp, i32, i32, i32, i32, i64, i64, f32, vp, i64, vp, i64, i32]
    for fn in ["gemm_create", "gemm_destroy", "gemm_set_stream", "gemm_run", "gemm_run_noalloc", "gemm_check_args",
               "gemm_query_policy", "gemm_set_policy", "gemm_lds_probe", "gemm_hw_probe", "gemm_policy_count",
               "gemm_run_mx", "gemm_quantize_mx", "gemm_syrk", "gemm_syr2k", "gemm_symm", "gemm_trmm",
               "gemm_trsm"]:
        getattr(lib, fn).restype = i32
    _lib = lib
    return lib


def version() -> str:
    return load_library().gemm_version().decode()


def policies():
    lib = load_library()
    return [lib.gemm_policy_name(i).decode() for i in range(lib.gemm_policy_count())]


def dtype_code(in_dtype: str, c_dtype: str) -> int:
    return {("bf16", "f32"): BF16_F32, ("bf16", "bf16"): BF16_BF16,
            ("e4m3", "bf16"): E4M3_BF16, ("e4m3", "f32"): E4M3_F32,
            ("e4m3", "e4m3"): E4M3_E4M3}[(in_dtype, c_dtype)]


def _c_kind(C) -> str:
    import torch
    if C.dtype == torch.float32:
        return "f32"
    if C.dtype == torch.float8_e4m3fn:
        return "e4m3"
    return "bf16"


def _current_stream(device) -> int:
    """Raw hipStream_t of torch's current stream on `device` (the cheap accessor when
    this torch has it)."""
    import torch
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return int(raw(device.index if device.index is not None else torch.cuda.current_device()))
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _ld(t) -> int:
    # row-major with unit column stride: the leading dimension is the row stride
    assert t.dim() == 2 and t.stride(1) == 1, "operands must be row-major 2-D views"
    return int(t.stride(0))


class Gemm:
    """A library handle on one device; calls enqueue on torch's current stream."""

    def __init__(self, device: int = 0):
        self.lib = load_library()
        self.device = device
        h = ctypes.c_void_p()
        st = self.lib.gemm_create(ctypes.byref(h), int(device))
        if st != 0:
            raise GemmError("gemm_create", st)
        self.handle = h
        self._stream = 0  # the stream the handle is bound to (gemm_create starts on NULL)

    def close(self):
        if self.handle is not None:
            self.lib.gemm_destroy(self.handle)
            self.handle = None

    def __del__(self):  # pragma: no cover
        try:
            self.close()
        except Exception:
            pass

    def set_policy(self, name: Optional[str]):
        st = self.lib.gemm_set_policy(self.handle, None if name is None else name.encode())
        if st != 0:
            raise GemmError("gemm_set_policy", st)

    def set_stream(self, stream_ptr: int):
        st = self.lib.gemm_set_stream(self.handle, ctypes.c_void_p(stream_ptr))
        if st != 0:
            raise GemmError("gemm_set_stream", st)
        self._stream = stream_ptr

    def run_raw(self, transA, transB, M, N, K, alpha, A_ptr, lda, B_ptr, ldb, beta, C_ptr, ldc,
                dtype, stream_ptr: Optional[int] = None) -> int:
        """Direct C-ABI call with raw device pointers; returns the status code."""
        if stream_ptr is not None and stream_ptr != self._stream:
            self.set_stream(stream_ptr)
        return self.lib.gemm_run(self.handle, int(transA), int(transB), int(M), int(N), int(K),
                                 float(alpha), ctypes.c_void_p(A_ptr), int(lda), ctypes.c_void_p(B_ptr),
                                 int(ldb), float(beta), ctypes.c_void_p(C_ptr), int(ldc), int(dtype))

    def __call__(self, A, B, C, transA: int = 0, transB: int = 0, alpha: float = 1.0,
                 beta: float = 0.0, dtype: Optional[int] = None):
        """C <- alpha*op(A)*op(B) + beta*C on torch tensors (row-major 2-D views).

        A and B are bf16 or float8_e4m3fn, C bf16 or float32 (or float8_e4m3fn for E4M3
        inputs); op(X) = X^T when the trans flag is 1, read in place from X's storage.
        """
        import torch
        if dtype is None:
            ind = "e4m3" if A.dtype == torch.float8_e4m3fn else "bf16"
            dtype = dtype_code(ind, _c_kind(C))
        M, N = C.shape
        K = A.shape[0] if transA else A.shape[1]
        stream = _current_stream(C.device)
        st = self.run_raw(transA, transB, M, N, K, alpha, _ptr(A), _ld(A), _ptr(B), _ld(B), beta,
                          _ptr(C), _ld(C), dtype, stream_ptr=stream)
        if st != 0:
            raise GemmError("gemm_run", st)
        return C

    def run_mx(self, A, SA, B, SB, C, alpha: float = 1.0, beta: float = 0.0):
        """Block-scaled E4M3 GEMM (gemm_run_mx) on torch tensors: A [M][K] and B [N][K] as
        float8_e4m3fn (or uint8 codes), SA [M][ceil(K/32)] and SB [N][ceil(K/32)] uint8
        UE8M0 scales, C bf16, float32 or float8_e4m3fn [M][N];
        C <- alpha*A*B^T(scaled) + beta*C."""
        import torch
        M, N = C.shape
        K = A.shape[1]
        dtype = {"f32": MXE4M3_F32, "e4m3": MXE4M3_E4M3, "bf16": MXE4M3_BF16}[_c_kind(C)]
        stream = _current_stream(C.device)
        if stream != self._stream:
            self.set_stream(stream)
        st = self.lib.gemm_run_mx(self.handle, int(M), int(N), int(K), float(alpha), ctypes.c_void_p(_ptr(A)),
                                  _ld(A), ctypes.c_void_p(_ptr(SA)), _ld(SA), ctypes.c_void_p(_ptr(B)), _ld(B),
                                  ctypes.c_void_p(_ptr(SB)), _ld(SB), float(beta), ctypes.c_void_p(_ptr(C)),
                                  _ld(C), int(dtype))
        if st != 0:
            raise GemmError("gemm_run_mx", st)
        return C

    def quantize_mx(self, src, dst, scales):
        """bf16 [rows][cols] -> E4M3 codes in dst [rows][cols] (uint8 or float8_e4m3fn) and
        UE8M0 scales [rows][ceil(cols/32)] (uint8), along rows (gemm_quantize_mx)."""
        rows, cols = src.shape
        stream = _current_stream(src.device)
        if stream != self._stream:
            self.set_stream(stream)
        st = self.lib.gemm_quantize_mx(self.handle, int(rows), int(cols), ctypes.c_void_p(_ptr(src)), _ld(src),
                                       ctypes.c_void_p(_ptr(dst)), _ld(dst), ctypes.c_void_p(_ptr(scales)),
                                       _ld(scales))
        if st != 0:
            raise GemmError("gemm_quantize_mx", st)
        return dst, scales

    def lds_probe(self, kind: int, offsets, iters: int, workgroups: int, stream_ptr: Optional[int] = None):
        """Enqueues the LDS read microbenchmark (gemm_lds_probe); offsets: 8 x 64 byte offsets."""
        flat = [int(v) for row in offsets for v in row]
        if len(flat) != 512:
            raise ValueError("offsets must be 8 rows of 64 lanes")
        if stream_ptr is not None and stream_ptr != self._stream:
            self.set_stream(stream_ptr)
        arr = (ctypes.c_uint32 * 512)(*flat)
        st = self.lib.gemm_lds_probe(self.handle, int(kind), arr, int(iters), int(workgroups))
        if st != 0:
            raise GemmError("gemm_lds_probe", st)

    # ---------------------------------------------------------------- BLAS3 family
    # Raw C-ABI calls (device pointers; the handle's current stream) return the status;
    # the tensor forms below bind torch's current stream and raise on an error.

    def hw_probe(self, kind: int, param: int, iters: int, workgroups: int, src=None, cycles=None):
        """Enqueues a hardware microbenchmark (gemm_hw_probe) on torch's current stream;
        `cycles` (int64 device tensor of `workgroups` values, allocated when None) receives
        each workgroup's shader-clock cycles.  Returns `cycles`."""
        import torch
        if cycles is None:
            cycles = torch.zeros(workgroups, dtype=torch.int64, device=f"cuda:{self.device}")
        self.set_stream(_current_stream(cycles.device))
        src_ptr = 0 if src is None else _ptr(src)
        src_bytes = 0 if src is None else src.numel() * src.element_size()
        st = self.lib.gemm_hw_probe(self.handle, int(kind), int(param), int(iters), int(workgroups),
                                    ctypes.c_void_p(src_ptr or None), int(src_bytes), ctypes.c_void_p(_ptr(cycles)))
        if st != 0:
            raise GemmError("gemm_hw_probe", st)
        return cycles

    def _bind(self, t):
        stream = _current_stream(t.device)
        if stream != self._stream:
            self.set_stream(stream)

    def syrk_raw(self, uplo, trans, N, K, alpha, A_ptr, lda, beta, C_ptr, ldc, dtype) -> int:
        return self.lib.gemm_syrk(self.handle, int(uplo), int(trans), int(N), int(K), float(alpha),
                                  ctypes.c_void_p(A_ptr), int(lda), float(beta), ctypes.c_void_p(C_ptr), int(ldc),
                                  int(dtype))

    def syr2k_raw(self, uplo, trans, N, K, alpha, A_ptr, lda, B_ptr, ldb, beta, C_ptr, ldc, dtype) -> int:
        return self.lib.gemm_syr2k(self.handle, int(uplo), int(trans), int(N), int(K), float(alpha),
                                   ctypes.c_void_p(A_ptr), int(lda), ctypes.c_void_p(B_ptr), int(ldb), float(beta),
                                   ctypes.c_void_p(C_ptr), int(ldc), int(dtype))

    def symm_raw(self, side, uplo, M, N, alpha, A_ptr, lda, B_ptr, ldb, beta, C_ptr, ldc, dtype) -> int:
        return self.lib.gemm_symm(self.handle, int(side), int(uplo), int(M), int(N), float(alpha),
                                  ctypes.c_void_p(A_ptr), int(lda), ctypes.c_void_p(B_ptr), int(ldb), float(beta),
                                  ctypes.c_void_p(C_ptr), int(ldc), int(dtype))

    def trmm_raw(self, side, uplo, transA, diag, M, N, alpha, A_ptr, lda, B_ptr, ldb, C_ptr, ldc, dtype) -> int:
        return self.lib.gemm_trmm(self.handle, int(side), int(uplo), int(transA), int(diag), int(M), int(N),
                                  float(alpha), ctypes.c_void_p(A_ptr), int(lda), ctypes.c_void_p(B_ptr), int(ldb),
                                  ctypes.c_void_p(C_ptr), int(ldc), int(dtype))

    def trsm_raw(self, side, uplo, transA, diag, M, N, alpha, A_ptr, lda, B_ptr, ldb, dtype=BF16_BF16) -> int:
        return self.lib.gemm_trsm(self.handle, int(side), int(uplo), int(transA), int(diag), int(M), int(N),
                                  float(alpha), ctypes.c_void_p(A_ptr), int(lda), ctypes.c_void_p(B_ptr), int(ldb),
                                  int(dtype))

    def syrk(self, A, C, uplo=LOWER, trans=0, alpha=1.0, beta=0.0):
        """C <- alpha*op(A)op(A)^T + beta*C on the uplo triangle (bf16 A; bf16 or fp32 C)."""
        self._bind(C)
        N = C.shape[0]
        K = A.shape[0] if trans else A.shape[1]
        st = self.syrk_raw(uplo, trans, N, K, alpha, _ptr(A), _ld(A), beta, _ptr(C), _ld(C),
                           dtype_code("bf16", _c_kind(C)))
        if st != 0:
            raise GemmError("gemm_syrk", st)
        return C

    def syr2k(self, A, B, C, uplo=LOWER, trans=0, alpha=1.0, beta=0.0):
        """C <- alpha*(op(A)op(B)^T + op(B)op(A)^T) + beta*C on the uplo triangle."""
        self._bind(C)
        N = C.shape[0]
        K = A.shape[0] if trans else A.shape[1]
        st = self.syr2k_raw(uplo, trans, N, K, alpha, _ptr(A), _ld(A), _ptr(B), _ld(B), beta, _ptr(C), _ld(C),
                            dtype_code("bf16", _c_kind(C)))
        if st != 0:
            raise GemmError("gemm_syr2k", st)
        return C

    def symm(self, A, B, C, side=LEFT, uplo=LOWER, alpha=1.0, beta=0.0):
        """C <- alpha*S*B (side LEFT) or alpha*B*S (RIGHT) + beta*C, S from A's uplo triangle."""
        self._bind(C)
        M, N = C.shape
        st = self.symm_raw(side, uplo, M, N, alpha, _ptr(A), _ld(A), _ptr(B), _ld(B), beta, _ptr(C), _ld(C),
                           dtype_code("bf16", _c_kind(C)))
        if st != 0:
            raise GemmError("gemm_symm", st)
        return C

    def trmm(self, A, B, C, side=LEFT, uplo=LOWER, transA=0, diag=NON_UNIT, alpha=1.0):
        """C <- alpha*op(T)*B (side LEFT) or alpha*B*op(T) (RIGHT), T from A's uplo triangle."""
        self._bind(C)
        M, N = C.shape
        st = self.trmm_raw(side, uplo, transA, diag, M, N, alpha, _ptr(A), _ld(A), _ptr(B), _ld(B), _ptr(C),
                           _ld(C), dtype_code("bf16", _c_kind(C)))
        if st != 0:
            raise GemmError("gemm_trmm", st)
        return C

    def trsm(self, A, B, side=LEFT, uplo=LOWER, transA=0, diag=NON_UNIT, alpha=1.0):
        """B <- X with op(T) X = alpha*B (side LEFT) or X op(T) = alpha*B (RIGHT), in place; bf16."""
        self._bind(B)
        M, N = B.shape
        st = self.trsm_raw(side, uplo, transA, diag, M, N, alpha, _ptr(A), _ld(A), _ptr(B), _ld(B))
        if st != 0:
            raise GemmError("gemm_trsm", st)
        return B

    def query_policy(self, M, N, K, transA=0, transB=0, dtype=BF16_BF16, A_ptr=0, lda=None,
                     B_ptr=0, ldb=None, C_ptr=0, ldc=None) -> str:
        return query_policy(M, N, K, transA, transB, dtype, A_ptr, lda, B_ptr, ldb, C_ptr, ldc,
                            handle=self.handle)


def query_policy(M, N, K, transA=0, transB=0, dtype=BF16_BF16, A_ptr=0, lda=None, B_ptr=0,
                 ldb=None, C_ptr=0, ldc=None, handle=None) -> str:
    """Name of the policy gemm_run would pick (pure host code; handle may be None)."""
    lib = load_library()
    lda = lda if lda is not None else (M if transA else K)
    ldb = ldb if ldb is not None else (K if transB else N)
    ldc = ldc if ldc is not None else N
    buf = ctypes.create_string_buffer(128)
    st = lib.gemm_query_policy(handle, transA, transB, M, N, K, ctypes.c_void_p(A_ptr), lda,
                               ctypes.c_void_p(B_ptr), ldb, ctypes.c_void_p(C_ptr), ldc, dtype, buf, 128)
    if st != 0:
        raise GemmError("gemm_query_policy", st)
    return buf.value.decode()


def check_args(transA, transB, M, N, K, alpha, A_ptr, lda, B_ptr, ldb, beta, C_ptr, ldc, dtype) -> int:
    lib = load_library()
    return lib.gemm_check_args(transA, transB, M, N, K, alpha, ctypes.c_void_p(A_ptr), lda,
                               ctypes.c_void_p(B_ptr), ldb, beta, ctypes.c_void_p(C_ptr), ldc, dtype)


def run_noalloc_raw(device, stream_ptr, policy, transA, transB, M, N, K, alpha, A_ptr, lda, B_ptr, ldb, beta,
                    C_ptr, ldc, dtype) -> int:
    """gemm_run_noalloc with raw pointers (stream_ptr 0: the default stream); returns the status."""
    lib = load_library()
    pol = None if policy is None else policy.encode()
    return lib.gemm_run_noalloc(int(device), ctypes.c_void_p(stream_ptr or None), pol, int(transA), int(transB),
                                int(M), int(N), int(K), float(alpha), ctypes.c_void_p(A_ptr), int(lda),
                                ctypes.c_void_p(B_ptr), int(ldb), float(beta), ctypes.c_void_p(C_ptr), int(ldc),
                                int(dtype))


def run_noalloc(A, B, C, transA: int = 0, transB: int = 0, alpha: float = 1.0, beta: float = 0.0,
                dtype: Optional[int] = None, policy: Optional[str] = None):
    """gemm_run_noalloc on torch tensors of one device, on torch's current stream there:
    the handle-free call that allocates nothing (its scratch is a static device array)."""
    import torch
    if dtype is None:
        ind = "e4m3" if A.dtype == torch.float8_e4m3fn else "bf16"
        dtype = dtype_code(ind, _c_kind(C))
    M, N = C.shape
    K = A.shape[0] if transA else A.shape[1]
    st = run_noalloc_raw(C.device.index or 0, _current_stream(C.device), policy, transA, transB, M, N, K, alpha,
                         _ptr(A), _ld(A), _ptr(B), _ld(B), beta, _ptr(C), _ld(C), dtype)
    if st != 0:
        raise GemmError("gemm_run_noalloc", st)
