// C-ABI of the GEMM library: handles, argument checks, policy choice and launch.
// The operation and its conventions are documented in include/gemm.h.
#include "gemm.h"

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <atomic>
#include <mutex>
#include <unordered_set>

#include "blas3_internal.h"

using namespace dbgemm;

namespace {

constexpr const char* kVersion = "dbgemm 0.1.0 policy-table 1";

// Device workspace, allocated once per handle at creation: split-K's fp32 partial tiles,
// and the BLAS3 calls' expanded, packed or transposed operands.
constexpr size_t kWorkspaceBytes = (size_t)256 << 20;
// Split-K partials use at most this much of it: the wave-time model's split costs were fitted
// with this bound (a larger one lets it split grids whose reduction costs more than it saves).
constexpr size_t kSplitBytes = (size_t)64 << 20;
// Stream-K hand-off flags, one int per stream-K workgroup; zero between calls (each owner
// clears the flags it waited for).  Kept apart from the workspace, which the BLAS3 calls
// overwrite with operands.
constexpr size_t kFlagBytes = (size_t)64 << 10;

// A policy pinned by name: table index (-1: shape-driven), split-K factor, and stream-K
// (0: off, -1: one stream-K workgroup per CU, > 0: that many).
struct Forced {
  int idx = -1;
  int splits = 1;
  int sk = 0;
};

struct Handle {
  int device = 0;
  int cu_count = 256;
  hipStream_t stream = nullptr;
  Forced forced;
  void* ws = nullptr;      // kWorkspaceBytes on `device`, or null (split-K and stream-K off)
  int* flags = nullptr;    // kFlagBytes on `device`, zeroed, or null (stream-K off)
  uint32_t epoch = 0;      // stream-K call counter (the flag value of the latest call)
  int64_t ws_floats() const { return ws ? (int64_t)(kSplitBytes / sizeof(float)) : 0; }
  int next_epoch() {
    if (++epoch == 0) ++epoch;
    return (int)epoch;
  }
};

// Live handles; a destroyed (or never created) handle is rejected instead of used.
std::mutex g_mu;
std::unordered_set<const void*> g_live;

bool live(gemm_handle_t h) {
  if (!h) return false;
  std::lock_guard<std::mutex> lk(g_mu);
  return g_live.count(h) != 0;
}

bool valid_op(int op) { return op == GEMM_OP_N || op == GEMM_OP_T; }
bool is_mx(int d) { return d == GEMM_MXE4M3_BF16 || d == GEMM_MXE4M3_F32 || d == GEMM_MXE4M3_E4M3; }
bool valid_query_dtype(int d) { return d >= GEMM_BF16_F32 && d <= GEMM_MXE4M3_E4M3; }
bool valid_dtype(int d) { return valid_query_dtype(d) && !is_mx(d); }  // gemm_run
int in_bytes(int d) { return (d == GEMM_BF16_F32 || d == GEMM_BF16_BF16) ? 2 : 1; }
int c_kind(int d) {
  if (d == GEMM_BF16_F32 || d == GEMM_E4M3_F32 || d == GEMM_MXE4M3_F32) return C_F32;
  if (d == GEMM_E4M3_E4M3 || d == GEMM_MXE4M3_E4M3) return C_E4M3;
  return C_BF16;
}
int out_bytes(int d) { return c_kind(d) == C_F32 ? 4 : c_kind(d) == C_E4M3 ? 1 : 2; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

Problem make_problem(int transA, int transB, int64_t M, int64_t N, int64_t K, const void* A,
                     int64_t lda, const void* B, int64_t ldb, const void* C, int64_t ldc,
                     int dtype, const void* sa = nullptr, int64_t ldsa = 4, const void* sb = nullptr,
                     int64_t ldsb = 4) {
  Problem pr;
  pr.transA = transA;
  pr.transB = transB;
  pr.M = M;
  pr.N = N;
  pr.K = K;
  pr.in_fp8 = in_bytes(dtype) == 1;
  pr.c_kind = c_kind(dtype);
  pr.mx = is_mx(dtype);
  pr.mx_words = ((uintptr_t)sa & 3u) == 0 && ((uintptr_t)sb & 3u) == 0 && ldsa % 4 == 0 && ldsb % 4 == 0;
  const int ie = in_bytes(dtype), oe = out_bytes(dtype);
  const int vec = 16 / ie;
  bool ok = aligned16(A) && aligned16(B) && aligned16(C);
  ok = ok && (lda * ie) % 16 == 0 && (ldb * ie) % 16 == 0 && (ldc * oe) % 16 == 0;
  // contiguous extent of each operand in whole 16-byte chunks
  ok = ok && (transA ? M % vec == 0 : K % vec == 0);
  ok = ok && (transB ? K % vec == 0 : N % vec == 0);
  // 32-bit buffer offsets: every operand span, plus one tile of rows of slack for
  // the out-of-range marker, stays below 2^31 bytes
  const double lim = 2147483647.0;
  const double a_rows = (double)(transA ? K : M) + 256.0;
  const double b_rows = (double)(transB ? N : K) + 256.0;
  ok = ok && a_rows * (double)lda * ie < lim && b_rows * (double)ldb * ie < lim;
  // block-scaled operands: the MFMA kernels take A [M][K] and B [N][K] only
  if (pr.mx) ok = ok && transA == 0 && transB == 1;
  pr.fast_ok = ok;
  return pr;
}

}  // namespace

namespace dbgemm {
hipError_t launch_mfma_dma(const Policy& p, const GemmArgs& a, hipStream_t s) {
  hipError_t e = hipErrorInvalidConfiguration;
  switch (a.transA * 2 + a.transB) {
    case 0: (void)(launch_mfma_dma_00_p0(p, a, s, &e) || launch_mfma_dma_00_p1(p, a, s, &e)); break;
    case 1: (void)(launch_mfma_dma_01_p0(p, a, s, &e) || launch_mfma_dma_01_p1(p, a, s, &e)); break;
    case 2: (void)(launch_mfma_dma_10_p0(p, a, s, &e) || launch_mfma_dma_10_p1(p, a, s, &e)); break;
    default: (void)(launch_mfma_dma_11_p0(p, a, s, &e) || launch_mfma_dma_11_p1(p, a, s, &e)); break;
  }
  return e;
}
hipError_t launch_mfma_staged(const Policy& p, const GemmArgs& a, hipStream_t s) {
  switch (a.transA * 2 + a.transB) {
    case 0: return launch_mfma_staged_00(p, a, s);
    case 1: return launch_mfma_staged_01(p, a, s);
    case 2: return launch_mfma_staged_10(p, a, s);
    default: return launch_mfma_staged_11(p, a, s);
  }
}
hipError_t launch_mfma_pp(const Policy& p, const GemmArgs& a, hipStream_t s) {
  switch (a.transA * 2 + a.transB) {
    case 0: return launch_mfma_pp_00(p, a, s);
    case 1: return launch_mfma_pp_01(p, a, s);
    case 2: return launch_mfma_pp_10(p, a, s);
    default: return launch_mfma_pp_11(p, a, s);
  }
}
}  // namespace dbgemm

extern "C" {

const char* gemm_version(void) { return kVersion; }

const char* gemm_status_string(int status) {
  switch (status) {
    case GEMM_STATUS_SUCCESS: return "GEMM_STATUS_SUCCESS";
    case GEMM_STATUS_INVALID_VALUE: return "GEMM_STATUS_INVALID_VALUE";
    case GEMM_STATUS_NOT_SUPPORTED: return "GEMM_STATUS_NOT_SUPPORTED";
    case GEMM_STATUS_NOT_INITIALIZED: return "GEMM_STATUS_NOT_INITIALIZED";
    case GEMM_STATUS_LAUNCH_FAILED: return "GEMM_STATUS_LAUNCH_FAILED";
    case GEMM_STATUS_INTERNAL: return "GEMM_STATUS_INTERNAL";
    default: return "GEMM_STATUS_UNKNOWN";
  }
}

int gemm_policy_count(void) { return policy_count(); }

const char* gemm_policy_name(int index) {
  if (index < 0 || index >= policy_count()) return nullptr;
  return policy_at(index).name;
}

gemm_status_t gemm_check_args(int transA, int transB, int64_t M, int64_t N, int64_t K, float alpha,
                              const void* A, int64_t lda, const void* B, int64_t ldb, float beta,
                              const void* C, int64_t ldc, int dtype) {
  if (!valid_op(transA) || !valid_op(transB) || !valid_dtype(dtype)) return GEMM_STATUS_INVALID_VALUE;
  if (M < 0 || N < 0 || K < 0) return GEMM_STATUS_INVALID_VALUE;
  const int64_t imax = 0x7FFFFFFF;
  if (M > imax || N > imax || K > imax) return GEMM_STATUS_INVALID_VALUE;
  // leading dimensions: at least the stored row length, and at least 1
  const int64_t a_cols = transA ? M : K, b_cols = transB ? K : N;
  if (lda < (a_cols > 1 ? a_cols : 1) || ldb < (b_cols > 1 ? b_cols : 1) || ldc < (N > 1 ? N : 1))
    return GEMM_STATUS_INVALID_VALUE;
  if (!std::isfinite(alpha) || !std::isfinite(beta)) return GEMM_STATUS_NOT_SUPPORTED;
  if (M == 0 || N == 0) return GEMM_STATUS_SUCCESS;
  if (!C) return GEMM_STATUS_INVALID_VALUE;
  if (K > 0 && alpha != 0.f && (!A || !B)) return GEMM_STATUS_INVALID_VALUE;
  return GEMM_STATUS_SUCCESS;
}

gemm_status_t gemm_create(gemm_handle_t* h, int device) {
  if (!h) return GEMM_STATUS_INVALID_VALUE;
  *h = nullptr;
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return GEMM_STATUS_NOT_INITIALIZED;
  }
  if (device < 0 || device >= n) return GEMM_STATUS_INVALID_VALUE;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) {
    (void)hipGetLastError();
    return GEMM_STATUS_INTERNAL;
  }
  Handle* p = new Handle();
  p->device = device;
  p->cu_count = cus > 0 ? cus : 256;
  // The workspace and the flags are optional: without them every call runs unsplit.
  int prev = -1;
  if (hipGetDevice(&prev) == hipSuccess && hipSetDevice(device) == hipSuccess) {
    void* ws = nullptr;
    if (hipMalloc(&ws, kWorkspaceBytes) == hipSuccess) p->ws = ws;
    void* fl = nullptr;
    if (hipMalloc(&fl, kFlagBytes) == hipSuccess) {
      if (hipMemset(fl, 0, kFlagBytes) == hipSuccess && hipDeviceSynchronize() == hipSuccess)
        p->flags = (int*)fl;
      else
        (void)hipFree(fl);
    }
    (void)hipSetDevice(prev);
  }
  (void)hipGetLastError();
  {
    std::lock_guard<std::mutex> lk(g_mu);
    g_live.insert(p);
  }
  *h = reinterpret_cast<gemm_handle_t>(p);
  return GEMM_STATUS_SUCCESS;
}

gemm_status_t gemm_destroy(gemm_handle_t h) {
  if (!h) return GEMM_STATUS_SUCCESS;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_live.erase(h) == 0) return GEMM_STATUS_NOT_INITIALIZED;
  }
  Handle* p = reinterpret_cast<Handle*>(h);
  if (p->ws || p->flags) {
    int prev = -1;
    if (hipGetDevice(&prev) == hipSuccess && hipSetDevice(p->device) == hipSuccess) {
      if (p->ws) (void)hipFree(p->ws);  // waits for the device's work in flight
      if (p->flags) (void)hipFree(p->flags);
      (void)hipSetDevice(prev);
    }
    (void)hipGetLastError();
  }
  delete p;
  return GEMM_STATUS_SUCCESS;
}

gemm_status_t gemm_set_stream(gemm_handle_t h, void* stream) {
  if (!live(h)) return GEMM_STATUS_NOT_INITIALIZED;
  reinterpret_cast<Handle*>(h)->stream = reinterpret_cast<hipStream_t>(stream);
  return GEMM_STATUS_SUCCESS;
}

}  // extern "C"

// A policy name as gemm_set_policy takes it: NULL or "auto" (shape-driven), "<policy>",
// "<policy>+sk<S>" with S in {2, 4, 8, 16} (split-K, ring policies), "<policy>+streamk" or
// "<policy>+streamk<G>" with 1 <= G <= 4096 (stream-K, ping-pong policies).
static gemm_status_t parse_policy(const char* name, Forced* f) {
  *f = Forced{};
  if (!name || std::strcmp(name, "auto") == 0) return GEMM_STATUS_SUCCESS;
  char base[128];
  Forced out;
  const char* plus = std::strchr(name, '+');
  const size_t n = plus ? (size_t)(plus - name) : std::strlen(name);
  if (n == 0 || n >= sizeof(base)) return GEMM_STATUS_INVALID_VALUE;
  std::memcpy(base, name, n);
  base[n] = 0;
  if (plus) {
    char* end = nullptr;
    if (std::strncmp(plus, "+streamk", 8) == 0) {
      out.sk = -1;
      if (plus[8] != 0) {
        const long v = std::strtol(plus + 8, &end, 10);
        if (!end || *end != 0 || v < 1 || v > 4096) return GEMM_STATUS_INVALID_VALUE;
        out.sk = (int)v;
      }
    } else if (std::strncmp(plus, "+sk", 3) == 0) {
      const long v = std::strtol(plus + 3, &end, 10);
      if (!end || *end != 0 || (v != 2 && v != 4 && v != 8 && v != 16)) return GEMM_STATUS_INVALID_VALUE;
      out.splits = (int)v;
    } else {
      return GEMM_STATUS_INVALID_VALUE;
    }
  }
  out.idx = policy_find(base);
  if (out.idx < 0) return GEMM_STATUS_INVALID_VALUE;
  if (out.splits > 1 && policy_at(out.idx).pipe != 1) return GEMM_STATUS_INVALID_VALUE;  // direct-to-LDS only
  if (out.sk != 0 && policy_at(out.idx).pipe != 2) return GEMM_STATUS_INVALID_VALUE;    // ping-pong only
  *f = out;
  return GEMM_STATUS_SUCCESS;
}

// The policy, split-K factor and stream-K plan a call runs with (`flags`: whether stream-K
// flags are available; `extras`: a BLAS3 call, which never splits); false when a forced
// policy cannot serve the call.  Stream-K runs only when forced by name; on a grid of
// whole rounds it runs plain.
static bool choose(const Problem& pr, int cu_count, int64_t ws_floats, bool flags, const Forced& f, bool extras,
                   int* idx, int* sp, StreamK* sk) {
  *sk = StreamK{};
  if (f.idx >= 0) {
    *idx = f.idx;
    *sp = f.splits;
    const Policy& pol = policy_at(*idx);
    if (!policy_serves(pol, pr) || !split_allowed(pol, pr, *sp, ws_floats) || (extras && (*sp != 1 || f.sk != 0)))
      return false;
    if (f.sk != 0) {
      if (!flags) return false;
      *sk = stream_k_plan(pol, pr, cu_count, f.sk > 0 ? f.sk : 0);
      if (sk->tiles > 0 && stream_k_ws_floats(pol, *sk) > ws_floats) return false;
    }
    return true;
  }
  *idx = policy_select(pr, cu_count, extras ? 0 : ws_floats, sp);
  return true;
}

extern "C" {

gemm_status_t gemm_set_policy(gemm_handle_t h, const char* name) {
  if (!live(h)) return GEMM_STATUS_NOT_INITIALIZED;
  Handle* p = reinterpret_cast<Handle*>(h);
  Forced f;
  const gemm_status_t st = parse_policy(name, &f);
  if (st != GEMM_STATUS_SUCCESS) return st;
  p->forced = f;
  return GEMM_STATUS_SUCCESS;
}

gemm_status_t gemm_query_policy(gemm_handle_t h, int transA, int transB, int64_t M, int64_t N,
                                int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                                const void* C, int64_t ldc, int dtype, char* name, size_t len) {
  if (!name || len == 0) return GEMM_STATUS_INVALID_VALUE;
  name[0] = 0;
  if (h && !live(h)) return GEMM_STATUS_NOT_INITIALIZED;
  if (!valid_op(transA) || !valid_op(transB) || !valid_query_dtype(dtype)) return GEMM_STATUS_INVALID_VALUE;
  if (M < 0 || N < 0 || K < 0) return GEMM_STATUS_INVALID_VALUE;
  const Handle* p = reinterpret_cast<const Handle*>(h);
  const Problem pr = make_problem(transA, transB, M, N, K, A, lda, B, ldb, C, ldc, dtype);
  // without a handle, the workspace and flags a new handle would have
  const int64_t wsf = p ? p->ws_floats() : (int64_t)(kSplitBytes / sizeof(float));
  const Forced f = p ? p->forced : Forced{};
  int idx = 0, sp = 1;
  StreamK sk;
  if (!choose(pr, p ? p->cu_count : 256, wsf, p ? p->flags != nullptr : true, f, false, &idx, &sp, &sk))
    return GEMM_STATUS_NOT_SUPPORTED;
  if (sp > 1)
    std::snprintf(name, len, "%s+sk%d", policy_at(idx).name, sp);
  else if (sk.tiles > 0 && f.sk > 0)
    std::snprintf(name, len, "%s+streamk%d", policy_at(idx).name, f.sk);
  else if (sk.tiles > 0)
    std::snprintf(name, len, "%s+streamk", policy_at(idx).name);
  else
    std::snprintf(name, len, "%s", policy_at(idx).name);
  return GEMM_STATUS_SUCCESS;
}

gemm_status_t gemm_lds_probe(gemm_handle_t h, int kind, const uint32_t* offsets, int iters,
                             int workgroups) {
  if (!live(h)) return GEMM_STATUS_NOT_INITIALIZED;
  const int w = lds_probe_width(kind);
  if (w == 0 || !offsets || iters < 1 || iters > (1 << 20) || workgroups < 1 || workgroups > 65536)
    return GEMM_STATUS_INVALID_VALUE;
  LdsProbeOffsets o;
  for (int j = 0; j < 8; ++j)
    for (int l = 0; l < 64; ++l) {
      const uint32_t v = offsets[j * 64 + l];
      if (v % (uint32_t)w != 0 || v > (uint32_t)(kLdsProbeBytes - lds_probe_span(kind))) return GEMM_STATUS_INVALID_VALUE;
      o.off[j][l] = v;
    }
  const Handle* p = reinterpret_cast<const Handle*>(h);
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return GEMM_STATUS_INTERNAL;
  if (cur != p->device && hipSetDevice(p->device) != hipSuccess) return GEMM_STATUS_INTERNAL;
  const hipError_t err = launch_lds_probe(kind, o, iters, workgroups, p->stream);
  if (cur != p->device) (void)hipSetDevice(cur);
  return err == hipSuccess ? GEMM_STATUS_SUCCESS : GEMM_STATUS_LAUNCH_FAILED;
}

gemm_status_t gemm_hw_probe(gemm_handle_t h, int kind, int param, int iters, int workgroups, const void* src,
                            int64_t src_bytes, unsigned long long* cycles) {
  if (!live(h)) return GEMM_STATUS_NOT_INITIALIZED;
  if (kind < 0 || kind > 2 || iters < 1 || iters > (1 << 20) || workgroups < 1 || workgroups > 65536 || !cycles)
    return GEMM_STATUS_INVALID_VALUE;
  if (kind < 2 && param != 0 && param != 1) return GEMM_STATUS_INVALID_VALUE;
  if (kind == 2) {
    const int64_t panel = 256 * kHwProbePitch;
    if (param != 64 && param != 128 && param != 256) return GEMM_STATUS_INVALID_VALUE;
    if (!src || src_bytes < panel || src_bytes % panel != 0 || src_bytes > ((int64_t)1 << 31) ||
        ((uintptr_t)src & 15u) != 0)
      return GEMM_STATUS_INVALID_VALUE;
  }
  const Handle* p = reinterpret_cast<const Handle*>(h);
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return GEMM_STATUS_INTERNAL;
  if (cur != p->device && hipSetDevice(p->device) != hipSuccess) return GEMM_STATUS_INTERNAL;
  const hipError_t err = launch_hw_probe(kind, param, iters, workgroups, src, src_bytes, cycles, p->stream);
  if (cur != p->device) (void)hipSetDevice(cur);
  return err == hipSuccess ? GEMM_STATUS_SUCCESS : GEMM_STATUS_LAUNCH_FAILED;
}

// Enqueues one checked GEMM on `stream` (the device is current).  `f` may pin a policy;
// *unsupported is set when that policy cannot serve the call.  `flags` (or null: no
// stream-K) and `epoch` (non-zero, new for each call) are the stream-K hand-off state.
static hipError_t enqueue_impl(int cu_count, hipStream_t stream, void* ws, int64_t ws_floats, int* flags, int epoch,
                               int transA, int transB,
                               int64_t M, int64_t N, int64_t K, float alpha, const void* A, int64_t lda,
                               const void* B, int64_t ldb, float beta, void* C, int64_t ldc, int dtype,
                               const uint8_t* sa, int64_t ldsa, const uint8_t* sb, int64_t ldsb,
                               const GemmExtras& x, const Forced& f, bool* unsupported) {
  *unsupported = false;
  if (M == 0 || N == 0) return hipSuccess;
  GemmArgs a{};
  a.A = A;
  a.B = B;
  a.C = C;
  a.lda = lda;
  a.ldb = ldb;
  a.ldc = ldc;
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  a.alpha = alpha;
  a.beta = beta;
  a.c_kind = c_kind(dtype);
  a.in_fp8 = in_bytes(dtype) == 1;
  a.transA = transA;
  a.transB = transB;
  a.splits = 1;
  a.mx = is_mx(dtype);
  a.sa = sa;
  a.sb = sb;
  a.ldsa = ldsa;
  a.ldsb = ldsb;
  a.tri = x.tri;
  a.kband = x.kband;
  a.band_off = x.band_off;
  a.dual = x.dual;
  a.A2 = x.A2;
  a.B2 = x.B2;
  a.lda2 = x.lda2;
  a.ldb2 = x.ldb2;
  const bool batched = x.batch_y > 1 || x.batch_z > 1;
  if (batched) {
    a.batch_y = x.batch_y;
    a.batch_z = x.batch_z;
    for (int i = 0; i < 2; ++i) {
      a.bsA[i] = x.bsA[i];
      a.bsB[i] = x.bsB[i];
      a.bsC[i] = x.bsC[i];
    }
  }
  const bool extras = x.tri != TRI_NONE || x.kband != KBAND_NONE || x.dual || batched;

  if (K == 0 || alpha == 0.f) {
    if (batched) {  // the scaling kernel runs one product
      *unsupported = true;
      return hipSuccess;
    }
    return launch_scale(a, stream);
  }
  Problem pr = make_problem(transA, transB, M, N, K, A, lda, B, ldb, C, ldc, dtype, sa, ldsa, sb, ldsb);
  if (extras) {
    pr.blas3 = true;
    pr.square_tiles = x.tri != TRI_NONE;
    pr.kband = x.kband != KBAND_NONE;
    if (x.dual) {  // two products in one sum: the bf16 A [M][K], B [N][K] kernels, equal strides
      const Problem p2 = make_problem(transA, transB, M, N, K, x.A2, x.lda2, x.B2, x.ldb2, C, ldc, dtype);
      pr.fast_ok = pr.fast_ok && p2.fast_ok && x.lda2 == lda && x.ldb2 == ldb && transA == 0 && transB == 1;
    }
  }
  int idx = 0, sp = 1;
  StreamK sk;
  if (!choose(pr, cu_count, ws_floats, flags != nullptr, f, extras, &idx, &sp, &sk)) {
    *unsupported = true;
    return hipSuccess;
  }
  const Policy& pol = policy_at(idx);
  // a batch runs only on the direct-to-LDS kernels, unsplit, with at most a K band (the
  // same band in every product)
  if (batched && (pol.pipe != 1 || sp > 1 || sk.tiles > 0 || x.tri != TRI_NONE || x.dual)) {
    *unsupported = true;
    return hipSuccess;
  }
  if (pol.kind == KIND_SIMT) {
    if ((M + 63) / 64 > 65535) {
      *unsupported = true;
      return hipSuccess;
    }
    return launch_simt(a, stream);
  }
  a.tiles_m = (int)((M + pol.BM - 1) / pol.BM);
  a.tiles_n = (int)((N + pol.BN - 1) / pol.BN);
  a.group = pol.group;
  a.raster_n = pol.raster_n;
  a.xcd = pol.xcd;
  const int64_t batch = (int64_t)(x.batch_y > 1 ? x.batch_y : 1) * (x.batch_z > 1 ? x.batch_z : 1);
  if (x.kband != KBAND_NONE && (int64_t)a.tiles_m * a.tiles_n * batch > cu_count) {
    // longest tiles first in dispatch order (tile_of): the XCDs take runs of four raster
    // positions in turn instead of one contiguous part each, and groups of tile rows (A
    // bands) or columns (B bands) are walked from the long end.  (In a single round every
    // tile starts at once: the order does not matter there, and the per-XCD split keeps
    // the operands' reuse in each L2.)
    a.xcd = pol.xcd > 1 ? -pol.xcd : 1;
    a.raster_n = (x.kband == KBAND_B_LOWER || x.kband == KBAND_B_UPPER) ? 1 : 0;
  }
  a.swizzle = pol.swizzle;
  a.krot = extras ? 0 : pol.krot;
  a.splits = sp;
  a.kt_per_split = (int)split_kt(pol, K, sp);
  if (sp > 1) a.ws = (float*)ws;
  if (sk.tiles > 0) {
    a.sk_dp = sk.dp;
    a.sk_tiles = sk.tiles;
    a.sk_grid = sk.grid;
    a.sk_iters = sk.iters;
    a.ws = (float*)ws;
    a.flags = flags;
    a.epoch = epoch;
  }
  if (pol.pipe == 2) return launch_mfma_pp(pol, a, stream);
  return pol.pipe == 1 ? launch_mfma_dma(pol, a, stream) : launch_mfma_staged(pol, a, stream);
}

// Shared by gemm_run and gemm_run_mx once the arguments are checked.
static gemm_status_t run_checked(Handle* p, int transA, int transB, int64_t M, int64_t N, int64_t K,
                                 float alpha, const void* A, int64_t lda, const void* B, int64_t ldb,
                                 float beta, void* C, int64_t ldc, int dtype, const uint8_t* sa,
                                 int64_t ldsa, const uint8_t* sb, int64_t ldsb) {
  if (M == 0 || N == 0) return GEMM_STATUS_SUCCESS;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return GEMM_STATUS_INTERNAL;
  if (cur != p->device && hipSetDevice(p->device) != hipSuccess) return GEMM_STATUS_INTERNAL;
  bool unsupported = false;
  const hipError_t err = enqueue_impl(p->cu_count, p->stream, p->ws, p->ws_floats(), p->flags, p->next_epoch(),
                                      transA, transB, M, N, K, alpha,
                                      A, lda, B, ldb, beta, C, ldc, dtype, sa, ldsa, sb, ldsb, GemmExtras{},
                                      p->forced, &unsupported);
  if (cur != p->device) (void)hipSetDevice(cur);
  if (unsupported) return GEMM_STATUS_NOT_SUPPORTED;
  if (err != hipSuccess) return GEMM_STATUS_LAUNCH_FAILED;
  return GEMM_STATUS_SUCCESS;
}

}  // extern "C"

namespace dbgemm {
bool handle_view(gemm_handle_t h, HandleView* v) {
  if (!live(h)) return false;
  const Handle* p = reinterpret_cast<const Handle*>(h);
  v->device = p->device;
  v->cu_count = p->cu_count;
  v->stream = p->stream;
  v->ws = p->ws;
  v->ws_bytes = p->ws ? kWorkspaceBytes : 0;
  return true;
}

hipError_t gemm_enqueue(const HandleView& hv, int transA, int transB, int64_t M, int64_t N, int64_t K, float alpha,
                        const void* A, int64_t lda, const void* B, int64_t ldb, float beta, void* C, int64_t ldc,
                        int dtype, const GemmExtras& x) {
  bool unsupported = false;
  // never split: the BLAS3 operations keep their operands in the workspace
  Forced f;
  f.idx = x.policy;
  const hipError_t e = enqueue_impl(hv.cu_count, hv.stream, nullptr, 0, nullptr, 0, transA,
                                    transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, dtype, nullptr, 0, nullptr,
                                    0, x, f, &unsupported);
  return unsupported ? hipErrorInvalidConfiguration : e;
}

bool gemm_fast_ok(int transA, int transB, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                  int64_t ldb, const void* C, int64_t ldc, int dtype) {
  return make_problem(transA, transB, M, N, K, A, lda, B, ldb, C, ldc, dtype).fast_ok;
}
}  // namespace dbgemm

extern "C" {

gemm_status_t gemm_run(gemm_handle_t h, int transA, int transB, int64_t M, int64_t N, int64_t K,
                       float alpha, const void* A, int64_t lda, const void* B, int64_t ldb,
                       float beta, void* C, int64_t ldc, int dtype) {
  if (!live(h)) return GEMM_STATUS_NOT_INITIALIZED;
  const gemm_status_t st = gemm_check_args(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C,
                                           ldc, dtype);
  if (st != GEMM_STATUS_SUCCESS) return st;
  return run_checked(reinterpret_cast<Handle*>(h), transA, transB, M, N, K, alpha, A, lda, B, ldb,
                     beta, C, ldc, dtype, nullptr, 0, nullptr, 0);
}

gemm_status_t gemm_run_mx(gemm_handle_t h, int64_t M, int64_t N, int64_t K, float alpha, const void* A,
                          int64_t lda, const uint8_t* scale_a, int64_t ld_scale_a, const void* B,
                          int64_t ldb, const uint8_t* scale_b, int64_t ld_scale_b, float beta, void* C,
                          int64_t ldc, int dtype) {
  if (!live(h)) return GEMM_STATUS_NOT_INITIALIZED;
  if (!is_mx(dtype)) return GEMM_STATUS_INVALID_VALUE;
  // the operand checks of gemm_run with the E4M3 dtype of the same C type
  const int plain = dtype == GEMM_MXE4M3_F32    ? GEMM_E4M3_F32
                    : dtype == GEMM_MXE4M3_E4M3 ? GEMM_E4M3_E4M3
                                                : GEMM_E4M3_BF16;
  const gemm_status_t st = gemm_check_args(GEMM_OP_N, GEMM_OP_T, M, N, K, alpha, A, lda, B, ldb, beta, C,
                                           ldc, plain);
  if (st != GEMM_STATUS_SUCCESS) return st;
  const int64_t nb = (K + 31) / 32;
  if (ld_scale_a < (nb > 1 ? nb : 1) || ld_scale_b < (nb > 1 ? nb : 1)) return GEMM_STATUS_INVALID_VALUE;
  if (M > 0 && N > 0 && K > 0 && alpha != 0.f && (!scale_a || !scale_b)) return GEMM_STATUS_INVALID_VALUE;
  // 32-bit offsets into the scale arrays
  if ((double)M * (double)ld_scale_a >= 2147483647.0 || (double)N * (double)ld_scale_b >= 2147483647.0)
    return GEMM_STATUS_NOT_SUPPORTED;
  return run_checked(reinterpret_cast<Handle*>(h), GEMM_OP_N, GEMM_OP_T, M, N, K, alpha, A, lda, B,
                     ldb, beta, C, ldc, dtype, scale_a, ld_scale_a, scale_b, ld_scale_b);
}

gemm_status_t gemm_quantize_mx(gemm_handle_t h, int64_t rows, int64_t cols, const void* src, int64_t ld_src,
                               void* dst, int64_t ld_dst, uint8_t* scales, int64_t ld_scales) {
  if (!live(h)) return GEMM_STATUS_NOT_INITIALIZED;
  if (rows < 0 || cols < 0) return GEMM_STATUS_INVALID_VALUE;
  const int64_t nb = (cols + 31) / 32;
  if (ld_src < (cols > 1 ? cols : 1) || ld_dst < (cols > 1 ? cols : 1) || ld_scales < (nb > 1 ? nb : 1))
    return GEMM_STATUS_INVALID_VALUE;
  if (rows == 0 || cols == 0) return GEMM_STATUS_SUCCESS;
  if (!src || !dst || !scales) return GEMM_STATUS_INVALID_VALUE;
  if (cols > kQuantizeMaxCols) return GEMM_STATUS_NOT_SUPPORTED;
  const Handle* p = reinterpret_cast<const Handle*>(h);
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return GEMM_STATUS_INTERNAL;
  if (cur != p->device && hipSetDevice(p->device) != hipSuccess) return GEMM_STATUS_INTERNAL;
  const hipError_t err = launch_quantize_mx(rows, cols, src, ld_src, dst, ld_dst, scales, ld_scales, p->stream);
  if (cur != p->device) (void)hipSetDevice(cur);
  return err == hipSuccess ? GEMM_STATUS_SUCCESS : GEMM_STATUS_LAUNCH_FAILED;
}

}  // extern "C"

// ---- gemm_run_noalloc: the scratch memory of a handle (the split-K and stream-K partials,
// then the stream-K flags) in a device array instead, so that a call allocates nothing.
// The code object's loader places one copy of the array on each device the library runs
// on, zeroed; it stays there until the process ends.  In host code `scratch` names a
// host-side stand-in, not the device address: the address comes from hipGetSymbolAddress,
// once per device, and only that pointer is ever passed to a kernel.
static_assert(GEMM_STATIC_SCRATCH_BYTES >= kSplitBytes, "the partials of any split a handle would choose");
static __device__ __align__(256) float scratch[(GEMM_STATIC_SCRATCH_BYTES + kFlagBytes) / sizeof(float)];

namespace {
constexpr int kMaxStaticDevices = 64;
struct StaticScratch {
  std::once_flag once;
  hipError_t err = hipErrorNotInitialized;
  void* ptr = nullptr;  // device address of `scratch` on this device
  int cu_count = 0;
  std::atomic<uint32_t> epoch{0};  // stream-K call counter
};
StaticScratch g_static[kMaxStaticDevices];
}  // namespace

extern "C" {

gemm_status_t gemm_run_noalloc(int device, void* stream, const char* policy, int transA, int transB, int64_t M,
                               int64_t N, int64_t K, float alpha, const void* A, int64_t lda, const void* B,
                               int64_t ldb, float beta, void* C, int64_t ldc, int dtype) {
  gemm_status_t st = gemm_check_args(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, dtype);
  if (st != GEMM_STATUS_SUCCESS) return st;
  Forced f;
  st = parse_policy(policy, &f);
  if (st != GEMM_STATUS_SUCCESS) return st;
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return GEMM_STATUS_NOT_INITIALIZED;
  }
  if (device < 0 || device >= n || device >= kMaxStaticDevices) return GEMM_STATUS_INVALID_VALUE;
  if (M == 0 || N == 0) return GEMM_STATUS_SUCCESS;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return GEMM_STATUS_INTERNAL;
  if (cur != device && hipSetDevice(device) != hipSuccess) return GEMM_STATUS_INTERNAL;
  StaticScratch& s = g_static[device];
  std::call_once(s.once, [&s, device] {  // with `device` current
    s.err = hipGetSymbolAddress(&s.ptr, HIP_SYMBOL(scratch));
    if (s.err == hipSuccess && hipDeviceGetAttribute(&s.cu_count, hipDeviceAttributeMultiprocessorCount, device) !=
                                   hipSuccess)
      s.err = hipErrorInvalidDevice;
    if (s.err != hipSuccess) (void)hipGetLastError();
  });
  gemm_status_t out = GEMM_STATUS_INTERNAL;
  if (s.err == hipSuccess && s.ptr) {
    bool unsupported = false;
    uint32_t e = ++s.epoch;
    if (e == 0) e = ++s.epoch;
    int* flags = (int*)((char*)s.ptr + GEMM_STATIC_SCRATCH_BYTES);
    const hipError_t err =
        enqueue_impl(s.cu_count > 0 ? s.cu_count : 256, reinterpret_cast<hipStream_t>(stream), s.ptr,
                     (int64_t)(GEMM_STATIC_SCRATCH_BYTES / sizeof(float)), flags, (int)e, transA, transB, M, N, K,
                     alpha, A, lda, B, ldb, beta, C, ldc, dtype, nullptr, 0, nullptr, 0, GemmExtras{}, f,
                     &unsupported);
    out = unsupported ? GEMM_STATUS_NOT_SUPPORTED : err == hipSuccess ? GEMM_STATUS_SUCCESS : GEMM_STATUS_LAUNCH_FAILED;
  }
  if (cur != device) (void)hipSetDevice(cur);
  return out;
}

}  // extern "C"
