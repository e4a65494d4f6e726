"""Benchmark of the dense GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--sweep]
                    [--ablation] [--ladder] [--lds-probe] [--policy NAME] [--workload NAME]
                    [--copy-calibration MiB]

A step is one call C = alpha*A*B + beta*C of the headline workload, 4096^3 bf16
row-major NN with bf16 C (alpha 1, beta 0), on inputs already resident in HBM.
W untimed warmup steps run first; then K steps run back to back between two device
synchronisations, with one pair of HIP events on the kernels' stream around them:
`value` is 2MNK*K over the host wall time of that region, `roofline.achieved` 2MNK over
the event time per step.  A separate pass afterwards times each launch between its own
pair of events (p50/p95).  Prints one JSON line, with the shader clock sampled from a host
thread during the timed region, the device, and (with the CPU baseline) the timed
output's rows checked against the fp64 oracle.

--sweep additionally times every other workload (10 warmup + 50 event-timed calls
each, p50/p95) and prints a Markdown table to stderr; the JSON line is unchanged.
--ablation times every applicable policy on the headline and the E4M3 workloads.
--ladder runs the ablation ladder (one variable per rung: global->LDS path and LDS stages,
LDS->register reads, B layout, swizzle) on three K values and a K x M/N heat map, and
--lds-probe the load-only LDS read microbenchmark, --mx the MXFP8 quantiser and GEMM at
the E4M3 forward shape, --blas3 the BLAS3 family (SYRK, SYR2K, SYMM, TRMM, TRSM) at 4096;
these print to stderr and exit without the JSON line.
--policy / --workload pin the policy or pick another workload for the timed steps
(used for profiling single kernels); the JSON line then names them in `config`.
--copy-calibration N runs only a plain device-to-device copy of N MiB (the known-size
reference that scales the rocprofv3 FETCH_SIZE / WRITE_SIZE counters) and exits.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import gemm_inputs as gi  # noqa: E402

PEAK_TFLOPS = {"bf16": 2516.6, "e4m3": 5033.2}  # 256 CU x 2.4 GHz x 4096 (8192 for fp8) FLOP/clk
HBM_GBS = 8000.0
METRIC = "TFLOP/s and % of MI355X dense MFMA peak, 4096³ bf16 GEMM (1 GPU)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_4096_bf16.md")
# the device code of the headline policy's kernel (the ping-pong kernel and its shared parts)
KERNEL_SOURCES = [os.path.join(ROOT, "dense_blas3_gemm_amd", "csrc", f)
                  for f in ("kernel_pingpong.hip", "policies_pp.inc", "mfma_common.h", "gemm_internal.h")]


def _dev(bits, kind):
    import torch
    if kind == "bf16":
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    if kind == "e4m3":
        return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.float8_e4m3fn).cuda()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.float32)).cuda()


def kernel_hash() -> str:
    """Hash of the headline kernel's sources with their // comments and blank lines removed
    (a change of wording alone keeps counters taken on the code valid)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, encoding="utf-8") as fh:
            for line in fh:
                code = re.sub(r"//.*", "", line).rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def measured_traffic(policy: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel sources and the same policy (else None)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for line in open(TRAFFIC_FILE):
        if line.startswith("traffic:"):
            for kv in line[len("traffic:"):].split():
                k, v = kv.split("=")
                vals[k] = v
    if vals.get("kernel_hash") != kernel_hash() or vals.get("policy") != policy:
        return None
    try:
        return float(vals["fetch_bytes"]) + float(vals["write_bytes"])
    except (KeyError, ValueError):
        return None


def _operands(p: gi.Gemm, data):
    import torch
    A = _dev(data["A"], p.in_dtype)
    B = _dev(data["B"], p.in_dtype)
    if "C" in data:
        C = _dev(data["C"], p.c_dtype)
    else:
        C = torch.zeros((p.M, p.N), dtype=torch.float32 if p.c_dtype == "f32" else torch.bfloat16,
                        device="cuda:0")
    return A, B, C


def time_problem(g, p: gi.Gemm, warmup: int, steps: int, data=None):
    """Event-timed launches: returns dict with wall ms/step, per-launch event durations (ms)
    and the policy name.  Each launch sits between its own pair of HIP events."""
    import torch
    data = data if data is not None else p.make()
    A, B, C = _operands(p, data)
    policy = g.query_policy(p.M, p.N, p.K, p.transA, p.transB, p.dtype_code, A.data_ptr(),
                            A.stride(0), B.data_ptr(), B.stride(0), C.data_ptr(), C.stride(0))
    stream = torch.cuda.current_stream()
    call = lambda: g(A, B, C, transA=p.transA, transB=p.transB, alpha=p.alpha, beta=p.beta,
                     dtype=p.dtype_code)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s, e in ev:
        s.record(stream)
        call()
        e.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    durs = np.array([s.elapsed_time(e) for s, e in ev])
    return {"wall_ms": wall * 1e3 / steps, "event_ms": durs, "policy": policy}


def time_headline(g, p: gi.Gemm, warmup: int, steps: int, data):
    """The bench step loop: W warmup launches, then K launches back to back between two
    device synchronisations, with one pair of HIP events on the kernels' stream around
    the whole timed region (no event between launches).  Returns wall and event ms per
    step, the policy, the output C and the operands (for the per-launch pass)."""
    import torch
    A, B, C = _operands(p, data)
    policy = g.query_policy(p.M, p.N, p.K, p.transA, p.transB, p.dtype_code, A.data_ptr(),
                            A.stride(0), B.data_ptr(), B.stride(0), C.data_ptr(), C.stride(0))
    stream = torch.cuda.current_stream()
    call = lambda: g(A, B, C, transA=p.transA, transB=p.transB, alpha=p.alpha, beta=p.beta,
                     dtype=p.dtype_code)
    for _ in range(warmup):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return {"wall_ms": wall * 1e3 / steps, "event_ms_per_step": e0.elapsed_time(e1) / steps, "policy": policy,
            "C": C}


def _sclk_files(device: int = 0):
    """The sysfs pp_dpm_sclk file of the GPU that HIP calls `device`, found by its PCI
    address (the host may list other GPUs, which this process does not see, before it);
    empty when there is none."""
    import os
    import torch
    try:
        pr = torch.cuda.get_device_properties(device)
        addr = "%04x:%02x:%02x.0" % (pr.pci_domain_id, pr.pci_bus_id, pr.pci_device_id)
    except (AttributeError, RuntimeError, AssertionError):
        return []
    f = os.path.join("/sys/bus/pci/devices", addr, "pp_dpm_sclk")
    return [f] if os.path.exists(f) else []


def gpu_clock_mhz(files=None):
    """Current shader clock (MHz) of the GPU, from its sysfs pp_dpm_sclk (the level marked
    '*'); None where it cannot be read."""
    for f in files if files is not None else _sclk_files():
        try:
            for line in open(f):
                if line.rstrip().endswith("*"):
                    return int(line.split(":")[1].strip().split("Mhz")[0].split("MHz")[0])
        except (OSError, ValueError, IndexError):
            continue
    return None


class ClockSampler:
    """Samples the shader clock from a host thread while the timed region runs (the clock
    read after a synchronisation is the idle one)."""

    def __init__(self, period_s: float = 0.0005):
        import threading
        self.files = _sclk_files()
        self.period = period_s
        self.samples = []
        self._stop = threading.Event()
        self._t = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        while not self._stop.is_set():
            v = gpu_clock_mhz(self.files)
            if v is not None:
                self.samples.append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        if self.files:
            self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self.files:
            self._t.join()

    def summary(self):
        if not self.samples:
            return None
        v = np.array(self.samples)
        return {"samples": int(v.size), "median": int(np.median(v)), "min": int(v.min()), "max": int(v.max()),
                "source": self.files[0]}


def build_info():
    """The build stamp written next to the library (git state at build time), if present."""
    f = os.path.join(ROOT, "dense_blas3_gemm_amd", "build_info.json")
    try:
        return json.load(open(f))
    except (OSError, ValueError):
        return {}


def cpu_baseline(p: gi.Gemm, target_s: float = 8.0):
    """The fp64 oracle on a bounded sample of output rows of the same workload."""
    import oracle
    threads = oracle.default_threads()
    data = p.make()
    calib = list(range(0, p.M, max(1, p.M // 16)))[:16]
    t0 = time.perf_counter()
    oracle.gemm_problem(p, data, rows=calib, with_abs=False, threads=threads)
    per_row = (time.perf_counter() - t0) / len(calib)
    nrows = int(max(len(calib), min(p.M, target_s / max(per_row, 1e-9))))
    rows = np.linspace(0, p.M - 1, nrows).round().astype(np.int64)
    t0 = time.perf_counter()
    oracle.gemm_problem(p, data, rows=rows, with_abs=False, threads=threads)
    dt = time.perf_counter() - t0
    flops = 2.0 * len(rows) * p.N * p.K
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(rows)} of {p.M} output rows of {p.name} (fp64 triple loop, "
                      f"{flops / 1e9:.1f} GFLOP in {dt:.1f} s)"}


def parity_sample(p: gi.Gemm, data, C_dev, nrows: int = 32):
    """The timed output on rows spread over every 256-row tile against the fp64 oracle (the
    CPU-baseline leg): elements past the stated bf16 bound (2^-8 |R| + 1e-6), past the bound
    with the probabilistic fp32 accumulation term (2^-24 sqrt(K) sum|a b|), the largest
    error / bound and the relative Frobenius error of those rows."""
    import oracle
    import torch
    rows = np.unique(np.linspace(0, p.M - 1, nrows).round().astype(np.int64))
    R, S = oracle.gemm_problem(p, data, rows=rows, with_abs=True, threads=oracle.default_threads())
    C = C_dev.detach()[torch.as_tensor(rows, device=C_dev.device)].float().cpu().numpy().astype(np.float64)
    err = np.abs(C - R)
    literal = 2.0 ** -8 * np.abs(R) + 1e-6 if p.c_dtype == "bf16" else 2.0 ** -23 * np.abs(R) + 1e-6
    bound = literal + 2.0 ** -24 * np.sqrt(p.K) * S
    return {"rows": int(len(rows)), "elements": int(err.size),
            "n_outside_literal_bound": int((err > literal).sum()),
            "n_outside_bound": int((err > bound).sum()),
            "max_err_over_bound": float((err / bound).max()),
            "frob_rel": float(np.linalg.norm(C - R) / np.linalg.norm(R)),
            "finite": bool(np.isfinite(C).all())}


def sweep(g, warmup: int = 10, steps: int = 50):
    rows = []
    probs = [gi.SMALL_256, gi.SQUARE_4096] + gi.SWEEP + [gi.PROJ_DX, gi.PROJ_DW, gi.FP8_FWD]
    for p in probs:
        r = time_problem(g, p, warmup, steps)
        p50, p95 = np.percentile(r["event_ms"], [50, 95])
        tf = p.flops / (p50 * 1e-3) / 1e12
        peak = PEAK_TFLOPS[p.in_dtype]
        gbs = p.algorithmic_bytes / (p50 * 1e-3) / 1e9
        rows.append((p.name, p.M, p.N, p.K, r["policy"], p50 * 1e3, p95 * 1e3, tf, 100 * tf / peak, gbs))
    print("| workload | M | N | K | policy | p50 us | p95 us | TFLOP/s | % peak | alg. GB/s |", file=sys.stderr)
    print("|---|---|---|---|---|---|---|---|---|---|", file=sys.stderr)
    for r in rows:
        print(f"| {r[0]} | {r[1]} | {r[2]} | {r[3]} | {r[4]} | {r[5]:.1f} | {r[6]:.1f} | {r[7]:.1f} | "
              f"{r[8]:.1f} | {r[9]:.0f} |", file=sys.stderr)
    return rows


def ablation(g, p: gi.Gemm, warmup: int = 10, steps: int = 50):
    """Times every policy of the table that can serve workload p (one variable per row:
    tile shape, waves, MFMA block, LDS swizzle, XCD remap, E4M3 widening)."""
    import dense_blas3_gemm_amd as d
    data = p.make()
    rows = []
    for name in d.policies():
        if name == "simt_generic" and p.flops > 2e10:
            continue
        want = "e4m3" if p.in_dtype == "e4m3" else "bf16_"
        if not (name.startswith(want) or name == "simt_generic"):
            continue
        g.set_policy(name)
        try:
            r = time_problem(g, p, warmup, steps, data=data)
        finally:
            g.set_policy(None)
        p50, p95 = np.percentile(r["event_ms"], [50, 95])
        tf = p.flops / (p50 * 1e-3) / 1e12
        rows.append((name, p50 * 1e3, p95 * 1e3, tf, 100 * tf / PEAK_TFLOPS[p.in_dtype]))
    print(f"ablation on {p.name}:", file=sys.stderr)
    print("| policy | p50 us | p95 us | TFLOP/s | % peak |", file=sys.stderr)
    print("|---|---|---|---|---|", file=sys.stderr)
    for r in rows:
        print(f"| {r[0]} | {r[1]:.1f} | {r[2]:.1f} | {r[3]:.1f} | {r[4]:.1f} |", file=sys.stderr)
    return rows


# The ablation ladder ("cp.async / ldmatrix ablation -- initial plan", sections 2-4) at a
# fixed 128x128x64 tile, 8 waves, 16x16x32 MFMA.  Global -> LDS rungs in the corrected
# order (section 2.3, first pitfall: a second buffer before the asynchronous path):
# register-staged loads with two LDS stages, then direct-to-LDS loads with two, three and
# four stages.  LDS -> register rungs on the last of them: element-wise reads, the
# layout most favourable to plain reads (B stored K-contiguous), transposing reads.
LADDER = [
    ("B0", "global -> VGPR -> ds_write, 2 LDS stages", "bf16_m128n128k64_w2x4_mt16_s2", 0),
    ("B1", "direct-to-LDS loads, 2 stages", "bf16_dma_m128n128k64_w2x4_mt16_s2", 0),
    ("B2", "direct-to-LDS loads, 3 stages", "bf16_dma_m128n128k64_w2x4_mt16_s3", 0),
    ("B3", "direct-to-LDS loads, 4 stages", "bf16_dma_m128n128k64_w2x4_mt16_s4", 0),
    ("A1", "B3, B read one element at a time (ds_read_u16)", "bf16_dma_m128n128k64_w2x4_mt16_s4_rd0", 0),
    ("A2", "B3, B stored K-contiguous (NT): plain ds_read_b128", "bf16_dma_m128n128k64_w2x4_mt16_s4", 1),
    ("A3", "B3, B read with ds_read_b64_tr_b16 (NN)", "bf16_dma_m128n128k64_w2x4_mt16_s4", 0),
    ("S0", "B3 without the LDS xor swizzle", "bf16_dma_m128n128k64_w2x4_mt16_s4_noswz", 0),
    ("S1", "B3 with the swizzle", "bf16_dma_m128n128k64_w2x4_mt16_s4", 0),
    ("P0", "256x256 tile, global -> VGPR -> ds_write", "bf16_m256n256k64_w2x4_mt16_s2", 0),
    ("P1", "256x256 tile, direct-to-LDS (the 4096^3 default)", "bf16_dma_m256n256k64_w2x4_mt16_s2", 0),
]


def ladder(g, rounds: int = 3, warmup: int = 3, steps: int = 20, heatmap: bool = True, quick: bool = False):
    """Each rung on K = 256, 4096, 8192 at M = N = 4096 (section 2.3, third pitfall: a
    single shape misleads), rounds interleaved; Markdown to stderr.  quick: 4096^3 only,
    one round, in LADDER order (for counter passes: 23 GEMM dispatches per rung)."""
    import dataclasses
    shapes = [gi.BY_NAME["sweep_mn4096_k256"], gi.SQUARE_4096, gi.BY_NAME["sweep_mn4096_k8192"]]
    if quick:
        shapes, rounds, heatmap = [gi.SQUARE_4096], 1, False
    res = {}
    for p in shapes:
        datas = {tb: dataclasses.replace(p, transB=tb).make() for tb in (0, 1)}
        times = {r[0]: [] for r in LADDER}
        for _ in range(rounds):
            for rung, _desc, pol, tb in LADDER:
                q = dataclasses.replace(p, transB=tb)
                g.set_policy(pol)
                try:
                    t = time_problem(g, q, warmup, steps, data=datas[tb])
                finally:
                    g.set_policy(None)
                times[rung].append(float(np.percentile(t["event_ms"], 50)))
        for rung in times:
            ms = float(np.median(times[rung]))
            res[(rung, p.name)] = (ms * 1e3, p.flops / (ms * 1e-3) / 1e12)
    out = sys.stderr
    print("ablation ladder (p50 of event-timed calls, median over rounds; delta vs the rung above)", file=out)
    hdr = "| rung | change | policy | " + " | ".join(f"{p.name} TFLOP/s | delta" for p in shapes) + " |"
    print(hdr, file=out)
    print("|" + "---|" * (3 + 2 * len(shapes)), file=out)
    prev = None
    for rung, desc, pol, tb in LADDER:
        cells = []
        for p in shapes:
            tf = res[(rung, p.name)][1]
            base = None
            if prev is not None and rung[0] == prev[0]:
                base = res[(prev, p.name)][1]
            cells.append(f"{tf:.1f} | " + (f"{100 * (tf / base - 1):+.1f}%" if base else ""))
        print(f"| {rung} | {desc} | {pol}{' (NT)' if tb else ''} | " + " | ".join(cells) + " |", file=out)
        prev = rung
    if heatmap:
        print("heat map (TFLOP/s, p50 of 20 event-timed calls): rows K, columns M = N", file=out)
        ks = sorted({w.K for w in gi.SWEEP})
        mns = sorted({w.M for w in gi.SWEEP})
        for label, pol in [("B0", LADDER[0][2]), ("B3", LADDER[3][2]), ("P1", LADDER[-1][2]), ("auto", None)]:
            print(f"{label} ({pol or 'shape-driven policy'})", file=out)
            print("| K | " + " | ".join(f"M=N={m}" for m in mns) + " |", file=out)
            print("|---|" + "---|" * len(mns), file=out)
            for k in ks:
                row = []
                for m in mns:
                    w = next(x for x in gi.SWEEP if x.K == k and x.M == m)
                    g.set_policy(pol)
                    try:
                        t = time_problem(g, w, warmup, steps)
                    finally:
                        g.set_policy(None)
                    row.append(f"{w.flops / (float(np.percentile(t['event_ms'], 50)) * 1e-3) / 1e12:.1f}")
                print(f"| {k} | " + " | ".join(row) + " |", file=out)
    return res


def lds_probe_patterns():
    """Per-lane LDS byte offsets of the kernels' 16x16x32 fragment reads (8 read slots).
    K-contiguous A fragments of a 128-byte-row tile (ds_read_b128, one read per fragment);
    M/N-contiguous B fragments of a 256-byte-row tile (128 wide): transposing reads (two
    per fragment) or one element per read (eight per fragment); with and without the row
    xor."""
    def kc(r, swz):
        return ((r >> 1) & 7) if swz else 0

    def mn(k, swz):
        return ((((k & 3) << 1) | ((k >> 3) & 1)) << 1) & 15 if swz else 0
    pats = []
    for swz in (1, 0):
        b128 = [[(16 * j + l % 16) * 128 + (((l // 16) ^ kc(16 * j + l % 16, swz)) & 7) * 16 for l in range(64)]
                for j in range(8)]
        tr = []
        for j in range(8):
            x0, h = 16 * (j // 2), j % 2
            row = []
            for l in range(64):
                g_, s_ = l >> 4, l & 15
                x, k = x0 + (s_ % 4) * 4, g_ * 8 + h * 4 + s_ // 4
                xb = 2 * x
                row.append(k * 256 + ((((xb >> 4) ^ mn(k, swz)) << 4) | (xb & 15)))
            tr.append(row)
        u16 = []
        for e in range(8):
            row = []
            for l in range(64):
                x, k = l % 16, (l // 16) * 8 + e
                xb = 2 * x
                row.append(k * 256 + ((((xb >> 4) ^ mn(k, swz)) << 4) | (xb & 15)))
            u16.append(row)
        tag = "swizzled" if swz else "plain"
        pats += [(f"A fragment, ds_read_b128, {tag}", 0, b128, 8),
                 (f"B fragment, ds_read_b64_tr_b16, {tag}", 1, tr, 4),
                 (f"B fragment, ds_read_u16 x8, {tag}", 2, u16, 1)]
    # E4M3 K-contiguous fragments of a 128-byte-row tile (8 bytes per lane: row l % 16, K
    # bytes 8 (l / 16) of the step's 32, chunk xor (r >> 1) & 7): one ds_read_b64 each, or
    # two fragments 16 rows apart in one ds_read2st64_b64 (the pairing a compiler makes of
    # such reads when it sees their constant distance)
    def e8(r, kb):
        return r * 128 + ((((kb >> 4) ^ ((r >> 1) & 7)) << 4) | (kb & 15))
    b64 = [[e8(16 * j + l % 16, (l // 16) * 8) for l in range(64)] for j in range(8)]
    pair = [[e8(32 * j + l % 16, (l // 16) * 8) for l in range(64)] for j in range(8)]
    pats += [("E4M3 K-contiguous fragment, ds_read_b64", 3, b64, 8),
             ("E4M3 K-contiguous fragments 16 rows apart, ds_read2st64_b64", 5, pair, 16)]
    return pats


def lds_probe(g, iters: int = 512, workgroups: int = 1024, reps: int = 5):
    """The load-only LDS microbenchmark (section 2.3, second pitfall): ns per 16x16x32
    fragment per CU for each read form, Markdown to stderr."""
    import torch
    stream = torch.cuda.current_stream()
    out = sys.stderr
    print("LDS read microbenchmark: 1024 workgroups x 4 waves, 512 iterations x 8 reads per lane", file=out)
    print("| read | reads per fragment | us per launch (p50) | ns per fragment per CU | fragment bytes per CU per ns |",
          file=out)
    print("|---|---|---|---|---|", file=out)
    rows = []
    for name, kind, offs, frags in lds_probe_patterns():
        ev = []
        for _ in range(reps + 1):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            g.lds_probe(kind, offs, iters, workgroups, stream_ptr=stream.cuda_stream)
            b.record(stream)
            ev.append((a, b))
        torch.cuda.synchronize()
        us = float(np.median([a.elapsed_time(b) for a, b in ev[1:]])) * 1e3
        total_frags = workgroups * 4 * iters * frags
        ns_per_frag_cu = us * 1e3 * 256 / total_frags
        per_frag = 8 / frags
        fbytes = 512 if kind in (3, 5) else 1024  # an E4M3 fragment is 64 lanes x 8 bytes
        rows.append((name, per_frag, us, ns_per_frag_cu))
        print(f"| {name} | {per_frag:g} | {us:.1f} | {ns_per_frag_cu:.2f} | {fbytes / ns_per_frag_cu:.1f} |",
              file=out)
    return rows


def hw_probes(g, reps: int = 5):
    """The hardware microbenchmarks (gemm_hw_probe): MFMA issue interval and the shader clock
    under full-chip and light load, and the direct-to-LDS copy rate per CU, Markdown to
    stderr.  Returns the rows."""
    import torch
    stream = torch.cuda.current_stream()
    out = sys.stderr
    src = torch.randint(-2 ** 15, 2 ** 15, ((64 << 20) // 2,), dtype=torch.int16, device="cuda:0")

    def run(kind, param, iters, wgs):
        cyc = torch.zeros(wgs, dtype=torch.int64, device="cuda:0")
        g.hw_probe(kind, param, iters, wgs, src if kind == 2 else None, cyc)  # warm-up
        torch.cuda.synchronize()
        us, cycles = [], []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            g.hw_probe(kind, param, iters, wgs, src if kind == 2 else None, cyc)
            b.record(stream)
            b.synchronize()
            us.append(a.elapsed_time(b) * 1e3)
            cycles.append(float(cyc.double().median().item()))
        return float(np.median(us)), float(np.median(cycles))

    rows = []
    print("MFMA issue (8 waves per workgroup, 2 per SIMD; 2048 clusters per wave):", file=out)
    print("| MFMA | schedule | workgroups | us | shader GHz (cycles / time) | cycles per MFMA per SIMD | TFLOP/s |",
          file=out)
    print("|---|---|---|---|---|---|---|", file=out)
    for kind, name, per, flop in ((0, "16x16x32 bf16", 32, 16384), (1, "32x32x16 bf16", 16, 32768)):
        for param, sched in ((0, "all 8 waves"), (1, "two groups in turn")):
            for wgs in (256, 32):
                iters = 2048
                us, cyc = run(kind, param, iters, wgs)
                ghz = cyc / (us * 1e3)
                per_mfma = cyc / (2 * iters * per)
                tf = wgs * 8 * iters * per * flop / (us * 1e-6) / 1e12
                rows.append(("mfma", name, sched, wgs, us, ghz, per_mfma, tf))
                print(f"| {name} | {sched} | {wgs} | {us:.1f} | {ghz:.3f} | {per_mfma:.2f} | {tf:.0f} |", file=out)
    print("Direct-to-LDS copy (256 workgroups of 8 waves, 256-row tiles, rows 8192 bytes apart):", file=out)
    print("| row bytes | us | shader GHz | bytes per clock per CU | TB/s (chip) |", file=out)
    print("|---|---|---|---|---|", file=out)
    for rb in (64, 128, 256):
        iters = 8192 * 64 // rb
        us, cyc = run(2, rb, iters, 256)
        per_clk = iters * 256 * rb / cyc
        tbs = 256 * iters * 256 * rb / (us * 1e-6) / 1e12
        rows.append(("copy", rb, us, cyc / (us * 1e3), per_clk, tbs))
        print(f"| {rb} | {us:.1f} | {cyc / (us * 1e3):.3f} | {per_clk:.1f} | {tbs:.1f} |", file=out)
    return rows


def mx_bench(g, warmup: int = 5, steps: int = 30):
    """Block-scaled E4M3 at the E4M3 forward shape: the quantiser on a bf16 [16384][5120]
    matrix (HBM bytes/s) and gemm_run_mx 16384 x 5120 x 5120 (TFLOP/s).  Returns a dict."""
    import torch
    M, N, K = gi.MX_FWD_SHAPE
    stream = torch.cuda.current_stream()
    src = _dev(gi.bf16_normal((M, K), 0), "bf16")
    dst = torch.empty((M, K), dtype=torch.uint8, device="cuda:0")
    sc = torch.empty((M, (K + 31) // 32), dtype=torch.uint8, device="cuda:0")

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in ev])
    q_ms = timed(lambda: g.quantize_mx(src, dst, sc))
    q_bytes = M * K * 2 + M * K + M * ((K + 31) // 32)
    d = gi.mx_operands(M, N, K, seeds=(0, 1, 2, 3))
    A, B = _dev(d["A"], "e4m3"), _dev(d["B"], "e4m3")
    SA = torch.from_numpy(d["SA"]).cuda()
    SB = torch.from_numpy(d["SB"]).cuda()
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    g_ms = timed(lambda: g.run_mx(A, SA, B, SB, C))
    g.set_policy("mxe4m3native_dma_m256n256k128_w2x4_mt32_s2")  # the scaled f8f6f4 MFMA
    try:
        n_ms = timed(lambda: g.run_mx(A, SA, B, SB, C))
        g.set_policy("mxe4m3_m128n128k64_w2x4_mt16_s2")  # widened with the scale while staged to LDS
        s_ms = timed(lambda: g.run_mx(A, SA, B, SB, C))
    finally:
        g.set_policy(None)
    flops = 2.0 * M * N * K
    qp50, gp50 = float(np.percentile(q_ms, 50)), float(np.percentile(g_ms, 50))
    np50 = float(np.percentile(n_ms, 50))
    out = {"quantize_us_p50": round(qp50 * 1e3, 1), "quantize_GBps": round(q_bytes / (qp50 * 1e-3) / 1e9, 1),
           "quantize_frac_hbm": round(q_bytes / (qp50 * 1e-3) / 1e9 / HBM_GBS, 3),
           "gemm_us_p50": round(gp50 * 1e3, 1), "gemm_tflops": round(flops / (gp50 * 1e-3) / 1e12, 1),
           "gemm_frac_bf16_peak": round(flops / (gp50 * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"], 4),
           "policy": g.query_policy(M, N, K, 0, 1, 4),
           "native_us_p50": round(np50 * 1e3, 1), "native_tflops": round(flops / (np50 * 1e-3) / 1e12, 1),
           "native_frac_fp8_peak": round(flops / (np50 * 1e-3) / 1e12 / PEAK_TFLOPS["e4m3"], 4),
           "staged_us_p50": round(float(np.percentile(s_ms, 50)) * 1e3, 1)}
    print("MXFP8 at 16384 x 5120 x 5120: " + json.dumps(out), file=sys.stderr)
    return out


# The BLAS3 family at 4096 (bf16 operands, fp32 accumulation, bf16 results): the
# operator set of "BLASMp development notes" on one GPU.  FLOP counts are the standard
# ones of each operation's useful work (the triangle only for SYRK / SYR2K, the
# triangular half for TRMM / TRSM): SYRK N(N+1)K, SYR2K 2N(N+1)K, SYMM 2M^2N (left),
# TRMM M^2N, TRSM M^2N (left).
BLAS3_N = 4096


def blas3_bench(g, warmup: int = 5, steps: int = 30, n: int = BLAS3_N, cpu: bool = True):
    """Event-timed p50 of each BLAS3 call at n x n (left side, lower, no transpose,
    non-unit diagonal); returns a list of dicts and prints a Markdown table to stderr."""
    import torch
    stream = torch.cuda.current_stream()
    A = _dev(gi.bf16_uniform((n, n), 0), "bf16")
    B = _dev(gi.bf16_uniform((n, n), 1), "bf16")
    Tm = _dev(gi.bf16_triangular(n, gi.LOWER, 2), "bf16")
    Tu = _dev(gi.bf16_triangular(n, gi.UPPER, 4), "bf16")
    Sm = _dev(gi.bf16_symmetric_stored(n, gi.LOWER, 3), "bf16")
    C = torch.zeros((n, n), dtype=torch.bfloat16, device="cuda:0")
    X = torch.empty_like(B)

    def timed(fn, pre=None):
        for _ in range(warmup):
            if pre:
                pre()
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in ev:
            if pre:
                pre()
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in ev])
    nn = float(n)
    ops = [
        ("gemm (context)", 2 * nn ** 3, lambda: g(A, B, C), None),
        ("syrk lower, N", nn * (nn + 1) * nn, lambda: g.syrk(A, C, uplo=0, trans=0), None),
        ("syr2k lower, N", 2 * nn * (nn + 1) * nn, lambda: g.syr2k(A, B, C, uplo=0, trans=0), None),
        ("symm left lower", 2 * nn ** 3, lambda: g.symm(Sm, B, C, side=0, uplo=0), None),
        ("trmm left lower N", nn ** 3, lambda: g.trmm(Tm, B, C, side=0, uplo=0, transA=0), None),
        # the solve overwrites its right-hand side: a fresh copy goes in before each call,
        # outside the event pair
        ("trsm left lower N", nn ** 3, lambda: g.trsm(Tm, X, side=0, uplo=0, transA=0), lambda: X.copy_(B)),
        # the other layouts: A read transposed (TN), the triangle on the right, upper, transposed
        ("syrk lower, T", nn * (nn + 1) * nn, lambda: g.syrk(A, C, uplo=0, trans=1), None),
        ("trmm right upper T", nn ** 3, lambda: g.trmm(Tu, B, C, side=1, uplo=1, transA=1), None),
        ("trsm right upper T", nn ** 3, lambda: g.trsm(Tu, X, side=1, uplo=1, transA=1), lambda: X.copy_(B)),
    ]
    rows = []
    for name, flops, fn, pre in ops:
        ms = timed(fn, pre)
        p50, p95 = float(np.percentile(ms, 50)), float(np.percentile(ms, 95))
        tf = flops / (p50 * 1e-3) / 1e12
        rows.append({"op": name, "n": n, "us_p50": round(p50 * 1e3, 1), "us_p95": round(p95 * 1e3, 1),
                     "tflops": round(tf, 1), "frac_bf16_peak": round(tf / PEAK_TFLOPS["bf16"], 4)})
    if cpu:
        for r, c in zip(rows, blas3_cpu_baseline()):
            r["cpu_oracle_gflops"] = c
    print(f"BLAS3 family at {n} (bf16 in, fp32 accumulate, bf16 out; p50 of {steps} event-timed calls)",
          file=sys.stderr)
    import oracle
    print(f"| op | us p50 | us p95 | TFLOP/s | frac of bf16 peak | oracle GFLOP/s (host, n = 1024, "
          f"{oracle.default_threads()} threads) |", file=sys.stderr)
    print("|---|---|---|---|---|---|", file=sys.stderr)
    for r in rows:
        print(f"| {r['op']} | {r['us_p50']} | {r['us_p95']} | {r['tflops']} | {r['frac_bf16_peak']} | "
              f"{r.get('cpu_oracle_gflops', '-')} |", file=sys.stderr)
    print("blas3: " + json.dumps(rows), file=sys.stderr)
    return rows


def blas3_cpu_baseline(n: int = 1024):
    """The oracle as it stands (float64 numpy, oracle/blas3.py; the C oracle for the plain
    GEMM), timed on the host for each operation of blas3_bench at n = 1024 instead of 4096
    (a bounded sample of the same workload: each takes under a few seconds).  Returns
    GFLOP/s in blas3_bench's order, counting the same useful FLOPs."""
    import oracle
    from oracle import blas3 as ob
    A, B = gi.bf16_uniform((n, n), 0), gi.bf16_uniform((n, n), 1)
    Tm, Sm = gi.bf16_triangular(n, gi.LOWER, 2), gi.bf16_symmetric_stored(n, gi.LOWER, 3)
    Tu = gi.bf16_triangular(n, gi.UPPER, 4)
    nn = float(n)
    calls = [
        (2 * nn ** 3, lambda: oracle.gemm(0, 0, n, n, n, 1.0, A, n, B, n, 0.0, None, n, oracle.IN_BF16,
                                          oracle.C_BF16, with_abs=False)),
        (nn * (nn + 1) * nn, lambda: ob.syrk(0, 0, n, n, 1.0, A, 0.0, None, oracle.C_BF16)),
        (2 * nn * (nn + 1) * nn, lambda: ob.syr2k(0, 0, n, n, 1.0, A, B, 0.0, None, oracle.C_BF16)),
        (2 * nn ** 3, lambda: ob.symm(0, 0, n, n, 1.0, Sm, B, 0.0, None, oracle.C_BF16)),
        (nn ** 3, lambda: ob.trmm(0, 0, 0, 0, n, n, 1.0, Tm, B)),
        (nn ** 3, lambda: ob.trsm(0, 0, 0, 0, n, n, 1.0, Tm, B)),
        (nn * (nn + 1) * nn, lambda: ob.syrk(0, 1, n, n, 1.0, A, 0.0, None, oracle.C_BF16)),
        (nn ** 3, lambda: ob.trmm(1, 1, 1, 0, n, n, 1.0, Tu, B)),
        (nn ** 3, lambda: ob.trsm(1, 1, 1, 0, n, n, 1.0, Tu, B)),
    ]
    out = []
    for flops, fn in calls:
        t0 = time.perf_counter()
        fn()
        out.append(round(flops / (time.perf_counter() - t0) / 1e9, 2))
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--ablation", action="store_true",
                    help="time every applicable policy on the 4096^3 bf16 and the E4M3 workloads")
    ap.add_argument("--ladder", action="store_true", help="run the ablation ladder and exit")
    ap.add_argument("--no-heatmap", action="store_true", help="with --ladder: skip the K x M/N heat map")
    ap.add_argument("--ladder-quick", action="store_true",
                    help="with --ladder: 4096^3 only, one round (3 + 20 calls per rung, in order)")
    ap.add_argument("--lds-probe", action="store_true", help="run the LDS read microbenchmark and exit")
    ap.add_argument("--hw-probes", action="store_true",
                    help="run the MFMA-issue and direct-to-LDS copy microbenchmarks and exit")
    ap.add_argument("--mx", action="store_true", help="time the MXFP8 quantiser and GEMM and exit")
    ap.add_argument("--blas3", action="store_true", help="time the BLAS3 family at 4096 and exit")
    ap.add_argument("--policy", default=None, help="force a named policy for the timed steps")
    ap.add_argument("--workload", default=gi.SQUARE_4096.name, choices=sorted(gi.BY_NAME))
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MiB")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this GEMM engine runs on a single MI355X "
              "(no sharding or collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import dense_blas3_gemm_amd as d

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": args.warmup + args.steps}))
        return
    g = d.Gemm(0)
    if args.ladder or args.lds_probe or args.mx or args.blas3 or args.hw_probes:
        if args.hw_probes:
            hw_probes(g)
        if args.blas3:
            blas3_bench(g, cpu=not args.no_cpu_baseline)
        if args.mx:
            mx_bench(g)
        if args.lds_probe:
            lds_probe(g)
        if args.ladder:
            ladder(g, heatmap=not args.no_heatmap, quick=args.ladder_quick)
        g.close()
        return
    p = gi.BY_NAME[args.workload]
    data = p.make()
    if args.policy:
        g.set_policy(args.policy)
    with ClockSampler() as clk:
        r = time_headline(g, p, args.warmup, args.steps, data)
    # per-launch distribution: a separate pass after the timed region, each launch between
    # its own pair of events
    dist = time_problem(g, p, 0, args.steps, data=data)["event_ms"]
    g.set_policy(None)
    ms = r["wall_ms"]
    value = p.flops / (ms * 1e-3) / 1e12
    ev_ms = r["event_ms_per_step"]
    achieved = p.flops / (ev_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[p.in_dtype]
    import torch
    props = torch.cuda.get_device_properties(0)
    out = {
        "metric": METRIC if p is gi.SQUARE_4096 else f"TFLOP/s and % of MI355X dense MFMA peak, {p.name} (1 GPU)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.in_dtype,
        "data": "synthetic",
        "pct_of_peak": round(100.0 * value / peak, 2),
        "config": {"workload": p.name, "M": p.M, "N": p.N, "K": p.K,
                   "layout": "row-major " + "NT"[p.transA] + "NT"[p.transB],
                   "inputs": f"{p.in_dtype} {p.dist} seeds {p.seeds[0]}/{p.seeds[1]}", "c_dtype": p.c_dtype,
                   "accumulate": "f32", "alpha": p.alpha, "beta": p.beta, "policy": r["policy"]},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic(r["policy"]) if p is gi.SQUARE_4096 and not args.policy else None,
                     "kernel_us_timed_region": round(ev_ms * 1e3, 2),
                     "launch_us_p50": round(float(np.percentile(dist, 50)) * 1e3, 2),
                     "launch_us_p95": round(float(np.percentile(dist, 95)) * 1e3, 2)},
        "device": {"name": props.name, "cus": props.multi_processor_count, "hip": torch.version.hip,
                   "sclk_mhz_during_timed_region": clk.summary(), "build": build_info()},
    }
    C_out = r["C"]
    if args.sweep:
        sweep(g)
    if args.ablation:
        ablation(g, p)
        ablation(g, gi.FP8_FWD)
    g.close()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(p)
        out["parity"] = parity_sample(p, data, C_out)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
