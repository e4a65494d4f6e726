"""Benchmark of the dense GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--sweep]
                    [--ablation] [--policy NAME] [--workload NAME] [--copy-calibration MiB]

A step is one call C = alpha*A*B + beta*C of the headline workload, 4096^3 bf16
row-major NN with bf16 C (alpha 1, beta 0), on inputs already resident in HBM.
W untimed warmup steps run first; then K steps are timed between two device
synchronisations, and each launch also sits between its own pair of HIP events
recorded on the stream the kernel runs on.  Prints one JSON line.

--sweep additionally times every other workload (10 warmup + 50 event-timed calls
each, p50/p95) and prints a Markdown table to stderr; the JSON line is unchanged.
--ablation times every applicable policy on the headline and the E4M3 workloads.
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
# the device code of the direct-to-LDS kernels (the headline policy's kernel)
KERNEL_SOURCES = [os.path.join(ROOT, "dense_blas3_gemm_amd", "csrc", f)
                  for f in ("kernel_mfma_dma.hip", "mfma_common.h", "gemm_internal.h")]


def _dev(bits, kind):
    import torch
    if kind == "bf16":
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    if kind == "e4m3":
        return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.float8_e4m3fn).cuda()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.float32)).cuda()


def kernel_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
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


def time_problem(g, p: gi.Gemm, warmup: int, steps: int, data=None):
    """Returns dict with wall ms/step, event durations (ms) and the policy name."""
    import torch
    data = data if data is not None else p.make()
    A = _dev(data["A"], p.in_dtype)
    B = _dev(data["B"], p.in_dtype)
    if "C" in data:
        C = _dev(data["C"], p.c_dtype)
    else:
        C = torch.zeros((p.M, p.N), dtype=torch.float32 if p.c_dtype == "f32" else torch.bfloat16,
                        device="cuda:0")
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--ablation", action="store_true",
                    help="time every applicable policy on the 4096^3 bf16 and the E4M3 workloads")
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
    p = gi.BY_NAME[args.workload]
    if args.policy:
        g.set_policy(args.policy)
    r = time_problem(g, p, args.warmup, args.steps)
    g.set_policy(None)
    ms = r["wall_ms"]
    value = p.flops / (ms * 1e-3) / 1e12
    ev = r["event_ms"]
    avg_launch_ms = float(ev.mean())
    achieved = p.flops / (avg_launch_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[p.in_dtype]
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
                     "launch_us_p50": round(float(np.percentile(ev, 50)) * 1e3, 2),
                     "launch_us_p95": round(float(np.percentile(ev, 95)) * 1e3, 2),
                     "launch_us_mean": round(avg_launch_ms * 1e3, 2)},
    }
    if args.sweep:
        sweep(g)
    if args.ablation:
        ablation(g, p)
        ablation(g, gi.FP8_FWD)
    g.close()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(p)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
