"""Builds libdbgemm.so (HIP kernels for gfx950 + the C-ABI) in the package folder.

    python -m dense_blas3_gemm_amd.build                 # or dense_blas3_gemm_amd.build.build()
    python -m dense_blas3_gemm_amd.build --incremental   # recompile only stale objects

Every translation unit is compiled by hipcc for gfx950 only.  Packed-fp32 VALU
instructions are disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libdbgemm.so")
BUILD = os.path.join(PKG, "_build")

# (source, object name, extra flags): the direct-to-LDS ring kernels are compiled once per
# transpose case and half of the policy table, the register-staged and ping-pong kernels
# once per transpose case, so that the groups of instantiations build in parallel
SOURCES = [("api.cpp", "api", []), ("policy.cpp", "policy", []), ("kernel_simt.hip", "kernel_simt", []),
           ("lds_probe.hip", "lds_probe", []), ("hw_probe.hip", "hw_probe", []),
           ("quantize_mx.hip", "quantize_mx", []),
           ("blas3.cpp", "blas3", []), ("blas3_kernels.hip", "blas3_kernels", [])] + [
    ("kernel_mfma.hip", f"kernel_mfma_{ta}{tb}", [f"-DDBGEMM_DMA_TA={ta}", f"-DDBGEMM_DMA_TB={tb}"])
    for ta in (0, 1) for tb in (0, 1)] + [
    ("kernel_mfma_dma.hip", f"kernel_mfma_dma_{ta}{tb}_p{part}",
     [f"-DDBGEMM_DMA_TA={ta}", f"-DDBGEMM_DMA_TB={tb}", f"-DDBGEMM_DMA_PART={part}"])
    for ta in (0, 1) for tb in (0, 1) for part in (0, 1)] + [
    ("kernel_pingpong.hip", f"kernel_pingpong_{ta}{tb}", [f"-DDBGEMM_DMA_TA={ta}", f"-DDBGEMM_DMA_TB={tb}"])
    for ta in (0, 1) for tb in (0, 1)]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-Xclang", "-target-feature",
         "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC]


def _deps(path: str, seen=None) -> set:
    """The file and the local headers it includes, recursively (quoted includes found in
    csrc/ or include/)."""
    import re
    seen = set() if seen is None else seen
    if path in seen or not os.path.exists(path):
        return seen
    seen.add(path)
    for inc in re.findall(r'^\s*#\s*include\s+"([^"]+)"', open(path).read(), re.M):
        for d in (CSRC, INCLUDE):
            cand = os.path.join(d, inc)
            if os.path.exists(cand):
                _deps(cand, seen)
                break
    return seen


def _stale(src: str, obj: str) -> bool:
    """An object is stale when it is older than its source or a header the source includes."""
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    return any(os.path.getmtime(d) > t for d in _deps(os.path.join(CSRC, src)))


def _compile(entry, incremental: bool = False) -> str:
    src, name, extra = entry
    obj = os.path.join(BUILD, name + ".o")
    if incremental and not _stale(src, obj):
        return obj
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC, *FLAGS, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _write_build_info() -> None:
    """Records the source state the library was built from (git describe, when the tree is
    a git checkout) beside it; bench.py reports it."""
    import json
    import time
    try:
        desc = subprocess.run(["git", "-C", ROOT, "describe", "--always", "--dirty", "--abbrev=12"],
                              capture_output=True, text=True, timeout=20).stdout.strip() or None
    except (OSError, subprocess.SubprocessError):
        desc = None
    with open(os.path.join(PKG, "build_info.json"), "w") as f:
        json.dump({"git": desc, "built": time.strftime("%Y-%m-%dT%H:%M:%SZ", time.gmtime()), "arch": ARCH}, f)


def build(verbose: bool = False, incremental: bool = False) -> str:
    """Compiles every translation unit (only the stale ones with `incremental`) and links."""
    os.makedirs(BUILD, exist_ok=True)
    # the slowest translation units first, so that they start at once
    order = sorted(SOURCES, key=lambda e: not e[0].startswith("kernel_mfma"))
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 8)) as ex:
        objs = list(ex.map(lambda e: _compile(e, incremental), order))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    _write_build_info()
    if verbose:
        print(f"built {OUT}")
    return OUT


SAN_BUILD = os.path.join(PKG, "_build_san")
SAN_OUT = os.path.join(SAN_BUILD, "libdbgemm_san.so")
# The host-logic translation units (argument checks, policy choice, split and stream-K
# sizing, the BLAS3 drivers) with AddressSanitizer and UndefinedBehaviorSanitizer on the
# host side only, linked with the kernels' objects of the regular build.
SAN_SOURCES = ("api.cpp", "policy.cpp", "blas3.cpp")
SAN_FLAGS = ["-O1", "-g", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-fno-omit-frame-pointer",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-fno-gpu-sanitize",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC]


def build_sanitized(verbose: bool = False) -> str:
    """The library with its host logic sanitized (stale objects only; the kernel objects
    come from the regular build, which must exist).  Load it with the ASan runtime
    preloaded and DBGEMM_LIB pointing at it."""
    os.makedirs(SAN_BUILD, exist_ok=True)
    objs = []
    for src, name, extra in SOURCES:
        if src in SAN_SOURCES:
            obj = os.path.join(SAN_BUILD, name + ".o")
            if _stale(src, obj):
                r = subprocess.run([HIPCC, *SAN_FLAGS, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj],
                                   capture_output=True, text=True)
                if r.returncode != 0:
                    raise RuntimeError(f"hipcc (sanitized host) failed for {src}:\n{r.stderr}")
        else:
            obj = os.path.join(BUILD, name + ".o")
            if not os.path.exists(obj):
                raise RuntimeError(f"{obj} is missing: run the regular build first")
        objs.append(obj)
    if not os.path.exists(SAN_OUT) or any(os.path.getmtime(o) > os.path.getmtime(SAN_OUT) for o in objs):
        cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Xarch_host", "-fsanitize=address",
               "-Xarch_host", "-fsanitize=undefined", "-o", SAN_OUT + ".tmp", *objs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"sanitized link failed:\n{r.stderr}")
        os.replace(SAN_OUT + ".tmp", SAN_OUT)
    if verbose:
        print(f"built {SAN_OUT}")
    return SAN_OUT


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        build_sanitized(verbose=True)
    else:
        build(verbose=True, incremental="--incremental" in sys.argv[1:])
    sys.exit(0)
