"""Builds libdbgemm.so (HIP kernels for gfx950 + the C-ABI) in the package folder.

    python -m dense_blas3_gemm_amd.build        # or dense_blas3_gemm_amd.build.build()

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

# (source, object name, extra flags): the direct-to-LDS kernels are compiled once per
# transpose case so that the four groups of instantiations build in parallel
SOURCES = [("api.cpp", "api", []), ("policy.cpp", "policy", []), ("kernel_simt.hip", "kernel_simt", []),
           ("kernel_mfma.hip", "kernel_mfma", []), ("lds_probe.hip", "lds_probe", []),
           ("quantize_mx.hip", "quantize_mx", []),
           ("blas3.cpp", "blas3", []), ("blas3_kernels.hip", "blas3_kernels", [])] + [
    ("kernel_mfma_dma.hip", f"kernel_mfma_dma_{ta}{tb}", [f"-DDBGEMM_DMA_TA={ta}", f"-DDBGEMM_DMA_TB={tb}"])
    for ta in (0, 1) for tb in (0, 1)]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-Xclang", "-target-feature",
         "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC]


def _compile(entry) -> str:
    src, name, extra = entry
    obj = os.path.join(BUILD, name + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC, *FLAGS, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
