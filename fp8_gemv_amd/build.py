"""Build the gfx950 HIP library ``libfp8_gemv.so`` in-tree with hipcc.

Every source is compiled for gfx950 only.  The producer is compiled without floating-point
contraction so that its f64/f32 operation sequence is exactly the one its comments state.
Packed FP32 instructions are disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfp8_gemv.so")
ARCH = "gfx950"

COMMON = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(HERE, "..", "include")]
SOURCES = {
    "producer.hip": ["-ffp-contract=off"],
    "gemv_e4m3.hip": [],
    # MFMA results straight into VGPRs (they feed VALU fmas; the AGPR form adds a copy each)
    "gemv_e4m3_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "gemv_q8_0.hip": [],
    "gemv_q8_0_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "read_ceiling.hip": [],
    "requant.hip": ["-ffp-contract=off"],
    "capi.hip": [],
}


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [hipcc(), *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(lambda kv: _compile(*kv), SOURCES.items()))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
