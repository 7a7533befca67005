"""Build librazer.so in-tree with hipcc for gfx950.

Every HIP source is compiled with the packed-FP32 target feature disabled.  The
encoder and decoder translation units are also compiled with
-ffp-contract=off, because their bytes must follow a fixed sequence of single
IEEE fp32 operations.  The products keep contraction on (they are checked
against a tolerance, not bit for bit).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "librazer.so")
# measurement probes loaded only by the bench (plain read, register-only MFMA loop)
CEILING_LIB = os.path.join(HERE, "libceiling.so")
CEILING_SRC = "rz_ceiling.hip"
BUILD_DIR = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
EXACT = ["-ffp-contract=off"]

SOURCES = {
    "rz_quantize.hip": EXACT,
    "rz_dequant.hip": EXACT,
    "rz_gemv.hip": [],
    "rz_gemm.hip": [],
    "rz_smallm.hip": [],
    # MFMA results in VGPRs: the epilogue of every block reads them with VALU
    "rz_bdiag.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "rz_w4a4.hip": [],
    "rz_api.cpp": [],
}


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD_DIR, src + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *COMMON, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the GPU target feature; that warning is expected
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _link(objs: list[str], out: str) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = list(SOURCES.items()) + [(CEILING_SRC, [])]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda kv: _compile(*kv), jobs))
    _link(objs[:-1], LIB)
    _link(objs[-1:], CEILING_LIB)
    if verbose:
        print(f"built {LIB} and {CEILING_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
