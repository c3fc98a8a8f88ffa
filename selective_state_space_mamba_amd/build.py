"""Build the HIP library (libssd_mi355x.so) for gfx950 with hipcc.

Every source under csrc/ is compiled separately (in parallel) and linked into
one shared library next to this file.  Run: ``python -m selective_state_space_mamba_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB_NAME = "libssd_mi355x.so"
ARCH = "gfx950"

SOURCES = ["ssd_state.hip", "ssd_chunk_fwd.hip", "ssd_chunk_bwd.hip", "ssd_bwd_bf16.hip", "ssd_bwd_fused.hip", "ssd_fwd_bf16.hip", "ssd_state_bf16.hip", "shell.hip", "gemm.cpp", "capi.cpp"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed f32 ALU ops stay off: only plain scalar/vector f32 code is emitted
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def lib_path() -> str:
    return os.path.join(HERE, LIB_NAME)


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), "-x", "hip", *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    out = lib_path()
    tmp = out + ".tmp%d" % os.getpid()
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-L" + os.path.join(rocm, "lib"),
           "-lrocblas", "-lhipblaslt", "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
