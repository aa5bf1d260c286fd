"""Build libqmm.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m bit_quantized_mat_quantize_amd.build

Every HIP source is compiled with hipcc for gfx950 only, with FMA contraction
off and correctly rounded fp32 division (the encoders must reproduce the
reference bytes exactly) and with packed-fp32 instructions disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
OUT = os.path.join(PKG, "libqmm.so")
BUILD_DIR = os.path.join(ROOT, "_build_asan" if os.environ.get("QMM_ASAN") else "_build")
SOURCES = ["api.hip", "quantize.hip", "repack.hip", "gemv.hip", "skinny.hip", "skinny16.hip", "skinny16r.hip", "skinny32r.hip", "q6k.hip", "q6k_gemm.hip", "q6k_skinny.hip",
           "q2k.hip", "q2k_gemm.hip", "q2k_skinny.hip", "q40_gemm.hip", "q40_skinny.hip", "moe.hip", "gemm.hip"]
PROBE_SOURCES = ["probe.hip"]
PROBE_OUT = os.path.join(PKG, "libqmm_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


# QMM_ASAN=1: AddressSanitizer on the host code only (argument validation,
# dispatch, launch set-up), for the CPU test run of tests/asan_cpu.sh; the GPU
# code is built as usual.
ASAN = bool(os.environ.get("QMM_ASAN"))
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *(HOST_ASAN if ASAN else []), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is noise
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if msg.strip() and verbose:
        print(msg)
    return obj


def _link(objs, out: str, verbose: bool) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *(["-shared-libsan", "-fsanitize=address"] if ASAN else []),
           "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """libqmm.so (the method) and libqmm_probe.so (the calibration probes the
    benchmark reports beside it)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    _link(objs[:len(SOURCES)], OUT, verbose)
    _link(objs[len(SOURCES):], PROBE_OUT, verbose)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
