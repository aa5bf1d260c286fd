"""CPU oracle for the quantized mul_mat -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and its
binding) never touches it, and it shares no code with that path.

This module is argument marshalling over ``qmm_oracle.c`` (plain C, built with
gcc); every computation lives in that file, which cites the passage of the pages
each function follows.  Arrays are numpy arrays; block data are ``uint8`` arrays
of the byte formats documented in ``qmm_oracle.h``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qmm_oracle.c")
_LIB = os.path.join(_HERE, "libqmm_oracle.so")

Q4_0_BYTES, Q8_0_BYTES, Q4_K_BYTES, Q8_K_BYTES, Q6_K_BYTES, Q2_K_BYTES = 18, 34, 144, 292, 210, 84
QK4_0, QK_K = 32, 256

_lib = None


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc (plain C11, OpenMP, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           "-o", _LIB + ".tmp", _SRC, "-lm"]
    if os.environ.get("ORACLE_ASAN"):  # AddressSanitizer build (tests/asan_cpu.sh)
        cmd[1:1] = ["-fsanitize=address", "-fno-omit-frame-pointer"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    sigs = {
        "orc_f32_to_f16": (ctypes.c_uint16, [ctypes.c_float]),
        "orc_f16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
        "orc_q4_K_get_scale_min": (None, [P, ctypes.c_int, P, P]),
        "orc_q4_K_pack_scales": (None, [P, P, P]),
        "orc_quantize_q4_0": (None, [P, I64, I64, P]),
        "orc_quantize_q4_K": (None, [P, I64, I64, P]),
        "orc_quantize_q8_0": (None, [P, I64, I64, P]),
        "orc_quantize_q8_K": (None, [P, I64, I64, P]),
        "orc_dequantize_q4_0": (None, [P, I64, I64, P]),
        "orc_dequantize_q4_K": (None, [P, I64, I64, P]),
        "orc_dequantize_q8_0": (None, [P, I64, I64, P]),
        "orc_dequantize_q8_K": (None, [P, I64, I64, P]),
        "orc_brute_force": (None, [P, P, I64, I64, I64, P, P]),
        "orc_mul_mat_q4_0_q8_0": (None, [P, P, I64, I64, I64, P, ctypes.c_int]),
        "orc_mul_mat_q4_K_q8_K": (None, [P, P, I64, I64, I64, P, ctypes.c_int]),
        "orc_q4_K_subblock_sums": (None, [P, P, I64, I64, I64, P]),
        "orc_q4_0_block_sums": (None, [P, P, I64, I64, I64, P]),
        "orc_sample_q4_K_q8_K": (None, [P, P, I64, I64, I64, P, P, I64, P, P]),
        "orc_sample_q4_0_q8_0": (None, [P, P, I64, I64, I64, P, P, I64, P, P]),
        "orc_repacked_bytes_q4_0": (I64, [I64, I64]),
        "orc_repacked_bytes_q4_K": (I64, [I64, I64]),
        "orc_repack_q4_0": (None, [P, I64, I64, P]),
        "orc_repack_q4_K": (None, [P, I64, I64, P]),
        "orc_q6_K_pack_codes": (None, [P, P]),
        "orc_quantize_q6_K": (None, [P, I64, I64, P]),
        "orc_dequantize_q6_K": (None, [P, I64, I64, P]),
        "orc_mul_mat_q6_K_q8_K": (None, [P, P, I64, I64, I64, P, ctypes.c_int]),
        "orc_q6_K_group_sums": (None, [P, P, I64, I64, I64, P]),
        "orc_sample_q6_K_q8_K": (None, [P, P, I64, I64, I64, P, P, I64, P, P]),
        "orc_repacked_bytes_q6_K": (I64, [I64, I64]),
        "orc_repack_q6_K": (None, [P, I64, I64, P]),
        "orc_q2_K_pack_codes": (None, [P, P]),
        "orc_quantize_q2_K": (None, [P, I64, I64, P]),
        "orc_dequantize_q2_K": (None, [P, I64, I64, P]),
        "orc_mul_mat_q2_K_q8_K": (None, [P, P, I64, I64, I64, P, ctypes.c_int]),
        "orc_q2_K_group_sums": (None, [P, P, I64, I64, I64, P]),
        "orc_sample_q2_K_q8_K": (None, [P, P, I64, I64, I64, P, P, I64, P, P]),
        "orc_repacked_bytes_q2_K": (I64, [I64, I64]),
        "orc_repack_q2_K": (None, [P, I64, I64, P]),
        "orc_mul_mat_id": (ctypes.c_int, [ctypes.c_int, P, I64, I64, I64, P, P, I64, I64, ctypes.c_int, P, P]),
        "orc_max_threads": (ctypes.c_int, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _nblocks(fmt: str, K: int) -> tuple[int, int]:
    return {"q4_0": (K // 32, Q4_0_BYTES), "q8_0": (K // 32, Q8_0_BYTES),
            "q4_K": (K // 256, Q4_K_BYTES), "q8_K": (K // 256, Q8_K_BYTES),
            "q6_K": (K // 256, Q6_K_BYTES), "q2_K": (K // 256, Q2_K_BYTES)}[fmt]


def f32_to_f16(x: float) -> int:
    return int(_load().orc_f32_to_f16(float(x)))


def f16_to_f32(h: int) -> float:
    return float(_load().orc_f16_to_f32(int(h)))


def get_scale_min(scales12: np.ndarray, j: int) -> tuple[int, int]:
    s = ctypes.c_uint8()
    m = ctypes.c_uint8()
    buf = _c(scales12, np.uint8)
    _load().orc_q4_K_get_scale_min(_p(buf), j, ctypes.byref(s), ctypes.byref(m))
    return s.value, m.value


def pack_scales(s, m) -> np.ndarray:
    s = _c(s, np.uint8)
    m = _c(m, np.uint8)
    out = np.zeros(12, np.uint8)
    _load().orc_q4_K_pack_scales(_p(s), _p(m), _p(out))
    return out


def quantize(fmt: str, x: np.ndarray) -> np.ndarray:
    """Encode a [rows, K] fp32 array into `fmt` blocks; returns [rows, nb*bytes]."""
    x = _c(x, np.float32)
    rows, K = x.shape
    nb, bb = _nblocks(fmt, K)
    out = np.zeros((rows, nb * bb), np.uint8)
    getattr(_load(), f"orc_quantize_{fmt}")(_p(x), rows, K, _p(out))
    return out


def dequantize(fmt: str, blocks: np.ndarray, rows: int, K: int) -> np.ndarray:
    blocks = _c(blocks, np.uint8)
    nb, bb = _nblocks(fmt, K)
    assert blocks.size == rows * nb * bb
    out = np.zeros((rows, K), np.float64)
    getattr(_load(), f"orc_dequantize_{fmt}")(_p(blocks), rows, K, _p(out))
    return out


def brute_force(w: np.ndarray, a: np.ndarray):
    """fp64 C[m,n] = sum_k a[m,k] w[n,k] and sum_k |a w|; w [N,K], a [M,K]."""
    w = _c(w, np.float64)
    a = _c(a, np.float64)
    N, K = w.shape
    M = a.shape[0]
    out = np.zeros((M, N), np.float64)
    terms = np.zeros((M, N), np.float64)
    _load().orc_brute_force(_p(w), _p(a), M, N, K, _p(out), _p(terms))
    return out, terms


def mul_mat(wfmt: str, w: np.ndarray, y: np.ndarray, M: int, N: int, K: int,
            nthreads: int = 0) -> np.ndarray:
    """Integer path; w canonical blocks [N,...], y activation blocks [M,...]."""
    w = _c(w, np.uint8)
    y = _c(y, np.uint8)
    out = np.zeros((M, N), np.float64)
    fn = {"q4_0": "orc_mul_mat_q4_0_q8_0", "q4_K": "orc_mul_mat_q4_K_q8_K",
          "q6_K": "orc_mul_mat_q6_K_q8_K", "q2_K": "orc_mul_mat_q2_K_q8_K"}[wfmt]
    getattr(_load(), fn)(_p(w), _p(y), M, N, K, _p(out), int(nthreads))
    return out


def subblock_sums(wfmt: str, w: np.ndarray, y: np.ndarray, M: int, N: int, K: int):
    """int32 P[m, n, K/32] (Q4_K sub-blocks, Q4_0 blocks) or P[m, n, K/16]
    (Q6_K and Q2_K 16-element groups)."""
    w = _c(w, np.uint8)
    y = _c(y, np.uint8)
    P = np.zeros((M, N, K // (16 if wfmt in ("q6_K", "q2_K") else 32)), np.int32)
    fn = {"q4_0": "orc_q4_0_block_sums", "q4_K": "orc_q4_K_subblock_sums",
          "q6_K": "orc_q6_K_group_sums", "q2_K": "orc_q2_K_group_sums"}[wfmt]
    getattr(_load(), fn)(_p(w), _p(y), M, N, K, _p(P))
    return P


def sample(wfmt: str, w: np.ndarray, y: np.ndarray, M: int, N: int, K: int,
           ms: np.ndarray, ns: np.ndarray):
    """Outputs and sum|terms| at the listed (m, n) pairs only."""
    w = _c(w, np.uint8)
    y = _c(y, np.uint8)
    ms = _c(ms, np.int64)
    ns = _c(ns, np.int64)
    assert ms.shape == ns.shape
    out = np.zeros(ms.shape, np.float64)
    terms = np.zeros(ms.shape, np.float64)
    fn = {"q4_0": "orc_sample_q4_0_q8_0", "q4_K": "orc_sample_q4_K_q8_K",
          "q6_K": "orc_sample_q6_K_q8_K", "q2_K": "orc_sample_q2_K_q8_K"}[wfmt]
    getattr(_load(), fn)(_p(w), _p(y), M, N, K, _p(ms), _p(ns), ms.size, _p(out), _p(terms))
    return out, terms


def repacked_bytes(wfmt: str, N: int, K: int) -> int:
    return int(getattr(_load(), f"orc_repacked_bytes_{wfmt}")(N, K))


def repack(wfmt: str, w: np.ndarray, N: int, K: int) -> np.ndarray:
    w = _c(w, np.uint8)
    out = np.zeros(repacked_bytes(wfmt, N, K), np.uint8)
    getattr(_load(), f"orc_repack_{wfmt}")(_p(w), N, K, _p(out))
    return out


def q6_K_pack_codes(q) -> np.ndarray:
    """ql[128] | qh[64] bytes of 256 signed 6-bit codes (the documented placement)."""
    q = _c(q, np.int8)
    assert q.size == 256
    out = np.zeros(192, np.uint8)
    _load().orc_q6_K_pack_codes(_p(q), _p(out))
    return out


_WFMT = {"q4_0": 0, "q4_K": 1, "q6_K": 2, "q2_K": 3}


def mul_mat_id(wfmt: str, w: np.ndarray, E: int, N: int, K: int, y: np.ndarray,
               ids: np.ndarray, y_per_slot: bool = False):
    """Expert-routed integer path: w is the canonical stack [E*N, ...], ids
    [T, U] int32; returns (out [T, U, N], sum|terms| [T, U, N]).  Raises
    ValueError for an id outside [0, E)."""
    w = _c(w, np.uint8)
    y = _c(y, np.uint8)
    ids = _c(ids, np.int32)
    T, U = ids.shape
    out = np.zeros((T, U, N), np.float64)
    terms = np.zeros((T, U, N), np.float64)
    rc = _load().orc_mul_mat_id(_WFMT[wfmt], _p(w), E, N, K, _p(y), _p(ids), T, U,
                                int(bool(y_per_slot)), _p(out), _p(terms))
    if rc != 0:
        raise ValueError("mul_mat_id: expert id out of range")
    return out, terms


def q2_K_pack_codes(q) -> np.ndarray:
    """qs[64] bytes of 256 2-bit codes (the documented placement)."""
    q = _c(q, np.uint8)
    assert q.size == 256
    out = np.zeros(64, np.uint8)
    _load().orc_q2_K_pack_codes(_p(q), _p(out))
    return out


def max_threads() -> int:
    return int(_load().orc_max_threads())
