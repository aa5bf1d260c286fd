"""ctypes binding of libqmm (include/qmm.h): argument marshalling only.

Every computation runs in the HIP kernels of ``libqmm.so``; this module checks
that it was handed torch tensors on the GPU, passes their device pointers and
the current HIP stream, and turns a non-zero status into :class:`QmmError`.
There is no fallback: if ``libqmm.so`` is missing, importing the entry points
raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libqmm.so")

# enums of include/qmm.h
Q8_0, Q8_K = 0, 1
Q4_0, Q4_K, Q6_K, Q2_K = 0, 1, 2, 3
CANONICAL, REPACKED = 0, 1
ALGO_AUTO, ALGO_GEMV, ALGO_MFMA, ALGO_SKINNY = 0, 1, 2, 3
STATUS = {0: "QMM_OK", 1: "QMM_EINVAL", 2: "QMM_EALIGN", 3: "QMM_EUNSUPPORTED", 4: "QMM_EDEVICE"}

_ACT = {"q8_0": Q8_0, "q8_K": Q8_K}
_WEIGHT = {"q4_0": Q4_0, "q4_K": Q4_K, "q6_K": Q6_K, "q2_K": Q2_K}
_LAYOUT = {"canonical": CANONICAL, "repacked": REPACKED}
_ALGO = {"auto": ALGO_AUTO, "gemv": ALGO_GEMV, "mfma": ALGO_MFMA, "skinny": ALGO_SKINNY}


class QmmError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}: {detail}")


_lib = None


def load() -> ctypes.CDLL:
    """Load libqmm.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m bit_quantized_mat_quantize_amd.build`")
    # torch first: its HIP runtime must be the one libqmm binds to (loading
    # libqmm first would bring in the system runtime under the same soname)
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, SZ, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
    sigs = {
        "qmm_act_bytes": (SZ, [I, I64, I64]),
        "qmm_weight_bytes": (SZ, [I, I, I64, I64]),
        "qmm_quantize_row_q8": (I, [I, P, I64, I64, P, SZ, P]),
        "qmm_quantize_weights": (I, [I, P, I64, I64, P, SZ, P]),
        "qmm_repack_weights": (I, [I, P, I64, I64, P, SZ, P]),
        "qmm_mul_mat_q4_0": (I, [P, SZ, I, P, SZ, P, SZ, I64, I64, I64, P]),
        "qmm_mul_mat_q4_K": (I, [P, SZ, I, P, SZ, P, SZ, I64, I64, I64, P]),
        "qmm_mul_mat_q4_K_ex": (I, [P, SZ, I, P, SZ, P, SZ, I64, I64, I64, I, P]),
        "qmm_mul_mat_q6_K": (I, [P, SZ, I, P, SZ, P, SZ, I64, I64, I64, P]),
        "qmm_mul_mat_q6_K_ex": (I, [P, SZ, I, P, SZ, P, SZ, I64, I64, I64, I, P]),
        "qmm_mul_mat_q2_K": (I, [P, SZ, I, P, SZ, P, SZ, I64, I64, I64, P]),
        "qmm_mul_mat_q4_0_ex": (I, [P, SZ, I, P, SZ, P, SZ, I64, I64, I64, I, P]),
        "qmm_mul_mat_id_workspace_bytes": (SZ, [I64, I64, I64]),
        "qmm_mul_mat_id_q4_K": (I, [P, SZ, I64, I, P, SZ, I, P, I64, I64, P, SZ, I64, I64, P, SZ, I, P]),
        "qmm_mul_mat_id": (I, [I, P, SZ, I64, I, P, SZ, I, P, I64, I64, P, SZ, I64, I64, P, SZ, I, P]),
        "qmm_mul_mat_id_noalloc": (I, [I, P, SZ, I64, I, P, SZ, I, P, I64, I64, P, SZ, I64, I64, I, P]),
        "qmm_mul_mat_q2_K_ex": (I, [P, SZ, I, P, SZ, P, SZ, I64, I64, I64, I, P]),
        "qmm_quantize_mul_mat": (I, [I, P, SZ, I, P, P, SZ, P, SZ, I64, I64, I64, P]),
        "qmm_debug_block_sums": (I, [I, P, SZ, I, P, SZ, P, SZ, I64, I64, I64, P]),
        "qmm_status_string": (ctypes.c_char_p, [I]),
        "qmm_last_error": (ctypes.c_char_p, []),
        "qmm_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int, where: str) -> None:
    if status != 0:
        raise QmmError(status, where, load().qmm_last_error().decode())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (got device {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr()), t.numel() * t.element_size()


def act_bytes(fmt: str, M: int, K: int) -> int:
    return int(load().qmm_act_bytes(_ACT[fmt], M, K))


def weight_bytes(fmt: str, layout: str, N: int, K: int) -> int:
    return int(load().qmm_weight_bytes(_WEIGHT[fmt], _LAYOUT[layout], N, K))


def quantize_row_q8(x, fmt: str = "q8_K", out=None, stream=None):
    """fp32 [M, K] GPU tensor -> uint8 activation blocks (bit-exact Q8_0/Q8_K)."""
    import torch
    M, K = x.shape
    if x.dtype != torch.float32:
        raise ValueError("x must be float32")
    if out is None:
        out = torch.empty(max(act_bytes(fmt, M, K), 1), dtype=torch.uint8, device=x.device)
    px, _ = _dev(x, "x")
    py, ny = _dev(out, "y")
    _check(load().qmm_quantize_row_q8(_ACT[fmt], px, M, K, py, ny, _stream(stream)),
           "qmm_quantize_row_q8")
    return out


def quantize_weights(w, fmt: str = "q4_K", out=None, stream=None):
    """fp32 [N, K] GPU tensor -> canonical uint8 weight blocks."""
    import torch
    N, K = w.shape
    if w.dtype != torch.float32:
        raise ValueError("w must be float32")
    if out is None:
        out = torch.empty(max(weight_bytes(fmt, "canonical", N, K), 1), dtype=torch.uint8,
                          device=w.device)
    pw, _ = _dev(w, "w")
    po, no = _dev(out, "out")
    _check(load().qmm_quantize_weights(_WEIGHT[fmt], pw, N, K, po, no, _stream(stream)),
           "qmm_quantize_weights")
    return out


def repack_weights(w, fmt: str, N: int, K: int, out=None, stream=None):
    import torch
    if out is None:
        out = torch.empty(max(weight_bytes(fmt, "repacked", N, K), 1), dtype=torch.uint8,
                          device=w.device)
    pw, _ = _dev(w, "w_canon")
    po, no = _dev(out, "w_repacked")
    _check(load().qmm_repack_weights(_WEIGHT[fmt], pw, N, K, po, no, _stream(stream)),
           "qmm_repack_weights")
    return out


def mul_mat_q4_0(w, y, M: int, N: int, K: int, layout: str = "canonical", algo: str = "auto",
                 out=None, stream=None):
    import torch
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=y.device)
    pw, nw = _dev(w, "w")
    py, ny = _dev(y, "y")
    po, no = _dev(out, "out")
    _check(load().qmm_mul_mat_q4_0_ex(pw, nw, _LAYOUT[layout], py, ny, po, no, M, N, K,
                                      _ALGO[algo], _stream(stream)), "qmm_mul_mat_q4_0")
    return out


def mul_mat_q4_K(w, y, M: int, N: int, K: int, layout: str = "canonical", algo: str = "auto",
                 out=None, stream=None):
    import torch
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=y.device)
    pw, nw = _dev(w, "w")
    py, ny = _dev(y, "y")
    po, no = _dev(out, "out")
    _check(load().qmm_mul_mat_q4_K_ex(pw, nw, _LAYOUT[layout], py, ny, po, no, M, N, K,
                                      _ALGO[algo], _stream(stream)), "qmm_mul_mat_q4_K")
    return out


def quantize_mul_mat(wfmt: str, w, x, N: int, layout: str = "canonical", y=None, out=None,
                     stream=None):
    """out = mul_mat(w, quantize_row_q8(x)) in one call; returns (out, y).

    x: fp32 [M, K] GPU tensor; y receives the Q8 activation bytes.  For Q4_K
    and M == 1 the quantization runs inside the GEMV launch."""
    import torch
    M, K = x.shape
    if x.dtype != torch.float32:
        raise ValueError("x must be float32")
    afmt = ACT_FOR[wfmt]
    if y is None:
        y = torch.empty(max(act_bytes(afmt, M, K), 1), dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    pw, nw = _dev(w, "w")
    px, _ = _dev(x, "x")
    py, ny = _dev(y, "y")
    po, no = _dev(out, "out")
    _check(load().qmm_quantize_mul_mat(_WEIGHT[wfmt], pw, nw, _LAYOUT[layout], px, py, ny, po, no,
                                       M, N, K, _stream(stream)), "qmm_quantize_mul_mat")
    return out, y


def mul_mat_q6_K(w, y, M: int, N: int, K: int, layout: str = "canonical", algo: str = "auto",
                 out=None, stream=None):
    import torch
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=y.device)
    pw, nw = _dev(w, "w")
    py, ny = _dev(y, "y")
    po, no = _dev(out, "out")
    _check(load().qmm_mul_mat_q6_K_ex(pw, nw, _LAYOUT[layout], py, ny, po, no, M, N, K,
                                      _ALGO[algo], _stream(stream)), "qmm_mul_mat_q6_K")
    return out


def mul_mat_q2_K(w, y, M: int, N: int, K: int, layout: str = "canonical", algo: str = "auto",
                 out=None, stream=None):
    import torch
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=y.device)
    pw, nw = _dev(w, "w")
    py, ny = _dev(y, "y")
    po, no = _dev(out, "out")
    _check(load().qmm_mul_mat_q2_K_ex(pw, nw, _LAYOUT[layout], py, ny, po, no, M, N, K,
                                      _ALGO[algo], _stream(stream)), "qmm_mul_mat_q2_K")
    return out


def mul_mat_id_workspace_bytes(T: int, U: int, E: int) -> int:
    return int(load().qmm_mul_mat_id_workspace_bytes(T, U, E))


def mul_mat_id(wfmt: str, w, E: int, y, ids, N: int, K: int, layout: str = "canonical",
               y_per_slot: bool = False, algo: str = "auto", out=None, workspace=None, stream=None):
    """out [T, U, N] fp32: slot u of token t multiplies expert ids[t, u]'s matrix
    in format `wfmt` (w = E matrices back to back) with activation row t (or
    t*U + u)."""
    import torch
    T, U = ids.shape
    if ids.dtype != torch.int32:
        raise ValueError("ids must be int32")
    if out is None:
        out = torch.empty((T, U, N), dtype=torch.float32, device=ids.device)
    if workspace is None:
        workspace = torch.empty(max(mul_mat_id_workspace_bytes(T, U, E), 16), dtype=torch.uint8,
                                device=ids.device)
    pw, nw = _dev(w, "w")
    py, ny = _dev(y, "y")
    pi, _ = _dev(ids, "ids")
    po, no = _dev(out, "out")
    pws, nws = _dev(workspace, "workspace")
    _check(load().qmm_mul_mat_id(_WEIGHT[wfmt], pw, nw, E, _LAYOUT[layout], py, ny, int(bool(y_per_slot)), pi,
                                 T, U, po, no, N, K, pws, nws, _ALGO[algo], _stream(stream)),
           "qmm_mul_mat_id")
    return out


def mul_mat_id_noalloc(wfmt: str, w, E: int, y, ids, N: int, K: int, layout: str = "canonical",
                       y_per_slot: bool = False, algo: str = "auto", out=None, stream=None):
    """mul_mat_id with the expert grouping in the library's own per-GPU scratch
    (no workspace argument; see qmm_mul_mat_id_noalloc)."""
    import torch
    T, U = ids.shape
    if ids.dtype != torch.int32:
        raise ValueError("ids must be int32")
    if out is None:
        out = torch.empty((T, U, N), dtype=torch.float32, device=ids.device)
    pw, nw = _dev(w, "w")
    py, ny = _dev(y, "y")
    pi, _ = _dev(ids, "ids")
    po, no = _dev(out, "out")
    _check(load().qmm_mul_mat_id_noalloc(_WEIGHT[wfmt], pw, nw, E, _LAYOUT[layout], py, ny, int(bool(y_per_slot)),
                                         pi, T, U, po, no, N, K, _ALGO[algo], _stream(stream)),
           "qmm_mul_mat_id_noalloc")
    return out


def mul_mat_id_q4_K(w, E: int, y, ids, N: int, K: int, layout: str = "canonical",
                    y_per_slot: bool = False, algo: str = "auto", out=None, workspace=None,
                    stream=None):
    return mul_mat_id("q4_K", w, E, y, ids, N, K, layout=layout, y_per_slot=y_per_slot, algo=algo,
                      out=out, workspace=workspace, stream=stream)


ACT_FOR = {"q4_0": "q8_0", "q4_K": "q8_K", "q6_K": "q8_K", "q2_K": "q8_K"}  # activation blocks each weight format takes


def mul_mat(wfmt: str, w, y, M: int, N: int, K: int, layout: str = "canonical", out=None,
            stream=None):
    """The mul_mat entry point of weight format `wfmt` (automatic dispatch by M)."""
    fn = {"q4_0": mul_mat_q4_0, "q4_K": mul_mat_q4_K, "q6_K": mul_mat_q6_K, "q2_K": mul_mat_q2_K}[wfmt]
    return fn(w, y, M, N, K, layout=layout, out=out, stream=stream)


def debug_block_sums(wfmt: str, w, y, M: int, N: int, K: int, layout: str = "canonical",
                     out=None, stream=None):
    """int32 [M, N, K/32] per-sub-block (Q4_K) or per-block (Q4_0) sums, or
    [M, N, K/16] per-group sums (Q6_K, Q2_K)."""
    import torch
    if out is None:
        out = torch.empty((M, N, K // (16 if wfmt in ("q6_K", "q2_K") else 32)), dtype=torch.int32,
                          device=y.device)
    pw, nw = _dev(w, "w")
    py, ny = _dev(y, "y")
    po, no = _dev(out, "P")
    _check(load().qmm_debug_block_sums(_WEIGHT[wfmt], pw, nw, _LAYOUT[layout], py, ny, po, no,
                                       M, N, K, _stream(stream)), "qmm_debug_block_sums")
    return out


def version() -> str:
    return load().qmm_version().decode()
