"""ctypes binding of libqmm_probe (include/qmm_probe.h): the calibration
kernels the benchmark reports beside the method's kernels.  Argument
marshalling only; both probes run as HIP kernels."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB_PATH = os.path.join(PKG, "libqmm_probe.so")

_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(PROBE_LIB_PATH):
        raise ImportError(f"{PROBE_LIB_PATH} is missing: build it with "
                          "`python -m bit_quantized_mat_quantize_amd.build`")
    # torch first: its HIP runtime must be the one libqmm binds to (loading
    # libqmm first would bring in the system runtime under the same soname)
    import torch  # noqa: F401
    lib = ctypes.CDLL(PROBE_LIB_PATH)
    P, SZ, I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    for name, res, args in (("qmm_probe_read", I, [P, SZ, I, P, P]),
                            ("qmm_probe_mfma_sink_bytes", SZ, []),
                            ("qmm_probe_mfma_ops", ctypes.c_double, [I]),
                            ("qmm_probe_mfma_i8", I, [P, SZ, I, I, P])):
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def probe_read(buf, offset: int, nbytes: int, sink, loads_per_thread: int = 4) -> None:
    """Read nbytes of the uint8 CUDA tensor buf starting at byte offset."""
    assert buf.is_cuda and sink.is_cuda and 0 <= offset and offset + nbytes <= buf.numel()
    st = load().qmm_probe_read(ctypes.c_void_p(buf.data_ptr() + offset), nbytes, loads_per_thread,
                               ctypes.c_void_p(sink.data_ptr()), _stream())
    if st != 0:
        raise RuntimeError(f"qmm_probe_read: status {st}")


def mfma_sink_bytes() -> int:
    return int(load().qmm_probe_mfma_sink_bytes())


def mfma_ops(iters: int) -> float:
    return float(load().qmm_probe_mfma_ops(iters))


def probe_mfma_i8(sink, iters: int, seed: int = 0) -> None:
    assert sink.is_cuda
    st = load().qmm_probe_mfma_i8(ctypes.c_void_p(sink.data_ptr()), sink.numel() * sink.element_size(), iters,
                                  seed, _stream())
    if st != 0:
        raise RuntimeError(f"qmm_probe_mfma_i8: status {st}")
