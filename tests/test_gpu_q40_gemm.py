"""Q4_0 x Q8_0 on the int8 MFMA GEMM (repacked layout, K % 256 == 0) against
the oracle.

* exactness window: Q4_0 blocks with d = 1 and integer activations with
  amax = 127 per 32-block (d_a = 1) keep every partial sum an integer below
  2^24, so the fp32 outputs equal the integer result exactly -- including the
  code extremes 0 and 15 (q - 8 = -8 and 7) against y = +-127.
* fp32 outputs: |gpu - oracle| <= 1e-4 * sum_k |w a| for every checked (m, n),
  on ragged row and column tiles, one K step and many.
* AUTO dispatch: GEMV up to M = 8, for the canonical layout and for K not a
  multiple of 256; the GEMM otherwise.
"""
import struct

import numpy as np
import pytest

import oracle
import bit_quantized_mat_quantize_amd as qmm
from bit_quantized_mat_quantize_amd.inputs import activations, weights_normal
from gpu_helpers import assert_close, full_reference, to_dev, to_host, upload_weights

pytestmark = pytest.mark.gpu


def _blocks(codes, d=1.0):
    N, K = codes.shape
    out = bytearray()
    for n in range(N):
        for b in range(K // 32):
            qq = codes[n, 32 * b:32 * b + 32]
            out += struct.pack("<e", d) + bytes(int(qq[l] | (qq[l + 16] << 4)) for l in range(16))
    return np.frombuffer(bytes(out), np.uint8).reshape(N, -1)


@pytest.mark.parametrize("extreme", [False, True])
def test_mfma_exactness_window(extreme):
    M, N, K = 130, 300, 512
    rng = np.random.default_rng(31)
    if extreme:
        codes = rng.choice([0, 15], (N, K))
        x = np.where(rng.random((M, K)) < 0.5, -127.0, 127.0).astype(np.float32)
    else:
        codes = rng.integers(0, 16, (N, K))
        x = rng.integers(-40, 41, (M, K)).astype(np.float32)
        x[:, ::32] = 127.0    # amax 127 per 32-block: d_a = 1 (exact in fp16)
    w = _blocks(codes)
    y = oracle.quantize("q8_0", x)
    want, terms = full_reference("q4_0", w, y, M, N, K)
    assert terms.max() < 2 ** 24
    wd = upload_weights("q4_0", w, N, K, "repacked")
    got = to_host(qmm.mul_mat_q4_0(wd, to_dev(y.reshape(-1)), M, N, K, layout="repacked", algo="mfma"))
    assert np.array_equal(got.astype(np.float64), want)


@pytest.mark.parametrize("M,N,K", [(9, 1, 256), (128, 256, 1024), (200, 257, 4096), (33, 40, 8192)])
def test_mfma_q4_0(M, N, K):
    w = oracle.quantize("q4_0", weights_normal([430, M + N], N, K))
    y = oracle.quantize("q8_0", activations([431, M + N], M, K, outlier_frac=0.01))
    want, terms = full_reference("q4_0", w, y, M, N, K)
    wd = upload_weights("q4_0", w, N, K, "repacked")
    got = to_host(qmm.mul_mat_q4_0(wd, to_dev(y.reshape(-1)), M, N, K, layout="repacked", algo="mfma"))
    assert_close(got, want, terms, f"q4_0 mfma M={M} N={N} K={K}")


def test_auto_dispatch():
    """Every AUTO choice (the GEMV for M = 1 and while M*N <= 30*8192 per 65536
    columns, for the canonical layout and for K % 256 != 0; the GEMM
    otherwise) is bit-identical to that path and agrees with the oracle."""
    for M, N, K in [(8, 70, 1024), (40, 70, 1024), (40, 70, 288), (40, 6200, 1024)]:
        w = oracle.quantize("q4_0", weights_normal([432, M + K], N, K))
        y = oracle.quantize("q8_0", activations([433, M + K], M, K))
        want, terms = full_reference("q4_0", w, y, M, N, K)
        for layout in ("canonical", "repacked"):
            wd = upload_weights("q4_0", w, N, K, layout)
            got = to_host(qmm.mul_mat_q4_0(wd, to_dev(y.reshape(-1)), M, N, K, layout=layout))
            assert_close(got, want, terms, f"q4_0 auto M={M} K={K} {layout}")
            gemv = (layout == "canonical" or K % 256 != 0 or M == 1
                    or M * N <= 30 * 8192 * ((N + 65535) // 65536))
            ref = to_host(qmm.mul_mat_q4_0(wd, to_dev(y.reshape(-1)), M, N, K, layout=layout,
                                           algo="gemv" if gemv else "mfma"))
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (M, N, K, layout)
    M, N, K = 40, 70, 288                                      # K % 256 != 0: no MFMA path
    w = oracle.quantize("q4_0", weights_normal([432, M + K], N, K))
    y = oracle.quantize("q8_0", activations([433, M + K], M, K))
    with pytest.raises(qmm.QmmError):
        qmm.mul_mat_q4_0(upload_weights("q4_0", w, N, K, "repacked"), to_dev(y.reshape(-1)), M, N, K,
                         layout="repacked", algo="mfma")
