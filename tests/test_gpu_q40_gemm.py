"""Q4_0 x Q8_0 on the int8 MFMA kernels (repacked layout, K % 256 == 0): the
prefill GEMM and the small-batch kernel, against the oracle.

* exactness window: Q4_0 blocks with d = 1 and integer activations with
  amax = 127 per 32-block (d_a = 1) keep every partial sum an integer below
  2^24, so the fp32 outputs equal the integer result exactly -- including the
  code extremes 0 and 15 (q - 8 = -8 and 7) against y = +-127.
* fp32 outputs: |gpu - oracle| <= 1e-4 * sum_k |w a| for every checked (m, n),
  on ragged row and column tiles, one K step and many; for the small-batch
  kernel also step counts that leave some of its eight K-split wavefronts with
  no step or one step more than the others, and several 32-row chunks.
* AUTO dispatch: each choice is bit-identical to the path it names.
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


@pytest.mark.parametrize("algo", ["mfma", "skinny"])
@pytest.mark.parametrize("extreme", [False, True])
def test_mfma_exactness_window(extreme, algo):
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
    got = to_host(qmm.mul_mat_q4_0(wd, to_dev(y.reshape(-1)), M, N, K, layout="repacked", algo=algo))
    assert np.array_equal(got.astype(np.float64), want)


@pytest.mark.parametrize("M,N,K", [(9, 1, 256), (128, 256, 1024), (200, 257, 4096), (33, 40, 8192)])
def test_mfma_q4_0(M, N, K):
    w = oracle.quantize("q4_0", weights_normal([430, M + N], N, K))
    y = oracle.quantize("q8_0", activations([431, M + N], M, K, outlier_frac=0.01))
    want, terms = full_reference("q4_0", w, y, M, N, K)
    wd = upload_weights("q4_0", w, N, K, "repacked")
    got = to_host(qmm.mul_mat_q4_0(wd, to_dev(y.reshape(-1)), M, N, K, layout="repacked", algo="mfma"))
    assert_close(got, want, terms, f"q4_0 mfma M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", [(2, 70, 256), (5, 33, 512), (8, 300, 2048), (9, 64, 4608), (17, 1, 256),
                                   (32, 257, 1024), (40, 100, 2048), (70, 130, 4608)])
def test_skinny_q4_0(M, N, K):
    w = oracle.quantize("q4_0", weights_normal([434, M + N], N, K))
    y = oracle.quantize("q8_0", activations([435, M + N], M, K, outlier_frac=0.01))
    want, terms = full_reference("q4_0", w, y, M, N, K)
    wd = upload_weights("q4_0", w, N, K, "repacked")
    got = to_host(qmm.mul_mat_q4_0(wd, to_dev(y.reshape(-1)), M, N, K, layout="repacked", algo="skinny"))
    assert_close(got, want, terms, f"q4_0 skinny M={M} N={N} K={K}")


@pytest.mark.parametrize("layout", ["canonical", "repacked"])
@pytest.mark.parametrize("M,N,K", [(1, 2048, 2048), (1, 4099, 1024), (2, 1031, 4096), (3, 8200, 512),
                                   (4, 512, 12288)])
def test_gemv_q4_0_staged(M, N, K, layout):
    """The GEMV with the activation rows staged in LDS (N*K >= 2^22, K % 64 == 0,
    M*K*5/4 <= 61440): the smallest staged N*K, ragged N, one block pair per row
    and the LDS boundary M = 4, K = 12288, both layouts; fp32 outputs against
    the oracle and the int32 block sums of the same kernel bit-exact."""
    w = oracle.quantize("q4_0", weights_normal([438, M + N], N, K))
    y = oracle.quantize("q8_0", activations([439, M + N], M, K, outlier_frac=0.01))
    want, terms = full_reference("q4_0", w, y, M, N, K)
    wd = upload_weights("q4_0", w, N, K, layout)
    yd = to_dev(y.reshape(-1))
    got = to_host(qmm.mul_mat_q4_0(wd, yd, M, N, K, layout=layout, algo="gemv"))
    assert_close(got, want, terms, f"q4_0 staged gemv M={M} N={N} K={K} {layout}")
    sums = to_host(qmm.debug_block_sums("q4_0", wd, yd, M, N, K, layout=layout))
    assert np.array_equal(sums, oracle.subblock_sums("q4_0", w, y, M, N, K))


def test_skinny_overwrites_and_rejects():
    """The small-batch kernel writes every output (no accumulation into a
    stale buffer) and refuses what it does not take: the canonical layout and
    K not a multiple of 256."""
    M, N, K = 20, 50, 512
    w = oracle.quantize("q4_0", weights_normal([436, 1], N, K))
    y = oracle.quantize("q8_0", activations([437, 1], M, K))
    want, terms = full_reference("q4_0", w, y, M, N, K)
    wd = upload_weights("q4_0", w, N, K, "repacked")
    import torch
    out = torch.full((M, N), float("nan"), device="cuda")
    qmm.mul_mat_q4_0(wd, to_dev(y.reshape(-1)), M, N, K, layout="repacked", algo="skinny", out=out)
    assert_close(to_host(out), want, terms, "q4_0 skinny into a NaN-filled buffer")
    with pytest.raises(qmm.QmmError):
        qmm.mul_mat_q4_0(upload_weights("q4_0", w, N, K, "canonical"), to_dev(y.reshape(-1)), M, N, K,
                         layout="canonical", algo="skinny")
    K = 288
    w = oracle.quantize("q4_0", weights_normal([436, 2], N, K))
    y = oracle.quantize("q8_0", activations([437, 2], M, K))
    with pytest.raises(qmm.QmmError):
        qmm.mul_mat_q4_0(upload_weights("q4_0", w, N, K, "repacked"), to_dev(y.reshape(-1)), M, N, K,
                         layout="repacked", algo="skinny")


def _auto_algo(M, N, K, layout):
    """The AUTO rule as the library documents it."""
    staged = K % 64 == 0 and M * K * 5 // 4 <= 61440
    if (layout == "canonical" or K % 256 != 0 or M == 1 or (staged and (M <= 4 or M * N <= 36864))
            or (M == 2 and N < 8192)):
        return "gemv"
    return "skinny" if (M + 31) // 32 * N <= 16 * 8192 else "mfma"


def test_auto_dispatch():
    """Every AUTO choice (the GEMV for M = 1, for M <= 4 or M*N <= 36864 while the
    rows fit its LDS staging, for M = 2 below 8192 columns, for the canonical
    layout and for K % 256 != 0; the small-batch kernel while ceil(M/32)*N <=
    16*8192; the GEMM above) is bit-identical to that path and agrees with the
    oracle."""
    for M, N, K in [(1, 70, 1024), (2, 70, 1024), (4, 300, 12288), (4, 300, 12544), (2, 8192, 256),
                    (8, 4608, 1024), (8, 4609, 1024), (40, 70, 288), (40, 6200, 1024), (100, 32768, 256),
                    (161, 26000, 256)]:
        w = oracle.quantize("q4_0", weights_normal([432, M + K], N, K))
        y = oracle.quantize("q8_0", activations([433, M + K], M, K))
        want, terms = full_reference("q4_0", w, y, M, N, K)
        for layout in ("canonical", "repacked"):
            wd = upload_weights("q4_0", w, N, K, layout)
            got = to_host(qmm.mul_mat_q4_0(wd, to_dev(y.reshape(-1)), M, N, K, layout=layout))
            assert_close(got, want, terms, f"q4_0 auto M={M} K={K} {layout}")
            algo = _auto_algo(M, N, K, layout)
            ref = to_host(qmm.mul_mat_q4_0(wd, to_dev(y.reshape(-1)), M, N, K, layout=layout, algo=algo))
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (M, N, K, layout, algo)
    seen = {_auto_algo(M, N, K, "repacked") for M, N, K in [(2, 70, 1024), (4, 300, 12544), (100, 32768, 256),
                                                              (161, 26000, 256)]}
    assert seen == {"gemv", "skinny", "mfma"}
    M, N, K = 40, 70, 288                                      # K % 256 != 0: no MFMA path
    w = oracle.quantize("q4_0", weights_normal([432, M + K], N, K))
    y = oracle.quantize("q8_0", activations([433, M + K], M, K))
    with pytest.raises(qmm.QmmError):
        qmm.mul_mat_q4_0(upload_weights("q4_0", w, N, K, "repacked"), to_dev(y.reshape(-1)), M, N, K,
                         layout="repacked", algo="mfma")
