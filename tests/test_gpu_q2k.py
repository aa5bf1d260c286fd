"""GPU Q2_K path against the oracle.

* GPU encoder and load-time repack: byte-identical to the oracle's.
* int32 group sums P[m][n][K/16] (the GEMV decode path): bit-exact.
* exactness windows (GEMV and MFMA GEMM): integer activations with amax = 127
  per block (d_a = 1) and weights with d = 1, dmin in {0, 1} keep every
  partial sum an integer below 2^24, so the fp32 outputs equal the integer
  result exactly -- including saturated scales, mins and codes (s = m = 15,
  q = 3) against y = +-127.
* fp32 outputs: |gpu - oracle| <= 1e-4 * sum_k |w a| for every checked (m, n).
Shapes: GEMV with one, two and four units per lane (K up to 53760), ragged N,
several activation rows, both layouts; GEMM with ragged row and column tiles,
K past the GEMV's limit; the small-batch kernel with 8, 16 and 32 staged rows,
ragged N, K not a multiple of eight super-blocks and several row chunks; and
AUTO dispatch.
"""
import struct

import numpy as np
import pytest

import oracle
import bit_quantized_mat_quantize_amd as qmm
from bit_quantized_mat_quantize_amd.inputs import activations, weights_t4_skewed
from gpu_helpers import assert_close, full_reference, to_dev, to_host

pytestmark = pytest.mark.gpu

LAYOUTS = ["canonical", "repacked"]
Q2K_MAX_K = 53760


def _upload(w, N, K, layout):
    wd = to_dev(np.ascontiguousarray(w).reshape(-1))
    return qmm.repack_weights(wd, "q2_K", N, K) if layout == "repacked" else wd


def _case(M, N, K, seed):
    w = oracle.quantize("q2_K", weights_t4_skewed([700, seed], N, K))
    y = oracle.quantize("q8_K", activations([701, seed], M, K, outlier_frac=0.01))
    return w, y


@pytest.mark.parametrize("N,K", [(1, 256), (7, 512), (33, 4096), (5, 14336)])
def test_encoder_bytes(N, K):
    x = weights_t4_skewed([702, N], N, K)
    x[0, :16] = 0.0                          # an all-zero group
    x[-1, 16:32] = np.abs(x[-1, 16:32])      # a group with no negative value (mn = 0)
    x[-1, 32:48] = np.float32(0.03)          # a constant group
    want = oracle.quantize("q2_K", x)
    got = to_host(qmm.quantize_weights(to_dev(x), "q2_K"))
    assert np.array_equal(got.reshape(-1), want.reshape(-1))


@pytest.mark.parametrize("N,K", [(1, 256), (9, 512), (130, 2048)])
def test_repack_bytes(N, K):
    w, _ = _case(1, N, K, N)
    want = oracle.repack("q2_K", w, N, K)
    got = to_host(qmm.repack_weights(to_dev(w.reshape(-1)), "q2_K", N, K))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("M,N,K", [(1, 5, 256), (2, 37, 4096), (3, 9, 14336), (1, 3, 33024)])
def test_group_sums_bit_exact(M, N, K, layout):
    w, y = _case(M, N, K, M * 100 + N)
    want = oracle.subblock_sums("q2_K", w, y, M, N, K)
    got = to_host(qmm.debug_block_sums("q2_K", _upload(w, N, K, layout), to_dev(y.reshape(-1)),
                                       M, N, K, layout=layout))
    assert np.array_equal(got, want)


def _q2k_block(d, dmin, scales, mins, codes):
    sc = bytes((int(s) & 15) | ((int(m) & 15) << 4) for s, m in zip(scales, mins))
    qs = bytearray(64)
    for k, q in enumerate(codes):
        h, rest = divmod(k, 128)
        sh, l = divmod(rest, 32)
        qs[32 * h + l] |= (int(q) & 3) << (2 * sh)
    return sc + bytes(qs) + struct.pack("<ee", d, dmin)


def _window(rng, N, K, dmin, scales, mins, codes):
    blocks = b"".join(_q2k_block(1.0, dmin, scales(rng), mins(rng), codes(rng))
                      for _ in range(N * K // 256))
    return np.frombuffer(blocks, np.uint8).reshape(N, -1)


@pytest.mark.parametrize("algo,M,N,K", [("gemv", 3, 41, 1024), ("mfma", 130, 300, 1024),
                                         ("skinny", 20, 70, 2304)])
@pytest.mark.parametrize("dmin", [0.0, 1.0])
def test_exactness_window(algo, M, N, K, dmin):
    rng = np.random.default_rng(21)
    w = _window(rng, N, K, dmin, lambda r: r.integers(0, 16, 16), lambda r: r.integers(0, 16, 16),
                lambda r: r.integers(0, 4, 256))
    x = rng.integers(-20, 21, (M, K)).astype(np.float32)
    x[:, ::256] = 127.0
    y = oracle.quantize("q8_K", x)
    want, terms = full_reference("q2_K", w, y, M, N, K)
    assert terms.max() < 2 ** 24
    for layout in (LAYOUTS if algo == "gemv" else ["repacked"]):
        got = to_host(qmm.mul_mat_q2_K(_upload(w, N, K, layout), to_dev(y.reshape(-1)), M, N, K,
                                       layout=layout, algo=algo))
        assert np.array_equal(got.astype(np.float64), want), layout


def test_saturated_window():
    """s = m = 15 and q = 3 everywhere against y = +-127: the largest group
    sums (|P_j| = 6096) and min terms the format allows, still exact."""
    M, N, K = 33, 40, 512
    rng = np.random.default_rng(22)
    w = _window(rng, N, K, 1.0, lambda r: np.full(16, 15), lambda r: np.full(16, 15),
                lambda r: np.full(256, 3))
    x = np.where(rng.random((M, K)) < 0.5, -127.0, 127.0).astype(np.float32)
    y = oracle.quantize("q8_K", x)
    want, terms = full_reference("q2_K", w, y, M, N, K)
    assert terms.max() < 2 ** 24
    for algo in ("gemv", "mfma", "skinny"):
        got = to_host(qmm.mul_mat_q2_K(_upload(w, N, K, "repacked"), to_dev(y.reshape(-1)), M, N, K,
                                       layout="repacked", algo=algo))
        assert np.array_equal(got.astype(np.float64), want), algo


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (1, 131, 3072), (4, 66, 4096), (2, 17, 14336),
                                   (1, 5, Q2K_MAX_K)])
def test_mul_mat_q2_K_gemv(M, N, K, layout):
    w, y = _case(M, N, K, 7 * M + N)
    want, terms = full_reference("q2_K", w, y, M, N, K)
    got = to_host(qmm.mul_mat_q2_K(_upload(w, N, K, layout), to_dev(y.reshape(-1)), M, N, K,
                                   layout=layout, algo="gemv"))
    assert_close(got, want, terms, f"q2_K gemv M={M} N={N} K={K} {layout}")


@pytest.mark.parametrize("M,N,K", [(9, 1, 256), (128, 256, 2048), (200, 257, 4096), (33, 40, Q2K_MAX_K + 256)])
def test_mul_mat_q2_K_mfma(M, N, K):
    w, y = _case(M, N, K, 11 * M + N)
    want, terms = full_reference("q2_K", w, y, M, N, K)
    got = to_host(qmm.mul_mat_q2_K(_upload(w, N, K, "repacked"), to_dev(y.reshape(-1)), M, N, K,
                                   layout="repacked", algo="mfma"))
    assert_close(got, want, terms, f"q2_K mfma M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", [(2, 70, 256), (5, 33, 512), (8, 300, 2048), (9, 64, 4608), (16, 40, 1024),
                                   (17, 1, 256), (32, 257, 1024), (40, 100, 2048), (70, 130, 4608),
                                   (3, 20, Q2K_MAX_K + 256)])
def test_mul_mat_q2_K_skinny(M, N, K):
    w, y = _case(M, N, K, 13 * M + N)
    want, terms = full_reference("q2_K", w, y, M, N, K)
    got = to_host(qmm.mul_mat_q2_K(_upload(w, N, K, "repacked"), to_dev(y.reshape(-1)), M, N, K,
                                   layout="repacked", algo="skinny"))
    assert_close(got, want, terms, f"q2_K skinny M={M} N={N} K={K}")


def test_skinny_overwrites_and_rejects():
    """The small-batch kernel writes every output, and refuses the canonical layout."""
    import torch
    M, N, K = 12, 50, 512
    w, y = _case(M, N, K, 77)
    want, terms = full_reference("q2_K", w, y, M, N, K)
    out = torch.full((M, N), float("nan"), device="cuda")
    qmm.mul_mat_q2_K(_upload(w, N, K, "repacked"), to_dev(y.reshape(-1)), M, N, K, layout="repacked",
                     algo="skinny", out=out)
    assert_close(to_host(out), want, terms, "q2_K skinny into a NaN-filled buffer")
    with pytest.raises(qmm.QmmError):
        qmm.mul_mat_q2_K(_upload(w, N, K, "canonical"), to_dev(y.reshape(-1)), M, N, K, layout="canonical",
                         algo="skinny")


SKINNY_MN = 6 * 8192


def _auto_algo(M, N, layout):
    """The AUTO rule as the library documents it (K within the GEMV's limit)."""
    if layout == "canonical" or M == 1 or (M == 2 and N < 8192):
        return "gemv"
    return "skinny" if (M + 31) // 32 * N <= SKINNY_MN else "mfma"


def test_auto_dispatch_and_fused():
    """AUTO (repacked): the GEMV for M = 1 and for M = 2 below 8192 columns,
    the small-batch kernel while ceil(M/32)*N <= SKINNY_MN, the GEMM above; the
    GEMV for the canonical layout.  AUTO is bit-identical to that path and
    agrees with the oracle; quantize_mul_mat equals quantize + mul_mat."""
    for M, N, K in ((1, 96, 2048), (2, 96, 2048), (8, 96, 2048), (64, 96, 2048), (64, 3400, 2048),
                    (2, 9000, 256), (3, 9000, 256), (64, 24576, 256), (65, 16400, 256)):
        w, _ = _case(M, N, K, 900 + M)
        x = activations([703, M], M, K)
        y = oracle.quantize("q8_K", x)
        want, terms = full_reference("q2_K", w, y, M, N, K)
        for layout in LAYOUTS:
            wd = _upload(w, N, K, layout)
            got = to_host(qmm.mul_mat_q2_K(wd, to_dev(y.reshape(-1)), M, N, K, layout=layout))
            assert_close(got, want, terms, f"q2_K auto M={M} N={N} {layout}")
            ref = to_host(qmm.mul_mat_q2_K(wd, to_dev(y.reshape(-1)), M, N, K, layout=layout,
                                           algo=_auto_algo(M, N, layout)))
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (M, N, layout)
            fused, yq = qmm.quantize_mul_mat("q2_K", wd, to_dev(x), N, layout=layout)
            assert np.array_equal(to_host(yq).reshape(-1), y.reshape(-1))
            assert np.array_equal(to_host(fused).view(np.uint32), got.view(np.uint32))
