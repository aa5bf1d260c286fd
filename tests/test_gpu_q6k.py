"""GPU Q6_K path against the oracle.

* GPU encoder and load-time repack: byte-identical to the oracle's.
* int32 group sums P[m][n][K/16] (the GEMV decode path): bit-exact.
* exactness windows (GEMV and MFMA GEMM): integer activations with amax = 127
  per block (d_a = 1), weights with d = 1 and scales/codes that keep every
  partial sum an integer below 2^24, so the fp32 outputs equal the integer
  result exactly -- including the extreme scales -128 and 127 with the extreme
  codes -32 and 31, the corners of the GEMM's digit split.
* fp32 outputs: |gpu - oracle| <= 1e-4 * sum_k |w a| for every checked (m, n).
Shapes: GEMV with one, two and four 16-byte piece units per lane (K <= 8192)
and two or four half-block units per lane (longer rows, K up to 53760, the last
with a second pass), ragged N, several activation rows, both layouts; GEMM with
ragged row and column tiles, K past the GEMV's limit, and AUTO dispatch; the
small-batch kernel with 8, 16 and 32 staged rows, several 32-row chunks, step
counts that leave wavefronts idle or uneven, and ragged N.
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
Q6K_MAX_K = 53760


def _upload(w, N, K, layout):
    wd = to_dev(np.ascontiguousarray(w).reshape(-1))
    return qmm.repack_weights(wd, "q6_K", N, K) if layout == "repacked" else wd


def _case(M, N, K, seed):
    w = oracle.quantize("q6_K", weights_t4_skewed([600, seed], N, K))
    y = oracle.quantize("q8_K", activations([601, seed], M, K, outlier_frac=0.01))
    return w, y


@pytest.mark.parametrize("N,K", [(1, 256), (7, 512), (33, 4096), (5, 14336)])
def test_encoder_bytes(N, K):
    x = weights_t4_skewed([602, N], N, K)
    x[0, :16] = 0.0                      # an all-zero group
    x[-1, 16:32] = np.float32(0.03)      # a group of equal magnitudes (first index wins)
    x[-1, 40] = np.float32(-0.03)
    want = oracle.quantize("q6_K", x)
    got = to_host(qmm.quantize_weights(to_dev(x), "q6_K"))
    assert np.array_equal(got.reshape(-1), want.reshape(-1))


@pytest.mark.parametrize("N,K", [(1, 256), (9, 512), (130, 2048)])
def test_repack_bytes(N, K):
    w, _ = _case(1, N, K, N)
    want = oracle.repack("q6_K", w, N, K)
    got = to_host(qmm.repack_weights(to_dev(w.reshape(-1)), "q6_K", N, K))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("M,N,K", [(1, 5, 256), (2, 37, 4096), (1, 6, 6144), (3, 9, 14336),
                                   (1, 3, 33024)])
def test_group_sums_bit_exact(M, N, K, layout):
    w, y = _case(M, N, K, M * 100 + N)
    want = oracle.subblock_sums("q6_K", w, y, M, N, K)
    got = to_host(qmm.debug_block_sums("q6_K", _upload(w, N, K, layout), to_dev(y.reshape(-1)),
                                       M, N, K, layout=layout))
    assert np.array_equal(got, want)


def _q6k_block(d, scales, codes):
    ql = bytearray(128)
    qh = bytearray(64)
    for k, q in enumerate(codes):
        u = int(q) + 32
        g, r = divmod(k, 64)
        ql[32 * g + r % 32] |= (u & 15) << (0 if r < 32 else 4)
        qh[r] |= ((u >> 4) & 3) << (2 * g)
    return bytes(ql) + bytes(qh) + np.asarray(scales, np.int8).tobytes() + struct.pack("<e", d)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_exactness_window(layout):
    M, N, K = 3, 41, 1024
    rng = np.random.default_rng(11)
    blocks = b"".join(_q6k_block(1.0, rng.integers(-3, 4, 16), rng.integers(-32, 32, 256))
                      for _ in range(N * K // 256))
    w = np.frombuffer(blocks, np.uint8).reshape(N, -1)
    x = rng.integers(-20, 21, (M, K)).astype(np.float32)
    x[:, ::256] = 127.0
    y = oracle.quantize("q8_K", x)
    want, terms = full_reference("q6_K", w, y, M, N, K)
    assert terms.max() < 2 ** 24
    got = to_host(qmm.mul_mat_q6_K(_upload(w, N, K, layout), to_dev(y.reshape(-1)), M, N, K,
                                   layout=layout))
    assert np.array_equal(got.astype(np.float64), want)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (1, 131, 3072), (4, 66, 4096), (1, 9, 6144),
                                   (2, 12, 8192), (2, 17, 14336), (1, 5, Q6K_MAX_K)])
def test_mul_mat_q6_K(M, N, K, layout):
    w, y = _case(M, N, K, 7 * M + N)
    want, terms = full_reference("q6_K", w, y, M, N, K)
    got = to_host(qmm.mul_mat_q6_K(_upload(w, N, K, layout), to_dev(y.reshape(-1)), M, N, K,
                                   layout=layout))
    assert_close(got, want, terms, f"q6_K M={M} N={N} K={K} {layout}")


def test_full_size_sampled():
    """N = K = 4096, M = 1 on sampled outputs, and through quantize_mul_mat."""
    M, N, K = 1, 4096, 4096
    w = oracle.quantize("q6_K", weights_t4_skewed([603, 0], N, K))
    x = activations([604, 0], M, K)
    y = oracle.quantize("q8_K", x)
    wd = _upload(w, N, K, "repacked")
    got = to_host(qmm.mul_mat_q6_K(wd, to_dev(y.reshape(-1)), M, N, K, layout="repacked"))
    fused, yq = qmm.quantize_mul_mat("q6_K", wd, to_dev(x), N, layout="repacked")
    assert np.array_equal(to_host(yq).reshape(-1), y.reshape(-1))
    assert np.array_equal(to_host(fused).view(np.uint32), got.view(np.uint32))
    ns = np.arange(0, N, 7)
    want, terms = oracle.sample("q6_K", w, y, M, N, K, np.zeros_like(ns), ns)
    assert_close(got[0, ns], want, terms, "q6_K 4096^2 sampled")


# ---------------------------------------------------------------- MFMA GEMM
def _window_blocks(rng, N, K, scales, codes):
    return np.frombuffer(b"".join(_q6k_block(1.0, scales(rng), codes(rng))
                                  for _ in range(N * K // 256)), np.uint8).reshape(N, -1)


def test_mfma_exactness_window():
    """Ragged tiles (M = 130, N = 300), d = 1, d_a = 1, small scales: exact."""
    M, N, K = 130, 300, 1024
    rng = np.random.default_rng(12)
    w = _window_blocks(rng, N, K, lambda r: r.integers(-3, 4, 16), lambda r: r.integers(-32, 32, 256))
    x = rng.integers(-20, 21, (M, K)).astype(np.float32)
    x[:, ::256] = 127.0
    y = oracle.quantize("q8_K", x)
    want, terms = full_reference("q6_K", w, y, M, N, K)
    assert terms.max() < 2 ** 24
    for algo in ("mfma", "skinny"):
        got = to_host(qmm.mul_mat_q6_K(_upload(w, N, K, "repacked"), to_dev(y.reshape(-1)), M, N, K,
                                       layout="repacked", algo=algo))
        assert np.array_equal(got.astype(np.float64), want), algo


def test_mfma_extreme_digits():
    """Scales in {-128, -127, -1, 0, 1, 127} and codes in {-32, -31, 0, 31}
    (t = s*q spans [-4064, 4096], both ends of the 256*hi + lo split), with
    activations that are 0 or +-1 apart from one 127 per block: every sum is an
    integer below 2^24, so the outputs are exact."""
    M, N, K = 40, 70, 512
    rng = np.random.default_rng(13)
    w = _window_blocks(rng, N, K, lambda r: r.choice([-128, -127, -1, 0, 1, 127], 16),
                       lambda r: r.choice([-32, -31, 0, 31], 256))
    x = rng.integers(-1, 2, (M, K)).astype(np.float32)
    x[:, ::256] = 127.0
    y = oracle.quantize("q8_K", x)
    want, terms = full_reference("q6_K", w, y, M, N, K)
    assert terms.max() < 2 ** 24
    for algo in ("mfma", "gemv", "skinny"):
        got = to_host(qmm.mul_mat_q6_K(_upload(w, N, K, "repacked"), to_dev(y.reshape(-1)), M, N,
                                       K, layout="repacked", algo=algo))
        assert np.array_equal(got.astype(np.float64), want), algo


@pytest.mark.parametrize("M,N,K", [(9, 1, 256), (128, 256, 2048), (200, 257, 4096), (33, 40, Q6K_MAX_K + 256)])
def test_mul_mat_q6_K_mfma(M, N, K):
    w, y = _case(M, N, K, 11 * M + N)
    want, terms = full_reference("q6_K", w, y, M, N, K)
    got = to_host(qmm.mul_mat_q6_K(_upload(w, N, K, "repacked"), to_dev(y.reshape(-1)), M, N, K,
                                   layout="repacked", algo="mfma"))
    assert_close(got, want, terms, f"q6_K mfma M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", [(2, 70, 256), (5, 33, 512), (8, 300, 2048), (9, 64, 4608), (16, 40, 1024),
                                   (17, 1, 256), (32, 257, 1024), (40, 100, 2048), (70, 130, 4608)])
def test_mul_mat_q6_K_skinny(M, N, K):
    w, y = _case(M, N, K, 13 * M + N)
    want, terms = full_reference("q6_K", w, y, M, N, K)
    got = to_host(qmm.mul_mat_q6_K(_upload(w, N, K, "repacked"), to_dev(y.reshape(-1)), M, N, K,
                                   layout="repacked", algo="skinny"))
    assert_close(got, want, terms, f"q6_K skinny M={M} N={N} K={K}")


def test_skinny_overwrites_and_rejects():
    """The small-batch kernel writes every output, and refuses the canonical layout."""
    import torch
    M, N, K = 12, 50, 512
    w, y = _case(M, N, K, 77)
    want, terms = full_reference("q6_K", w, y, M, N, K)
    out = torch.full((M, N), float("nan"), device="cuda")
    qmm.mul_mat_q6_K(_upload(w, N, K, "repacked"), to_dev(y.reshape(-1)), M, N, K, layout="repacked",
                     algo="skinny", out=out)
    assert_close(to_host(out), want, terms, "q6_K skinny into a NaN-filled buffer")
    with pytest.raises(qmm.QmmError):
        qmm.mul_mat_q6_K(_upload(w, N, K, "canonical"), to_dev(y.reshape(-1)), M, N, K, layout="canonical",
                         algo="skinny")


def _auto_algo(M, N, layout):
    """The AUTO rule as the library documents it (K within the GEMV's limit)."""
    if layout == "canonical" or M == 1 or (M == 2 and N < 8192):
        return "gemv"
    return "skinny" if (M + 31) // 32 * N <= 8 * 8192 else "mfma"


def test_auto_dispatch():
    """AUTO (repacked): the GEMV for M = 1 and for M = 2 below 8192 columns, the
    small-batch kernel while ceil(M/32)*N <= 8*8192, the GEMM above; the GEMV
    for the canonical layout at any M.  AUTO is bit-identical to that path and
    agrees with the oracle."""
    for M, N, K in ((1, 96, 2048), (2, 96, 2048), (2, 8192, 512), (8, 96, 2048), (64, 2100, 2048),
                    (64, 32768, 256), (65, 22000, 256)):
        w, y = _case(M, N, K, 900 + M)
        want, terms = full_reference("q6_K", w, y, M, N, K)
        for layout in LAYOUTS:
            wd, yd = _upload(w, N, K, layout), to_dev(y.reshape(-1))
            got = to_host(qmm.mul_mat_q6_K(wd, yd, M, N, K, layout=layout))
            assert_close(got, want, terms, f"q6_K auto M={M} N={N} {layout}")
            algo = _auto_algo(M, N, layout)
            ref = to_host(qmm.mul_mat_q6_K(wd, yd, M, N, K, layout=layout, algo=algo))
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (M, N, layout, algo)
    assert {_auto_algo(M, N, "repacked") for M, N in ((2, 96), (64, 32768), (65, 22000))} == {"gemv", "skinny", "mfma"}
