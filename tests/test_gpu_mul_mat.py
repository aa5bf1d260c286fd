"""GPU mul_mat against the oracle.

* int32 per-(sub-)block sums: bit-exact (qmm_debug_block_sums uses the GEMV
  decode and dot-product code).
* exactness windows through the public entry points: integer activations with
  amax = 127 per block give d_a = 1 exactly; weights with d = 1 and dmin in
  {0, 1} and small codes keep every partial sum below 2^24, so the fp32 output
  must equal the integer result exactly, in any summation order.
* fp32 outputs: |gpu - oracle| <= 1e-4 * sum_k |w a| for every checked (m, n).
"""
import numpy as np
import pytest

import oracle
import bit_quantized_mat_quantize_amd as qmm
from bit_quantized_mat_quantize_amd.inputs import activations, weights_normal, weights_t4_skewed
from gpu_helpers import assert_close, full_reference, to_dev, to_host, upload_weights

pytestmark = pytest.mark.gpu

LAYOUTS = ["canonical", "repacked"]


def _case(wfmt, M, N, K, seed):
    if wfmt == "q4_K":
        w = oracle.quantize("q4_K", weights_t4_skewed([400, seed], N, K))
        x = activations([401, seed], M, K, outlier_frac=0.01)
        afmt = "q8_K"
    else:
        w = oracle.quantize("q4_0", weights_normal([402, seed], N, K))
        x = activations([403, seed], M, K)
        afmt = "q8_0"
    y = oracle.quantize(afmt, x)
    return w, x, y, afmt


# ------------------------------------------------------------ int32 sums
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("wfmt,M,N,K", [("q4_K", 1, 5, 256), ("q4_K", 3, 37, 1024),
                                        ("q4_K", 8, 66, 2048), ("q4_K", 11, 9, 512),
                                        ("q4_0", 1, 3, 32), ("q4_0", 5, 41, 1024),
                                        ("q4_0", 9, 7, 96)])
def test_block_sums_bit_exact(wfmt, M, N, K, layout):
    w, x, y, afmt = _case(wfmt, M, N, K, M * 1000 + N)
    want = oracle.subblock_sums(wfmt, w, y, M, N, K)
    wd = upload_weights(wfmt, w, N, K, layout)
    got = to_host(qmm.debug_block_sums(wfmt, wd, to_dev(y.reshape(-1)), M, N, K, layout=layout))
    assert np.array_equal(got, want)


def test_block_sums_saturated_codes():
    """q = 15 against y = +-127 everywhere: |P_j| = 60960, the largest value."""
    M, N, K = 2, 3, 512
    w = oracle.quantize("q4_K", np.ones((N, K), np.float32))  # all q = 15 after the search
    codes = np.frombuffer(w.tobytes(), np.uint8).reshape(N, -1, 144)[:, :, 16:]
    assert (codes == 0xFF).all()
    x = np.full((M, K), 127.0, np.float32)
    x[1] = -127.0
    y = oracle.quantize("q8_K", x)
    want = oracle.subblock_sums("q4_K", w, y, M, N, K)
    assert np.abs(want).max() == 60960
    got = to_host(qmm.debug_block_sums("q4_K", to_dev(w.reshape(-1)), to_dev(y.reshape(-1)),
                                       M, N, K))
    assert np.array_equal(got, want)


# ------------------------------------------------------ exactness windows
def _window_weights(N, K, rng, dmin_one=True, smax=3, qmax=15, mmax=7):
    import struct
    blocks = bytearray()
    nbk = K // 256
    for _ in range(N * nbk):
        s = [int(v) for v in rng.integers(0, smax + 1, 8)]
        m = [int(v) for v in rng.integers(0, mmax + 1, 8)] if dmin_one else [0] * 8
        q = rng.integers(0, qmax + 1, 256)
        qs = bytearray(128)
        for g in range(4):
            for l in range(32):
                qs[32 * g + l] = int(q[64 * g + l] | (q[64 * g + 32 + l] << 4))
        blocks += struct.pack("<e", 1.0) + struct.pack("<e", 1.0 if dmin_one else 0.0)
        blocks += oracle.pack_scales(s, m).tobytes() + bytes(qs)
    return np.frombuffer(bytes(blocks), np.uint8).reshape(N, -1)


@pytest.mark.parametrize("algo,M,N,K", [("gemv", 1, 70, 1024), ("gemv", 8, 33, 2048),
                                        ("mfma", 1, 130, 512), ("mfma", 40, 257, 1024),
                                        ("mfma", 129, 64, 2048), ("skinny", 2, 70, 1024),
                                        ("skinny", 16, 8230, 512), ("skinny", 32, 33, 4608)])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_exactness_window_q4_K(algo, M, N, K, layout):
    rng = np.random.default_rng(M * 7 + N)
    w = _window_weights(N, K, rng)
    # integer activations, every block holding +-127 once: d_a = 1 exactly
    x = rng.integers(-20, 21, (M, K)).astype(np.float32)
    x[:, ::256] = 127.0
    y = oracle.quantize("q8_K", x)
    assert (np.frombuffer(y.tobytes(), np.uint8).reshape(M, -1, 292)[:, :, :4].view(np.float32) == 1.0).all()
    want, terms = full_reference("q4_K", w, y, M, N, K)
    # every partial sum is an integer below 2^24 in magnitude: fp32 is exact
    assert terms.max() < 2 ** 24
    wd = upload_weights("q4_K", w, N, K, layout)
    got = to_host(qmm.mul_mat_q4_K(wd, to_dev(y.reshape(-1)), M, N, K, layout=layout, algo=algo))
    assert np.array_equal(got.astype(np.float64), want), \
        f"max |diff| {np.abs(got - want).max()}"


@pytest.mark.parametrize("layout", LAYOUTS)
def test_exactness_window_q4_0(layout):
    M, N, K = 3, 50, 1024
    rng = np.random.default_rng(5)
    import struct
    q = rng.integers(0, 16, (N, K))
    blocks = bytearray()
    for n in range(N):
        for b in range(K // 32):
            qq = q[n, 32 * b:32 * b + 32]
            blocks += struct.pack("<e", 1.0) + bytes(int(qq[l] | (qq[l + 16] << 4)) for l in range(16))
    w = np.frombuffer(bytes(blocks), np.uint8).reshape(N, -1)
    x = rng.integers(-40, 41, (M, K)).astype(np.float32)
    x[:, ::32] = 127.0    # amax 127 per 32-block: d_a = 1 (exact in fp16)
    y = oracle.quantize("q8_0", x)
    want, terms = full_reference("q4_0", w, y, M, N, K)
    assert terms.max() < 2 ** 24
    wd = upload_weights("q4_0", w, N, K, layout)
    got = to_host(qmm.mul_mat_q4_0(wd, to_dev(y.reshape(-1)), M, N, K, layout=layout))
    assert np.array_equal(got.astype(np.float64), want)


def test_special_scale_cases():
    """s_j = 0 (min term only), m_j = 0 (symmetric), d = dmin = 0 (zero block),
    through GEMV and MFMA."""
    import struct
    rng = np.random.default_rng(77)
    N, K, M = 40, 512, 33
    blocks = bytearray()
    for n in range(N):
        for b in range(K // 256):
            kind = (n + b) % 4
            s = [0] * 8 if kind == 0 else [int(v) for v in rng.integers(0, 64, 8)]
            m = [0] * 8 if kind == 1 else [int(v) for v in rng.integers(0, 64, 8)]
            d, dmin = (0.0, 0.0) if kind == 2 else (float(rng.uniform(1e-4, 1e-3)), float(rng.uniform(1e-4, 1e-3)))
            q = rng.integers(0, 16, 256)
            qs = bytes(int(q[64 * g + l] | (q[64 * g + 32 + l] << 4)) for g in range(4) for l in range(32))
            blocks += struct.pack("<e", d) + struct.pack("<e", dmin) + oracle.pack_scales(s, m).tobytes() + qs
    w = np.frombuffer(bytes(blocks), np.uint8).reshape(N, -1)
    y = oracle.quantize("q8_K", activations(78, M, K))
    want, terms = full_reference("q4_K", w, y, M, N, K)
    yd = to_dev(y.reshape(-1))
    for algo, mm in (("gemv", 8), ("mfma", M), ("skinny", 16), ("skinny", 32)):
        got = to_host(qmm.mul_mat_q4_K(to_dev(w.reshape(-1)), yd, mm, N, K, algo=algo))
        assert_close(got, want[:mm], terms[:mm], f"special {algo}")


# --------------------------------------------------------- fp32 parity
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
def test_gemv_q4_K(M, layout):
    N, K = 131, 3072   # ragged N (not a multiple of the 4-wave block), 12 super-blocks
    w, x, y, _ = _case("q4_K", M, N, K, 10 + M)
    want, terms = full_reference("q4_K", w, y, M, N, K)
    wd = upload_weights("q4_K", w, N, K, layout)
    got = to_host(qmm.mul_mat_q4_K(wd, to_dev(y.reshape(-1)), M, N, K, layout=layout, algo="gemv"))
    assert_close(got, want, terms, f"gemv M={M} {layout}")


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (9, 130, 512), (31, 257, 1024), (33, 128, 768),
                                   (128, 128, 256), (200, 333, 2048), (257, 65, 1280)])
def test_mfma_q4_K(M, N, K, layout):
    w, x, y, _ = _case("q4_K", M, N, K, M + 3 * N)
    want, terms = full_reference("q4_K", w, y, M, N, K)
    wd = upload_weights("q4_K", w, N, K, layout)
    got = to_host(qmm.mul_mat_q4_K(wd, to_dev(y.reshape(-1)), M, N, K, layout=layout, algo="mfma"))
    assert_close(got, want, terms, f"mfma M={M} N={N} K={K} {layout}")


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("M,N,K", [(2, 1, 256), (2, 33, 512), (3, 100, 2304), (5, 64, 4096),
                                   (8, 257, 6144), (9, 40, 1536), (16, 64, 2560), (17, 45, 1024),
                                   (32, 96, 3840), (1, 70, 2048), (40, 50, 1024), (65, 33, 512),
                                   (97, 70, 2304), (4, 8200, 768), (13, 8192, 512), (16, 9000, 1280),
                                   (7, 6000, 1280), (6, 17, 3328), (1, 4100, 512), (32, 8200, 768),
                                   (20, 16400, 512), (25, 4100, 1280), (31, 33, 2304), (32, 8192, 256),
                                   (12, 16400, 512), (10, 4100, 1280)])
def test_skinny_q4_K(M, N, K, layout):
    """Small-batch MFMA paths: ragged N, K splits of 1..3 super-blocks per
    wavefront (odd and even counts, wavefronts without work); up to 8 rows
    of the repacked layout the producer/consumer ring kernel (stages of four
    super-blocks with 1..3 of them past K; one, two and three or more
    workgroups per CU, i.e. 3, 2 and 1 stages in flight), from 9 to 32 rows
    of the repacked layout the ring with one or two 16-row blocks (16 columns
    per workgroup below N = 8192, 32 from there; one or two stages in flight;
    stages with super-blocks past K), the 16 x 16-tile kernel up to 16 rows of
    the canonical layout (8 wavefronts per 16 columns below N = 8192), and the
    32 x 32 kernel above with 8, 16 and 32 staged activation rows and several
    32-row chunks (grid.y) with a ragged last chunk."""
    w, x, y, _ = _case("q4_K", M, N, K, 7 * M + N)
    want, terms = full_reference("q4_K", w, y, M, N, K)
    wd = upload_weights("q4_K", w, N, K, layout)
    got = to_host(qmm.mul_mat_q4_K(wd, to_dev(y.reshape(-1)), M, N, K, layout=layout, algo="skinny"))
    assert_close(got, want, terms, f"skinny M={M} N={N} K={K} {layout}")


def test_skinny_rejects_unsupported():
    with pytest.raises(qmm.QmmError):   # K not a multiple of 256
        qmm.mul_mat_q4_K(to_dev(np.zeros(64 * 144, np.uint8)), to_dev(np.zeros(33 * 292, np.uint8)),
                         33, 64, 200, algo="skinny")


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("M,N,K", [(1, 256, 1024), (3, 77, 4096), (8, 9, 64), (13, 40, 512)])
def test_q4_0(M, N, K, layout):
    w, x, y, _ = _case("q4_0", M, N, K, M + N)
    want, terms = full_reference("q4_0", w, y, M, N, K)
    wd = upload_weights("q4_0", w, N, K, layout)
    got = to_host(qmm.mul_mat_q4_0(wd, to_dev(y.reshape(-1)), M, N, K, layout=layout))
    assert_close(got, want, terms, f"q4_0 M={M} N={N} K={K} {layout}")


def test_auto_dispatch_and_overwrite():
    """AUTO picks the GEMV for M = 1, the small-batch kernels up to M = 32
    and while ceil(M/32)*N <= 9*8192, the GEMM above, and is bit-identical to
    that path; `out` is overwritten."""
    import torch
    K = 512
    for M, N in ((1, 64), (2, 64), (2, 8192), (8, 64), (9, 64), (32, 64), (33, 64), (100, 64), (33, 40000)):
        w, x, y, _ = _case("q4_K", M, N, K, 900 + M)
        want, terms = full_reference("q4_K", w, y, M, N, K)
        wd, yd = to_dev(w.reshape(-1)), to_dev(y.reshape(-1))
        out = torch.full((M, N), 1e9, device="cuda")
        qmm.mul_mat_q4_K(wd, yd, M, N, K, out=out)
        assert_close(to_host(out), want, terms, f"auto M={M} N={N}")
        algo = ("gemv" if M == 1 else
                "skinny" if M <= 32 or (M + 31) // 32 * N <= 9 * 8192 else "mfma")
        ref = to_host(qmm.mul_mat_q4_K(wd, yd, M, N, K, algo=algo))
        assert np.array_equal(to_host(out).view(np.uint32), ref.view(np.uint32)), (M, N, algo)


def test_end_to_end_quantize_then_mul_mat():
    """fp32 activations quantized on the GPU feed mul_mat directly."""
    M, N, K = 5, 96, 2048
    w, x, y, _ = _case("q4_K", M, N, K, 55)
    yd = qmm.quantize_row_q8(to_dev(x), "q8_K")
    assert np.array_equal(to_host(yd), y.reshape(-1))
    want, terms = full_reference("q4_K", w, y, M, N, K)
    got = to_host(qmm.mul_mat_q4_K(to_dev(w.reshape(-1)), yd, M, N, K))
    assert_close(got, want, terms, "end to end")
