"""GPU quantize_mul_mat (quantize + mul_mat in one call) against the oracle.

For Q4_K with M = 1 the activation row is quantized inside the GEMV launch.
Checks, on the same seeded inputs:
* the Q8 bytes it returns equal the oracle's quantizer (bit-exact);
* the fp32 outputs are within 1e-4 * sum_k |w a| of the oracle;
* the outputs equal, bit for bit, those of quantize_row_q8 followed by
  mul_mat (the same per-row arithmetic in the same order).
Shapes cover one, two, four and eight pieces per lane (eight: the first row's
requests split around the quantization), rows looped over by the persistent
workgroups (N above 16 rows per CU, also with eight pieces), ragged N tails,
the largest K of the one-launch kernel and K above it (two-launch path),
M > 1, and the one-launch kernels of Q4_0, Q6_K and Q2_K.
"""
import numpy as np
import pytest

import oracle
import bit_quantized_mat_quantize_amd as qmm
from bit_quantized_mat_quantize_amd.inputs import activations, weights_normal, weights_t4_skewed
from gpu_helpers import assert_close, full_reference, to_dev, to_host, upload_weights

pytestmark = pytest.mark.gpu

FUSED_MAX_K = 16384  # largest K of the one-launch path (eight 16-byte pieces per lane)


def _inputs(wfmt, M, N, K, seed):
    if wfmt in ("q4_K", "q6_K", "q2_K"):
        w = oracle.quantize(wfmt, weights_t4_skewed([500, seed], N, K))
        x = activations([501, seed], M, K, outlier_frac=0.01)
    else:
        w = oracle.quantize("q4_0", weights_normal([502, seed], N, K))
        x = activations([503, seed], M, K)
    return w, x


def _check(wfmt, M, N, K, layout, seed, sample=None):
    import torch
    afmt = "q8_0" if wfmt == "q4_0" else "q8_K"
    w, x = _inputs(wfmt, M, N, K, seed)
    y_want = oracle.quantize(afmt, x)
    wd = upload_weights(wfmt, w, N, K, layout)
    xd = to_dev(x)
    out, y = qmm.quantize_mul_mat(wfmt, wd, xd, N, layout=layout)
    got, got_y = to_host(out), to_host(y)
    assert np.array_equal(got_y.reshape(-1), y_want.reshape(-1)), "Q8 bytes differ from the oracle"
    # the two-call path on the same device bytes
    y2 = qmm.quantize_row_q8(xd, afmt)
    ref = to_host(qmm.mul_mat(wfmt, wd, y2, M, N, K, layout=layout))
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), "fused != quantize + mul_mat"
    if sample is None:
        want, terms = full_reference(wfmt, w, y_want, M, N, K)
        assert_close(got, want, terms, f"{wfmt} M={M} N={N} K={K} {layout}")
    else:
        rng = np.random.default_rng(seed)
        ms = rng.integers(0, M, sample)
        ns = rng.integers(0, N, sample)
        ns[:2] = [0, N - 1]
        want, terms = oracle.sample(wfmt, w, y_want, M, N, K, ms, ns)
        assert_close(got[ms, ns], want, terms, f"{wfmt} M={M} N={N} K={K} {layout} sampled")
    torch.cuda.synchronize()


@pytest.mark.parametrize("layout", ["canonical", "repacked"])
@pytest.mark.parametrize("N,K", [(1, 256), (7, 512), (131, 2048), (64, 4096), (77, 8192),
                                 (45, 14336), (19, 20480), (9000, 1024), (5003, 4096), (4500, 16384),
                                 (4200, 12288)])
def test_fused_q4_K_m1(N, K, layout):
    _check("q4_K", 1, N, K, layout, seed=N * 7 + K)


@pytest.mark.parametrize("K", [FUSED_MAX_K, FUSED_MAX_K + 256])
def test_fused_q4_K_m1_k_limit(K):
    """The largest one-launch K and the first one that takes the two-launch path."""
    _check("q4_K", 1, 9, K, "repacked", seed=K, sample=None)


@pytest.mark.parametrize("M,N,K", [(2, 33, 1024), (8, 17, 512), (40, 96, 1024)])
def test_quantize_mul_mat_q4_K_multi_row(M, N, K):
    _check("q4_K", M, N, K, "repacked", seed=M * 31 + N)


@pytest.mark.parametrize("M,N,K", [(1, 256, 1024), (5, 41, 96)])
def test_quantize_mul_mat_q4_0(M, N, K):
    _check("q4_0", M, N, K, "repacked", seed=M * 13 + N)


@pytest.mark.parametrize("layout", ["canonical", "repacked"])
@pytest.mark.parametrize("N,K", [(77, 64), (3, 4096), (1024, 4096), (4096, 1024), (4097, 1024), (10, 96),
                                 (1, 4160), (3, 16384)])
def test_fused_q4_0_m1(N, K, layout):
    """Q4_0 at M = 1: one launch (quantization in every workgroup) for K % 64 == 0,
    K <= 4096 and N*K <= 2^22 -- one to four 32-block quantization passes (the
    first with its values and each lane's first weight block requested ahead),
    fewer than 32 blocks, the N*K limit itself -- and two launches past those
    limits."""
    _check("q4_0", 1, N, K, layout, seed=N * 3 + K)


def test_fused_full_size_headline_shape():
    """N = K = 4096, M = 1 (the decode shape) on sampled outputs."""
    _check("q4_K", 1, 4096, 4096, "repacked", seed=4096, sample=3000)


def test_fused_gate_up_concatenated():
    """gate||up as one N = 2*14336 matrix: equals the two projections computed apart."""
    import torch
    K, Nh = 4096, 14336
    rng_seed = 77
    w_gate = oracle.quantize("q4_K", weights_t4_skewed([510, 0], Nh, K))
    w_up = oracle.quantize("q4_K", weights_t4_skewed([510, 1], Nh, K))
    x = activations([511, rng_seed], 1, K)
    cat = np.concatenate([w_gate.reshape(-1), w_up.reshape(-1)])
    wd = upload_weights("q4_K", cat, 2 * Nh, K, "repacked")
    out, y = qmm.quantize_mul_mat("q4_K", wd, to_dev(x), 2 * Nh, layout="repacked")
    got = to_host(out)
    y_host = oracle.quantize("q8_K", x)
    assert np.array_equal(to_host(y).reshape(-1), y_host.reshape(-1))
    for half, wc in enumerate((w_gate, w_up)):
        g = to_host(qmm.mul_mat_q4_K(upload_weights("q4_K", wc, Nh, K, "repacked"),
                                     to_dev(y_host.reshape(-1)), 1, Nh, K, layout="repacked"))
        assert np.array_equal(got[:, half * Nh:(half + 1) * Nh].view(np.uint32), g.view(np.uint32))
    ns = np.arange(0, 2 * Nh, 97)
    want, terms = oracle.sample("q4_K", cat, y_host, 1, 2 * Nh, K, np.zeros_like(ns), ns)
    assert_close(got[0, ns], want, terms, "gate||up sampled")
    torch.cuda.synchronize()


def test_fused_zero_rows_and_quantize_only():
    """N = 0 quantizes only; M = 0 is an empty call."""
    import torch
    K = 1024
    x = activations([520, 0], 1, K)
    xd = to_dev(x)
    y = torch.full((qmm.act_bytes("q8_K", 1, K),), 0xAB, dtype=torch.uint8, device=xd.device)
    w = torch.zeros(16, dtype=torch.uint8, device=xd.device)
    out = torch.zeros(4, dtype=torch.float32, device=xd.device)
    qmm.quantize_mul_mat("q4_K", w, xd, 0, y=y, out=out)
    assert np.array_equal(to_host(y), oracle.quantize("q8_K", x).reshape(-1))
    x0 = torch.zeros((0, K), dtype=torch.float32, device=xd.device)
    qmm.quantize_mul_mat("q4_K", w, x0, 4, y=y, out=out)


def test_fused_graph_replay():
    """Captured in a HIP graph, replays equal the eager result."""
    import torch
    N, K = 96, 4096
    w, x = _inputs("q4_K", 1, N, K, 9)
    wd = upload_weights("q4_K", w, N, K, "repacked")
    xd = to_dev(x)
    eager, _ = qmm.quantize_mul_mat("q4_K", wd, xd, N, layout="repacked")
    eager = to_host(eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    y = torch.empty(qmm.act_bytes("q8_K", 1, K), dtype=torch.uint8, device=xd.device)
    out = torch.empty((1, N), dtype=torch.float32, device=xd.device)
    with torch.cuda.stream(s):
        qmm.quantize_mul_mat("q4_K", wd, xd, N, layout="repacked", y=y, out=out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        qmm.quantize_mul_mat("q4_K", wd, xd, N, layout="repacked", y=y, out=out)
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(out).view(np.uint32), eager.view(np.uint32))


@pytest.mark.parametrize("layout", ["canonical", "repacked"])
@pytest.mark.parametrize("N,K", [(77, 256), (4096, 4096), (8192, 1024), (100, 8192), (4096, 8192),
                                 (8193, 1024), (4097, 8192), (3, 8448)])
def test_fused_q6_K_m1(N, K, layout):
    """Q6_K at M = 1: one launch (quantization in every workgroup) for K <= 4096
    and N <= 32 rows per CU (one or two rows per wavefront, one or two piece
    units per lane) and for K <= 8192 and N <= 16 rows per CU (one row of four
    units), and two launches just past those limits."""
    sample = 3000 if N * K > (1 << 24) else None
    _check("q6_K", 1, N, K, layout, seed=N * 5 + K, sample=sample)


@pytest.mark.parametrize("layout", ["canonical", "repacked"])
@pytest.mark.parametrize("N,K", [(77, 256), (4096, 4096), (8192, 1024), (100, 8192), (4100, 12288),
                                 (5, 16384), (8193, 1024), (3, 16640)])
def test_fused_q2_K_m1(N, K, layout):
    """Q2_K at M = 1: one launch (quantization in every workgroup) for K <= 16384
    and N <= 32 rows per CU -- one and two rows per wavefront, one, two and
    four units per lane -- and two launches just past those limits."""
    sample = 3000 if N * K > (1 << 24) else None
    _check("q2_K", 1, N, K, layout, seed=N * 7 + K, sample=sample)
