"""The measured workloads at full size, in the launch configuration the
benchmark times (repacked weights, automatic GEMV/MFMA dispatch).

The weights are encoded on the GPU exactly as the benchmark does it and must be
byte-identical to the oracle's encoding; activations likewise.  Outputs are
compared element by element with the oracle for the GEMV workloads and on a
sample of (m, n) pairs for the prefill GEMM: one whole 128 x 256 workgroup
tile (every lane and result register of all eight wavefronts and four row
tiles), tile corners and random pairs.  The M = 1 workloads also run through
quantize_mul_mat (the fused form the benchmark times), which must give the
same Q8 bytes and the same outputs bit for bit.
"""
import numpy as np
import pytest

import oracle
import bit_quantized_mat_quantize_amd as qmm
from bit_quantized_mat_quantize_amd.inputs import workload
from gpu_helpers import assert_close, full_reference, to_dev, to_host

pytestmark = pytest.mark.gpu


def _run_projection(p, full: bool):
    afmt = qmm.ACT_FOR[p.wfmt]
    wf = p.weights()
    w_gpu = qmm.quantize_weights(to_dev(wf), p.wfmt)
    w_orc = oracle.quantize(p.wfmt, wf)
    assert np.array_equal(to_host(w_gpu), w_orc.reshape(-1)), f"{p.name}: weight bytes differ"
    x = p.acts()
    y_gpu = qmm.quantize_row_q8(to_dev(x), afmt)
    y_orc = oracle.quantize(afmt, x)
    assert np.array_equal(to_host(y_gpu), y_orc.reshape(-1)), f"{p.name}: activation bytes differ"
    wr = qmm.repack_weights(w_gpu, p.wfmt, p.N, p.K)
    got = to_host(qmm.mul_mat(p.wfmt, wr, y_gpu, p.M, p.N, p.K, layout="repacked"))
    if p.M == 1:
        out_f, y_f = qmm.quantize_mul_mat(p.wfmt, wr, to_dev(x), p.N, layout="repacked")
        assert np.array_equal(to_host(y_f).reshape(-1), y_orc.reshape(-1)), f"{p.name}: fused Q8 bytes differ"
        assert np.array_equal(to_host(out_f).view(np.uint32), got.view(np.uint32)), f"{p.name}: fused != two-call"
    if full:
        want, terms = full_reference(p.wfmt, w_orc, y_orc, p.M, p.N, p.K)
        assert_close(got, want, terms, p.name)
    else:
        rng = np.random.default_rng(7)
        ms = [0, p.M - 1] + [127, 128, 255, 256] + list(rng.integers(0, p.M, 2000))
        ns = [0, p.N - 1] + [127, 128, 129, 255] + list(rng.integers(0, p.N, 2000))
        ms = np.array([m for m in ms if m < p.M][: len(ns)], np.int64)
        ns = np.array(ns[: len(ms)], np.int64)
        # one whole workgroup tile of the last row tile: rows 128 t .. + 127, columns 256 c .. + 255
        t, c = (p.M - 1) // 128, int(rng.integers(0, p.N // 256))
        tm, tn = np.meshgrid(np.arange(128 * t, min(128 * t + 128, p.M)), np.arange(256 * c, 256 * c + 256),
                             indexing="ij")
        ms = np.concatenate([ms, tm.ravel()])
        ns = np.concatenate([ns, tn.ravel()])
        want, terms = oracle.sample(p.wfmt, w_orc, y_orc, p.M, p.N, p.K, ms, ns)
        assert_close(got[ms, ns], want, terms, p.name + " (sampled)")


@pytest.mark.parametrize("key", ["c1", "c2", "c3", "c4_m4", "c4_m8", "c4_m32", "q6K_c2", "q6K_down",
                                 "q2K_c2"])
def test_decode_workloads(key):
    for p in workload(key).projections:
        _run_projection(p, full=True)


@pytest.mark.parametrize("key", ["c5_m512", "c5_m2048", "q6K_c5_m512", "q2K_c5_m512", "q40_c5_m512"])
def test_prefill_workloads(key):
    for p in workload(key).projections:
        _run_projection(p, full=False)
