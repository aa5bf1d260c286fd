"""Launch-size edges: the kernels whose activation rows or (token, slot) pairs
go to grid.y split them into launches of at most 65535; these cases cross that
split (rows or pairs 0, 65534, 65535, 65536 and the last one are checked
against the oracle), with tiny N and K so the oracle stays fast."""
import numpy as np
import pytest

import oracle
import bit_quantized_mat_quantize_amd as qmm
from bit_quantized_mat_quantize_amd.inputs import activations, weights_t4_skewed
from gpu_helpers import assert_close, to_dev, to_host

pytestmark = pytest.mark.gpu

EDGE = np.array([0, 1, 65534, 65535, 65536, 65537], np.int64)


@pytest.mark.parametrize("wfmt", ["q6_K", "q2_K"])
def test_gemv_rows_past_grid_limit(wfmt):
    M, N, K = 65538, 3, 256
    w = oracle.quantize(wfmt, weights_t4_skewed([910, 6 if wfmt == "q6_K" else 2], N, K))
    y = oracle.quantize("q8_K", activations([911, 0], M, K))
    fn = qmm.mul_mat_q6_K if wfmt == "q6_K" else qmm.mul_mat_q2_K
    got = to_host(fn(to_dev(w.reshape(-1)), to_dev(y.reshape(-1)), M, N, K, layout="canonical", algo="gemv"))
    ms = np.repeat(EDGE, N)
    ns = np.tile(np.arange(N), len(EDGE))
    want, terms = oracle.sample(wfmt, w, y, M, N, K, ms, ns)
    assert_close(got[ms, ns], want, terms, f"{wfmt} rows past 65535")


def test_mul_mat_id_pairs_past_grid_limit():
    T, U, E, N, K = 32769, 2, 4, 2, 256        # 65538 pairs through the per-pair GEMV
    w = np.concatenate([oracle.quantize("q4_K", weights_t4_skewed([912, e], N, K)) for e in range(E)])
    y = oracle.quantize("q8_K", activations([913, 0], T, K))
    rng = np.random.default_rng(914)
    ids = np.stack([rng.choice(E, U, replace=False) for _ in range(T)]).astype(np.int32)
    got = to_host(qmm.mul_mat_id_q4_K(to_dev(w.reshape(-1)), E, to_dev(y.reshape(-1)), to_dev(ids), N, K,
                                      algo="gemv"))
    pairs = EDGE
    ts, us = pairs // U, pairs % U
    sub_t = np.unique(ts)
    want, terms = oracle.mul_mat_id("q4_K", w, E, N, K, y.reshape(T, -1)[sub_t], ids[sub_t])
    for p, t, u in zip(pairs, ts, us):
        i = int(np.searchsorted(sub_t, t))
        assert_close(got[t, u], want[i, u], terms[i, u], f"pair {p}")
