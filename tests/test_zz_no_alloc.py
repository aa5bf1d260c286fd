"""mul_mat_id without a workspace (qmm_mul_mat_id_noalloc), through the C ABI.

The entry point for callers that cannot allocate keeps the expert grouping in
the library's own per-GPU scratch array.  It must give what qmm_mul_mat_id with
a caller workspace gives (the same kernels, so bit for bit) and stay within the
oracle's tolerance, on two calls in a row where the second has fewer pairs (the
scratch keeps the first call's tables; the second must not read them).
"""
import numpy as np
import pytest

import oracle
import bit_quantized_mat_quantize_amd as qmm
from bit_quantized_mat_quantize_amd.inputs import activations, weights_t4_skewed
from gpu_helpers import assert_close, to_dev, to_host

pytestmark = pytest.mark.gpu


def _routing(rng, T, U, E):
    return np.stack([rng.choice(E, U, replace=False) for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("fmt", ["q4_K", "q6_K"])
def test_noalloc_matches_workspace_path_twice(fmt):
    E, N, K = 6, 200, 1024
    w = np.concatenate([oracle.quantize(fmt, weights_t4_skewed([850, e], N, K)) for e in range(E)])
    per = w.size // E
    wd0 = to_dev(w.reshape(-1))
    import torch
    wd = torch.cat([qmm.repack_weights(wd0[e * per:(e + 1) * per], fmt, N, K) for e in range(E)])
    rng = np.random.default_rng(851)
    for T, U in ((300, 3), (70, 2)):          # the second call is smaller
        print(f"noalloc {fmt} T={T} U={U} E={E} N={N} K={K}", flush=True)
        y = oracle.quantize("q8_K", activations([852, T], T, K, outlier_frac=0.01))
        ids = _routing(rng, T, U, E)
        yd, idd = to_dev(y.reshape(-1)), to_dev(ids)
        for algo in ("mfma", "auto"):
            ref = to_host(qmm.mul_mat_id(fmt, wd, E, yd, idd, N, K, layout="repacked", algo=algo))
            out = torch.full((T, U, N), float("nan"), dtype=torch.float32, device=yd.device)
            got = to_host(qmm.mul_mat_id_noalloc(fmt, wd, E, yd, idd, N, K, layout="repacked", algo=algo,
                                                 out=out))
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (fmt, T, algo)
            want, terms = oracle.mul_mat_id(fmt, w, E, N, K, y, ids, False)
            assert_close(got, want, terms, f"noalloc {fmt} T={T} {algo}")


def test_noalloc_bad_ids_and_gemv():
    """Out-of-range ids give NaN rows through the scratch path too; the GEMV
    path (no grouping) also works without a workspace."""
    E, N, K, T, U = 4, 64, 512, 90, 2
    w = np.concatenate([oracle.quantize("q4_K", weights_t4_skewed([853, e], N, K)) for e in range(E)])
    wd = to_dev(w.reshape(-1))
    rng = np.random.default_rng(854)
    y = oracle.quantize("q8_K", activations([855, 0], T, K))
    ids = _routing(rng, T, U, E)
    bad = ids.copy()
    bad[5, 1], bad[80, 0] = E, -1
    good = np.ones((T, U), bool)
    good[5, 1] = good[80, 0] = False
    want, terms = oracle.mul_mat_id("q4_K", w, E, N, K, y, np.where(good, bad, 0).astype(np.int32), False)
    for algo in ("mfma", "gemv"):
        got = to_host(qmm.mul_mat_id_noalloc("q4_K", wd, E, to_dev(y.reshape(-1)), to_dev(bad), N, K,
                                             layout="canonical", algo=algo))
        assert np.isnan(got[~good]).all(), algo
        assert_close(got[good], want[good], terms[good], f"noalloc {algo} with bad ids")
