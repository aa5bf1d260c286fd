"""Shared helpers for the GPU parity tests: inputs come from the seeded
generators, expected values from the oracle, results from the HIP library."""
import numpy as np

import oracle
import bit_quantized_mat_quantize_amd as qmm

TOL = 1e-4   # |gpu - oracle| <= TOL * sum_k |w a|  (fp32 outputs)


def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def to_dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def to_host(t) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def upload_weights(wfmt, w_canon: np.ndarray, N, K, layout):
    """Canonical bytes from the oracle encoder, on the GPU in `layout`."""
    wd = to_dev(w_canon.reshape(-1))
    if layout == "repacked":
        wd = qmm.repack_weights(wd, wfmt, N, K)
    return wd


def assert_close(got: np.ndarray, want: np.ndarray, terms: np.ndarray, what: str, tol=TOL):
    got = np.asarray(got, np.float64).reshape(want.shape)
    err = np.abs(got - want)
    bound = tol * terms + 1e-30
    bad = err > bound
    if bad.any():
        i = np.flatnonzero(bad.ravel())[:5]
        raise AssertionError(
            f"{what}: {bad.sum()} of {bad.size} outside {tol}*sum|terms|; first at flat {i}: "
            f"got {got.ravel()[i]}, want {want.ravel()[i]}, terms {terms.ravel()[i]}")


def full_reference(wfmt, w_canon, y_canon, M, N, K):
    """Oracle outputs and sum|terms| for every (m, n)."""
    ms = np.repeat(np.arange(M), N)
    ns = np.tile(np.arange(N), M)
    out, terms = oracle.sample(wfmt, w_canon, y_canon, M, N, K, ms, ns)
    return out.reshape(M, N), terms.reshape(M, N)
