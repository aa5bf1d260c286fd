"""Graph capture of the hot path (the benchmark replays captured steps): every
replay must reproduce the eager result exactly, with eager work and
synchronizations between replays.  The kernels are deterministic (no atomics,
fixed reduction order), so equality is bitwise."""
import numpy as np
import pytest

import oracle
import bit_quantized_mat_quantize_amd as qmm
from bit_quantized_mat_quantize_amd.inputs import activations, weights_t4_skewed
from gpu_helpers import to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,algo", [(1, "gemv"), (4, "gemv"), (64, "mfma")])
def test_graph_replays_match_eager(M, algo):
    import torch
    N, K = 200, 2048
    w = qmm.repack_weights(to_dev(oracle.quantize("q4_K", weights_t4_skewed(8, N, K)).reshape(-1)),
                           "q4_K", N, K)
    x1 = to_dev(activations(9, M, K))
    x2 = to_dev(activations(10, M, K))
    y = torch.empty(qmm.act_bytes("q8_K", M, K), dtype=torch.uint8, device="cuda")
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")

    def step(x):
        qmm.quantize_row_q8(x, "q8_K", out=y)
        qmm.mul_mat_q4_K(w, y, M, N, K, layout="repacked", algo=algo, out=out)

    step(x1)
    eager1 = to_host(out).copy()
    step(x2)
    eager2 = to_host(out).copy()
    assert not np.array_equal(eager1, eager2)

    xin = torch.empty_like(x1)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        xin.copy_(x1)
        step(xin)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step(xin)
    for rep in range(4):
        src = x1 if rep % 2 == 0 else x2
        xin.copy_(src)
        out.fill_(-1.0)                       # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        got = to_host(out)
        want = eager1 if rep % 2 == 0 else eager2
        assert np.array_equal(got, want), f"replay {rep} differs"
