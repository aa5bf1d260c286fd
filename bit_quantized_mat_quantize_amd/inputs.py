"""Seeded synthetic inputs (fp32 arrays) for the five measured workloads.

This module draws random numbers and nothing else: it holds none of the
quantization or dot-product arithmetic.  Both the oracle-based tests and the GPU
benchmark take their fp32 weights and activations from here, so the two sides
always start from identical inputs.

The pages measure on real GGUF models (Llama-3.1-8B / Llama-3.2-1B, ggml-cpu
mul_mat page, "真实数字" section); no model file is available, so these seeded
arrays of the same projection shapes (7B: 4096 / 14336; 70B: 8192 / 28672) stand
in for them.

Recipes (numpy ``default_rng``; rows drawn in order, in chunks of ``_CHUNK``):
  * ``normal(sigma)``      -- N(0, sigma^2)
  * ``t4_skewed``          -- 0.02 * Student-t(df=4); a seeded choice of
                              round(0.25 * N) rows is shifted by +0.01 (half the
                              0.02 scale), so those rows need a non-zero min
  * activations            -- N(0, 1); with ``outliers`` a seeded 1% of the K
                              channels is multiplied by 20 in every row
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

_CHUNK = 4096


def _rows(rng: np.random.Generator, n: int, k: int, draw) -> np.ndarray:
    out = np.empty((n, k), np.float32)
    for r0 in range(0, n, _CHUNK):
        r1 = min(n, r0 + _CHUNK)
        out[r0:r1] = draw(rng, (r1 - r0, k))
    return out


def weights_normal(seed, n: int, k: int, sigma: float = 0.02) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return _rows(rng, n, k, lambda g, s: g.normal(0.0, sigma, s))


def weights_t4_skewed(seed, n: int, k: int, scale: float = 0.02,
                      shift_frac: float = 0.25) -> np.ndarray:
    rng = np.random.default_rng(seed)
    w = _rows(rng, n, k, lambda g, s: scale * g.standard_t(4.0, s))
    n_shift = int(round(shift_frac * n))
    rows = rng.choice(n, size=n_shift, replace=False)
    w[rows] += np.float32(0.5 * scale)
    return w


def activations(seed, m: int, k: int, outlier_frac: float = 0.0,
                outlier_gain: float = 20.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    a = _rows(rng, m, k, lambda g, s: g.standard_normal(s))
    if outlier_frac > 0.0:
        n_out = int(round(outlier_frac * k))
        ch = rng.choice(k, size=n_out, replace=False)
        a[:, ch] *= np.float32(outlier_gain)
    return a


@dataclass
class Projection:
    """One weight matrix [N, K] in format `wfmt` and its activations [M, K]."""
    name: str
    wfmt: str           # "q4_0", "q4_K", "q6_K" or "q2_K"
    M: int
    N: int
    K: int
    w_seed: object
    a_seed: object
    w_kind: str = "t4_skewed"
    outliers: float = 0.0
    act_key: str = ""   # projections with the same key share one activation array

    def weights(self) -> np.ndarray:
        if self.w_kind == "normal":
            return weights_normal(self.w_seed, self.N, self.K)
        return weights_t4_skewed(self.w_seed, self.N, self.K)

    def acts(self) -> np.ndarray:
        return activations(self.a_seed, self.M, self.K, self.outliers)


@dataclass
class Workload:
    key: str
    description: str
    projections: list = field(default_factory=list)

    @property
    def weight_bytes(self) -> int:
        per = {"q4_0": 18 / 32, "q4_K": 144 / 256, "q6_K": 210 / 256, "q2_K": 84 / 256}
        return int(sum(p.N * p.K * per[p.wfmt] for p in self.projections))

    @property
    def ops(self) -> int:
        return int(sum(2 * p.M * p.N * p.K for p in self.projections))


def workload(key: str) -> Workload:
    """The measured configurations, by key:

    c1        Q4_0 x Q8_0 GEMV, M=1, N=256, K=1024, weights N(0, 0.02) seed 0
    c2        Q4_K x Q8_K GEMV, M=1, N=K=4096 (7B attention projection)
    c3        Q4_K FFN at M=1: gate, up (N=14336, K=4096), down (N=4096, K=14336)
    c4_m{4,8,32}   Q4_K, N=K=8192 (70B projection), M in {4, 8, 32}
    c5_m{512,2048} Q4_K prefill, N=28672, K=8192, activations with 1% outliers x20
    q6K_c2    Q6_K x Q8_K GEMV, M=1, N=K=4096, the weights of c2 in 6-bit form
    q6K_down  Q6_K x Q8_K GEMV, M=1, N=4096, K=14336 (the FFN down projection,
              the matrix 4-bit model files commonly keep at 6 bits)
    q6K_c5_m{512,2048}  Q6_K prefill on the c5 shapes (N=28672, K=8192)
    q2K_c2    Q2_K x Q8_K GEMV, M=1, N=K=4096, the weights of c2 in 2-bit form
    q2K_c5_m{512,2048}  Q2_K prefill on the c5 shapes
    q40_c5_m{512,2048}  Q4_0 x Q8_0 prefill on the c5 shapes, weights N(0, 0.02)
                        as in c1
    """
    if key == "c1":
        return Workload(key, "Q4_0xQ8_0 GEMV M=1 N=256 K=1024", [
            Projection("w", "q4_0", 1, 256, 1024, 0, 101, w_kind="normal")])
    if key == "c2":
        return Workload(key, "Q4_KxQ8_K GEMV M=1 N=4096 K=4096", [
            Projection("w", "q4_K", 1, 4096, 4096, 2, 102)])
    if key == "c3":
        return Workload(key, "Q4_K FFN M=1 gate/up 14336x4096 + down 4096x14336", [
            Projection("gate", "q4_K", 1, 14336, 4096, [3, 0], 103, act_key="x"),
            Projection("up", "q4_K", 1, 14336, 4096, [3, 1], 103, act_key="x"),
            Projection("down", "q4_K", 1, 4096, 14336, [3, 2], [103, 1], act_key="h")])
    if key.startswith("c4_m"):
        m = int(key[4:])
        assert m in (4, 8, 32)
        return Workload(key, f"Q4_K M={m} N=8192 K=8192", [
            Projection("w", "q4_K", m, 8192, 8192, 4, [104, m])])
    if key.startswith("c5_m"):
        m = int(key[4:])
        assert m in (512, 2048)
        return Workload(key, f"Q4_K prefill M={m} N=28672 K=8192", [
            Projection("w", "q4_K", m, 28672, 8192, 5, [105, m], outliers=0.01)])
    if key == "q6K_c2":
        return Workload(key, "Q6_KxQ8_K GEMV M=1 N=4096 K=4096", [
            Projection("w", "q6_K", 1, 4096, 4096, 2, 102)])
    if key == "q6K_down":
        return Workload(key, "Q6_KxQ8_K GEMV M=1 N=4096 K=14336", [
            Projection("down", "q6_K", 1, 4096, 14336, [3, 2], [103, 1])])
    if key.startswith("q6K_c5_m"):
        m = int(key[8:])
        assert m in (512, 2048)
        return Workload(key, f"Q6_K prefill M={m} N=28672 K=8192", [
            Projection("w", "q6_K", m, 28672, 8192, 5, [105, m], outliers=0.01)])
    if key == "q2K_c2":
        return Workload(key, "Q2_KxQ8_K GEMV M=1 N=4096 K=4096", [
            Projection("w", "q2_K", 1, 4096, 4096, 2, 102)])
    if key.startswith("q2K_c5_m"):
        m = int(key[8:])
        assert m in (512, 2048)
        return Workload(key, f"Q2_K prefill M={m} N=28672 K=8192", [
            Projection("w", "q2_K", m, 28672, 8192, 5, [105, m], outliers=0.01)])
    if key.startswith("q40_c5_m"):
        m = int(key[8:])
        assert m in (512, 2048)
        return Workload(key, f"Q4_0xQ8_0 prefill M={m} N=28672 K=8192", [
            Projection("w", "q4_0", m, 28672, 8192, 5, [105, m], w_kind="normal", outliers=0.01)])
    raise KeyError(key)


ALL_WORKLOADS = ["c1", "c2", "c3", "c4_m4", "c4_m8", "c4_m32", "c5_m512", "c5_m2048",
                 "q6K_c2", "q6K_down", "q6K_c5_m512", "q6K_c5_m2048",
                 "q2K_c2", "q2K_c5_m512", "q2K_c5_m2048", "q40_c5_m512", "q40_c5_m2048"]
