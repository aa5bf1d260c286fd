"""Quantized mul_mat (Q4_0 / Q4_K / Q6_K / Q2_K weights x Q8_0 / Q8_K activations) on MI355X.

The computation lives in ``libqmm.so`` (hand-written HIP kernels for gfx950
behind the C ABI of ``include/qmm.h``); this package is its thin binding.
"""
from ._binding import (  # noqa: F401
    ALGO_AUTO, ALGO_GEMV, ALGO_MFMA, ALGO_SKINNY, CANONICAL, LIB_PATH, Q2_K, Q4_0, Q4_K, Q6_K, Q8_0, Q8_K, REPACKED,
    ACT_FOR, QmmError, act_bytes, debug_block_sums, load, mul_mat, mul_mat_id, mul_mat_id_noalloc, mul_mat_id_q4_K,
    mul_mat_id_workspace_bytes, mul_mat_q2_K, mul_mat_q4_0, mul_mat_q4_K, mul_mat_q6_K, quantize_mul_mat,
    quantize_row_q8, quantize_weights, repack_weights, version, weight_bytes,
)
