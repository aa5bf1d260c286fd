"""AUTO kernel choice, read from the QMM_LOG line each mul_mat call prints.

The dispatch decision is host logic: it is taken and logged after argument
validation and before the kernel launch.  Without a GPU the launch then fails
with QMM_EDEVICE, so the decision can be checked on the CPU for any shape.  The
pointers below are aligned placeholders and must never reach a device: the
test runs only where no GPU device node exists, in a child process (QMM_LOG is
read once per process).
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(os.path.exists("/dev/kfd"),
                                reason="placeholder pointers are only passed where no GPU exists")

CHILD = r"""
import ctypes, json, sys
sys.path.insert(0, sys.argv[1])
from bit_quantized_mat_quantize_amd import _binding
lib = _binding.load()
hip = ctypes.CDLL("libamdhip64.so")
n = ctypes.c_int(0)
if hip.hipGetDeviceCount(ctypes.byref(n)) == 0 and n.value > 0:
    sys.exit(3)                      # a device exists: placeholder pointers must not be launched
P, I, S = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
FN = {"q4_0": lib.qmm_mul_mat_q4_0_ex, "q4_K": lib.qmm_mul_mat_q4_K_ex,
      "q6_K": lib.qmm_mul_mat_q6_K_ex, "q2_K": lib.qmm_mul_mat_q2_K_ex}
big = 1 << 40
for fmt, layout, M, N, K, algo in json.loads(sys.argv[2]):
    f = FN[fmt]
    st = f(P(1 << 20), S(big), layout, P(2 << 20), S(big), P(3 << 20), S(big), I(M), I(N), I(K), algo, None)
    print("status", st, flush=True)
"""

# (format, layout, M, N, K, expected family under AUTO)
CASES = [
    # Q4_K: GEMV at M = 1 and at M = 2 below 8192 columns; small batch up to
    # M = 32 and while ceil(M/32)*N <= 9*8192; GEMM above
    ("q4_K", 1, 1, 4096, 4096, "GEMV"),
    ("q4_K", 0, 1, 4096, 4096, "GEMV"),
    ("q4_K", 1, 2, 4096, 4096, "SKINNY"),
    ("q4_K", 1, 2, 8192, 8192, "SKINNY"),
    ("q4_K", 1, 4, 8192, 8192, "SKINNY"),
    ("q4_K", 1, 32, 28672, 8192, "SKINNY"),
    ("q4_K", 1, 288, 8192, 8192, "SKINNY"),
    ("q4_K", 1, 289, 8192, 8192, "MFMA"),
    ("q4_K", 1, 512, 28672, 8192, "MFMA"),
    # Q4_0: GEMV at M = 1 and while its LDS staging fits (M <= 4 or M*N <= 36864)
    ("q4_0", 1, 1, 256, 1024, "GEMV"),
    ("q4_0", 1, 4, 28672, 8192, "GEMV"),
    ("q4_0", 1, 8, 4096, 4096, "GEMV"),
    ("q4_0", 1, 8, 8192, 8192, "SKINNY"),
    ("q4_0", 1, 512, 28672, 8192, "MFMA"),
    ("q4_0", 0, 512, 28672, 8192, "GEMV"),       # canonical: no MFMA kernel
    ("q4_0", 1, 512, 28672, 8224, "GEMV"),       # K % 256 != 0: no MFMA kernel
    # Q6_K / Q2_K repacked: GEMV at M = 1 and M = 2 below 8192 columns, small
    # batch while ceil(M/32)*N <= 8*8192 (Q6_K) / 6*8192 (Q2_K), GEMM above
    ("q6_K", 1, 1, 4096, 4096, "GEMV"),
    ("q6_K", 1, 2, 4096, 4096, "GEMV"),
    ("q6_K", 1, 8, 8192, 8192, "SKINNY"),
    ("q6_K", 1, 256, 8192, 8192, "SKINNY"),
    ("q6_K", 1, 257, 8192, 8192, "MFMA"),
    ("q2_K", 1, 192, 8192, 8192, "SKINNY"),
    ("q2_K", 1, 193, 8192, 8192, "MFMA"),
    # a K above the GEMV's limit sends M = 1 down the small-batch rule
    ("q6_K", 1, 1, 4096, 65536, "SKINNY"),
    ("q2_K", 1, 1, 4096, 65536, "SKINNY"),
    ("q6_K", 1, 1, 70000, 65536, "MFMA"),
    # the canonical layout has only the GEMV, whatever M
    ("q6_K", 0, 1, 4096, 4096, "GEMV"),
    ("q6_K", 0, 4096, 8192, 8192, "GEMV"),
    ("q2_K", 0, 4096, 8192, 8192, "GEMV"),
]


def test_auto_choice_logged():
    fmts = {"q4_0": "Q4_0", "q4_K": "Q4_K", "q6_K": "Q6_K", "q2_K": "Q2_K"}
    calls = [[f, lay, M, N, K, 0] for f, lay, M, N, K, _ in CASES]
    env = dict(os.environ, QMM_LOG="1")
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT, json.dumps(calls)], env=env,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    logs = [l for l in r.stderr.splitlines() if l.startswith("qmm: mul_mat ")]
    stats = [int(l.split()[1]) for l in r.stdout.splitlines() if l.startswith("status")]
    assert len(logs) == len(CASES) and len(stats) == len(CASES), (r.stdout, r.stderr)
    for (f, lay, M, N, K, want), line, st in zip(CASES, logs, stats):
        assert st == 4, (f, M, N, K, st)             # QMM_EDEVICE: no device to launch on
        head = f"qmm: mul_mat {fmts[f]} M={M} N={N} K={K} layout={'repacked' if lay else 'canonical'}"
        assert line.startswith(head), (line, head)
        assert f"algo=AUTO -> {want} (" in line, (line, want)


def test_log_off_by_default():
    env = {k: v for k, v in os.environ.items() if k != "QMM_LOG"}
    calls = [["q4_K", 1, 1, 4096, 4096, 0]]
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT, json.dumps(calls)], env=env,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "qmm:" not in r.stderr
