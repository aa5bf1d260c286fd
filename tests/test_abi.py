"""The C ABI without a GPU: every symbol declared in include/qmm.h is exported
by libqmm.so, the size helpers agree with the formats, and every validation
error is returned by the host before any HIP call (the pointers below are never
dereferenced)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmm.h")

OK, EINVAL, EALIGN, EUNSUP = 0, 1, 2, 3


@pytest.fixture(scope="module")
def lib():
    from bit_quantized_mat_quantize_amd import _binding
    return _binding.load()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qmm_[A-Za-z0-9_]+)\s*\(", src)))


def test_header_symbols_exported(lib):
    names = _declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    # the exports are exactly the declared entry points (no stray C symbols)
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", lib._name], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted({l.split()[-1] for l in out.splitlines() if re.search(r" T qmm_", l)})
    assert exported == names


def test_probe_header_symbols_exported():
    """libqmm_probe.so exports exactly what include/qmm_probe.h declares, and
    its argument checks answer without a GPU."""
    import subprocess
    from bit_quantized_mat_quantize_amd import _probe
    plib = _probe.load()
    src = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "qmm_probe.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(qmm_[A-Za-z0-9_]+)\s*\(", src)))
    out = subprocess.run(["nm", "-D", "--defined-only", plib._name], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted({l.split()[-1] for l in out.splitlines() if re.search(r" T qmm_", l)})
    assert exported == names and len(names) == 4
    assert plib.qmm_probe_mfma_sink_bytes() == 256 * 8 * 256 * 4
    assert plib.qmm_probe_mfma_ops(1) == 256 * 8 * 4 * 4 * 2 * 32 ** 3
    P = ctypes.c_void_p
    assert plib.qmm_probe_read(None, 16, 4, P(16), None) == 1      # null buffer
    assert plib.qmm_probe_read(P(16), 24, 4, P(16), None) == 1     # not a multiple of 16
    assert plib.qmm_probe_read(P(16), 32, 3, P(16), None) == 1     # unsupported loads per thread
    assert plib.qmm_probe_read(P(8), 32, 4, P(16), None) == 1      # misaligned
    assert plib.qmm_probe_mfma_i8(P(16), 16, 8, 0, None) == 1      # sink too small


def test_size_helpers(lib):
    assert lib.qmm_act_bytes(0, 3, 64) == 3 * 2 * 34
    assert lib.qmm_act_bytes(1, 3, 512) == 3 * 2 * 292
    assert lib.qmm_act_bytes(1, 3, 500) == 0
    assert lib.qmm_weight_bytes(1, 0, 5, 512) == 5 * 2 * 144
    assert lib.qmm_weight_bytes(1, 1, 5, 512) == 5 * 2 * 144
    assert lib.qmm_weight_bytes(0, 0, 5, 64) == 5 * 2 * 18
    # repacked Q4_0: scale section padded to 256 B, then 16 B per block
    assert lib.qmm_weight_bytes(0, 1, 5, 64) == 256 + 5 * 2 * 16
    assert lib.qmm_weight_bytes(0, 1, 256, 1024) == (2 * 256 * 32 + 255) // 256 * 256 + 16 * 256 * 32
    assert lib.qmm_weight_bytes(7, 0, 5, 64) == 0
    # Q6_K: 210 B per 256; repacked adds the padding of its d section
    assert lib.qmm_weight_bytes(2, 0, 5, 512) == 5 * 2 * 210
    assert lib.qmm_weight_bytes(2, 1, 5, 512) == 256 + 5 * 2 * 208
    assert lib.qmm_weight_bytes(2, 0, 5, 100) == 0
    # Q2_K: 84 B per 256; repacked pads its (d, dmin) section to 256 B
    assert lib.qmm_weight_bytes(3, 0, 5, 512) == 5 * 2 * 84
    assert lib.qmm_weight_bytes(3, 1, 5, 512) == 256 + 5 * 2 * 80
    assert lib.qmm_weight_bytes(3, 1, 64, 512) == 64 * 2 * 4 + 64 * 2 * 80
    assert lib.qmm_weight_bytes(3, 0, 5, 128) == 0


def _last(lib):
    return lib.qmm_last_error().decode()


A = 0x10000  # a 16-byte-aligned fake address, never dereferenced


def test_quantize_validation(lib):
    q = lib.qmm_quantize_row_q8
    assert q(1, A, 2, 300, A, 10**6, None) == EUNSUP and "multiple of 256" in _last(lib)
    assert q(0, A, 2, 48, A, 10**6, None) == EUNSUP
    assert q(1, A, 2, 0, A, 10**6, None) == EUNSUP
    assert q(1, A, -1, 256, A, 10**6, None) == EINVAL
    assert q(1, A, 2**24 + 1, 256, A, 10**9, None) == EUNSUP
    assert q(1, A, 2, 2**21, A, 10**9, None) == EUNSUP
    assert q(1, None, 2, 256, A, 10**6, None) == EINVAL and "x is NULL" in _last(lib)
    assert q(1, A + 4, 2, 256, A, 10**6, None) == EALIGN
    assert q(1, A, 2, 256, A + 8, 10**6, None) == EALIGN
    assert q(1, A, 2, 256, A, 2 * 292 - 1, None) == EINVAL and "needed" in _last(lib)
    assert q(5, A, 2, 256, A, 10**6, None) == EUNSUP
    # empty is a valid no-op (nothing is launched, pointers may be NULL)
    assert q(1, None, 0, 256, None, 0, None) == OK


def test_mul_mat_validation(lib):
    f = lib.qmm_mul_mat_q4_K_ex
    big = 10**9
    args = dict(w=A, wb=big, l=0, y=A, yb=big, o=A, ob=big, M=4, N=8, K=512, algo=0)

    def call(**kw):
        a = {**args, **kw}
        return f(a["w"], a["wb"], a["l"], a["y"], a["yb"], a["o"], a["ob"], a["M"], a["N"], a["K"],
                 a["algo"], None)

    assert call(K=384) == EUNSUP
    assert call(l=2) == EUNSUP
    assert call(algo=9) == EUNSUP
    # SKINNY: 32-row chunks on grid.y, at most 65535 of them
    mmax = 65535 * 32
    assert call(M=mmax + 1, yb=2**40, ob=2**40, algo=3) == EUNSUP
    assert call(M=mmax, N=0, yb=2**40, ob=2**40, algo=3) == OK     # valid, nothing to do
    assert call(M=-1) == EINVAL
    assert call(N=-3) == EINVAL
    assert call(w=None) == EINVAL
    assert call(y=A + 2) == EALIGN
    assert call(o=A + 4) == EALIGN
    assert call(wb=8 * 2 * 144 - 1) == EINVAL
    assert call(yb=4 * 2 * 292 - 1) == EINVAL
    assert call(ob=4 * 8 * 4 - 1) == EINVAL
    assert call(M=9, algo=1) == EUNSUP and "M <= 8" in _last(lib)
    assert call(M=0, w=None, y=None, o=None) == OK
    assert call(N=0) == OK
    g = lib.qmm_mul_mat_q4_0
    assert g(A, big, 0, A, big, A, big, 1, 256, 1000, None) == EUNSUP
    assert g(A, 18 * 32 * 256 - 1, 0, A, big, A, big, 1, 256, 1024, None) == EINVAL
    # repacked Q4_0 needs the padded size
    need = lib.qmm_weight_bytes(0, 1, 3, 64)
    assert g(A, need - 1, 1, A, big, A, big, 1, 3, 64, None) == EINVAL
    gx = lib.qmm_mul_mat_q4_0_ex
    # SKINNY: repacked layout, K % 256 == 0, M <= 65535*32; unknown families refused
    assert gx(A, big, 0, A, big, A, big, 4, 8, 512, 3, None) == EUNSUP and "SKINNY" in _last(lib)
    assert gx(A, big, 1, A, big, A, big, 4, 8, 288, 3, None) == EUNSUP
    assert gx(A, 2**40, 1, A, 2**40, A, 2**40, mmax + 1, 8, 512, 3, None) == EUNSUP
    assert gx(A, 2**40, 1, A, 2**40, A, 2**40, mmax, 0, 512, 3, None) == OK
    assert gx(A, big, 1, A, big, A, big, 4, 8, 512, 7, None) == EUNSUP and "unknown algo" in _last(lib)


def test_quantize_mul_mat_validation(lib):
    f = lib.qmm_quantize_mul_mat
    big = 10**9
    args = dict(t=1, w=A, wb=big, l=1, x=A, y=A, yb=big, o=A, ob=big, M=1, N=8, K=512)

    def call(**kw):
        a = {**args, **kw}
        return f(a["t"], a["w"], a["wb"], a["l"], a["x"], a["y"], a["yb"], a["o"], a["ob"],
                 a["M"], a["N"], a["K"], None)

    assert call(t=4) == EUNSUP
    assert call(l=3) == EUNSUP
    assert call(K=300) == EUNSUP
    assert call(t=0, K=48) == EUNSUP
    assert call(M=-2) == EINVAL
    assert call(N=-1) == EINVAL
    assert call(x=None) == EINVAL and "x is NULL" in _last(lib)
    assert call(x=A + 4) == EALIGN
    assert call(y=None) == EINVAL
    assert call(yb=2 * 292 - 1) == EINVAL and "needed" in _last(lib)
    assert call(t=0, yb=16 * 34 - 1) == EINVAL
    assert call(w=None) == EINVAL
    assert call(o=A + 8) == EALIGN
    assert call(wb=8 * 2 * 144 - 1) == EINVAL
    assert call(ob=8 * 4 - 1) == EINVAL
    # w and out are not checked when N == 0 would only quantize; M == 0 is empty
    assert call(M=0, x=None, y=None, w=None, o=None) == OK


def test_q6_K_validation(lib):
    f = lib.qmm_mul_mat_q6_K
    big = 10**9
    assert f(A, big, 1, A, big, A, big, 2, 8, 384, None) == EUNSUP          # K % 256
    # K beyond the GEMV's LDS limit: only the MFMA path (repacked layout) takes it
    assert f(A, big, 0, A, big, A, big, 2, 8, 53760 + 256, None) == EUNSUP
    assert "needs the repacked layout" in _last(lib)
    fx = lib.qmm_mul_mat_q6_K_ex
    assert fx(A, big, 1, A, big, A, big, 2, 8, 53760 + 256, 1, None) == EUNSUP  # GEMV
    assert "Q6_K GEMV takes K" in _last(lib)
    assert fx(A, big, 0, A, big, A, big, 2, 8, 512, 2, None) == EUNSUP  # MFMA, canonical
    assert "repacked layout" in _last(lib)
    # SKINNY: repacked layout, M <= 65535*32
    assert fx(A, big, 0, A, big, A, big, 2, 8, 512, 3, None) == EUNSUP and "SKINNY" in _last(lib)
    assert fx(A, 2**40, 1, A, 2**40, A, 2**40, 65535 * 32 + 1, 8, 512, 3, None) == EUNSUP
    assert fx(A, 2**40, 1, A, 2**40, A, 2**40, 65535 * 32, 0, 512, 3, None) == OK
    assert fx(A, big, 1, A, big, A, big, 2, 8, 512, 9, None) == EUNSUP  # unknown
    # 32-bit offsets: a weight matrix of 4 GiB or more rules the MFMA path out
    kk = 1 << 20
    n4g = (1 << 32) // (kk // 256 * 208) + 1  # repacked rows of K = 2^20 past 4 GiB
    assert fx(A, 2**62, 1, A, 2**40, A, 2**40, 2, n4g, kk, 2, None) == EUNSUP
    assert "below 4 GiB" in _last(lib)
    n4g = (1 << 32) // 288 + 1  # Q4_K rows of K = 512 (288 B each) past 4 GiB, N < 2^24
    assert lib.qmm_mul_mat_q4_K_ex(A, 2**62, 0, A, big, A, 2**40, 2, n4g, 512, 2, None) == EUNSUP
    assert "below 4 GiB" in _last(lib)
    assert f(A, 8 * 2 * 210 - 1, 0, A, big, A, big, 2, 8, 512, None) == EINVAL
    assert f(A, 256 + 8 * 2 * 208 - 1, 1, A, big, A, big, 2, 8, 512, None) == EINVAL
    assert f(A, big, 1, A, 2 * 2 * 292 - 1, A, big, 2, 8, 512, None) == EINVAL
    assert f(A, big, 1, A + 2, big, A, big, 2, 8, 512, None) == EALIGN
    assert f(None, 0, 1, None, 0, None, 0, 0, 8, 512, None) == OK
    assert lib.qmm_quantize_weights(2, A, 4, 300, A, 10**6, None) == EUNSUP
    assert lib.qmm_quantize_weights(2, A, 4, 256, A, 4 * 210 - 1, None) == EINVAL
    assert lib.qmm_repack_weights(2, A, 4, 256, A + 10**6, 256 + 4 * 208 - 1, None) == EINVAL


def test_q2_K_validation(lib):
    f = lib.qmm_mul_mat_q2_K
    fx = lib.qmm_mul_mat_q2_K_ex
    big = 10**9
    assert f(A, big, 1, A, big, A, big, 2, 8, 384, None) == EUNSUP          # K % 256
    assert f(A, big, 0, A, big, A, big, 2, 8, 53760 + 256, None) == EUNSUP
    assert "Q2_K with K" in _last(lib)
    assert fx(A, big, 1, A, big, A, big, 2, 8, 53760 + 256, 1, None) == EUNSUP  # GEMV
    assert fx(A, big, 0, A, big, A, big, 2, 8, 512, 2, None) == EUNSUP        # MFMA, canonical
    # SKINNY: repacked layout, M <= 65535*32
    assert fx(A, big, 0, A, big, A, big, 2, 8, 512, 3, None) == EUNSUP and "SKINNY" in _last(lib)
    assert fx(A, 2**40, 1, A, 2**40, A, 2**40, 65535 * 32 + 1, 8, 512, 3, None) == EUNSUP
    assert fx(A, 2**40, 1, A, 2**40, A, 2**40, 65535 * 32, 0, 512, 3, None) == OK
    assert f(A, 8 * 2 * 84 - 1, 0, A, big, A, big, 2, 8, 512, None) == EINVAL
    assert f(A, 256 + 8 * 2 * 80 - 1, 1, A, big, A, big, 2, 8, 512, None) == EINVAL
    assert f(A, big, 1, A, 2 * 2 * 292 - 1, A, big, 2, 8, 512, None) == EINVAL
    assert f(A, big, 1, A, big, A + 4, big, 2, 8, 512, None) == EALIGN
    assert f(None, 0, 1, None, 0, None, 0, 2, 0, 512, None) == OK
    assert lib.qmm_quantize_weights(3, A, 4, 300, A, 10**6, None) == EUNSUP
    assert lib.qmm_quantize_weights(3, A, 4, 256, A, 4 * 84 - 1, None) == EINVAL
    assert lib.qmm_repack_weights(3, A, 4, 256, A + 10**6, 256 + 4 * 80 - 1, None) == EINVAL
    assert lib.qmm_debug_block_sums(3, A, 10**9, 0, A, 10**9, A, 4 * 8 * 32 * 4 - 1,
                                    4, 8, 512, None) == EINVAL


def test_mul_mat_id_validation(lib):
    f = lib.qmm_mul_mat_id_q4_K
    big = 10**9
    wsb = lib.qmm_mul_mat_id_workspace_bytes
    # int32 words: start[E+1], tile_e/tile_r0[ceil(P/128)+E], ntiles, sorted[P], 16-byte sections
    up4 = lambda v: (v + 3) // 4 * 4
    for T, U, E in ((3, 2, 8), (300, 8, 64), (1, 1, 1)):
        mt = (T * U + 127) // 128 + E
        assert wsb(T, U, E) == 4 * (up4(E + 1) + 2 * up4(mt) + 4 + up4(T * U))
    assert wsb(3, 0, 8) == 0 and wsb(3, 2, 0) == 0 and wsb(3, 2, 4097) == 0

    def call(**kw):
        a = dict(w=A, wb=big, E=4, l=1, y=A, yb=big, yps=0, ids=A, T=3, U=2, o=A, ob=big, N=8, K=512,
                 ws=A, wsb=big, algo=0)
        a.update(kw)
        return f(a["w"], a["wb"], a["E"], a["l"], a["y"], a["yb"], a["yps"], a["ids"], a["T"], a["U"],
                 a["o"], a["ob"], a["N"], a["K"], a["ws"], a["wsb"], a["algo"], None)

    assert call(E=0) == EUNSUP and call(E=4097) == EUNSUP
    assert call(U=0) == EINVAL and call(U=5) == EINVAL
    assert call(yps=2) == EINVAL
    assert call(K=384) == EUNSUP
    assert call(l=2) == EUNSUP
    assert call(algo=3) == EUNSUP
    assert call(T=0, w=None, y=None, ids=None, o=None, ws=None) == OK
    assert call(ids=None) == EINVAL and "ids" in _last(lib)
    assert call(ids=A + 4) == EALIGN
    assert call(wb=4 * 8 * 2 * 144 - 1) == EINVAL          # four expert matrices
    assert call(yb=3 * 2 * 292 - 1) == EINVAL               # one row per token
    assert call(yps=1, yb=6 * 2 * 292 - 1) == EINVAL        # one row per (token, slot)
    assert call(ob=3 * 2 * 8 * 4 - 1) == EINVAL
    assert call(algo=1, K=53760 + 256) == EUNSUP            # GEMV row limit
    # the MFMA path needs its workspace
    assert call(algo=2, ws=None) == EINVAL
    assert call(algo=2, wsb=wsb(3, 2, 4) - 1) == EINVAL



def test_mul_mat_id_generic_validation(lib):
    f = lib.qmm_mul_mat_id
    big = 10**9
    wsb = lib.qmm_mul_mat_id_workspace_bytes

    def call(t, **kw):
        a = dict(w=A, wb=big, E=4, l=1, y=A, yb=big, yps=0, ids=A, T=3, U=2, o=A, ob=big, N=8, K=512,
                 ws=A, wsb=big, algo=0)
        a.update(kw)
        return f(t, a["w"], a["wb"], a["E"], a["l"], a["y"], a["yb"], a["yps"], a["ids"], a["T"], a["U"],
                 a["o"], a["ob"], a["N"], a["K"], a["ws"], a["wsb"], a["algo"], None)

    assert call(7) == EUNSUP and "weight type" in _last(lib)
    # Q4_0 rows of 32-weight blocks against Q8_0 activations (34 bytes per 32)
    assert call(0, K=96, algo=1, wb=4 * 8 * 3 * 18 - 1) == EINVAL
    assert call(0, K=96, algo=1, yb=3 * 3 * 34 - 1) == EINVAL
    assert call(0, K=100) == EUNSUP                          # K not a multiple of 32
    assert call(0, K=96, algo=2) == EUNSUP                   # MFMA path steps K by 256
    assert call(0, K=512, algo=2, l=0) == EUNSUP             # ... and reads the repacked layout
    # Q6_K and Q2_K: canonical matrices only through the GEMV
    for t, per in ((2, 210), (3, 84)):
        assert call(t, algo=2, l=0) == EUNSUP
        assert call(t, algo=1, wb=4 * 8 * 2 * per - 1, l=0) == EINVAL
        assert call(t, algo=1, K=53760 + 256) == EUNSUP      # one Q8_K row staged in LDS
        assert call(t, algo=2, wsb=wsb(3, 2, 4) - 1) == EINVAL
        assert call(t, T=0, w=None, y=None, ids=None, o=None, ws=None) == OK
    # the Q4_K entry point is the generic one with its type fixed
    assert call(1, algo=1, K=53760 + 256) == EUNSUP


def test_mul_mat_id_noalloc_validation(lib):
    """The no-workspace variant refuses, before any HIP call, a grouping that
    does not fit the library's 2 MiB scratch (unless the call is forced onto
    the per-pair GEMV, which needs none), and validates like qmm_mul_mat_id."""
    f = lib.qmm_mul_mat_id_noalloc
    big = 10**12
    wsb = lib.qmm_mul_mat_id_workspace_bytes

    def call(t, **kw):
        a = dict(w=A, wb=big, E=8, l=1, y=A, yb=big, yps=0, ids=A, T=3, U=2, o=A, ob=big, N=8, K=512, algo=0)
        a.update(kw)
        return f(t, a["w"], a["wb"], a["E"], a["l"], a["y"], a["yb"], a["yps"], a["ids"], a["T"], a["U"],
                 a["o"], a["ob"], a["N"], a["K"], a["algo"], None)

    limit = 2 << 20
    T_fit = 1
    while wsb(2 * T_fit, 2, 8) <= limit:
        T_fit *= 2
    while wsb(T_fit + 1, 2, 8) <= limit:
        T_fit += 1
    assert wsb(T_fit, 2, 8) <= limit < wsb(T_fit + 1, 2, 8)
    for algo in (0, 2):                                   # AUTO, MFMA
        assert call(1, T=T_fit + 1, algo=algo) == EUNSUP and "scratch" in _last(lib)
    assert call(7) == EUNSUP and "weight type" in _last(lib)
    assert call(1, algo=2, l=1, ids=None) == EINVAL
    assert call(0, K=96, algo=2) == EUNSUP               # MFMA path steps K by 256
    assert call(1, U=9) == EINVAL                        # U > E
    assert call(1, T=0, w=None, y=None, ids=None, o=None) == OK


def test_other_validation(lib):
    assert lib.qmm_quantize_weights(1, A, 4, 100, A, 10**6, None) == EUNSUP
    assert lib.qmm_quantize_weights(0, A, 4, 64, A, 4 * 2 * 18 - 1, None) == EINVAL
    assert lib.qmm_quantize_weights(7, A, 4, 256, A, 10**6, None) == EUNSUP   # unknown type
    assert lib.qmm_repack_weights(1, A, 4, 256, A + 4 * 144 - 16, 10**6, None) == EINVAL  # overlap
    assert "overlap" in _last(lib)
    assert lib.qmm_repack_weights(1, A, 4, 256, A + 10**6, 4 * 144 - 1, None) == EINVAL
    assert lib.qmm_debug_block_sums(1, A, 10**9, 0, A, 10**9, A, 4 * 8 * 16 * 4 - 1,
                                    4, 8, 512, None) == EINVAL
    assert lib.qmm_debug_block_sums(7, A, 10**9, 0, A, 10**9, A, 10**9, 4, 8, 512, None) == EUNSUP
    # Q6_K group sums: K/16 int32 per (m, n)
    assert lib.qmm_debug_block_sums(2, A, 10**9, 0, A, 10**9, A, 4 * 8 * 32 * 4 - 1,
                                    4, 8, 512, None) == EINVAL


def test_status_strings(lib):
    for s in range(5):
        assert lib.qmm_status_string(s)
    assert lib.qmm_version().startswith(b"qmm")


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from bit_quantized_mat_quantize_amd import _binding
    monkeypatch.setattr(_binding, "_lib", None)
    monkeypatch.setattr(_binding, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        _binding.load()


def test_product_path_does_not_import_oracle():
    """The product package must not reach the oracle (test infrastructure)."""
    pkg = os.path.join(ROOT, "bit_quantized_mat_quantize_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                txt = open(os.path.join(dirpath, fn), encoding="utf-8").read()
                assert not re.search(r"\bimport oracle\b|from oracle\b|qmm_oracle", txt), fn
