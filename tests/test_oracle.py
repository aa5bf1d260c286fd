"""Pins for the CPU oracle (no GPU).

Each test ties the oracle to something other than itself: values the pages
print (golden fixtures), the format definitions, closed forms, invariants of
the encoders, and brute force on tiny inputs.  A plausible slip in the oracle
(a swapped nibble, a dropped min term, a wrong scale bit, a wrong sign) fails
at least one of them.
"""
import json
import os
import struct

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _f16(x):
    return struct.pack("<e", x)


# --------------------------------------------------------------------- fp16
def test_fp16_encodings(orc):
    for val, hexbits in _gold("fp16_values.json")["cases"]:
        assert orc.f32_to_f16(val) == int(hexbits, 16), (val, hexbits)


def test_fp16_matches_numpy_rne(orc):
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(3000) * 10.0 ** rng.integers(-9, 5, 3000),
        rng.uniform(-65000, 65000, 500)]).astype(np.float32)
    want = x.astype(np.float16).view(np.uint16)
    got = np.array([orc.f32_to_f16(v) for v in x], np.uint16)
    assert np.array_equal(got, want)
    back = np.array([orc.f16_to_f32(h) for h in want], np.float32)
    assert np.array_equal(back, want.view(np.float16).astype(np.float32))


# -------------------------------------------------------------- block sizes
def test_block_sizes(orc):
    g = _gold("block_sizes.json")
    for fmt, K in (("q4_0", 64), ("q8_0", 64), ("q4_K", 512), ("q8_K", 512), ("q6_K", 512),
                   ("q2_K", 512)):
        x = np.zeros((3, K), np.float32)
        b = orc.quantize(fmt, x)
        per = g[fmt]
        assert b.shape == (3, K // per["elements"] * per["bytes"])
        assert per["bytes"] * 8 / per["elements"] == per["bpw"]


# ------------------------------------------------- Q4_K scale/min bit field
def test_scale_pack_roundtrip_exhaustive(orc):
    rng = np.random.default_rng(2)
    for j in range(8):
        for v in range(64):
            s = rng.integers(0, 64, 8).astype(np.uint8)
            m = rng.integers(0, 64, 8).astype(np.uint8)
            s[j] = v
            m[j] = 63 - v
            packed = orc.pack_scales(s, m)
            for jj in range(8):
                assert orc.get_scale_min(packed, jj) == (s[jj], m[jj])


def test_scale_field_word_parallel_rule(orc):
    """The page's word-parallel unpack (three 32-bit masks, "6-bit 参数是怎么塞进
    12 字节的"): the mins of sub-blocks 4..7 are the high nibbles of bytes 8..11
    joined with the top two bits of bytes 4..7 shifted up by four.  Checked
    against the per-j decode on random fields (every bit pattern is valid)."""
    rng = np.random.default_rng(3)
    for _ in range(2000):
        f = rng.integers(0, 256, 12).astype(np.uint8)
        w0, w1, w2 = struct.unpack("<III", f.tobytes())
        word = ((w2 >> 4) & 0x0F0F0F0F) | (((w1 >> 6) & 0x03030303) << 4)
        mins_hi = [(word >> (8 * i)) & 0xFF for i in range(4)]
        assert mins_hi == [orc.get_scale_min(f, 4 + i)[1] for i in range(4)]
        # the scales of sub-blocks 4..7: low nibbles of bytes 8..11 joined with
        # the top two bits of bytes 0..3
        word = (w2 & 0x0F0F0F0F) | (((w0 >> 6) & 0x03030303) << 4)
        scales_hi = [(word >> (8 * i)) & 0xFF for i in range(4)]
        assert scales_hi == [orc.get_scale_min(f, 4 + i)[0] for i in range(4)]
        # and the first four: low six bits of bytes 0..3 (scales), 4..7 (mins)
        assert [orc.get_scale_min(f, i)[0] for i in range(4)] == [b & 63 for b in f[:4]]
        assert [orc.get_scale_min(f, i)[1] for i in range(4)] == [b & 63 for b in f[4:8]]


# ------------------------------------------------------ hand-built blocks
def _q4K_block(d, dmin, s, m, q):
    """Bytes of one Q4_K block built by hand from the page's packing rule:
    for each 64-element group, byte l = q[l] | q[l+32] << 4."""
    from oracle import pack_scales  # scale field pinned above
    qs = bytearray(128)
    for g in range(4):
        for l in range(32):
            qs[32 * g + l] = q[64 * g + l] | (q[64 * g + 32 + l] << 4)
    return np.frombuffer(_f16(d) + _f16(dmin) + pack_scales(s, m).tobytes() + bytes(qs),
                         np.uint8).copy()


def _q8K_block(d, y):
    y = np.asarray(y, np.int8)
    bs = [int(y[16 * g:16 * g + 16].astype(np.int32).sum()) for g in range(16)]
    return np.frombuffer(struct.pack("<f", d) + y.tobytes() + struct.pack("<16h", *bs),
                         np.uint8).copy()


def test_worked_example(orc):
    """Hand-computed sub-block of the ggml-cpu page: d=0.5, dmin=0.25, s=4,
    m=1, q=3, d_a=0.02, y=10 -> 36.8 per 32-element sub-block."""
    g = _gold("worked_example_q4_K.json")
    W, A = g["weights"], g["activations"]
    for j in range(8):
        s = [0] * 8
        m = [0] * 8
        s[j], m[j] = W["s_j"], W["m_j"]
        w = _q4K_block(W["d"], W["dmin"], s, m, [W["q"]] * 256)
        y = _q8K_block(A["d_a"], [A["y"]] * 256)
        deq_w = orc.dequantize("q4_K", w, 1, 256)
        deq_a = orc.dequantize("q8_K", y, 1, 256)
        sb = slice(32 * j, 32 * j + 32)
        assert np.all(deq_w[0, sb] == g["dequantized_weight"])
        assert np.allclose(deq_a[0], g["dequantized_activation"], rtol=1e-7)
        P = orc.subblock_sums("q4_K", w, y, 1, 1, 256)
        assert P[0, 0, j] == g["integer_path"]["sum_q_y"]
        out = orc.mul_mat("q4_K", w, y, 1, 1, 256)[0, 0]
        # d_a = 0.02 is not exact in fp32: allow its representation error only
        assert abs(out - g["integer_path"]["result"]) < 1e-6
        bf, _ = orc.brute_force(deq_w, deq_a)
        assert abs(bf[0, 0] - g["dequant_path_result"]) < 1e-6
    # all eight sub-blocks carrying the example
    w = _q4K_block(W["d"], W["dmin"], [W["s_j"]] * 8, [W["m_j"]] * 8, [W["q"]] * 256)
    y = _q8K_block(A["d_a"], [A["y"]] * 256)
    assert abs(orc.mul_mat("q4_K", w, y, 1, 1, 256)[0, 0] - 8 * 36.8) < 1e-5


def test_q4K_nibble_order_and_pack_identity(orc):
    """Element order of the 128 payload bytes, and the packing identity of the
    BitBLAS page (q_i = (u >> 4i) & 15 for a 32-bit word u): in word t of
    64-element group g, nibble 2b is element 64g+4t+b, nibble 2b+1 is element
    64g+32+4t+b."""
    rng = np.random.default_rng(4)
    q = rng.integers(0, 16, 256)
    w = _q4K_block(1.0, 0.0, [1] * 8, [0] * 8, list(q))
    deq = orc.dequantize("q4_K", w, 1, 256)[0]
    assert np.array_equal(deq, q.astype(np.float64))
    words = np.frombuffer(w[16:].tobytes(), "<u4")
    for g in range(4):
        for t in range(8):
            u = int(words[8 * g + t])
            for i in range(8):
                b, hi = divmod(i, 2)
                k = 64 * g + 32 * hi + 4 * t + b
                assert (u >> (4 * i)) & 15 == q[k]


def test_q4_0_layout_and_formula(orc):
    """Q4_0: w = d (q - 8) (page: "最基础的两块"); byte l holds element l in
    its low nibble and l+16 in its high nibble (the reading taken)."""
    rng = np.random.default_rng(5)
    q = rng.integers(0, 16, 32)
    qs = bytes(int(q[l] | (q[l + 16] << 4)) for l in range(16))
    blk = np.frombuffer(_f16(0.5) + qs, np.uint8).copy()
    deq = orc.dequantize("q4_0", blk, 1, 32)[0]
    assert np.array_equal(deq, 0.5 * (q - 8))
    u = np.frombuffer(qs, "<u4")
    for t in range(4):
        for i in range(8):
            b, hi = divmod(i, 2)
            assert (int(u[t]) >> (4 * i)) & 15 == q[16 * hi + 4 * t + b]


# ----------------------------------------------------- activation encoders
@pytest.mark.parametrize("fmt,QK", [("q8_0", 32), ("q8_K", 256)])
def test_q8_invariants(orc, fmt, QK):
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((5, 4 * QK)) * rng.uniform(0.01, 100, (5, 1))).astype(np.float32)
    x[2, :QK] = 0.0                      # an all-zero block
    x[3, QK:2 * QK] = 7.0                # a constant block
    b = orc.quantize(fmt, x)
    nb, bb = 4, {"q8_0": 34, "q8_K": 292}[fmt]
    for r in range(5):
        for blk in range(nb):
            raw = b[r, blk * bb:(blk + 1) * bb].tobytes()
            if fmt == "q8_0":
                d = float(np.frombuffer(raw[:2], np.float16)[0])
                y = np.frombuffer(raw[2:], np.int8).astype(np.int64)
            else:
                d = float(np.frombuffer(raw[:4], np.float32)[0])
                y = np.frombuffer(raw[4:260], np.int8).astype(np.int64)
                bs = np.frombuffer(raw[260:], "<i2")
                assert np.array_equal(bs, y.reshape(16, 16).sum(1))
            xb = x[r, blk * QK:(blk + 1) * QK].astype(np.float64)
            amax = np.abs(xb).max()
            if amax == 0:
                assert d == 0 and not y.any()
                continue
            i = int(np.abs(xb).argmax())
            assert abs(y[i]) == 127 and np.sign(y[i]) == np.sign(xb[i])
            assert np.abs(y).max() == 127
            d32 = np.float32(amax) / np.float32(127)
            assert abs(d - d32) <= (0 if fmt == "q8_K" else 2.0 ** -10 * d32)
            err = np.abs(xb - float(d32) * y)
            assert err.max() <= 0.5 * float(d32) * (1 + 1e-5)


def test_q8_exact_window_and_ties(orc):
    """amax = 127 gives d = 1 exactly, so integers pass through unchanged and
    halves round to even (the rounding reading taken)."""
    x = np.zeros((1, 256), np.float32)
    x[0, 0] = 127.0
    x[0, 1:6] = [2.5, 3.5, -2.5, -0.5, 0.5]
    x[0, 6:40] = np.arange(-17, 17)
    b = orc.quantize("q8_K", x)[0]
    assert np.frombuffer(b[:4].tobytes(), np.float32)[0] == 1.0
    y = np.frombuffer(b[4:260].tobytes(), np.int8)
    assert list(y[:6]) == [127, 2, 4, -2, 0, 0]
    assert list(y[6:40]) == list(range(-17, 17))


# ------------------------------------------------------- weight encoders
def test_q4_0_encoder_roundtrip(orc):
    """Blocks whose largest-magnitude element decodes from q=0 and whose d is a
    power of two are reproduced exactly by encode(decode(block))."""
    rng = np.random.default_rng(7)
    rows, K = 6, 128
    blocks = bytearray()
    for _ in range(rows * K // 32):
        q = rng.integers(1, 16, 32)
        q[rng.integers(0, 32)] = 0
        d = float(2.0 ** rng.integers(-12, 2)) * (1 if rng.random() < 0.5 else -1)
        blocks += _f16(d) + bytes(int(q[l] | (q[l + 16] << 4)) for l in range(16))
    blocks = np.frombuffer(bytes(blocks), np.uint8).reshape(rows, -1)
    x = orc.dequantize("q4_0", blocks, rows, K).astype(np.float32)
    assert np.array_equal(orc.quantize("q4_0", x), blocks)


def test_q4_K_encoder_roundtrip(orc):
    """A super-block whose sub-blocks all contain q=0 and q=15, whose largest
    s_j and m_j are 63, and whose d, dmin are powers of two is reproduced
    exactly: the min/max search recovers s_j, m_j, d, dmin and every q."""
    rng = np.random.default_rng(8)
    rows, nbk = 4, 3
    blocks = []
    for _ in range(rows * nbk):
        s = rng.integers(1, 64, 8)
        m = rng.integers(0, 64, 8)
        s[rng.integers(0, 8)] = 63
        m[rng.integers(0, 8)] = 63
        q = rng.integers(0, 16, 256)
        for j in range(8):
            a, b = rng.choice(32, 2, replace=False)
            q[32 * j + a], q[32 * j + b] = 0, 15
        d = float(2.0 ** rng.integers(-14, -4))
        dmin = float(2.0 ** rng.integers(-14, -4))
        blocks.append(_q4K_block(d, dmin, list(s), list(m), list(q)))
    blocks = np.concatenate(blocks).reshape(rows, -1)
    x = orc.dequantize("q4_K", blocks, rows, 256 * nbk).astype(np.float32)
    assert np.array_equal(orc.quantize("q4_K", x), blocks)


def test_q4_K_encoder_error_bound(orc):
    """On skewed heavy-tailed rows the decoded weight stays within half a step
    (plus the 6-bit/fp16 rounding of the step) of the input."""
    from bit_quantized_mat_quantize_amd.inputs import weights_t4_skewed
    x = weights_t4_skewed(11, 16, 1024)
    b = orc.quantize("q4_K", x)
    w = orc.dequantize("q4_K", b, 16, 1024)
    for r in range(16):
        for blk in range(4):
            raw = b[r, blk * 144:(blk + 1) * 144]
            d = float(np.frombuffer(raw[:2].tobytes(), np.float16)[0])
            for j in range(8):
                s, m = orc.get_scale_min(raw[4:16], j)
                sl = slice(blk * 256 + 32 * j, blk * 256 + 32 * j + 32)
                # q is clamped to [0,15]; when the rounded step is smaller than
                # the exact one the top of the range may clip by up to 15*|rounding|
                step = d * s
                err = np.abs(x[r, sl] - w[r, sl]).max()
                assert err <= 0.5 * step + 16 * 0.5 * d + 1e-6


def test_zero_inputs(orc):
    z = np.zeros((2, 512), np.float32)
    for fmt in ("q4_K", "q8_0", "q8_K"):
        b = orc.quantize(fmt, z)
        assert not b.any()
    # Q4_0 has no zero code: q = 8 decodes to 0 under any d, and d is +0
    b = orc.quantize("q4_0", z).reshape(-1, 18)
    assert not b[:, :2].any() and (b[:, 2:] == 0x88).all()
    assert not orc.dequantize("q4_0", b, 2, 512).any()


# ---------------------------------------------------- integer path vs brute
@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (2, 3, 512), (3, 5, 256), (7, 2, 768)])
def test_q4K_integer_path_vs_brute_force(orc, M, N, K):
    from bit_quantized_mat_quantize_amd.inputs import activations, weights_t4_skewed
    w = orc.quantize("q4_K", weights_t4_skewed(20 + M, N, K))
    y = orc.quantize("q8_K", activations(30 + M, M, K, outlier_frac=0.02))
    bf, terms = orc.brute_force(orc.dequantize("q4_K", w, N, K), orc.dequantize("q8_K", y, M, K))
    out = orc.mul_mat("q4_K", w, y, M, N, K)
    assert np.all(np.abs(out - bf) <= 1e-12 * terms + 1e-300)
    so, st = orc.sample("q4_K", w, y, M, N, K, np.repeat(np.arange(M), N), np.tile(np.arange(N), M))
    assert np.array_equal(so, out.ravel())
    assert np.allclose(st, terms.ravel(), rtol=1e-12)
    # the per-sub-block sums equal the integer dot products of the codes
    P = orc.subblock_sums("q4_K", w, y, M, N, K)
    qy = orc.dequantize("q8_K", y, M, K)  # not used for P; codes taken below
    del qy
    codes_w = np.zeros((N, K), np.int64)
    for n in range(N):
        for b in range(K // 256):
            raw = w[n, 144 * b:144 * b + 144]
            for k in range(256):
                g, r = divmod(k, 64)
                byte = int(raw[16 + 32 * g + r % 32])
                codes_w[n, 256 * b + k] = byte & 15 if r < 32 else byte >> 4
    codes_y = np.stack([np.concatenate([np.frombuffer(y[m, 292 * b + 4:292 * b + 260].tobytes(), np.int8)
                                        for b in range(K // 256)]) for m in range(M)]).astype(np.int64)
    want = (codes_y[:, None, :] * codes_w[None, :, :]).reshape(M, N, K // 32, 32).sum(-1)
    assert np.array_equal(P, want)


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (2, 3, 64), (3, 4, 1024)])
def test_q4_0_integer_path_vs_brute_force(orc, M, N, K):
    from bit_quantized_mat_quantize_amd.inputs import activations, weights_normal
    w = orc.quantize("q4_0", weights_normal(40 + M, N, K))
    y = orc.quantize("q8_0", activations(50 + M, M, K))
    bf, terms = orc.brute_force(orc.dequantize("q4_0", w, N, K), orc.dequantize("q8_0", y, M, K))
    out = orc.mul_mat("q4_0", w, y, M, N, K)
    assert np.all(np.abs(out - bf) <= 1e-12 * terms + 1e-300)
    # the sampler, asked for every (m, n) in a shuffled order, returns the same
    # outputs and the brute-force sum|w a|: a wrong activation or weight stride
    # in the sampler picks another row and fails here
    perm = np.random.default_rng(M * 131 + N).permutation(M * N)
    ms, ns = perm // N, perm % N
    so, st = orc.sample("q4_0", w, y, M, N, K, ms, ns)
    assert np.array_equal(so, out[ms, ns])
    assert np.allclose(st, terms[ms, ns], rtol=1e-12, atol=0)
    # the block sums equal sum (q - 8) y over each 32-block, with the codes read
    # straight from the block bytes (d first, then element l low / l+16 high)
    P = orc.subblock_sums("q4_0", w, y, M, N, K)
    nb = K // 32
    qw = np.zeros((N, K), np.int64)
    for n in range(N):
        for b in range(nb):
            qs = w[n, 18 * b + 2:18 * b + 18].astype(np.int64)
            qw[n, 32 * b:32 * b + 16] = (qs & 15) - 8
            qw[n, 32 * b + 16:32 * b + 32] = (qs >> 4) - 8
    qy = np.stack([np.concatenate([y[m, 34 * b + 2:34 * b + 34].view(np.int8) for b in range(nb)])
                   for m in range(M)]).astype(np.int64)
    want = (qy[:, None, :] * qw[None, :, :]).reshape(M, N, nb, 32).sum(-1)
    assert np.array_equal(P, want)


def test_special_cases(orc):
    """s_j = 0 leaves only the min term; m_j = 0 makes the block symmetric;
    all q = c gives P_j = c * Y_j; d = dmin = 0 gives 0."""
    rng = np.random.default_rng(9)
    y_codes = rng.integers(-127, 128, 256)
    y = _q8K_block(0.125, y_codes)
    Y = y_codes.reshape(8, 32).sum(1)
    s = [0, 5, 0, 7, 0, 0, 63, 1]
    m = [3, 0, 9, 0, 0, 63, 0, 2]
    w = _q4K_block(0.5, 0.25, s, m, [6] * 256)
    P = orc.subblock_sums("q4_K", w, y, 1, 1, 256)[0, 0]
    assert np.array_equal(P, 6 * Y)
    want = 0.125 * (0.5 * sum(si * 6 * Yi for si, Yi in zip(s, Y)) - 0.25 * sum(mi * Yi for mi, Yi in zip(m, Y)))
    assert abs(orc.mul_mat("q4_K", w, y, 1, 1, 256)[0, 0] - want) < 1e-9
    w0 = _q4K_block(0.0, 0.0, s, m, list(rng.integers(0, 16, 256)))
    assert orc.mul_mat("q4_K", w0, y, 1, 1, 256)[0, 0] == 0.0


def test_repack_is_a_permutation(orc):
    from bit_quantized_mat_quantize_amd.inputs import weights_normal
    N, K = 5, 512
    for fmt in ("q4_K", "q4_0"):
        w = orc.quantize(fmt, weights_normal(60, N, K))
        r = orc.repack(fmt, w, N, K)
        assert r.size == orc.repacked_bytes(fmt, N, K)
        nb = K // (256 if fmt == "q4_K" else 32)
        if fmt == "q4_K":
            hdr = r[:16 * N * nb].reshape(N * nb, 16)
            pay = r[16 * N * nb:].reshape(N * nb, 128)
            canon = w.reshape(N * nb, 144)
            assert np.array_equal(hdr, canon[:, :16]) and np.array_equal(pay, canon[:, 16:])
        else:
            dsec = r.size - 16 * N * nb
            assert dsec % 256 == 0 and dsec >= 2 * N * nb
            canon = w.reshape(N * nb, 18)
            assert np.array_equal(r[:2 * N * nb].reshape(-1, 2), canon[:, :2])
            assert not r[2 * N * nb:dsec].any()
            assert np.array_equal(r[dsec:].reshape(-1, 16), canon[:, 2:])
