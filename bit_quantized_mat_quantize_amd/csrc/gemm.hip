// gemm.hip -- compute-bound quantized GEMM (prefill-sized M) on int8 MFMA, gfx950.
//
// Long prefill is bound by matrix-core throughput (BitBLAS page, "调度与自动调优"
// shape table; "性能判断" roofline), so each weight column is decoded once per
// K step and contracted on v_mfma_i32_32x32x32_i8, whose K of 32 is one Q4_K
// sub-block.  Scales stay outside the integer sums (ggml-cpu mul_mat page,
// "正确性:缩放系数可以提到求和号外面"):
//
//   per super-block b, output (m, n):
//     S  = sum_j s_j * P_j,  P_j = sum_{k in j} q_k y_k          (int32, exact)
//     Mn = sum_g m_{g/2} * bsums[g]                              (exact)
//     acc += d_a * (d * S - dmin * Mn)                           (fp32)
//
// The 6-bit sub-block scale is folded into the weight operand as two int8
// digit planes, s_j = 8*hi_j + lo_j with hi_j, lo_j in [0, 7], so every plane
// value hi_j*q, lo_j*q is at most 105 and the MFMA accumulates the whole
// super-block without touching the vector ALU:
//     ACC_hi += A_j x (hi_j * Q_j),  ACC_lo += A_j x (lo_j * Q_j),  S = 8*ACC_hi + ACC_lo
// The planes are built from packed nibbles with packed 16-bit multiplies (no
// carries: each byte product is < 256).  The min term runs on fp16 MFMAs:
// |bsums| <= 2032 is exact in fp16 and -dmin*m_j (17 significant bits) is the
// exact sum of two fp16 values, so only the fp32 accumulation rounds.
//
// Workgroup: 512 threads = 8 wavefronts, two per SIMD (256 registers per
// lane each); tile 128 (M) x 256 (N); wavefront w owns columns 32w..32w+31
// (one 32-column tile) for all 128 rows (four 32-row tiles), so each weight
// column is decoded by exactly one wavefront and the decoded planes feed four
// row tiles' MFMAs.  K advances one 256-element super-block per step.  The
// int8 activation codes of step b+1 stream into the other of two LDS buffers
// with direct global->LDS loads (buffer_load ... lds, no registers involved)
// while step b is computed; bsums and d_a of step b+1 travel through
// registers (converted to fp16 on the way).  The weights do not go through
// LDS: no other wavefront reads a column, so each lane loads the 80 bytes of
// its column it needs (the 16-byte header and the payload pieces of its
// K-slice) straight into registers, one step ahead.  One barrier per step.
// Per buffer:
//   A   int8 codes   [128][256]  16-byte piece p of row r at position p ^ (r & 15)
//   BS  bsums, fp16  [128][24]   stride 48 B
//   DA  d_a          [128]
// (the XOR placement makes the 16-byte reads down 16 consecutive rows hit
// distinct banks).  Each wavefront walks its four row tiles once per step.
// The eight sub-block planes of its column tile are built inside row tile 0,
// plane j just before the first MFMAs that read it, so the decode of j + 1
// issues while the MFMAs of j run; the next step's weights are loaded once
// the planes are built.  The tail of row tile i (S = 8*ACC_hi + ACC_lo,
// t = d*S on the vector ALU, the min term added by two fp16 MFMAs that take
// t as their accumulator input, acc += d_a*t) is placed after the MFMAs of
// row tile i + 1 for the same reason.
//
// MFMA operand convention (v_mfma_*_32x32xK): lane l supplies row (A) or
// column (B) l % 32 and the K-slice selected by l / 32; A and B use the same
// slice assignment, so the sum over a sub-block is complete whatever the
// hardware order inside the slice.  Result register r of lane l holds row
// 8*(r/4) + 4*(l/32) + r%4, column l % 32.
#include "mfma_common.h"
#include "qmm_device.h"
#include "qmm_launch.h"

namespace qmm {
namespace {

constexpr int BM = 128, BN = 256, MT = BM / 32, NWAVE = 8, NTHR = 64 * NWAVE;
constexpr int CT = BN / 32 / NWAVE;  // column tiles per wavefront (one)
constexpr int A_OFF = 0, A_BYTES = BM * 256;
constexpr int BS_OFF = A_OFF + A_BYTES, BS_STRIDE = 48, BS_BYTES = BM * BS_STRIDE;
constexpr int DA_OFF = BS_OFF + BS_BYTES, DA_BYTES = BM * 4;
constexpr int BUF_BYTES = DA_OFF + DA_BYTES;
constexpr int LDS_BYTES = 2 * BUF_BYTES;
constexpr int A_INSTR = A_BYTES / 1024;  // 64-lane x 16-byte loads per buffer
constexpr int A_PER_WAVE = A_INSTR / NWAVE;
static_assert(A_INSTR % NWAVE == 0, "staging must split evenly over the wavefronts");
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of a gfx950 CU");
static_assert(CT == 1 && 2 * BM <= NTHR, "one column tile per wavefront; bsums staged by 2*BM threads");

template <bool REPACKED, bool GROUPED>
__global__ __launch_bounds__(NTHR, 1) void k_gemm_q4_K(const uint8_t *__restrict__ W,
                                                       const uint8_t *__restrict__ Y,
                                                       float *__restrict__ out, int64_t M, int64_t N,
                                                       int64_t K, int tiles_m, int tiles_n, Grouping grp) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hh = lane >> 5;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // scalar: a uniform branch

    // XCD-aware tile order: workgroups are dealt round-robin to the 8 XCDs, so
    // each XCD gets a contiguous range of the index v; v walks groups of GM
    // row tiles with the row tile fastest, so the 32 workgroups an XCD runs
    // at once cover GM row tiles x 32/GM column tiles and share both their
    // activation and weight tiles through that XCD's L2.
    constexpr int GM = 4;
    const int nwg = tiles_m * tiles_n;
    const int bid = blockIdx.x;
    int tile_m, tile_n, m_last_g = 0, r0 = 0;
    if constexpr (GROUPED) {
        int e;
        tile_m = 0;
        if (!grouped_tile(grp, bid, tiles_n, BM, tile_n, r0, m_last_g, e)) return;  // uniform
        W += (int64_t)e * grp.w_stride;
    } else {
        const int v = (nwg % 8 == 0) ? (bid % 8) * (nwg / 8) + bid / 8 : bid;
        const int group = v / (GM * tiles_n), first_m = group * GM;
        const int gm = tiles_m - first_m < GM ? tiles_m - first_m : GM;
        const int in_group = v - group * GM * tiles_n;
        // (the division runs on the vector ALU; readfirstlane keeps the tile uniform)
        tile_m = __builtin_amdgcn_readfirstlane(first_m + in_group % gm);
        tile_n = __builtin_amdgcn_readfirstlane(in_group / gm);
    }
    const int64_t m_base = (int64_t)tile_m * BM, n_base = (int64_t)tile_n * BN;
    const int64_t nb = K / QK_K;

    // ---- staging sources.  Rows past M and columns past N are clamped to the
    // last valid one (their results are never stored), so every load is in
    // bounds and none is predicated.
    const int m_last = GROUPED ? m_last_g : (int)(M - 1 - m_base < BM - 1 ? M - 1 - m_base : BM - 1);
    const int mt_used = m_last / 32 + 1;  // 32-row tiles holding valid rows
    const int n_last = (int)(N - 1 - n_base < BN - 1 ? N - 1 - n_base : BN - 1);
    const uint32_t a_rowstride = (uint32_t)(nb * kQ8_KBytes);
    const int64_t a_first = m_base * nb * kQ8_KBytes;
    const int64_t a_bytes = M * nb * kQ8_KBytes - a_first;
    // byte offset (from Y + a_first) of tile row rr <= m_last
    auto arow = [&](int rr) -> uint32_t {
        if constexpr (GROUPED) {
            return (uint32_t)grouped_row(grp, r0, rr) * a_rowstride;
        } else {
            return (uint32_t)rr * a_rowstride;
        }
    };
    uint32_t a_goff[A_PER_WAVE];
#pragma unroll
    for (int t = 0; t < A_PER_WAVE; ++t) {
        const int row = (wave * A_PER_WAVE + t) * 4 + (lane >> 4);
        const int gp = (lane & 15) ^ (row & 15);  // global piece stored at position lane & 15
        const int rr = row < m_last ? row : m_last;
        a_goff[t] = arow(rr) + 4 + 16 * gp;
    }
    // this lane's weight column (clamped), straight into registers
    const uint32_t hdr_step = REPACKED ? 16 : kQ4_KBytes, pay_step = REPACKED ? 128 : kQ4_KBytes;
    const int64_t w_bytes = N * nb * kQ4_KBytes;
    const int64_t n_lane = n_base + wave * 32 + l32 < N ? n_base + wave * 32 + l32 : N - 1;
    const int64_t i0 = n_lane * nb;
    const uint32_t v_hdr = (uint32_t)(hdr_step * i0);
    const uint32_t v_pay = (uint32_t)(REPACKED ? 16 * N * nb + 128 * i0 + 16 * hh : kQ4_KBytes * i0 + 16 + 16 * hh);
    // bsums: row tid>>1, 16-byte half tid&1 (threads < 256); d_a: row tid (threads < 128)
    const int s_row = (tid >> 1) & (BM - 1);
    const uint32_t s_off = arow(s_row < m_last ? s_row : m_last) + 260 + 16 * (tid & 1);
    const uint32_t d_off = arow((tid & (BM - 1)) < m_last ? (tid & (BM - 1)) : m_last);

    auto issue = [&](int64_t b, uint8_t *buf) {
        const rsrc_t ra = make_rsrc(Y + a_first, a_bytes);
        const uint32_t sa = (uint32_t)b * kQ8_KBytes;
#pragma unroll
        for (int t = 0; t < A_PER_WAVE; ++t)
            dma16(ra, a_goff[t], sa, buf + A_OFF + (wave * A_PER_WAVE + t) * 1024);
    };
    struct WStage {
        uint4 hdr, pay[4];
    };
    auto wload = [&](int64_t b, WStage &x) {
        const rsrc_t rw = make_rsrc(W, w_bytes);
        const uint32_t bb = (uint32_t)b;
        x.hdr = bld16(rw, v_hdr, hdr_step * bb);
#pragma unroll
        for (int g = 0; g < 4; ++g) x.pay[g] = bld16(rw, v_pay + 32 * g, pay_step * bb);
    };
    auto prefetch = [&](int64_t b, uint4 &raw, uint32_t &draw) {
        const rsrc_t ra = make_rsrc(Y + a_first, a_bytes);
        const uint32_t sa = (uint32_t)b * kQ8_KBytes;
        if (tid < 2 * BM) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(ra, s_off, sa, 0);
            raw = make_uint4(v.x, v.y, v.z, v.w);
        }
        if (tid < BM) draw = __builtin_amdgcn_raw_buffer_load_b32(ra, d_off, sa, 0);
    };
    auto commit = [&](const uint4 &raw, uint32_t draw, uint8_t *buf) {
        if (tid < 2 * BM) {
            const uint4 hv = make_uint4(h2_bits((int16_t)(raw.x & 0xffff), (int16_t)(raw.x >> 16)),
                                        h2_bits((int16_t)(raw.y & 0xffff), (int16_t)(raw.y >> 16)),
                                        h2_bits((int16_t)(raw.z & 0xffff), (int16_t)(raw.z >> 16)),
                                        h2_bits((int16_t)(raw.w & 0xffff), (int16_t)(raw.w >> 16)));
            *reinterpret_cast<uint4 *>(buf + BS_OFF + s_row * BS_STRIDE + 16 * (tid & 1)) = hv;
        }
        if (tid < BM) *reinterpret_cast<uint32_t *>(buf + DA_OFF + 4 * tid) = draw;
    };

    float acc[MT][CT][16];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][c][r] = 0.0f;

    uint4 raw = make_uint4(0, 0, 0, 0);
    uint32_t draw = 0;
    WStage wx;
    issue(0, lds);
    prefetch(0, raw, draw);
    wload(0, wx);

    for (int64_t b = 0; b < nb; ++b) {
        uint8_t *buf = lds + (b & 1) * BUF_BYTES;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's loads of step b
        commit(raw, draw, buf);
        __syncthreads();  // every thread's step-b data is in LDS; step b-1 is fully consumed
        if (b + 1 < nb) {
            issue(b + 1, lds + ((b + 1) & 1) * BUF_BYTES);
            prefetch(b + 1, raw, draw);
        }
        // ---------------- this lane's column: header; the 8 sub-block planes are
        // built inside row tile 0, each just before its first MFMAs, so the
        // decode of sub-block j + 1 overlaps the MFMAs of sub-block j
        const uint4 hdr = wx.hdr;
        const float dcol = f16_bits_to_f32(hdr.x & 0xffff);
        const float dmcol = f16_bits_to_f32(hdr.x >> 16);
        const Q4KScales sc = unpack_scales(hdr.y, hdr.z, hdr.w);
        v4i bhi[8], blo[8];
        auto build = [&](int j) {
            const uint4 pw = wx.pay[j >> 1];
            const uint32_t sw = j < 4 ? sc.s_lo : sc.s_hi;
            const int shift = (j & 1) * 4;  // low nibbles: sub-block 2g, high: 2g + 1
            const uint32_t q0 = (pw.x >> shift) & 0x0f0f0f0fu, q1 = (pw.y >> shift) & 0x0f0f0f0fu;
            const uint32_t q2 = (pw.z >> shift) & 0x0f0f0f0fu, q3 = (pw.w >> shift) & 0x0f0f0f0fu;
            const uint32_t sj = (sw >> (8 * (j & 3))) & 0xff;
            const uint32_t hi2 = (sj >> 3) * 0x00010001u, lo2 = (sj & 7) * 0x00010001u;
            bhi[j] = v4i{plane(q0, hi2), plane(q1, hi2), plane(q2, hi2), plane(q3, hi2)};
            blo[j] = v4i{plane(q0, lo2), plane(q1, lo2), plane(q2, lo2), plane(q3, lo2)};
        };
        // min-term operand: -dmin*m_j has at most 17 significant bits, so it is
        // the exact sum of two fp16 values (hi = fp16(-dmin*m), lo = remainder);
        // two fp16 MFMAs against the exact fp16 bsums add -dmin*Mn to d*S in
        // fp32 (the MFMA's accumulator input carries d*S).
        v8h bmh, bml;
        {
            const uint32_t mw = hh == 0 ? sc.m_lo : sc.m_hi;  // m_{4hh .. 4hh+3}
            uint32_t bh[4], bl[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float vv = -dmcol * (float)((mw >> (8 * e)) & 0xff);  // exact in fp32
                const uint32_t hb = f32_to_f16_bits(vv);
                const uint32_t lb = f32_to_f16_bits(vv - f16_bits_to_f32(hb));
                bh[e] = hb | (hb << 16);
                bl[e] = lb | (lb << 16);
            }
            __builtin_memcpy(&bmh, bh, 16);
            __builtin_memcpy(&bml, bl, 16);
        }
        const float *da = reinterpret_cast<const float *>(buf + DA_OFF);

        // ---------------- the four row tiles of this column tile.  The tail of
        // row tile i - 1 (conversion, min term, accumulation) is placed after the
        // MFMAs of row tile i, so its vector work can issue while they run.
        v16i s_prev;
        v8h bs_prev;
        auto tail = [&](int i, const v16i &S, const v8h &a_bs) {
            v16f t;
#pragma unroll
            for (int r = 0; r < 16; ++r) t[r] = dcol * (float)S[r];
            t = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_bs, bmh, t, 0, 0, 0);
            t = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_bs, bml, t, 0, 0, 0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 d4 = *reinterpret_cast<const float4 *>(da + i * 32 + 8 * q + 4 * hh);
                const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][0][4 * q + e] = fmaf(dv[e], t[4 * q + e], acc[i][0][4 * q + e]);
            }
        };
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            // The two wavefronts of a SIMD (w and w + 4) take turns at high issue
            // priority, one row tile each, so one issues its MFMAs while the other's
            // vector work fills the gaps (c5, alternating runs: M = 2048 1045 against
            // 1085-1096 us, M = 512 317-322 against 321-326 us; priority for the
            // plane-building row tile only, or for the MFMAs against the tails, gained
            // about half of that).  Priority changes no result.
            if (((wave_u >> 2) ^ i) & 1)
                __builtin_amdgcn_s_setprio(0);
            else
                __builtin_amdgcn_s_setprio(2);
            // row tiles past the last valid row (a short tail tile, or an
            // expert's remainder rows under mul_mat_id) are skipped; row tile 0
            // always runs (it builds the planes and requests the next weights)
            if (i > 0 && i >= mt_used) continue;  // wavefront-uniform
            const int row = i * 32 + l32;
            const v16i zero = {};
            v16i ah, al;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                v4i a_op[4];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int j = 4 * half + jj;
                    const uint4 a = *reinterpret_cast<const uint4 *>(buf + A_OFF + row * 256 +
                                                                     16 * ((2 * j + hh) ^ (row & 15)));
                    a_op[jj] = v4i{(int)a.x, (int)a.y, (int)a.z, (int)a.w};
                }
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int j = 4 * half + jj;
                    if (i == 0) build(j);
                    ah = __builtin_amdgcn_mfma_i32_32x32x32_i8(a_op[jj], bhi[j], j ? ah : zero, 0, 0, 0);
                    al = __builtin_amdgcn_mfma_i32_32x32x32_i8(a_op[jj], blo[j], j ? al : zero, 0, 0, 0);
                }
            }
            if (i == 0 && b + 1 < nb) wload(b + 1, wx);  // the planes no longer need wx
            if (i > 0) tail(i - 1, s_prev, bs_prev);
            {
                const uint4 au = *reinterpret_cast<const uint4 *>(buf + BS_OFF + row * BS_STRIDE + 16 * hh);
                __builtin_memcpy(&bs_prev, &au, 16);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) s_prev[r] = (ah[r] << 3) + al[r];
        }
        // the tail of the last row tile run
        if (mt_used == MT) tail(MT - 1, s_prev, bs_prev);
#pragma unroll
        for (int i = 0; i < MT - 1; ++i)
            if (mt_used == i + 1) tail(i, s_prev, bs_prev);
    }

    // ---- store: register r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32
#pragma unroll
    for (int c = 0; c < CT; ++c) {
        const int64_t n = n_base + wave * 32 + l32;
        if (n < N) {
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    if constexpr (GROUPED) {
                        const int lm = i * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
                        if (lm <= m_last) out[(int64_t)grp.sorted[r0 + lm] * N + n] = acc[i][c][r];
                    } else {
                        const int64_t m = m_base + i * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
                        if (m < M) out[m * N + n] = acc[i][c][r];
                    }
                }
        }
    }
}

// tiles_m is the row-tile count (GROUPED: the most tiles any routing can
// produce; surplus workgroups exit at once)
template <bool REPACKED, bool GROUPED>
hipError_t launch(const uint8_t *w, const uint8_t *y, float *out, int64_t M, int64_t N, int64_t K,
                  int tiles_m, const Grouping &g, hipStream_t s) {
    static std::atomic<uint64_t> lds_set{0};  // the LDS budget above 64 KiB, per device
    const hipError_t e = ensure_lds_bytes((const void *)k_gemm_q4_K<REPACKED, GROUPED>, LDS_BYTES, lds_set);
    if (e != hipSuccess) return e;
    const int tiles_n = (int)((N + BN - 1) / BN);
    hipLaunchKernelGGL((k_gemm_q4_K<REPACKED, GROUPED>), dim3((unsigned)(tiles_m * tiles_n)), dim3(NTHR),
                       LDS_BYTES, s, w, y, out, M, N, K, tiles_m, tiles_n, g);
    return hipGetLastError();
}

}  // namespace

int gemm_tile_rows() { return BM; }

hipError_t launch_gemm_q4_K(const uint8_t *w, bool repacked, const uint8_t *y, float *out,
                            int64_t M, int64_t N, int64_t K, hipStream_t s) {
    const int tiles_m = (int)((M + BM - 1) / BM);
    return repacked ? launch<true, false>(w, y, out, M, N, K, tiles_m, Grouping{}, s)
                    : launch<false, false>(w, y, out, M, N, K, tiles_m, Grouping{}, s);
}

hipError_t launch_gemm_id_q4_K(const uint8_t *w, bool repacked, int64_t w_stride, const uint8_t *y,
                               int64_t y_rows, int y_per_slot, int64_t U, const int32_t *group_ws,
                               int64_t E, int64_t P, float *out, int64_t N, int64_t K, hipStream_t s) {
    const MoeGroupLayout L = moe_group_layout(P, E, BM);
    const Grouping g{group_ws + L.start, group_ws + L.tile_e, group_ws + L.tile_r0, group_ws + L.ntiles,
                     group_ws + L.sorted, U, w_stride, y_per_slot};
    return repacked ? launch<true, true>(w, y, out, y_rows, N, K, (int)L.max_tiles, g, s)
                    : launch<false, true>(w, y, out, y_rows, N, K, (int)L.max_tiles, g, s);
}

}  // namespace qmm
