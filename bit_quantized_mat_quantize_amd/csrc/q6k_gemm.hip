// q6k_gemm.hip -- Q6_K weights x Q8_K activations on int8 MFMA (prefill-sized
// M), gfx950, for the load-time (repacked) weight layout.
//
// Format and integer path: ggml-cpu mul_mat page, "更低的比特:Q6_K 与 Q2_K 的取舍"
// (ql/qh 6-bit codes, int8 scale per 16-element group, fp16 d, no min) and
// "正确性:缩放系数可以提到求和号外面" (scales outside the integer sums):
//   per super-block b, output (m, n):  S = sum_j s_j * sum_{i in j} q_i y_i,
//   acc += d_a * d * S.
//
// Tiling as in the Q4_K GEMM: 512 threads = 8 wavefronts, tile 128 (M) x 256
// (N), wavefront w owns the 32-column tile 32w..32w+31 for all four 32-row
// tiles, K advances one super-block per step, the int8 activation tile is
// double-buffered in LDS (direct global->LDS loads, XOR-swizzled pieces) with
// d_a beside it.  The weights do not go through LDS: no other wavefront reads
// a column, so each lane loads the 112 bytes of its column it needs straight
// into registers, one step ahead.
// Step order as in the Q4_K GEMM: the weight operands of chunk c are built
// inside row tile 0 just before its first MFMAs (the next step's weights load
// once they are built), and the tail of row tile i sits after the MFMAs of
// row tile i + 1, so vector and matrix work of one wavefront overlap.
//
// MFMA K-slices: in v_mfma_i32_32x32x32_i8 lane l supplies the 16 consecutive
// elements 16*(l/32).. of a 32-element chunk, i.e. exactly one 16-element
// group, so the group scale is one value per lane.  The lane forms per element
// the scaled code t = s * q in [-4064, 4096] and splits it into two int8
// digits, t = 256 * hi + lo with lo the signed low byte (hi in [-16, 16]);
// two MFMAs per chunk accumulate H = sum hi*y and L = sum lo*y over the
// super-block, and S = 256 H + L exactly (|S| <= 256 * 4096 * 127 < 2^31).
// The products are formed in packed 16-bit lanes: with the stored code
// u = q + 32, t + 128 = s*u + (128 - 32s) is one v_pk_mad per two codes, its
// high byte is hi and its low byte with the top bit flipped is lo, and
// v_perm_b32 moves bytes between the 8-bit and 16-bit lane layouts.  No bsums
// and no min term: the epilogue is acc += d_a * (d * S).
#include "mfma_common.h"
#include "qmm_device.h"
#include "qmm_launch.h"

namespace qmm {
namespace {

constexpr int BM = 128, BN = 256, MT = BM / 32, NWAVE = 8, NTHR = 64 * NWAVE;
constexpr int A_OFF = 0, A_BYTES = BM * 256;
constexpr int DA_OFF = A_OFF + A_BYTES, DA_BYTES = BM * 4;
constexpr int BUF_BYTES = DA_OFF + DA_BYTES;
constexpr int LDS_BYTES = 2 * BUF_BYTES;
constexpr int A_INSTR = A_BYTES / 1024;  // 64-lane x 16-byte loads per buffer
constexpr int A_PER_WAVE = A_INSTR / NWAVE;
static_assert(A_INSTR % NWAVE == 0, "activation staging must split evenly over the wavefronts");
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of a gfx950 CU");
static_assert(BN == 32 * NWAVE && BM <= NTHR, "one column tile per wavefront; d_a staged by BM threads");

// The weight side of one super-block for lane (column c, slice h): the ql
// pieces 2g + h (both nibbles used), the qh pieces h and h + 2, the block's
// 16 scales and its fp16 d.
struct Q6KStage {
    uint4 ql[4];
    uint4 qa, qb;
    uint4 sc;
    uint32_t d;
};

template <bool GROUPED>
__global__ __launch_bounds__(NTHR, 1) void k_gemm_q6_K(const uint8_t *__restrict__ W, int64_t w_bytes,
                                                       const uint8_t *__restrict__ Y,
                                                       float *__restrict__ out, int64_t M, int64_t N,
                                                       int64_t K, int tiles_m, int tiles_n, Grouping grp) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hh = lane >> 5;

    // XCD-aware tile order (as in the Q4_K GEMM): each XCD gets a contiguous
    // range of v, and v walks groups of GM row tiles with the row tile fastest.
    constexpr int GM = 4;
    const int nwg = tiles_m * tiles_n;
    const int bid = blockIdx.x;
    int tile_m, tile_n, m_last_g = 0, r0 = 0;
    if constexpr (GROUPED) {  // mul_mat_id: tile from the expert grouping
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

    // ---- activation staging (rows past M clamped to the last valid one)
    const int m_last = GROUPED ? m_last_g : (int)(M - 1 - m_base < BM - 1 ? M - 1 - m_base : BM - 1);
    const uint32_t a_rowstride = (uint32_t)(nb * kQ8_KBytes);
    const int64_t a_first = m_base * nb * kQ8_KBytes;
    const int64_t a_bytes = M * nb * kQ8_KBytes - a_first;
    // byte offset (from Y + a_first) of tile row rr <= m_last
    auto arow = [&](int rr) -> uint32_t {
        if constexpr (GROUPED) return (uint32_t)grouped_row(grp, r0, rr) * a_rowstride;
        else return (uint32_t)rr * a_rowstride;
    };
    uint32_t a_goff[A_PER_WAVE];
#pragma unroll
    for (int t = 0; t < A_PER_WAVE; ++t) {
        const int row = (wave * A_PER_WAVE + t) * 4 + (lane >> 4);
        const int gp = (lane & 15) ^ (row & 15);  // global piece stored at position lane & 15
        const int rr = row < m_last ? row : m_last;
        a_goff[t] = arow(rr) + 4 + 16 * gp;
    }
    const uint32_t d_off = arow((tid & (BM - 1)) < m_last ? (tid & (BM - 1)) : m_last);

    // ---- this lane's weight column (columns past N clamped; never stored)
    const int64_t NB = N * nb;
    const int64_t dsec = (2 * NB + 255) / 256 * 256;
    const int64_t n_lane = n_base + wave * 32 + l32 < N ? n_base + wave * 32 + l32 : N - 1;
    const int64_t i0 = n_lane * nb;  // block index of the column's first super-block
    const uint32_t v_d = (uint32_t)(2 * i0);
    const uint32_t v_sc = (uint32_t)(dsec + 16 * i0);
    const uint32_t v_ql = (uint32_t)(dsec + 16 * NB + 128 * i0 + 16 * hh);
    const uint32_t v_qh = (uint32_t)(dsec + 144 * NB + 64 * i0 + 16 * hh);

    auto issue = [&](int64_t b, uint8_t *buf) {
        const rsrc_t ra = make_rsrc(Y + a_first, a_bytes);
        const uint32_t sa = (uint32_t)b * kQ8_KBytes;
#pragma unroll
        for (int t = 0; t < A_PER_WAVE; ++t)
            dma16(ra, a_goff[t], sa, buf + A_OFF + (wave * A_PER_WAVE + t) * 1024);
    };
    auto prefetch = [&](int64_t b, uint32_t &draw) {
        const rsrc_t ra = make_rsrc(Y + a_first, a_bytes);
        if (tid < BM) draw = __builtin_amdgcn_raw_buffer_load_b32(ra, d_off, (uint32_t)b * kQ8_KBytes, 0);
    };
    auto wload = [&](int64_t b, Q6KStage &x) {
        const rsrc_t rw = make_rsrc(W, w_bytes);
        const uint32_t bb = (uint32_t)b;
#pragma unroll
        for (int g = 0; g < 4; ++g) x.ql[g] = bld16(rw, v_ql + 32 * g, 128 * bb);
        x.qa = bld16(rw, v_qh, 64 * bb);
        x.qb = bld16(rw, v_qh + 32, 64 * bb);
        x.sc = bld16(rw, v_sc, 16 * bb);
        x.d = __builtin_amdgcn_raw_buffer_load_b16(rw, v_d, 2 * bb, 0);
    };

    float acc[MT][16];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;

    uint32_t draw = 0;
    Q6KStage wx;
    issue(0, lds);
    prefetch(0, draw);
    wload(0, wx);

    for (int64_t b = 0; b < nb; ++b) {
        uint8_t *buf = lds + (b & 1) * BUF_BYTES;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's loads of step b
        if (tid < BM) *reinterpret_cast<uint32_t *>(buf + DA_OFF + 4 * tid) = draw;

        __syncthreads();  // every thread's step-b data is in LDS; step b-1 is fully consumed
        if (b + 1 < nb) {
            issue(b + 1, lds + ((b + 1) & 1) * BUF_BYTES);
            prefetch(b + 1, draw);
        }
        const float *da = reinterpret_cast<const float *>(buf + DA_OFF);

        // ---------------- decode: chunk c holds group G = 2c + hh of this lane.
        // The planes are built inside row tile 0, chunk c just before its first
        // MFMAs, so the decode of c + 1 issues while the MFMAs of c run.
        const float dcol = f16_bits_to_f32(wx.d);
        v4i bhi[8], blo[8];
        auto build = [&](int c) {
            const uint32_t sw[4] = {wx.sc.x, wx.sc.y, wx.sc.z, wx.sc.w};
            const int g = c >> 1, hi_nib = c & 1;
            const int s = (int)(int8_t)(sw[g] >> (16 * hi_nib + 8 * hh));  // scale byte 2c + hh
            const s16x2 s2 = {(short)s, (short)s};
            const s16x2 c2 = {(short)(128 - 32 * s), (short)(128 - 32 * s)};
            const uint32_t ql[4] = {wx.ql[g].x, wx.ql[g].y, wx.ql[g].z, wx.ql[g].w};
            const uint4 qhp = hi_nib ? wx.qb : wx.qa;
            const uint32_t qh[4] = {qhp.x, qhp.y, qhp.z, qhp.w};
            uint32_t hw[4], lw[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t u = ((ql[w] >> (4 * hi_nib)) & 0x0f0f0f0fu) |
                                   (((qh[w] >> (2 * g)) & 0x03030303u) << 4);
                t_digits(u, s2, c2, hw[w], lw[w]);
            }
            bhi[c] = v4i{(int)hw[0], (int)hw[1], (int)hw[2], (int)hw[3]};
            blo[c] = v4i{(int)lw[0], (int)lw[1], (int)lw[2], (int)lw[3]};
        };

        // ---------------- the four row tiles of this column tile.  The tail of
        // row tile i - 1 (conversion and accumulation) is placed after the MFMAs
        // of row tile i, so its vector work can issue while they run.
        v16i s_prev;
        auto tail = [&](int i, const v16i &S) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 d4 = *reinterpret_cast<const float4 *>(da + i * 32 + 8 * q + 4 * hh);
                const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * q + e;
                    acc[i][r] = fmaf(dv[e], dcol * (float)S[r], acc[i][r]);
                }
            }
        };
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            const int row = i * 32 + l32;
            const v16i zero = {};
            v16i ah, al;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                v4i a_op[4];
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) {
                    const int c = 4 * half + cc;
                    const uint4 a = *reinterpret_cast<const uint4 *>(buf + A_OFF + row * 256 +
                                                                     16 * ((2 * c + hh) ^ (row & 15)));
                    a_op[cc] = v4i{(int)a.x, (int)a.y, (int)a.z, (int)a.w};
                }
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) {
                    const int c = 4 * half + cc;
                    if (i == 0) build(c);
                    ah = __builtin_amdgcn_mfma_i32_32x32x32_i8(a_op[cc], bhi[c], c ? ah : zero, 0, 0, 0);
                    al = __builtin_amdgcn_mfma_i32_32x32x32_i8(a_op[cc], blo[c], c ? al : zero, 0, 0, 0);
                }
            }
            if (i == 0 && b + 1 < nb) wload(b + 1, wx);  // the planes no longer need wx
            if (i > 0) tail(i - 1, s_prev);
#pragma unroll
            for (int r = 0; r < 16; ++r) s_prev[r] = (ah[r] << 8) + al[r];  // |S| <= 256 * 4096 * 127
        }
        tail(MT - 1, s_prev);
    }

    // ---- store: register r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32
    const int64_t n = n_base + wave * 32 + l32;
    if (n < N) {
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if constexpr (GROUPED) {
                    const int lm = i * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
                    if (lm <= m_last) out[(int64_t)grp.sorted[r0 + lm] * N + n] = acc[i][r];
                } else {
                    const int64_t m = m_base + i * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
                    if (m < M) out[m * N + n] = acc[i][r];
                }
            }
    }
}

}  // namespace

namespace {
template <bool GROUPED>
hipError_t launch_t(const uint8_t *w, int64_t w_bytes, const uint8_t *y, float *out, int64_t M, int64_t N,
                    int64_t K, int tiles_m, const Grouping &g, hipStream_t s) {
    static std::atomic<uint64_t> lds_set{0};  // the LDS budget above 64 KiB, per device
    const hipError_t e = ensure_lds_bytes((const void *)k_gemm_q6_K<GROUPED>, LDS_BYTES, lds_set);
    if (e != hipSuccess) return e;
    const int tiles_n = (int)((N + BN - 1) / BN);
    hipLaunchKernelGGL((k_gemm_q6_K<GROUPED>), dim3((unsigned)(tiles_m * tiles_n)), dim3(NTHR), LDS_BYTES, s,
                       w, w_bytes, y, out, M, N, K, tiles_m, tiles_n, g);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm_q6_K(const uint8_t *w, int64_t w_bytes, const uint8_t *y, float *out,
                            int64_t M, int64_t N, int64_t K, hipStream_t s) {
    return launch_t<false>(w, w_bytes, y, out, M, N, K, (int)((M + BM - 1) / BM), Grouping{}, s);
}

// mul_mat_id: w_bytes and w_stride are the bytes of one expert matrix
hipError_t launch_gemm_id_q6_K(const uint8_t *w, int64_t w_bytes, const uint8_t *y, int64_t y_rows,
                               int y_per_slot, int64_t U, const int32_t *group_ws, int64_t E, int64_t P,
                               float *out, int64_t N, int64_t K, hipStream_t s) {
    const MoeGroupLayout L = moe_group_layout(P, E, BM);
    const Grouping g{group_ws + L.start, group_ws + L.tile_e, group_ws + L.tile_r0, group_ws + L.ntiles,
                     group_ws + L.sorted, U, w_bytes, y_per_slot};
    return launch_t<true>(w, w_bytes, y, out, y_rows, N, K, (int)L.max_tiles, g, s);
}

}  // namespace qmm
