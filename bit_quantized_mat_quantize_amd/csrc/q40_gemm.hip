// q40_gemm.hip -- Q4_0 weights x Q8_0 activations on int8 MFMA (prefill-sized
// M), gfx950, for the load-time (repacked) weight layout and K a multiple of
// 256.
//
// Arithmetic (ggml-cpu mul_mat page, "最基础的两块:Q4_0 与 Q8_0" and
// "正确性:缩放系数可以提到求和号外面"), per 32-element block b and output (m, n):
//   P_b = sum_{i in b} (q_i - 8) * y_i  (int32),   acc += d_a[m,b] * d_w[n,b] * P_b.
//
// A Q4_0 block is one K = 32 chunk of v_mfma_i32_32x32x32_i8, so the codes go
// straight into the weight operand as the int8 values q - 8 and one MFMA per
// chunk gives P_b for a 32 x 32 tile.  Unlike the K-quants, both scales change
// every 32 elements, so every MFMA result needs its own fp32 epilogue (convert,
// times d_w, fused multiply-add with d_a): three vector instructions per
// output value per block against one MFMA per 32 x 32 x 32 -- this kernel is
// bound by that epilogue, not by the matrix cores.  (The ggml-cpu page finds
// Q4_0 faster than the K-quants for CPU prefill because its unpack is
// cheaper; on the matrix cores the per-block scale traffic dominates instead.)
//
// Tiling as in the K-quant GEMMs: 512 threads = 8 wavefronts, tile 128 (M) x
// 256 (N), wavefront w owns the 32-column tile 32w..32w+31 for all four
// 32-row tiles; K advances 256 elements (8 blocks) per step.  Activations:
// a step of a Q8_0 row is 8 blocks of 34 bytes = 272 bytes, 16-byte aligned,
// but the codes of every other block sit at a 2-byte offset, so the tile is
// staged through registers: each thread loads one block pair (68 bytes, four
// dwordx4 + one dword, one step ahead), realigns the first block's codes with
// v_alignbyte, and writes codes and d_a to LDS (double-buffered; codes
// XOR-swizzled by 16-byte piece, d_a block-major so that four consecutive
// rows are one 8-byte read).  Weights: each lane loads its column's eight
// 16-byte payloads and eight fp16 d straight into registers, one step ahead.
#include "mfma_common.h"
#include "qmm_device.h"
#include "qmm_launch.h"

namespace qmm {
namespace {

constexpr int BM = 128, BN = 256, MT = BM / 32, NWAVE = 8, NTHR = 64 * NWAVE;
constexpr int A_OFF = 0, A_BYTES = BM * 256;
constexpr int DA_OFF = A_OFF + A_BYTES, DA_BYTES = 8 * BM * 2;  // fp16 [8 blocks][128 rows]
constexpr int BUF_BYTES = DA_OFF + DA_BYTES;
constexpr int LDS_BYTES = 2 * BUF_BYTES;
constexpr int kStepBytes = 8 * kQ8_0Bytes;  // 272: one K step of a Q8_0 row
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of a gfx950 CU");
static_assert(BN == 32 * NWAVE && 4 * BM == NTHR, "one column tile per wavefront; one block pair per thread");

struct Q40Stage {
    uint4 pay[8];  // payloads of blocks 8b..8b+7 of this lane's column
    uint4 d;       // their fp16 d
};

template <bool GROUPED>
__global__ __launch_bounds__(NTHR, 1) void k_gemm_q4_0(const uint8_t *__restrict__ W, int64_t w_bytes,
                                                       const uint8_t *__restrict__ Y,
                                                       float *__restrict__ out, int64_t M, int64_t N,
                                                       int64_t K, int tiles_m, int tiles_n, Grouping grp) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hh = lane >> 5;

    // XCD-aware tile order (as in the Q4_K GEMM)
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
    const int64_t nsteps = K / 256, nb32 = K / 32;

    // ---- activation staging: thread t takes row t/4 (clamped to the last
    // valid row) and block pair t%4 of each step
    const int m_last = GROUPED ? m_last_g : (int)(M - 1 - m_base < BM - 1 ? M - 1 - m_base : BM - 1);
    const int s_row = tid >> 2, s_pair = tid & 3;
    const uint32_t a_rowstride = (uint32_t)(nb32 * kQ8_0Bytes);
    const int64_t a_first = m_base * nb32 * kQ8_0Bytes;
    const int64_t a_bytes = M * nb32 * kQ8_0Bytes - a_first;
    // byte offset (from Y + a_first) of tile row rr <= m_last
    auto arow = [&](int rr) -> uint32_t {
        if constexpr (GROUPED) return (uint32_t)grouped_row(grp, r0, rr) * a_rowstride;
        else return (uint32_t)rr * a_rowstride;
    };
    const uint32_t a_off = arow(s_row < m_last ? s_row : m_last) + 68 * s_pair;

    // ---- this lane's weight column (columns past N clamped; never stored)
    const int64_t NB = N * nb32;
    const int64_t dsec = (2 * NB + 255) / 256 * 256;
    const int64_t n_lane = n_base + wave * 32 + l32 < N ? n_base + wave * 32 + l32 : N - 1;
    const uint32_t v_pay = (uint32_t)(dsec + 16 * n_lane * nb32);
    const uint32_t v_d = (uint32_t)(2 * n_lane * nb32);

    struct ARaw {
        uint4 q[4];
        uint32_t t;
    };
    auto aload = [&](int64_t b, ARaw &r) {
        const rsrc_t ra = make_rsrc(Y + a_first, a_bytes);
        const uint32_t sa = (uint32_t)b * kStepBytes;
#pragma unroll
        for (int k = 0; k < 4; ++k) r.q[k] = bld16(ra, a_off + 16 * k, sa);
        r.t = __builtin_amdgcn_raw_buffer_load_b32(ra, a_off + 64, sa, 0);
    };
    // bytes of the pair: [d0 | 32 codes of block 2p | d1 | 32 codes of block 2p+1]
    auto acommit = [&](const ARaw &r, uint8_t *buf) {
        const uint32_t w[17] = {r.q[0].x, r.q[0].y, r.q[0].z, r.q[0].w, r.q[1].x, r.q[1].y,
                                r.q[1].z, r.q[1].w, r.q[2].x, r.q[2].y, r.q[2].z, r.q[2].w,
                                r.q[3].x, r.q[3].y, r.q[3].z, r.q[3].w, r.t};
        uint32_t c0[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) c0[j] = __builtin_amdgcn_alignbyte(w[j + 1], w[j], 2);
        uint8_t *arow_p = buf + A_OFF + s_row * 256;
        const int blk0 = 2 * s_pair, blk1 = 2 * s_pair + 1;
        *reinterpret_cast<uint4 *>(arow_p + 16 * ((2 * blk0) ^ (s_row & 15))) = make_uint4(c0[0], c0[1], c0[2], c0[3]);
        *reinterpret_cast<uint4 *>(arow_p + 16 * ((2 * blk0 + 1) ^ (s_row & 15))) = make_uint4(c0[4], c0[5], c0[6], c0[7]);
        *reinterpret_cast<uint4 *>(arow_p + 16 * ((2 * blk1) ^ (s_row & 15))) = make_uint4(w[9], w[10], w[11], w[12]);
        *reinterpret_cast<uint4 *>(arow_p + 16 * ((2 * blk1 + 1) ^ (s_row & 15))) = make_uint4(w[13], w[14], w[15], w[16]);
        uint16_t *da = reinterpret_cast<uint16_t *>(buf + DA_OFF);
        da[blk0 * BM + s_row] = (uint16_t)(w[0] & 0xffff);
        da[blk1 * BM + s_row] = (uint16_t)(w[8] >> 16);
    };
    auto wload = [&](int64_t b, Q40Stage &x) {
        const rsrc_t rw = make_rsrc(W, w_bytes);
        const uint32_t bb = (uint32_t)b;
#pragma unroll
        for (int c = 0; c < 8; ++c) x.pay[c] = bld16(rw, v_pay + 16 * c, 128 * bb);
        x.d = bld16(rw, v_d, 16 * bb);
    };

    float acc[MT][16];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;

    ARaw ar;
    Q40Stage wx;
    aload(0, ar);
    wload(0, wx);

    for (int64_t b = 0; b < nsteps; ++b) {
        uint8_t *buf = lds + (b & 1) * BUF_BYTES;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's loads of step b
        acommit(ar, buf);

        // ---------------- decode: lane half hh takes the low (hh = 0) or high
        // nibbles of each payload (elements 16hh..16hh+15 of the block) as the
        // int8 values q - 8: ((q | 0x80) - 8) ^ 0x80 per byte, no borrow
        // crossing bytes
        v4i bq[8];
        float dw[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const uint32_t pw[4] = {wx.pay[c].x, wx.pay[c].y, wx.pay[c].z, wx.pay[c].w};
            uint32_t o[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                o[k] = ((((pw[k] >> (4 * hh)) & 0x0f0f0f0fu) | 0x80808080u) - 0x08080808u) ^ 0x80808080u;
            bq[c] = v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
        }
        {
            const uint32_t dd[4] = {wx.d.x, wx.d.y, wx.d.z, wx.d.w};
#pragma unroll
            for (int c = 0; c < 8; ++c) dw[c] = f16_bits_to_f32((dd[c >> 1] >> (16 * (c & 1))) & 0xffff);
        }

        __syncthreads();  // every thread's step-b data is in LDS; step b-1 is fully consumed
        if (b + 1 < nsteps) {
            aload(b + 1, ar);
            wload(b + 1, wx);
        }
        const _Float16 *da = reinterpret_cast<const _Float16 *>(buf + DA_OFF);

        // ---------------- the four row tiles of this column tile
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            const int row = i * 32 + l32;
            const v16i zero = {};
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const uint4 a = *reinterpret_cast<const uint4 *>(buf + A_OFF + row * 256 +
                                                                 16 * ((2 * c + hh) ^ (row & 15)));
                const v16i P = __builtin_amdgcn_mfma_i32_32x32x32_i8(v4i{(int)a.x, (int)a.y, (int)a.z, (int)a.w},
                                                                     bq[c], zero, 0, 0, 0);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    // d_a of rows 32i + 8q + 4hh .. +3 (one 8-byte read)
                    const uint2 dq = *reinterpret_cast<const uint2 *>(da + c * BM + i * 32 + 8 * q + 4 * hh);
                    const _Float16 *dh = reinterpret_cast<const _Float16 *>(&dq);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * q + e;
                        acc[i][r] = fmaf((float)dh[e], dw[c] * (float)P[r], acc[i][r]);
                    }
                }
            }
        }
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
    static bool attr_set = false;  // the LDS budget above 64 KiB must be opted into once
    if (!attr_set) {
        const hipError_t e = hipFuncSetAttribute((const void *)k_gemm_q4_0<GROUPED>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int tiles_n = (int)((N + BN - 1) / BN);
    hipLaunchKernelGGL((k_gemm_q4_0<GROUPED>), dim3((unsigned)(tiles_m * tiles_n)), dim3(NTHR), LDS_BYTES, s,
                       w, w_bytes, y, out, M, N, K, tiles_m, tiles_n, g);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm_q4_0(const uint8_t *w, int64_t w_bytes, const uint8_t *y, float *out,
                            int64_t M, int64_t N, int64_t K, hipStream_t s) {
    return launch_t<false>(w, w_bytes, y, out, M, N, K, (int)((M + BM - 1) / BM), Grouping{}, s);
}

// mul_mat_id: w_bytes and w_stride are the bytes of one expert matrix
hipError_t launch_gemm_id_q4_0(const uint8_t *w, int64_t w_bytes, const uint8_t *y, int64_t y_rows,
                               int y_per_slot, int64_t U, const int32_t *group_ws, int64_t E, int64_t P,
                               float *out, int64_t N, int64_t K, hipStream_t s) {
    const MoeGroupLayout L = moe_group_layout(P, E, BM);
    const Grouping g{group_ws + L.start, group_ws + L.tile_e, group_ws + L.tile_r0, group_ws + L.ntiles,
                     group_ws + L.sorted, U, w_bytes, y_per_slot};
    return launch_t<true>(w, w_bytes, y, out, y_rows, N, K, (int)L.max_tiles, g, s);
}

}  // namespace qmm
