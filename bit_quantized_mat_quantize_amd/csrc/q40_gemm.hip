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
// every 32 elements, so every MFMA result needs its own fp32 epilogue.  The
// scale products S_b[m][n] = d_a[m,b] * d_w[n,b] of a 32 x 32 tile come from
// one fp16 MFMA (v_mfma_f32_32x32x16_f16): the A operand holds the eight
// blocks' d_a of a row in K slots 0..7, the B operand holds d_w of block b in
// slot b and zeros elsewhere, so S_b is the single product, exact in fp32.
// The epilogue is then two vector instructions per output value per block
// (convert P_b, fused multiply-add with S_b) against two MFMAs per 32 x 32 x 32
// -- still the bound of this kernel, ahead of the matrix cores.  (The ggml-cpu
// page finds Q4_0 faster than the K-quants for CPU prefill because its unpack
// is cheaper; on the matrix cores the per-block scale traffic dominates.)
//
// Tiling as in the K-quant GEMMs: 512 threads = 8 wavefronts, tile 128 (M) x
// 256 (N), wavefront w owns the 32-column tile 32w..32w+31 for all four
// 32-row tiles; K advances 256 elements (8 blocks) per step.  Activations:
// a step of a Q8_0 row is 8 blocks of 34 bytes = 272 bytes, 16-byte aligned,
// but the codes of every other block sit at a 2-byte offset, so the tile is
// staged through registers: each thread loads one block pair (68 bytes, four
// dwordx4 + one dword, one step ahead), realigns the first block's codes with
// v_alignbyte, and writes codes and d_a to LDS (double-buffered; d_a
// row-major so that a row's eight blocks are one 16-byte read).  Code rows
// are padded to 272 bytes, an odd number of 16-byte slots, so the lanes
// reading one piece of consecutive rows hit distinct banks.  Within a row,
// piece k (16 bytes) of block pair p sits at slot 8*(k/2) + 2p + k%2: a
// 16-byte store serves 8 lanes together (two rows, four pairs, one piece k),
// and their slots are then the four even and the four odd ones modulo 8 --
// with pairs at 64-byte strides, pairs 0 and 2 of a row would share banks.
// Weights: each wavefront moves its 32 columns' step
// (eight 16-byte payloads and 16 bytes of fp16 d per column) with direct
// global->LDS loads into its own region of the next buffer, one step ahead;
// piece c of column col sits at slot c ^ (col & 7) ^ ((col >> 3) & 3) of the
// column's 128 bytes, so 8, 16 or 32 consecutive columns reading one piece
// fall in distinct 16-byte slots of 128, 256 or 512 bytes.  No
// other wavefront reads that region, so the loads need only this wavefront's
// wait.  Per step the blocks are the outer loop and the four row tiles the
// inner one, which keeps one decoded weight operand live.
#include "mfma_common.h"
#include "qmm_device.h"
#include "qmm_launch.h"

namespace qmm {
namespace {

constexpr int BM = 128, BN = 256, MT = BM / 32, NWAVE = 8, NTHR = 64 * NWAVE;
constexpr int A_ROW = 272;  // 256 code bytes + 16 bytes of padding per row
constexpr int A_OFF = 0, A_BYTES = BM * A_ROW;
constexpr int DA_OFF = A_OFF + A_BYTES, DA_BYTES = 8 * BM * 2;  // fp16 [128 rows][8 blocks]
constexpr int WP_OFF = DA_OFF + DA_BYTES, WP_WAVE = 32 * 128;    // payloads [wave][32 columns][8 slots]
constexpr int WD_OFF = WP_OFF + NWAVE * WP_WAVE, WD_WAVE = 32 * 16;  // d_w [wave][32 columns][8 fp16]
constexpr int BUF_BYTES = WD_OFF + NWAVE * WD_WAVE;
constexpr int ZERO_OFF = 2 * BUF_BYTES;    // 16 zero bytes: the scale MFMA's K slots 8..15
constexpr int LDS_BYTES = ZERO_OFF + 16;
constexpr int kStepBytes = 8 * kQ8_0Bytes;  // 272: one K step of a Q8_0 row
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of a gfx950 CU");
static_assert(BN == 32 * NWAVE && 4 * BM == NTHR, "one column tile per wavefront; one block pair per thread");

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

    // ---- weight DMA of this wavefront's 32 columns (columns past N clamped;
    // never stored): instruction t moves columns 8t..8t+7, lane l the piece
    // (l & 7) ^ wsw(col) of column col = 8t + l/8 to slot l & 7; lanes 0..31 of
    // one more move the 16 bytes of d of column l
    const int64_t NB = N * nb32;
    const int64_t dsec = (2 * NB + 255) / 256 * 256;
    auto wcol = [&](int col) -> int64_t {
        const int64_t n = n_base + wave * 32 + col;
        return n < N ? n : N - 1;
    };
    auto wsw_of = [](int col) { return (col & 7) ^ ((col >> 3) & 3); };
    uint32_t wp_goff[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int col = 8 * t + (lane >> 3);
        wp_goff[t] = (uint32_t)(dsec + 16 * wcol(col) * nb32 + 16 * ((lane & 7) ^ wsw_of(col)));
    }
    const uint32_t wd_goff = (uint32_t)(2 * wcol(l32) * nb32);
    auto wdma = [&](int64_t b, uint8_t *buf) {
        const rsrc_t rw = make_rsrc(W, w_bytes);
        const uint32_t bb = (uint32_t)b;
#pragma unroll
        for (int t = 0; t < 4; ++t) dma16(rw, wp_goff[t], 128 * bb, buf + WP_OFF + wave * WP_WAVE + 1024 * t);
        if (lane < 32) dma16(rw, wd_goff, 16 * bb, buf + WD_OFF + wave * WD_WAVE);
    };

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
        uint4 *arow_p = reinterpret_cast<uint4 *>(buf + A_OFF + s_row * A_ROW + 32 * s_pair);
        arow_p[0] = make_uint4(c0[0], c0[1], c0[2], c0[3]);
        arow_p[1] = make_uint4(c0[4], c0[5], c0[6], c0[7]);
        arow_p[8] = make_uint4(w[9], w[10], w[11], w[12]);
        arow_p[9] = make_uint4(w[13], w[14], w[15], w[16]);
        // d_a of blocks 2 s_pair and 2 s_pair + 1 of row s_row: adjacent halves
        *reinterpret_cast<uint32_t *>(buf + DA_OFF + s_row * 16 + 4 * s_pair) = (w[0] & 0xffffu) | (w[8] & 0xffff0000u);
    };

    float acc[MT][16];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;

    ARaw ar;
    aload(0, ar);
    wdma(0, lds);
    if (tid == 0) *reinterpret_cast<uint4 *>(lds + ZERO_OFF) = make_uint4(0, 0, 0, 0);  // read after a barrier
    // scale MFMA A operand: lanes 0..31 read their row's eight d_a (K slots
    // 0..7), lanes 32..63 the zero bytes (K slots 8..15)
    const int da_lane = hh ? ZERO_OFF : DA_OFF + l32 * 16;
    const uint32_t bmask = hh ? 0u : 0xffffffffu;  // B operand: K slots 8..15 are zero
    const int wp_lane = WP_OFF + wave * WP_WAVE + l32 * 128, wsw = wsw_of(l32);
    const int wd_lane = WD_OFF + wave * WD_WAVE + l32 * 16;

    for (int64_t b = 0; b < nsteps; ++b) {
        uint8_t *buf = lds + (b & 1) * BUF_BYTES;
        // this thread's activation loads and this wavefront's weight DMA of step b
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        acommit(ar, buf);
        __syncthreads();  // every thread's step-b activations are in LDS; step b-1 is fully consumed
        if (b + 1 < nsteps) {
            aload(b + 1, ar);
            wdma(b + 1, lds + ((b + 1) & 1) * BUF_BYTES);
        }
        const uint8_t *da_base = (hh ? lds : buf) + da_lane;  // the zero bytes are outside the buffers
        v8h a_da[MT];
#pragma unroll
        for (int i = 0; i < MT; ++i)
            a_da[i] = __builtin_bit_cast(v8h, *reinterpret_cast<const uint4 *>(da_base + (hh ? 0 : i * 32 * 16)));
        const uint4 dv = *reinterpret_cast<const uint4 *>(buf + wd_lane);
        const uint32_t dd[4] = {dv.x & bmask, dv.y & bmask, dv.z & bmask, dv.w & bmask};

        // The 32 (block, row tile) pairs run as a pipeline: the two MFMAs of
        // pair t + 1 are issued before the epilogue of pair t (convert P,
        // fused multiply-add with S), so the matrix cores work while the
        // vector ALU does the epilogue; scheduling barriers and the empty asm
        // statements keep that order.
        v4i bq[2];
        v8h b_dw[2];
        v16i P[2];
        v16f S[2];
        uint4 av[2], pv[2];
        auto read_a = [&](int t) {
            const int c = t >> 2, row = (t & 3) * 32 + l32;
            av[t & 1] = *reinterpret_cast<const uint4 *>(buf + A_OFF + row * A_ROW + 128 * (c & 1) + 32 * (c >> 1) +
                                                         16 * hh);
        };
        auto read_w = [&](int c) {
            pv[c & 1] = *reinterpret_cast<const uint4 *>(buf + wp_lane + 16 * (c ^ wsw));
        };
        // LDS reads run one pair (codes) or three pairs (payloads) ahead of
        // the MFMAs that take them
        auto issue = [&](int t) {
            const int c = t >> 2, i = t & 3;
            if (t + 1 < 8 * MT) read_a(t + 1);
            if (i == 1 && c + 1 < 8) read_w(c + 1);
            if (i == 0) {
                // decode: lane half hh takes the low (hh = 0) or high nibbles of
                // the payload (elements 16hh..16hh+15 of block c) into the high
                // half of each byte, XOR 0x80: the signed byte 16 * (q - 8).
                // The factor 16 is removed, exactly, at the store.  d_w of
                // block c goes to K slot c of the scale MFMA's B operand
                // (dword c/2, half c%2), zeros elsewhere.
                const uint32_t pw[4] = {pv[c & 1].x, pv[c & 1].y, pv[c & 1].z, pv[c & 1].w};
                uint32_t o[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) o[k] = ((pw[k] << (4 - 4 * hh)) & 0xf0f0f0f0u) ^ 0x80808080u;
                bq[c & 1] = v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
                uint32_t bs[4] = {0u, 0u, 0u, 0u};
                bs[c >> 1] = dd[c >> 1] & ((c & 1) ? 0xffff0000u : 0x0000ffffu);
                b_dw[c & 1] = __builtin_bit_cast(v8h, make_uint4(bs[0], bs[1], bs[2], bs[3]));
            }
            const uint4 a = av[t & 1];
            P[t & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(v4i{(int)a.x, (int)a.y, (int)a.z, (int)a.w},
                                                             bq[c & 1], v16i{}, 0, 0, 0);
            S[t & 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_da[i], b_dw[c & 1], v16f{}, 0, 0, 0);
        };
        read_w(0);
        read_a(0);
        issue(0);
#pragma unroll
        for (int t = 0; t < 8 * MT; ++t) {
            if (t + 1 < 8 * MT) issue(t + 1);
            __builtin_amdgcn_sched_barrier(0);
            const int i = t & 3;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][r] = fmaf((float)P[t & 1][r], S[t & 1][r], acc[i][r]);
#pragma unroll
            for (int r = 0; r < 16; ++r) asm volatile("" : "+v"(acc[i][r]));
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // ---- store: register r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column
    // l%32; the weight operand carried 16 * (q - 8), and scaling by 1/16 is exact
    const int64_t n = n_base + wave * 32 + l32;
    if (n < N) {
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if constexpr (GROUPED) {
                    const int lm = i * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
                    if (lm <= m_last) out[(int64_t)grp.sorted[r0 + lm] * N + n] = acc[i][r] * 0.0625f;
                } else {
                    const int64_t m = m_base + i * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
                    if (m < M) out[m * N + n] = acc[i][r] * 0.0625f;
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
    const hipError_t e = ensure_lds_bytes((const void *)k_gemm_q4_0<GROUPED>, LDS_BYTES, lds_set);
    if (e != hipSuccess) return e;
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
