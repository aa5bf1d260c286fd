// q40_skinny.hip -- Q4_0 weights x Q8_0 activations for small batches on int8
// MFMA, gfx950, repacked layout, K a multiple of 256.
//
// Arithmetic (ggml-cpu mul_mat page, "最基础的两块:Q4_0 与 Q8_0" and
// "正确性:缩放系数可以提到求和号外面"), per 32-element block b and output (m, n):
//   P_b = sum_{i in b} (q_i - 8) * y_i  (int32),   acc += d_a[m,b] * d_w[n,b] * P_b.
//
// A few activation rows still read every weight once, so a small batch is
// bound by the weight stream (BitBLAS page, "调度与自动调优"), but the Q4_0 GEMV
// repeats its per-row work for every row, and a single-row-tile GEMM runs too
// few workgroups.  Here, as in the Q4_K small-batch kernel, a workgroup owns
// 32 output columns and 32 activation rows (more rows take more grid rows,
// blockIdx.y), and its 8 wavefronts split K: wavefront w takes the 256-element
// steps w, w + 8, ... and the eight partial tiles are summed through LDS.
//
// Per step a wavefront loads its column's eight 16-byte payloads and eight
// fp16 d straight into registers (no other wavefront reads them), one step
// ahead.  Q8_0 blocks are 34 bytes, so their codes are only 2-byte aligned:
// each lane loads two 68-byte block pairs of the activation rows (four
// dwordx4 + one dword each, dword-aligned), also one step ahead.  After the
// step's MFMAs it realigns the first block's codes with v_alignbyte and writes
// codes and d_a into the other of its wavefront's two LDS stages (code rows
// padded to 272 bytes, so the 32 rows of one block read at a 68-dword stride
// fall in distinct bank groups and each block's read address is the lane's
// base plus an immediate; d_a block-major).  No other wavefront reads those
// stages, so a wavefront barrier suffices until the final reduction.  Each
// block is one K = 32 chunk of v_mfma_i32_32x32x32_i8 with q - 8 as the signed
// weight operand, followed by the per-block fp32 epilogue (convert, times d_w,
// fused multiply-add with d_a), which runs after the next block's MFMA is
// issued.
//
// MFMA operand convention (v_mfma_*_32x32xK): lane l supplies row (A) or
// column (B) l % 32 and the K-slice selected by l / 32; the result register r
// of lane l holds row 8*(r/4) + 4*(l/32) + r%4, column l % 32.
#include "mfma_common.h"
#include "qmm_device.h"
#include "qmm_launch.h"

namespace qmm {
namespace {

constexpr int QS_WAVES = 8, QS_THREADS = 64 * QS_WAVES;
constexpr int QS_ROWS = 32;                                 // activation rows per workgroup
constexpr int64_t QS_MAX_M = 65535ll * QS_ROWS;             // row chunks go to grid.y
// Per-wavefront LDS stage: codes [32 rows][272] (256 code bytes and a
// 16-byte pad per row), then d_a as fp16 [8 blocks][32 rows].
constexpr int QS_ROWB = 272;
constexpr int QS_A = 0, QS_DA = QS_ROWS * QS_ROWB, QS_STAGE = QS_DA + 8 * QS_ROWS * 2;
constexpr int QS_RED = QS_WAVES * 16 * 64 * 4;              // partial tiles at the end
constexpr int QS_LDS = 2 * QS_WAVES * QS_STAGE > QS_RED ? 2 * QS_WAVES * QS_STAGE : QS_RED;  // two stages
static_assert(QS_LDS <= 160 * 1024, "LDS budget of a gfx950 CU");
constexpr int kStep = 8 * kQ8_0Bytes;  // 272: one 256-element step of a Q8_0 row

struct QSWeights {
    uint4 pay[8];  // payloads of the step's eight blocks, this lane's column
    uint4 d;       // their fp16 d
};
struct QSActs {
    uint4 q[2][4];  // two 68-byte block pairs: [d0 | 32 codes | d1 | 32 codes]
    uint32_t t[2];
};

__global__ __launch_bounds__(QS_THREADS, 1) void k_skinny_q4_0(const uint8_t *__restrict__ W, int64_t w_bytes,
                                                              const uint8_t *__restrict__ Y,
                                                              float *__restrict__ out, int64_t M, int64_t N,
                                                              int64_t K) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    // this workgroup's chunk of at most 32 activation rows (grid.y)
    const int64_t nb32 = K / QK4_0, nsteps = K / 256;
    const int64_t m0 = (int64_t)blockIdx.y * QS_ROWS;
    Y += m0 * nb32 * kQ8_0Bytes;
    out += m0 * N;
    M = M - m0 < QS_ROWS ? M - m0 : QS_ROWS;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: feeds scalar offsets
    const int l32 = lane & 31, hh = lane >> 5;
    const int64_t n_base = (int64_t)blockIdx.x * 32;
    const int64_t col = n_base + l32 < N ? n_base + l32 : N - 1;  // clamped: loads stay in bounds
    uint8_t *const my = lds + wave * 2 * QS_STAGE;                 // this wavefront's two stages

    // weights (repacked: d section of 2 bytes per block padded to 256 bytes,
    // then the 16-byte payloads), offsets relative to the matrix start
    const int64_t dsec = (2 * N * nb32 + 255) / 256 * 256;
    const uint32_t v_pay = (uint32_t)(dsec + 16 * col * nb32);
    const uint32_t v_d = (uint32_t)(2 * col * nb32);
    // activations: pair k of this lane is row (lane + 64k) / 4 (clamped to M - 1),
    // block pair (lane + 64k) % 4 of the step
    const uint32_t a_rowstride = (uint32_t)(nb32 * kQ8_0Bytes);
    const int64_t y_bytes = M * nb32 * kQ8_0Bytes;
    uint32_t a_off[2];
    int s_row[2], s_pair[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int pi = lane + 64 * k;
        s_row[k] = pi >> 2;
        s_pair[k] = pi & 3;
        const int rr = s_row[k] < M ? s_row[k] : (int)M - 1;
        a_off[k] = (uint32_t)rr * a_rowstride + 68 * s_pair[k];
    }

    auto wload = [&](int64_t b, QSWeights &x) {
        const rsrc_t rw = make_rsrc(W, w_bytes);
        const uint32_t bb = (uint32_t)b;
#pragma unroll
        // constant offsets go to the scalar offset: a vector add would be
        // hoisted out of the loop and cost a register per block
        for (int c = 0; c < 8; ++c) x.pay[c] = bld16(rw, v_pay, 128 * bb + 16 * c);
        x.d = bld16(rw, v_d, 16 * bb);
    };
    auto aload = [&](int64_t b, QSActs &r) {
        const rsrc_t ra = make_rsrc(Y, y_bytes);
        const uint32_t sa = (uint32_t)b * kStep;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
#pragma unroll
            for (int j = 0; j < 4; ++j) r.q[k][j] = bld16(ra, a_off[k], sa + 16 * j);
            r.t[k] = __builtin_amdgcn_raw_buffer_load_b32(ra, a_off[k], sa + 64, 0);
        }
    };
    // realign and write stage st of this wavefront
    auto acommit = [&](const QSActs &r, uint8_t *st) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const uint32_t w[17] = {r.q[k][0].x, r.q[k][0].y, r.q[k][0].z, r.q[k][0].w, r.q[k][1].x,
                                    r.q[k][1].y, r.q[k][1].z, r.q[k][1].w, r.q[k][2].x, r.q[k][2].y,
                                    r.q[k][2].z, r.q[k][2].w, r.q[k][3].x, r.q[k][3].y, r.q[k][3].z,
                                    r.q[k][3].w, r.t[k]};
            uint32_t c0[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) c0[j] = __builtin_amdgcn_alignbyte(w[j + 1], w[j], 2);
            const int row = s_row[k], blk0 = 2 * s_pair[k], blk1 = blk0 + 1;
            uint4 *arow_p = reinterpret_cast<uint4 *>(st + QS_A + row * QS_ROWB + 64 * s_pair[k]);
            arow_p[0] = make_uint4(c0[0], c0[1], c0[2], c0[3]);
            arow_p[1] = make_uint4(c0[4], c0[5], c0[6], c0[7]);
            arow_p[2] = make_uint4(w[9], w[10], w[11], w[12]);
            arow_p[3] = make_uint4(w[13], w[14], w[15], w[16]);
            uint16_t *da = reinterpret_cast<uint16_t *>(st + QS_DA);
            da[blk0 * QS_ROWS + row] = (uint16_t)(w[0] & 0xffff);
            da[blk1 * QS_ROWS + row] = (uint16_t)(w[8] >> 16);
        }
    };

    float acc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;

    // One step: start the next step's loads (weights into the other register
    // stage, activation pairs into registers; a wavefront past its last step
    // reloads that step: in bounds, unused), then decode, contraction and
    // epilogue from this step's LDS stage, then realign the next step's
    // activations into the other stage (their loads had the compute to land).
    // Two weight register stages alternate (the loop is unrolled by two) so no
    // register copy forces a wait.
    QSActs ar;
    auto step = [&](int64_t b, int si, const QSWeights &cw, QSWeights &nw) {
        const uint8_t *st = my + si * QS_STAGE;
        const int64_t bn = b + QS_WAVES < nsteps ? b + QS_WAVES : b;
        aload(bn, ar);
        wload(bn, nw);

        // weight operand: lane half hh takes the low (hh = 0) or high nibbles of
        // each payload (elements 16hh..16hh+15 of the block) as the int8 values
        // q - 8: ((q | 0x80) - 8) ^ 0x80 per byte, no borrow crossing bytes.
        // The epilogue of block c runs after the MFMA of block c + 1 is issued,
        // and the empty asm statements pin the accumulators there: without
        // them the epilogues sink below all eight MFMAs, whose results then
        // hold 128 registers.
        const uint32_t dd[4] = {cw.d.x, cw.d.y, cw.d.z, cw.d.w};
        const uint8_t *arow = st + QS_A + l32 * QS_ROWB + 16 * hh;
        const _Float16 *da = reinterpret_cast<const _Float16 *>(st + QS_DA) + 4 * hh;
        const v16i zero = {};
        auto epilogue = [&](int c, const v16i &P) {
            const float dw = f16_bits_to_f32((dd[c >> 1] >> (16 * (c & 1))) & 0xffff);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                // d_a of rows 8q + 4hh .. +3 (one 8-byte read)
                const uint2 dq = *reinterpret_cast<const uint2 *>(da + c * QS_ROWS + 8 * q);
                const _Float16 *dh = reinterpret_cast<const _Float16 *>(&dq);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * q + e;
                    acc[r] = fmaf((float)dh[e], dw * (float)P[r], acc[r]);
                }
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) asm volatile("" : "+v"(acc[r]));
        };
        v16i Pp;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const uint32_t pw[4] = {cw.pay[c].x, cw.pay[c].y, cw.pay[c].z, cw.pay[c].w};
            uint32_t o[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                o[k] = ((((pw[k] >> (4 * hh)) & 0x0f0f0f0fu) | 0x80808080u) - 0x08080808u) ^ 0x80808080u;
            const uint4 a = *reinterpret_cast<const uint4 *>(arow + 32 * c);
            const v16i P = __builtin_amdgcn_mfma_i32_32x32x32_i8(v4i{(int)a.x, (int)a.y, (int)a.z, (int)a.w},
                                                                 v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]},
                                                                 zero, 0, 0, 0);
            if (c > 0) epilogue(c - 1, Pp);
            Pp = P;
        }
        epilogue(7, Pp);
        acommit(ar, my + (si ^ 1) * QS_STAGE);
        __builtin_amdgcn_wave_barrier();  // the stage is read by other lanes next step
    };

    const int64_t b0 = wave < nsteps ? wave : nsteps - 1;
    QSWeights w0, w1;
    aload(b0, ar);
    wload(b0, w0);
    acommit(ar, my);
    __builtin_amdgcn_wave_barrier();
    for (int64_t b = wave; b < nsteps; b += 2 * QS_WAVES) {
        step(b, 0, w0, w1);
        if (b + QS_WAVES < nsteps) step(b + QS_WAVES, 1, w1, w0);
    }

    // ---- sum the eight K-split partial tiles (in the stage LDS, now free)
    // and store the valid outputs
    __syncthreads();
    float *red = reinterpret_cast<float *>(lds);  // [QS_WAVES][16][64]
#pragma unroll
    for (int r = 0; r < 16; ++r) red[(wave * 16 + r) * 64 + lane] = acc[r];
    __syncthreads();
    for (int o = tid; o < 32 * 32; o += QS_THREADS) {
        const int m = o >> 5, c = o & 31;      // output row m, column n_base + c
        const int r = 4 * (m >> 3) + (m & 3);  // register holding row m ...
        const int l = c + 32 * ((m >> 2) & 1); // ... in lane l
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < QS_WAVES; ++w) s += red[(w * 16 + r) * 64 + l];
        if (m < M && n_base + c < N) out[(int64_t)m * N + n_base + c] = s;
    }
}

}  // namespace

int64_t skinny_q4_0_max_m() { return QS_MAX_M; }

hipError_t launch_skinny_q4_0(const uint8_t *w, int64_t w_bytes, const uint8_t *y, float *out, int64_t M,
                              int64_t N, int64_t K, hipStream_t s) {
    static std::atomic<uint64_t> lds_set{0};  // the LDS budget above 64 KiB, per device
    const hipError_t e = ensure_lds_bytes((const void *)k_skinny_q4_0, QS_LDS, lds_set);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)((N + 31) / 32), (unsigned)((M + QS_ROWS - 1) / QS_ROWS));
    hipLaunchKernelGGL(k_skinny_q4_0, grid, dim3(QS_THREADS), QS_LDS, s, w, w_bytes, y, out, M, N, K);
    return hipGetLastError();
}

}  // namespace qmm
