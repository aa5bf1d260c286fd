// q6k_skinny.hip -- Q6_K weights x Q8_K activations for small batches on int8
// MFMA, gfx950, repacked layout.
//
// Format and integer path: ggml-cpu mul_mat page, "更低的比特:Q6_K 与 Q2_K 的取舍"
// (ql/qh 6-bit codes, int8 scale per 16-element group, fp16 d, no min) and
// "正确性:缩放系数可以提到求和号外面":
//   per super-block b, output (m, n):  S = sum_j s_j * sum_{i in j} q_i y_i,
//   acc += d_a * d * S.
//
// A few activation rows still read every weight once (BitBLAS page,
// "调度与自动调优": small batches sit on the memory side of the roofline), but
// the GEMV repeats its dot products for every row and a single-row-tile GEMM
// runs too few workgroups.  As in the Q4_K small-batch kernel, a workgroup owns
// 32 output columns and up to 32 activation rows (more rows take more grid
// rows, blockIdx.y), and its 8 wavefronts split K: wavefront w takes the
// super-blocks w, w + 8, ... and the eight partial tiles are summed through LDS.
//
// Weights: each lane loads the part of its column's super-block that the Q6_K
// GEMM's lane loads (ql pieces 2g + h, qh pieces h and h + 2, the 16 scales,
// d) straight into registers, one step ahead, in two alternating register
// stages (the loop is unrolled by two).  Decode as in the GEMM: per 32-element
// chunk the scaled codes t = s*q are split into two int8 digits
// (t = 256 hi + lo) and take two MFMAs, S = 256 H + L.
// Activations: the R = 8, 16 or 32 rows M needs of the wavefront's super-block
// go into its own LDS stage by direct global->LDS loads, 16 lanes per 256-byte
// row (pieces XOR-swizzled by row), with d_a beside them, one step ahead.
// Each step reads all of its stage before it issues the next step's loads:
// the compiler makes an LDS read wait for every direct global->LDS load issued
// before it, and those would otherwise be the next step's.
//
// MFMA operand convention (v_mfma_*_32x32xK): lane l supplies row (A) or
// column (B) l % 32 and the K-slice selected by l / 32; the result register r
// of lane l holds row 8*(r/4) + 4*(l/32) + r%4, column l % 32.
#include "mfma_common.h"
#include "qmm_device.h"
#include "qmm_launch.h"

namespace qmm {
namespace {

constexpr int Q6S_WAVES = 8, Q6S_THREADS = 64 * Q6S_WAVES;
constexpr int Q6S_ROWS = 32;                       // activation rows per workgroup
constexpr int64_t Q6S_MAX_M = 65535ll * Q6S_ROWS;  // row chunks go to grid.y
// Per-wavefront LDS stage for R staged rows: codes [R][256] (16-byte piece p
// of row r at position p ^ (r & 15)), then d_a [64] (rows l % 32 of the loading
// lane l).  Sized by R, so that at R = 8 several workgroups share a CU.
constexpr int Q6S_A = 0;
constexpr int Q6S_RED = Q6S_WAVES * 16 * 64 * 4;  // the partial tiles at the end
template <int R>
struct Q6SLds {
    static constexpr int DA = R * 256, STAGE = DA + 64 * 4, BYTES = Q6S_WAVES * 2 * STAGE;
    static_assert(BYTES <= 160 * 1024 && Q6S_RED <= BYTES, "LDS budget of a gfx950 CU");
};

// The weight side of one super-block for lane (column l % 32, slice h = l / 32).
struct Q6SW {
    uint4 ql[4];  // ql pieces 2g + h
    uint4 qa, qb; // qh pieces h and h + 2
    uint4 sc;     // the 16 int8 scales
    uint32_t d;   // fp16 d
};

template <int R>
__global__ __launch_bounds__(Q6S_THREADS, 1) void k_skinny_q6_K(const uint8_t *__restrict__ W, int64_t w_bytes,
                                                               const uint8_t *__restrict__ Y,
                                                               float *__restrict__ out, int64_t M, int64_t N,
                                                               int64_t K) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    constexpr int STAGE = Q6SLds<R>::STAGE, DA = Q6SLds<R>::DA;

    // this workgroup's chunk of at most 32 activation rows (grid.y)
    const int64_t nb = K / QK_K;
    const int64_t m0 = (int64_t)blockIdx.y * Q6S_ROWS;
    Y += m0 * nb * kQ8_KBytes;
    out += m0 * N;
    M = M - m0 < Q6S_ROWS ? M - m0 : Q6S_ROWS;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: feeds scalar offsets
    const int l32 = lane & 31, hh = lane >> 5;
    const int64_t n_base = (int64_t)blockIdx.x * 32;
    const int64_t col = n_base + l32 < N ? n_base + l32 : N - 1;  // clamped: loads stay in bounds
    uint8_t *const my = lds + wave * 2 * STAGE;                // this wavefront's two stages

    // weights (repacked Q6_K: d section of 2 bytes per super-block padded to
    // 256 bytes, then scales 16 B, ql 128 B and qh 64 B per super-block, each
    // section [N][nb]); offsets relative to the matrix start
    const int64_t NB = N * nb;
    const int64_t dsec = (2 * NB + 255) / 256 * 256;
    const int64_t i0 = col * nb;  // the column's first super-block
    const uint32_t v_d = (uint32_t)(2 * i0);
    const uint32_t v_sc = (uint32_t)(dsec + 16 * i0);
    const uint32_t v_ql = (uint32_t)(dsec + 16 * NB + 128 * i0 + 16 * hh);
    const uint32_t v_qh = (uint32_t)(dsec + 144 * NB + 64 * i0 + 16 * hh);
    // constant offsets go to the scalar offset (a vector add would be hoisted
    // out of the loop and hold a register per load)
    auto wload = [&](int64_t b, Q6SW &x) {
        const rsrc_t rw = make_rsrc(W, w_bytes);
        const uint32_t bb = (uint32_t)b;
#pragma unroll
        for (int g = 0; g < 4; ++g) x.ql[g] = bld16(rw, v_ql, 128 * bb + 32 * g);
        x.qa = bld16(rw, v_qh, 64 * bb);
        x.qb = bld16(rw, v_qh, 64 * bb + 32);
        x.sc = bld16(rw, v_sc, 16 * bb);
        x.d = __builtin_amdgcn_raw_buffer_load_b16(rw, v_d, 2 * bb, 0);
    };

    // activations: rows past M - 1 are clamped to it (loaded, never stored)
    const int64_t y_bytes = M * nb * kQ8_KBytes;
    const uint32_t row_stride = (uint32_t)(nb * kQ8_KBytes);
    auto row_off = [&](int r) -> uint32_t { return (uint32_t)(r < M ? r : M - 1) * row_stride; };
    // codes: instruction t moves rows 4t .. 4t+3, 16 lanes per 256-byte row
    const int c_row = lane >> 4, c_pos = lane & 15;
    uint32_t a_goff[R / 4];
#pragma unroll
    for (int t = 0; t < R / 4; ++t) {
        const int r = 4 * t + c_row;
        a_goff[t] = row_off(r) + 4 + 16 * (uint32_t)(c_pos ^ (r & 15));
    }
    const uint32_t da_off = row_off(l32);
    auto aload = [&](int64_t b, uint8_t *st) {
        const rsrc_t ry = make_rsrc(Y, y_bytes);
        const uint32_t sy = (uint32_t)b * kQ8_KBytes;
#pragma unroll
        for (int t = 0; t < R / 4; ++t) dma16(ry, a_goff[t], sy, st + Q6S_A + 1024 * t);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ry, (lds_void *)(st + DA), 4, da_off, sy, 0, 0);
    };
    // MFMA row l32 reads staged row l32 & (R - 1) (rows >= M are never stored)
    const int arow = l32 & (R - 1);

    float acc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;

    // One step: wait for this step's data, read the whole stage, start the
    // next step's loads (a wavefront past its last step reloads that step: in
    // bounds, unused), then decode, contraction and epilogue.
    auto step = [&](int64_t b, int si, const Q6SW &cur, Q6SW &nxt) {
        const int64_t bn = b + Q6S_WAVES < nb ? b + Q6S_WAVES : b;
        const uint8_t *st = my + si * STAGE;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this step's weights and LDS rows
        uint4 a[8];
#pragma unroll
        for (int c = 0; c < 8; ++c)
            a[c] = *reinterpret_cast<const uint4 *>(st + Q6S_A + arow * 256 + 16 * ((2 * c + hh) ^ (arow & 15)));
        float4 d4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) d4[q] = *reinterpret_cast<const float4 *>(st + DA + 4 * (8 * q + 4 * hh));
        aload(bn, my + (si ^ 1) * STAGE);
        wload(bn, nxt);

        // chunk c holds group 2c + hh of this lane (see the Q6_K GEMM)
        const float dcol = f16_bits_to_f32(cur.d);
        const uint32_t sw[4] = {cur.sc.x, cur.sc.y, cur.sc.z, cur.sc.w};
        const v16i zero = {};
        v16i ah = zero, al = zero;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int g = c >> 1, hi_nib = c & 1;
            const int s = (int)(int8_t)(sw[g] >> (16 * hi_nib + 8 * hh));  // scale byte 2c + hh
            const s16x2 s2 = {(short)s, (short)s};
            const s16x2 c2 = {(short)(128 - 32 * s), (short)(128 - 32 * s)};
            const uint32_t ql[4] = {cur.ql[g].x, cur.ql[g].y, cur.ql[g].z, cur.ql[g].w};
            const uint4 qhp = hi_nib ? cur.qb : cur.qa;
            const uint32_t qh[4] = {qhp.x, qhp.y, qhp.z, qhp.w};
            uint32_t hw[4], lw[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t u = ((ql[w] >> (4 * hi_nib)) & 0x0f0f0f0fu) | (((qh[w] >> (2 * g)) & 0x03030303u) << 4);
                t_digits(u, s2, c2, hw[w], lw[w]);
            }
            const v4i av = v4i{(int)a[c].x, (int)a[c].y, (int)a[c].z, (int)a[c].w};
            ah = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, v4i{(int)hw[0], (int)hw[1], (int)hw[2], (int)hw[3]}, ah,
                                                       0, 0, 0);
            al = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, v4i{(int)lw[0], (int)lw[1], (int)lw[2], (int)lw[3]}, al,
                                                       0, 0, 0);
        }
        // epilogue: acc += d_a * (d * S), S = 256 H + L (|S| <= 256 * 4096 * 127)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float dv[4] = {d4[q].x, d4[q].y, d4[q].z, d4[q].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * q + e;
                acc[r] = fmaf(dv[e], dcol * (float)((ah[r] << 8) + al[r]), acc[r]);
            }
        }
        // the epilogue stays in this step: sunk into the next one it would
        // keep this step's MFMA results live across that step
#pragma unroll
        for (int r = 0; r < 16; ++r) asm volatile("" : "+v"(acc[r]));
    };

    const int64_t b0 = wave < nb ? wave : nb - 1;
    Q6SW w0, w1;
    aload(b0, my);
    wload(b0, w0);
    for (int64_t b = wave; b < nb; b += 2 * Q6S_WAVES) {
        step(b, 0, w0, w1);
        if (b + Q6S_WAVES < nb) step(b + Q6S_WAVES, 1, w1, w0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no transfer into LDS outlives the loop

    // ---- sum the eight K-split partial tiles (in the stage LDS, now free)
    // and store the valid outputs
    __syncthreads();
    float *red = reinterpret_cast<float *>(lds);  // [Q6S_WAVES][16][64]
#pragma unroll
    for (int r = 0; r < 16; ++r) red[(wave * 16 + r) * 64 + lane] = acc[r];
    __syncthreads();
    for (int o = tid; o < 32 * 32; o += Q6S_THREADS) {
        const int m = o >> 5, c = o & 31;      // output row m, column n_base + c
        const int r = 4 * (m >> 3) + (m & 3);  // register holding row m ...
        const int l = c + 32 * ((m >> 2) & 1); // ... in lane l
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < Q6S_WAVES; ++w) s += red[(w * 16 + r) * 64 + l];
        if (m < M && n_base + c < N) out[(int64_t)m * N + n_base + c] = s;
    }
}

template <int R>
hipError_t launch_q6s(const uint8_t *w, int64_t w_bytes, const uint8_t *y, float *out, int64_t M, int64_t N,
                      int64_t K, hipStream_t s) {
    static std::atomic<uint64_t> lds_set{0};  // the LDS budget above 64 KiB, per device
    const hipError_t e = ensure_lds_bytes((const void *)k_skinny_q6_K<R>, Q6SLds<R>::BYTES, lds_set);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)((N + 31) / 32), (unsigned)((M + Q6S_ROWS - 1) / Q6S_ROWS));
    hipLaunchKernelGGL((k_skinny_q6_K<R>), grid, dim3(Q6S_THREADS), Q6SLds<R>::BYTES, s, w, w_bytes, y, out, M, N, K);
    return hipGetLastError();
}

}  // namespace

int64_t skinny_q6_K_max_m() { return Q6S_MAX_M; }

hipError_t launch_skinny_q6_K(const uint8_t *w, int64_t w_bytes, const uint8_t *y, float *out, int64_t M,
                              int64_t N, int64_t K, hipStream_t s) {
    // rows staged per super-block: the power of two >= M among 8, 16, 32
    if (M <= 8) return launch_q6s<8>(w, w_bytes, y, out, M, N, K, s);
    if (M <= 16) return launch_q6s<16>(w, w_bytes, y, out, M, N, K, s);
    return launch_q6s<32>(w, w_bytes, y, out, M, N, K, s);
}

}  // namespace qmm
