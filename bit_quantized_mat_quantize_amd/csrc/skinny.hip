// skinny.hip -- quantized mul_mat for small batches on int8 MFMA, gfx950.
//
// A batch of a few activation rows still reads every weight once, so the
// operation stays bound by the weight stream (BitBLAS page, "调度与自动调优":
// small-M shapes sit on the memory side of the roofline), but the per-row
// vector dot products of the GEMV grow with M.  Here the contraction runs on
// the matrix cores instead: a workgroup's (at most 32) activation rows are one
// MFMA row tile, so every weight column is decoded once per super-block and
// then costs a handful of v_mfma_i32_32x32x32_i8 no matter how many rows
// there are.  Larger batches take one 32-row chunk per grid row (blockIdx.y);
// the chunks of a column tile read the same weights, the later ones mostly
// from L2 or the MALL.  A single-row-tile GEMM would run only N/256
// workgroups, so up to a few hundred rows (fewer for large N) this kernel is
// the faster one.
//
// Arithmetic (ggml-cpu mul_mat page, "正确性:缩放系数可以提到求和号外面" and
// "min 项与最终归约"), per super-block b and output (m, n):
//     S  = sum_j s_j P_j,  P_j = sum_{k in j} q_k y_k    (int32, exact)
//     Mn = sum_g m_{g/2} bsums[g]
//     out += d_a (d S - dmin Mn)                         (fp32)
// with the 6-bit s_j folded into two int8 digit planes (s = 8 hi + lo, every
// plane value <= 105) so that S = 8 (Y x hiQ) + (Y x loQ) on the MFMA, and
// -dmin m_j split into two fp16 values for an exact fp16 MFMA against the
// fp16 bsums (|bsums| <= 2032).
//
// Workgroup: 8 wavefronts (two per SIMD) own one 32-column tile of the output;
// wavefront w takes the super-blocks b = w, w + 8, ... (a split of K), and the
// eight partial tiles are summed through LDS at the end.  Each wavefront
// streams its columns' weights straight from memory into registers (no LDS
// staging: every byte is used by exactly one wavefront).  The activation rows
// come from L2, where all workgroups share them.  Up to 8 rows, each lane
// loads its row's operands straight into MFMA operand registers at the start
// of the step (the loads touch few distinct rows).  With more rows every lane
// would read a different row and one load would touch up to 64 cache lines,
// so the rows of the wavefront's super-block go into its own LDS stage by
// direct global->LDS loads instead, 16 lanes per contiguous 256-byte row (only
// the rows M needs: 16 or 32).  The weights (and the staged rows) of
// super-block b + 8 are requested before b is computed.
//
// MFMA operand convention (v_mfma_*_32x32xK): lane l supplies row (A) or
// column (B) l % 32 and the K-slice selected by l / 32; the result register r
// of lane l holds row 8*(r/4) + 4*(l/32) + r%4, column l % 32.
#include "mfma_common.h"
#include "qmm_device.h"
#include "qmm_launch.h"

namespace qmm {
namespace {

constexpr int SK_WAVES = 8, SK_THREADS = 64 * SK_WAVES;
constexpr int SK_ROWS = 32;                   // activation rows per workgroup (one MFMA row tile)
constexpr int64_t SK_MAX_M = 65535ll * SK_ROWS;  // row chunks go to grid.y
// Per-wavefront LDS stage: the activation rows of one super-block.
//   A   int8 codes [32][256]   16-byte piece p of row r at position p ^ (r & 15)
//   BS  bsums      [32][2][16 B]
//   DA  d_a        [64] (rows l % 32)
constexpr int ST_A = 0, ST_BS = 32 * 256, ST_DA = ST_BS + 32 * 32, ST_BYTES = ST_DA + 64 * 4;
constexpr int SK_LDS = SK_WAVES * 2 * ST_BYTES;
constexpr int RED_BYTES = SK_WAVES * 16 * 64 * 4;
static_assert(SK_LDS <= 160 * 1024 && RED_BYTES <= SK_LDS, "LDS budget of a gfx950 CU");

// One super-block in this lane's registers (loaded one step ahead): the
// weight side, and with activation registers also the row's bsums and d_a.
struct Stage {
    uint4 hdr;      // Q4_K header of column l%32
    uint4 pay[4];   // payload pieces 2g + l/32, g = 0..3
    uint4 bs;       // bsums 8*(l/32)..+7 of row l%32 (activation registers)
    uint32_t da;    // d_a of row l%32 (activation registers)
};
// LDS of the activation-register variant: the partial tiles, then d_a per wavefront
constexpr int SK_LDS_REG = RED_BYTES + SK_WAVES * 32 * 4;

// LDS_ACT: activation rows staged in LDS (M > 8); otherwise each lane loads its
// row's operands into registers at the start of the step (few distinct rows,
// so few cache lines per load).
template <bool REPACKED, bool LDS_ACT>
__global__ __launch_bounds__(SK_THREADS, 1) void k_skinny_q4_K(const uint8_t *__restrict__ W,
                                                             const uint8_t *__restrict__ Y,
                                                             float *__restrict__ out, int64_t M,
                                                             int64_t N, int64_t K) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    // this workgroup's chunk of at most 32 activation rows (grid.y)
    const int64_t m0 = (int64_t)blockIdx.y * SK_ROWS;
    Y += m0 * (K / QK_K) * kQ8_KBytes;
    out += m0 * N;
    M = M - m0 < SK_ROWS ? M - m0 : SK_ROWS;

    const int tid = threadIdx.x, lane = tid & 63;
    // wavefront-uniform, and known to be: the super-block index derived from it
    // goes into the scalar offset of the buffer loads
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hh = lane >> 5;
    const int64_t nb = K / QK_K;
    const int64_t n_base = (int64_t)blockIdx.x * 32;
    const int64_t col = n_base + l32 < N ? n_base + l32 : N - 1;  // clamped: loads stay in bounds
    uint8_t *const my = lds + wave * 2 * ST_BYTES;                // this wavefront's two stages

    // weights: this lane's column; offsets relative to the matrix start
    // (buffer resources are built where they are used: one held across the
    // lambdas below would be treated as divergent and waterfall-looped)
    const int64_t w_bytes = N * nb * kQ4_KBytes, y_bytes = M * nb * kQ8_KBytes;
    const uint32_t hdr_step = REPACKED ? 16 : kQ4_KBytes, pay_step = REPACKED ? 128 : kQ4_KBytes;
    const uint32_t h_off = (uint32_t)(col * nb) * hdr_step;
    const uint32_t p_off = REPACKED ? (uint32_t)(16 * N * nb + 128 * col * nb) + 16 * hh
                                    : (uint32_t)(kQ4_KBytes * col * nb) + 16 + 16 * hh;
    // activations: rows past M - 1 are clamped to it (loaded, never stored)
    const uint32_t row_stride = (uint32_t)(nb * kQ8_KBytes);
    auto row_off = [&](int r) -> uint32_t { return (uint32_t)(r < M ? r : M - 1) * row_stride; };
    // codes: instruction t moves rows 4t .. 4t+3, 16 lanes per 256-byte row
    const int c_row = lane >> 4, c_pos = lane & 15;
    const uint32_t bs_off = row_off(lane >> 1) + 260 + 16 * (lane & 1);
    const uint32_t da_off = row_off(l32);
    // rows staged: the power of two >= M among 8, 16, 32; MFMA row l32 reads
    // staged row l32 & (R - 1) (rows >= M are computed and never stored)
    const int R = M <= 8 ? 8 : (M <= 16 ? 16 : 32);
    const int arow = l32 & (R - 1);

    auto wload = [&](int64_t b, Stage &st) {
        const rsrc_t rw = make_rsrc(W, w_bytes);
        st.hdr = bld16(rw, h_off, (uint32_t)b * hdr_step);
#pragma unroll
        for (int g = 0; g < 4; ++g) st.pay[g] = bld16(rw, p_off + 32 * g, (uint32_t)b * pay_step);
    };
    // activation-register variant: the row's bsums and d_a with the weights
    const uint32_t y_off = row_off(l32);
    auto sload = [&](int64_t b, Stage &st) {
        const rsrc_t ry = make_rsrc(Y, y_bytes);
        const uint32_t sy = (uint32_t)b * kQ8_KBytes;
        st.bs = bld16(ry, y_off + 260 + 16 * hh, sy);
        st.da = __builtin_amdgcn_raw_buffer_load_b32(ry, y_off, sy, 0);
    };
    float *const s_da = reinterpret_cast<float *>(lds + RED_BYTES) + 32 * wave;
    // activation rows of super-block b into stage buffer st (direct global->LDS)
    auto aload = [&](int64_t b, uint8_t *st) {
        const rsrc_t ry = make_rsrc(Y, y_bytes);
        const uint32_t sy = (uint32_t)b * kQ8_KBytes;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            if (4 * t >= R) break;  // wavefront-uniform
            const int r = 4 * t + c_row;
            dma16(ry, row_off(r) + 4 + 16 * (uint32_t)(c_pos ^ (r & 15)), sy, st + ST_A + 1024 * t);
        }
        dma16(ry, bs_off, sy, st + ST_BS);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ry, (lds_void *)(st + ST_DA), 4, da_off, sy, 0, 0);
    };

    float acc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;

    // Register loads are never predicated (a branch around a load makes the
    // compiler wait for every outstanding load before the next use): a wavefront without
    // super-blocks loads block nb - 1 and skips the loop; the step after its
    // last one loads that block again (from L2) and leaves it unused.
    // One step: wait for this step's data, start the next step's (activations
    // into the other LDS stage, weights into the other register stage), then
    // decode, contraction and epilogue.  Two register stages alternate (the
    // loop is unrolled by two) so no register copy forces a wait.
    auto step = [&](int64_t b, int si, const Stage &cur, Stage &nxt) {
        const int64_t bn = b + SK_WAVES < nb ? b + SK_WAVES : b;
        const uint8_t *st = my + si * ST_BYTES;
        uint4 act[8];
        if constexpr (LDS_ACT) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this step's weights and LDS rows
            aload(bn, my + (si ^ 1) * ST_BYTES);
            wload(bn, nxt);
        } else {
            // this step's activation operands first, then the next step's loads
            // (waiting for the activations leaves that prefetch in flight)
            const rsrc_t ry = make_rsrc(Y, y_bytes);
            const uint32_t sy = (uint32_t)b * kQ8_KBytes;
#pragma unroll
            for (int j = 0; j < 8; ++j) act[j] = bld16(ry, y_off + 4 + 32 * j + 16 * hh, sy);
            wload(bn, nxt);
            sload(bn, nxt);
            if (hh == 0) s_da[l32] = __uint_as_float(cur.da);
        }

        const float dcol = f16_bits_to_f32(cur.hdr.x & 0xffff);
        const float dmcol = f16_bits_to_f32(cur.hdr.x >> 16);
        const Q4KScales sc = unpack_scales(cur.hdr.y, cur.hdr.z, cur.hdr.w);
        // plane j is built just before the two MFMAs that read it
        auto build = [&](int j, v4i &bh, v4i &bl) {
            const uint4 pw = cur.pay[j >> 1];
            const uint32_t sw = j < 4 ? sc.s_lo : sc.s_hi;
            const int shift = (j & 1) * 4;  // low nibbles: sub-block 2g, high: 2g + 1
            const uint32_t q0 = (pw.x >> shift) & 0x0f0f0f0fu, q1 = (pw.y >> shift) & 0x0f0f0f0fu;
            const uint32_t q2 = (pw.z >> shift) & 0x0f0f0f0fu, q3 = (pw.w >> shift) & 0x0f0f0f0fu;
            const uint32_t sj = (sw >> (8 * (j & 3))) & 0xff;
            const uint32_t hi2 = (sj >> 3) * 0x00010001u, lo2 = (sj & 7) * 0x00010001u;
            bh = v4i{plane(q0, hi2), plane(q1, hi2), plane(q2, hi2), plane(q3, hi2)};
            bl = v4i{plane(q0, lo2), plane(q1, lo2), plane(q2, lo2), plane(q3, lo2)};
        };
        // min-term operands: -dmin*m_j = hi + lo exactly in fp16; bsums exact in fp16
        v8h bmh, bml, a_bs;
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
            const uint4 r = LDS_ACT ? *reinterpret_cast<const uint4 *>(st + ST_BS + 16 * (2 * arow + hh)) : cur.bs;
            const uint4 hv = make_uint4(h2_bits((int16_t)(r.x & 0xffff), (int16_t)(r.x >> 16)),
                                        h2_bits((int16_t)(r.y & 0xffff), (int16_t)(r.y >> 16)),
                                        h2_bits((int16_t)(r.z & 0xffff), (int16_t)(r.z >> 16)),
                                        h2_bits((int16_t)(r.w & 0xffff), (int16_t)(r.w >> 16)));
            __builtin_memcpy(&a_bs, &hv, 16);
        }

        // ---- contraction: 16 int8 MFMAs (two planes x 8 sub-blocks), 2 fp16 MFMAs
        const v16i zero = {};
        v16i ah = zero, al = zero;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint4 av = LDS_ACT ? *reinterpret_cast<const uint4 *>(st + ST_A + arow * 256 +
                                                                        16 * ((2 * j + hh) ^ (arow & 15)))
                                     : act[j];
            const v4i a = v4i{(int)av.x, (int)av.y, (int)av.z, (int)av.w};
            v4i bh, bl;
            build(j, bh, bl);
            ah = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bh, ah, 0, 0, 0);
            al = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bl, al, 0, 0, 0);
        }
        const v16f zf = {};
        v16f mn = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_bs, bmh, zf, 0, 0, 0);
        mn = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_bs, bml, mn, 0, 0, 0);

        // ---- epilogue: acc += d_a * (d * S - dmin * Mn)
        const float *da = LDS_ACT ? reinterpret_cast<const float *>(st + ST_DA) : s_da;
        if constexpr (!LDS_ACT) __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 d4 = *reinterpret_cast<const float4 *>(da + 8 * q + 4 * hh);
            const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * q + e;
                const int S = (ah[r] << 3) + al[r];
                const float t = fmaf(dcol, (float)S, mn[r]);
                acc[r] = fmaf(dv[e], t, acc[r]);
            }
        }
        if constexpr (!LDS_ACT) __builtin_amdgcn_wave_barrier();  // s_da is rewritten next step
    };

    const int64_t b0 = wave < nb ? wave : nb - 1;
    Stage st0, st1;
    if constexpr (LDS_ACT) aload(b0, my);
    else sload(b0, st0);
    wload(b0, st0);
    for (int64_t b = wave; b < nb; b += 2 * SK_WAVES) {
        step(b, 0, st0, st1);
        if (b + SK_WAVES < nb) step(b + SK_WAVES, 1, st1, st0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no transfer into LDS outlives the loop

    // ---- sum the eight K-split partial tiles (in the staging LDS, now free)
    // and store the valid outputs
    __syncthreads();
    float *red = reinterpret_cast<float *>(lds);  // [SK_WAVES][16][64]
#pragma unroll
    for (int r = 0; r < 16; ++r) red[(wave * 16 + r) * 64 + lane] = acc[r];
    __syncthreads();
    for (int o = tid; o < 32 * 32; o += SK_THREADS) {
        const int m = o >> 5, c = o & 31;            // output row m, column n_base + c
        const int r = 4 * (m >> 3) + (m & 3);        // register holding row m ...
        const int l = c + 32 * ((m >> 2) & 1);       // ... in lane l
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < SK_WAVES; ++w) s += red[(w * 16 + r) * 64 + l];
        if (m < M && n_base + c < N) out[(int64_t)m * N + n_base + c] = s;
    }
}

}  // namespace

int64_t skinny_max_m() { return SK_MAX_M; }

hipError_t launch_skinny_q4_K(const uint8_t *w, bool repacked, const uint8_t *y, float *out,
                              int64_t M, int64_t N, int64_t K, hipStream_t s) {
    // 17 to 32 rows of the repacked layout: the producer/consumer ring
    // (skinny32r.hip; N = K = 8192, M = 32: 17.0 against 20.7 us here)
    if (repacked && M > 16 && M <= 32) return launch_skinny32r_q4_K(w, y, out, M, N, K, s);
    static std::atomic<uint64_t> lds_set[2] = {{0}, {0}};  // the LDS budget above 64 KiB, per device
    const hipError_t e = ensure_lds_bytes(
        repacked ? (const void *)k_skinny_q4_K<true, true> : (const void *)k_skinny_q4_K<false, true>, SK_LDS,
        lds_set[repacked]);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)((N + 31) / 32), (unsigned)((M + SK_ROWS - 1) / SK_ROWS)), block(SK_THREADS);
    // up to 8 rows the per-lane operand loads touch few cache lines and beat
    // the LDS staging; more rows are staged
    const bool lds_act = M > 8;
    const unsigned lds = lds_act ? SK_LDS : SK_LDS_REG;
#define QMM_SKINNY(RP, LA) hipLaunchKernelGGL((k_skinny_q4_K<RP, LA>), grid, block, lds, s, w, y, out, M, N, K)
    if (repacked) {
        if (lds_act) QMM_SKINNY(true, true); else QMM_SKINNY(true, false);
    } else {
        if (lds_act) QMM_SKINNY(false, true); else QMM_SKINNY(false, false);
    }
#undef QMM_SKINNY
    return hipGetLastError();
}

}  // namespace qmm
