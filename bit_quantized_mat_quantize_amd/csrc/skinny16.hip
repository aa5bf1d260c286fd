// skinny16.hip -- Q4_K weights x Q8_K activations for batches of up to 16
// rows on 16 x 16 int8 MFMA tiles, gfx950.
//
// A small batch reads every weight once, so the weight stream bounds it
// (BitBLAS page, "调度与自动调优": small-M shapes sit on the memory side of the
// roofline).  The 32 x 32 tiles of skinny.hip spend 16 int8 and 2 fp16 MFMAs
// of 32 cycles per step on 32 rows of which a batch of a few uses only M, and
// their 162 registers leave one 8-wavefront workgroup per CU, so a matrix
// with fewer than ~256 tiles of 32 columns leaves CUs idle.  Here an MFMA
// tile is 16 x 16 (v_mfma_i32_16x16x64_i8): half the MFMA cycles per column,
// a quarter of the epilogue per lane, and registers for more wavefronts per
// CU.  A workgroup of WAVES wavefronts owns TILES 16-column tiles (all tiles
// share each activation operand); the launcher picks 8 x 1 for matrices of
// few columns (more workgroups) and 4 x 2 otherwise.
//
// Arithmetic (ggml-cpu mul_mat page, "正确性:缩放系数可以提到求和号外面" and
// "min 项与最终归约"), per super-block b and output (m, n):
//     S  = sum_j s_j P_j,  P_j = sum_{k in j} q_k y_k    (int32, exact)
//     Mn = sum_g m_{g/2} bsums[g]
//     out += d_a (d S - dmin Mn)                         (fp32)
// with s_j folded into two int8 digit planes (s = 8 hi + lo; plane bytes
// q * hi and q * lo are below 128), so S = 8 (Y x hiQ) + (Y x loQ), and
// -dmin m_j split into two fp16 parts (hi + lo exactly) for the min term.
//
// Operand layout (v_mfma_i32_16x16x64_i8): lane l supplies row (A) or column
// (B) l % 16 and the 16 K-values of quarter h = l / 16; result register r of
// lane l holds row 4h + r, column l % 16.  The K order inside a super-block is
// free as long as both operands use it: in MFMA t (t = 0..3) quarter h takes
// the 8 elements 64h + 8t + i (low nibbles of payload bytes 32h + 8t + i,
// sub-block 2h) and the 8 elements 64h + 32 + 8t + i (high nibbles of the same
// bytes, sub-block 2h + 1).  So a lane reads 32 contiguous payload bytes (group
// h) of its column and 64 contiguous activation codes of its row, and its two
// sub-block scales stay fixed for the whole super-block.
// The min term is one v_mfma_f32_16x16x32_f16: K-values 8h + i are the
// bsums 8(h & 1) + i (A) against the hi part (h < 2) or lo part (h >= 2) of
// -dmin * m of their sub-block (B).
//
// Wavefront w takes super-blocks w, w + WAVES, ... (a split of K) for every
// tile of its workgroup, and the partial tiles are summed through LDS at the
// end.  Each lane holds the weights, bsums and d_a of its next super-block in
// registers (loaded one step ahead); its row's codes come from L2 at the
// start of each step, issued before the next step's loads so that waiting for
// them leaves that prefetch in flight (loads complete in issue order).
#include "mfma_common.h"
#include "qmm_device.h"
#include "qmm_launch.h"

namespace qmm {
namespace {

constexpr int S16_ROWS = 16;                      // activation rows per workgroup (one MFMA row tile)
constexpr int64_t S16_MAX_M = 65535ll * S16_ROWS;  // row chunks go to grid.y

typedef _Float16 v8h16 __attribute__((ext_vector_type(8)));
typedef int v4i16 __attribute__((ext_vector_type(4)));
typedef float v4f16 __attribute__((ext_vector_type(4)));

// One super-block of this lane's operands (the activation codes excepted).
template <int TILES>
struct S16Stage {
    uint4 hdr[TILES];     // Q4_K header of column 16t + l % 16
    uint4 pay[TILES][2];  // payload bytes 32h .. 32h + 31 of that column
    uint4 bs;             // bsums 8 (h & 1) .. + 7 of row l % 16
    uint32_t da;          // d_a of row l % 16
};

template <bool REPACKED, int WAVES, int TILES>
__global__ __launch_bounds__(64 * WAVES) void k_skinny16_q4_K(const uint8_t *__restrict__ W,
                                                             const uint8_t *__restrict__ Y,
                                                             float *__restrict__ out, int64_t M,
                                                             int64_t N, int64_t K) {
    __shared__ float s_da[WAVES][16];
    __shared__ float red[WAVES][TILES][4][64];

    // this workgroup's chunk of at most 16 activation rows (grid.y)
    const int64_t m0 = (int64_t)blockIdx.y * S16_ROWS;
    Y += m0 * (K / QK_K) * kQ8_KBytes;
    out += m0 * N;
    M = M - m0 < S16_ROWS ? M - m0 : S16_ROWS;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, h = lane >> 4;
    const int64_t nb = K / QK_K;
    const int64_t n_base = (int64_t)blockIdx.x * 16 * TILES;
    const int row = l16 < M ? l16 : (int)M - 1;  // rows past M: computed, never stored

    const int64_t w_bytes = N * nb * kQ4_KBytes, y_bytes = M * nb * kQ8_KBytes;
    const uint32_t hdr_step = REPACKED ? 16 : kQ4_KBytes, pay_step = REPACKED ? 128 : kQ4_KBytes;
    uint32_t h_off[TILES], p_off[TILES];
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
        const int64_t c = n_base + 16 * t + l16;
        const int64_t col = c < N ? c : N - 1;  // clamped: loads stay in bounds
        h_off[t] = (uint32_t)(col * nb) * hdr_step;
        p_off[t] = REPACKED ? (uint32_t)(16 * N * nb + 128 * col * nb) + 32 * h
                            : (uint32_t)(kQ4_KBytes * col * nb) + 16 + 32 * h;
    }
    const uint32_t y_off = (uint32_t)row * (uint32_t)(nb * kQ8_KBytes);

    auto load = [&](int64_t b, S16Stage<TILES> &st) {
        const rsrc_t rw = make_rsrc(W, w_bytes);
#pragma unroll
        for (int t = 0; t < TILES; ++t) {
            st.hdr[t] = bld16(rw, h_off[t], (uint32_t)b * hdr_step);
            st.pay[t][0] = bld16(rw, p_off[t], (uint32_t)b * pay_step);
            st.pay[t][1] = bld16(rw, p_off[t] + 16, (uint32_t)b * pay_step);
        }
        const rsrc_t ry = make_rsrc(Y, y_bytes);
        const uint32_t sy = (uint32_t)b * kQ8_KBytes;
        st.bs = bld16(ry, y_off + 260 + 16 * (h & 1), sy);
        st.da = __builtin_amdgcn_raw_buffer_load_b32(ry, y_off, sy, 0);
    };

    v4f16 acc[TILES];
#pragma unroll
    for (int t = 0; t < TILES; ++t) acc[t] = v4f16{0.0f, 0.0f, 0.0f, 0.0f};

    // One step: request super-block bn's operands (into nxt), then contract
    // super-block b from cur.  Loads are never predicated (a branch around a
    // load makes the compiler wait for every outstanding load before the next
    // use): past the end a wavefront reloads its current block (from L2).
    auto step = [&](int64_t b, const S16Stage<TILES> &cur, S16Stage<TILES> &nxt) {
        const int64_t bn = b + WAVES < nb ? b + WAVES : b;
        uint4 act[4];  // this step's activation codes first, then the next step's loads
        {
            const rsrc_t ry = make_rsrc(Y, y_bytes);
            const uint32_t sy = (uint32_t)b * kQ8_KBytes;
#pragma unroll
            for (int i = 0; i < 4; ++i) act[i] = bld16(ry, y_off + 4 + 64 * h + 16 * i, sy);
        }
        load(bn, nxt);
        if (h == 0) s_da[wave][l16] = __uint_as_float(cur.da);

        const uint32_t aw[16] = {act[0].x, act[0].y, act[0].z, act[0].w, act[1].x, act[1].y, act[1].z, act[1].w,
                                 act[2].x, act[2].y, act[2].z, act[2].w, act[3].x, act[3].y, act[3].z, act[3].w};
        v8h16 a_bs;  // bsums as fp16 (exact, |bsum| <= 2032): the min term's A operand
        {
            const uint4 r = cur.bs;
            const uint4 hv = make_uint4(h2_bits((int16_t)(r.x & 0xffff), (int16_t)(r.x >> 16)),
                                        h2_bits((int16_t)(r.y & 0xffff), (int16_t)(r.y >> 16)),
                                        h2_bits((int16_t)(r.z & 0xffff), (int16_t)(r.z >> 16)),
                                        h2_bits((int16_t)(r.w & 0xffff), (int16_t)(r.w >> 16)));
            __builtin_memcpy(&a_bs, &hv, 16);
        }
        __builtin_amdgcn_wave_barrier();
        const float4 d4 = *reinterpret_cast<const float4 *>(&s_da[wave][4 * h]);
        const float dv[4] = {d4.x, d4.y, d4.z, d4.w};  // d_a of rows 4h .. 4h + 3
#pragma unroll
        for (int tt = 0; tt < TILES; ++tt) {
            const uint4 hd = cur.hdr[tt];
            const float dcol = f16_bits_to_f32(hd.x & 0xffff);
            const float dmcol = f16_bits_to_f32(hd.x >> 16);
            const Q4KScales sc = unpack_scales(hd.y, hd.z, hd.w);
            // this lane's sub-blocks 2h (low nibbles) and 2h + 1 (high nibbles)
            const uint32_t sw = h < 2 ? sc.s_lo : sc.s_hi;
            const uint32_t sa = (sw >> (16 * (h & 1))) & 0xff, sb = (sw >> (16 * (h & 1) + 8)) & 0xff;
            const uint32_t ha = (sa >> 3) * 0x00010001u, la = (sa & 7) * 0x00010001u;
            const uint32_t hb = (sb >> 3) * 0x00010001u, lb = (sb & 7) * 0x00010001u;
            const uint32_t pw[8] = {cur.pay[tt][0].x, cur.pay[tt][0].y, cur.pay[tt][0].z, cur.pay[tt][0].w,
                                    cur.pay[tt][1].x, cur.pay[tt][1].y, cur.pay[tt][1].z, cur.pay[tt][1].w};

            // contraction: 8 int8 MFMAs (two planes x four K-slices of 64)
            const v4i16 zero = {0, 0, 0, 0};
            v4i16 ah = zero, al = zero;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint32_t w0 = pw[2 * t], w1 = pw[2 * t + 1];
                const uint32_t q0 = w0 & 0x0f0f0f0fu, q1 = w1 & 0x0f0f0f0fu;
                const uint32_t q2 = (w0 >> 4) & 0x0f0f0f0fu, q3 = (w1 >> 4) & 0x0f0f0f0fu;
                const v4i16 a = {(int)aw[2 * t], (int)aw[2 * t + 1], (int)aw[8 + 2 * t], (int)aw[9 + 2 * t]};
                const v4i16 bh = {plane(q0, ha), plane(q1, ha), plane(q2, hb), plane(q3, hb)};
                const v4i16 bl = {plane(q0, la), plane(q1, la), plane(q2, lb), plane(q3, lb)};
                ah = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bh, ah, 0, 0, 0);
                al = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bl, al, 0, 0, 0);
            }

            // min term: the bsums against the hi or lo part of -dmin * m_j
            // for the four sub-blocks 4 (h & 1) .. + 3
            v8h16 b_m;
            {
                const uint32_t mw = (h & 1) == 0 ? sc.m_lo : sc.m_hi;
                uint32_t bm[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float vv = -dmcol * (float)((mw >> (8 * e)) & 0xff);  // exact in fp32
                    const uint32_t hbits = f32_to_f16_bits(vv);
                    const uint32_t part = h < 2 ? hbits : f32_to_f16_bits(vv - f16_bits_to_f32(hbits));
                    bm[e] = part | (part << 16);
                }
                __builtin_memcpy(&b_m, bm, 16);
            }
            const v4f16 zf = {0.0f, 0.0f, 0.0f, 0.0f};
            const v4f16 mn = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_bs, b_m, zf, 0, 0, 0);

            // epilogue: acc += d_a * (d * S - dmin * Mn) for rows 4h .. 4h + 3
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int S = (ah[r] << 3) + al[r];
                const float u = fmaf(dcol, (float)S, mn[r]);
                acc[tt][r] = fmaf(dv[r], u, acc[tt][r]);
            }
        }
        __builtin_amdgcn_wave_barrier();  // s_da is rewritten next step
    };

    const int64_t b0 = wave < nb ? wave : nb - 1;
    S16Stage<TILES> st0, st1;
    load(b0, st0);
    for (int64_t b = wave; b < nb; b += 2 * WAVES) {
        step(b, st0, st1);
        if (b + WAVES < nb) step(b + WAVES, st1, st0);
    }

    // ---- sum the K-split partial tiles and store the valid outputs
#pragma unroll
    for (int t = 0; t < TILES; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][t][r][lane] = acc[t][r];
    __syncthreads();
    for (int o = tid; o < 256 * TILES; o += 64 * WAVES) {
        const int t = o >> 8, m = (o >> 4) & 15, c = o & 15;  // output row m, column n_base + 16t + c
        const int r = m & 3, l = c + 16 * (m >> 2);           // register r of lane l holds it
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) s += red[w][t][r][l];
        if (m < M && n_base + 16 * t + c < N) out[(int64_t)m * N + n_base + 16 * t + c] = s;
    }
}

template <int WAVES, int TILES>
hipError_t launch_cfg(const uint8_t *w, bool repacked, const uint8_t *y, float *out, int64_t M, int64_t N,
                      int64_t K, hipStream_t s) {
    const dim3 grid((unsigned)((N + 16 * TILES - 1) / (16 * TILES)), (unsigned)((M + S16_ROWS - 1) / S16_ROWS)),
        block(64 * WAVES);
    if (repacked)
        hipLaunchKernelGGL((k_skinny16_q4_K<true, WAVES, TILES>), grid, block, 0, s, w, y, out, M, N, K);
    else
        hipLaunchKernelGGL((k_skinny16_q4_K<false, WAVES, TILES>), grid, block, 0, s, w, y, out, M, N, K);
    return hipGetLastError();
}

}  // namespace

int64_t skinny16_max_m() { return S16_MAX_M; }

hipError_t launch_skinny16_q4_K(const uint8_t *w, bool repacked, const uint8_t *y, float *out,
                                int64_t M, int64_t N, int64_t K, hipStream_t s) {
    // Up to 8 rows of the repacked layout the producer/consumer kernel of
    // skinny16r.hip streams the weights faster (N = K = 8192: 11.6 / 12.1
    // against 14.0 / 14.2 us at M = 4 / 8; 5-25% on the other shapes).
    if (repacked && M <= 8) return launch_skinny16r_q4_K(w, y, out, M, N, K, s);
    // 9 to 16 rows of the repacked layout: the three-producer ring with one
    // 16-row block (skinny32r.hip; M = 16, N = K = 8192: 13.6 against 16.6 us
    // here, N = 28672, K = 4096: 21.7 against 28.8 us)
    if (repacked) return launch_skinny32r_q4_K(w, y, out, M, N, K, s);
    // Below 8192 columns (fewer than 256 tiles of 32) 8 wavefronts per
    // 16-column tile give twice the workgroups; wider matrices take 4
    // wavefronts per 32 columns, whose workgroups share a CU three at a time.
    // Measured (M = 4): N = 4096, K = 14336: 11.3 against 14.8 us;
    // N = 28672, K = 4096: 21.3 against 25.0 us.
    if (N < 8192) return launch_cfg<8, 1>(w, repacked, y, out, M, N, K, s);
    return launch_cfg<4, 2>(w, repacked, y, out, M, N, K, s);
}

}  // namespace qmm
