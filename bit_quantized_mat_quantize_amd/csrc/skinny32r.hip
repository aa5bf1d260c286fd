// skinny32r.hip -- Q4_K weights (repacked layout) x Q8_K activations for
// batches of 9 to 32 rows, gfx950: the producer/consumer LDS ring of
// skinny16r.hip, widened to RB = 1 or 2 blocks of 16 activation rows (16 or
// 32 rows), with one producer wavefront for the weights and one per row block
// for the activation codes.
//
// A small batch reads every weight once, so the weight stream bounds it
// (BitBLAS page, "调度与自动调优": small-M shapes sit on the memory side of the
// roofline).  With 32 rows the activation codes outweigh the weights a
// workgroup streams: per super-block and 16 columns, 2.3 KB of weights against
// 9.3 KB of codes, bsums and scales.  So a workgroup takes COLS = 32 columns
// where that still gives every CU a workgroup (each stage's codes then serve
// twice the weight bytes), else 16, and a stage holds SB = 64 / COLS
// super-blocks (one 64-lane load of headers).  A stage is 28 (COLS = 32) or
// 47 (COLS = 16) load instructions of 64 lanes, more than one wavefront's
// in-order load counter (63) holds for two stages in flight, so the loads are
// shared: producer 0 takes the headers, payloads, bsums and d_a, producer 1
// the codes of rows 0-15 and (RB = 2) producer 2 those of rows 16-31.  Each
// waits for its own part of the oldest stage (loads complete in issue order),
// then every wavefront meets at one workgroup barrier, which releases the
// stage to the four consumers; consumer c contracts super-block SB S + c % SB
// of stage S for the 16 columns 16 (c / SB) .. + 15 and every row block.  D
// stages are in flight: two with one workgroup per CU, one where the grid
// gives two per CU (their rings share the LDS).  Measured at M = 32 against
// the 32 x 32-tile kernel (skinny.hip): N = K = 8192 17.0 against 20.7 us,
// N = 28672, K = 4096 27.0 against 36.9, N = 4096, K = 14336 18.4 against
// 28.4 (16 columns; with 32 only half the CUs get a workgroup); deeper rings
// were slower (N = K = 8192, 32 columns: 17.4 us with D = 3, 18.2 with D = 4).
// At M = 16 (RB = 1) against the 16 x 16-tile kernel (skinny16.hip): 13.6
// against 16.6 us at N = K = 8192, 21.7 against 28.8 at N = 28672, K = 4096,
// 13.2 against 17.2 at N = 4096, K = 14336.
//
// Arithmetic, per super-block and output (m, n), as in skinny16r.hip (ggml-cpu
// mul_mat page, "正确性:缩放系数可以提到求和号外面" and "min 项与最终归约"):
// S = sum_j s_j P_j on two int8 digit planes of the sub-block scales
// (s = 8 hi + lo) on v_mfma_i32_16x16x64_i8, the min term -dmin * sum_j m_j
// bsums_j on one fp16 MFMA (bsums exact in fp16, -dmin m_j the exact sum of
// two fp16 parts), then acc += d_a (d S - dmin Mn).  The planes of a K-slice
// are built once and feed both row blocks.  Operand layout of the MFMAs: lane
// l supplies row (A) or column (B) l % 16 and K-values 16 (l / 16) .. + 15;
// result register r of lane l holds row 4 (l / 16) + r of the block, column
// l % 16.  Consumer c accumulates the super-blocks c % 2, c % 2 + 2, ...; the
// two partial tiles of a column group are summed through LDS at the end.
//
// Ring slot (COLS columns, super-blocks SB S .. SB S + SB - 1, 32 activation
// rows; RPB = 32 / SB rows per bsums load, RPD = 64 / SB rows per d_a load):
//   HDR  1 KB       header of super-block l / COLS, column l % COLS at 16 l
//   PAY  8 KB       super-block b, payload piece p of column c at 16 (8 COLS b + 8 c + (p ^ (c % 8)))
//   ACT  8 KB SB    row r, super-block b: code piece q at
//                   1024 SB (r / 4) + 1024 b + 16 (16 (r % 4) + (q ^ (r % 16)))
//   BSM  1 KB SB    row r, super-block b, bsums half e at
//                   1024 (r / RPB) + 16 (2 RPB b + 2 (r % RPB) + e)
//   DA   128 B SB   row r, super-block b at 256 (r / RPD) + 4 (RPD b + r % RPD)
// Rows past M, columns past N and super-blocks past K load the last valid
// one (every load in bounds, none predicated); their results are dropped.
#include "mfma_common.h"
#include "qmm_device.h"
#include "qmm_launch.h"

namespace qmm {
namespace {

typedef _Float16 v8h32r __attribute__((ext_vector_type(8)));
typedef int v4i32r __attribute__((ext_vector_type(4)));
typedef float v4f32r __attribute__((ext_vector_type(4)));

constexpr int kR32Consumers = 4;
// RB row blocks of 16 activation rows: one producer for the weights, bsums and
// d_a and one per row block for the codes
template <int RB>
constexpr int r32_threads() { return 64 * (kR32Consumers + 1 + RB); }

// Geometry for COLS columns per workgroup (16 or 32): a stage holds SB =
// 64 / COLS super-blocks, so its headers are one 64-lane load.
template <int COLS, int RB>
struct R32 {
    static_assert(COLS == 16 || COLS == 32, "16 or 32 columns per workgroup");
    static_assert(RB == 1 || RB == 2, "16 or 32 activation rows");
    static constexpr int SB = 64 / COLS;      // super-blocks per stage
    static constexpr int RPB = 32 / SB;       // rows per bsums load (8 or 16)
    static constexpr int RPD = 64 / SB;       // rows per d_a load (16 or 32)
    static constexpr int NBS = 16 * RB / RPB;               // bsums loads
    static constexpr int NDA = (16 * RB + RPD - 1) / RPD;   // d_a loads
    static constexpr int HDR = 0, PAY = 1024, ACT = PAY + 8192, BSM = ACT + 4096 * SB * RB, DA = BSM + 1024 * NBS;
    static constexpr int STAGE = DA + 256 * NDA;
    static constexpr int L0 = 1 + 8 + NBS + NDA;  // producer 0: header, payloads, bsums, d_a
    static constexpr int L1 = 4 * SB;             // producers 1 (and 2): codes of 16 rows
};
template <int COLS, int D, int RB>
struct R32Ring {
    using G = R32<COLS, RB>;
    static_assert(D >= 1 && D * G::L0 <= 63 && D * G::L1 <= 63, "the wait counter holds 63 loads");
    static constexpr int R = D + 1;  // slots: D in flight, one being contracted
    static constexpr int BYTES = R * G::STAGE;
    static_assert(BYTES <= 160 * 1024, "LDS budget of a gfx950 CU");
};

template <int N>
__device__ __forceinline__ void r32_wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// wait until at most n * L loads are outstanding (0 <= n, wave-uniform)
template <int L, int D>
__device__ __forceinline__ void r32_wait_stages(int n) {
    if constexpr (D >= 0) {
        if (n >= D) {
            r32_wait_vmcnt<D * L>();
            return;
        }
        r32_wait_stages<L, D - 1>(n);
    }
}
// a workgroup barrier that the compiler does not move memory operations across
__device__ __forceinline__ void r32_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
__device__ __forceinline__ void r32_dma4(rsrc_t r, uint32_t voff, uint32_t soff, uint8_t *lds_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds_base, 4, voff, soff, 0, 0);
}

template <int COLS, int D, int RB>
__global__ __launch_bounds__(r32_threads<RB>(), 1) void k_skinny32r_q4_K(const uint8_t *__restrict__ W,
                                                                  const uint8_t *__restrict__ Y,
                                                                  float *__restrict__ out, int64_t M,
                                                                  int64_t N, int64_t K) {
    using RS = R32Ring<COLS, D, RB>;
    using G = R32<COLS, RB>;
    constexpr int kRows = 16 * RB, kThreads = r32_threads<RB>();
    constexpr int SB = G::SB;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int Mc = (int)M;  // 1 <= M <= 16 RB
    const int nb = (int)(K / QK_K), nst = (nb + SB - 1) / SB;
    const int64_t n_base = (int64_t)blockIdx.x * COLS;

    if (wave >= kR32Consumers) {
        // ---------------- producers
        const int p = wave - kR32Consumers;
        const int64_t w_bytes = N * (int64_t)nb * kQ4_KBytes, y_bytes = (int64_t)Mc * nb * kQ8_KBytes;
        const int64_t col = n_base + (lane % COLS) < N ? n_base + (lane % COLS) : N - 1;
        const uint32_t rowb = (uint32_t)(nb * kQ8_KBytes);
        const int g = lane / COLS;  // the super-block of a stage this lane's header comes from
        auto clamp_b = [&](int b) { return b < nb ? b : nb - 1; };
        auto clamp_r = [&](int r) { return r < Mc ? r : Mc - 1; };
        auto issue = [&](int S) {
            uint8_t *base = lds + (S % RS::R) * G::STAGE;
            const rsrc_t ra = make_rsrc(Y, y_bytes);
            if (p == 0) {
                const rsrc_t rw = make_rsrc(W, w_bytes);
                dma16(rw, (uint32_t)(16 * (col * nb + clamp_b(SB * S + g))), 0, base + G::HDR);
                constexpr int KC = COLS / 8;  // payload loads per super-block
#pragma unroll
                for (int k = 0; k < 8; ++k) {  // super-block k / KC, columns 8 (k % KC) .. + 7
                    const int cc = 8 * (k % KC) + (lane >> 3);
                    const int64_t ck = n_base + cc < N ? n_base + cc : N - 1;
                    const int pc = (lane & 7) ^ (cc & 7);  // the piece stored at position lane
                    dma16(rw, (uint32_t)(16 * N * nb + 128 * (ck * nb + clamp_b(SB * S + k / KC)) + 16 * pc), 0,
                          base + G::PAY + 1024 * k);
                }
#pragma unroll
                for (int j = 0; j < G::NBS; ++j) {  // bsums of rows RPB j .. + RPB - 1
                    const int gb = lane / (2 * G::RPB);
                    const int rr = clamp_r(G::RPB * j + ((lane >> 1) % G::RPB));
                    dma16(ra, (uint32_t)rr * rowb + (uint32_t)clamp_b(SB * S + gb) * kQ8_KBytes + 260 + 16 * (lane & 1),
                          0, base + G::BSM + 1024 * j);
                }
#pragma unroll
                for (int j = 0; j < G::NDA; ++j) {  // d_a of rows RPD j .. + RPD - 1
                    const int gd = lane / G::RPD;
                    const int rr = clamp_r(G::RPD * j + lane % G::RPD);
                    r32_dma4(ra, (uint32_t)rr * rowb + (uint32_t)clamp_b(SB * S + gd) * kQ8_KBytes, 0,
                             base + G::DA + 256 * j);
                }
            } else {
#pragma unroll
                for (int bb = 0; bb < SB; ++bb) {
                    const uint32_t sb = (uint32_t)clamp_b(SB * S + bb) * kQ8_KBytes;
#pragma unroll
                    for (int gg = 0; gg < 4; ++gg) {
                        const int rg = 4 * (p - 1) + gg;  // row group: rows 4 rg .. 4 rg + 3
                        const int r = 4 * rg + (lane >> 4);
                        const int q = (lane & 15) ^ (r & 15);  // the code piece stored at position lane % 16
                        dma16(ra, (uint32_t)clamp_r(r) * rowb + sb + 4 + 16 * q, 0,
                              base + G::ACT + 1024 * SB * rg + 1024 * bb);
                    }
                }
            }
        };
        const int first = nst < D ? nst : D;
        for (int S = 0; S < first; ++S) issue(S);
        for (int S = 0; S < nst; ++S) {
            // stage S has landed once no more than the later stages' loads are outstanding
            const int later = nst - 1 - S < D - 1 ? nst - 1 - S : D - 1;
            if (p == 0)
                r32_wait_stages<G::L0, D - 1>(later);
            else
                r32_wait_stages<G::L1, D - 1>(later);
            r32_barrier();
            // into the slot of stage S - 1, which every consumer finished before this barrier
            if (S + D < nst) issue(S + D);
        }
        r32_barrier();  // the consumers' final barrier
    } else {
        // ---------------- consumer c: super-block SB S + c % SB of every stage S, columns 16 (c / SB) .. + 15
        const int c = wave, gsb = c % SB, l16 = lane & 15, h = lane >> 4;
        const int cl = 16 * (c / SB) + l16;  // this lane's column of the workgroup's COLS
        v4f32r acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};  // row blocks 0, 1
        for (int S = 0; S < nst; ++S) {
            r32_barrier();
            if (SB * S + gsb < nb) {  // wavefront-uniform
                const uint8_t *base = lds + (S % RS::R) * G::STAGE;
                const uint4 hd = *reinterpret_cast<const uint4 *>(base + G::HDR + 16 * (COLS * gsb + cl));
                const int pb = G::PAY + 16 * (8 * COLS * gsb + 8 * cl);
                const uint4 p0 = *reinterpret_cast<const uint4 *>(base + pb + 16 * ((2 * h) ^ (l16 & 7)));
                const uint4 p1 = *reinterpret_cast<const uint4 *>(base + pb + 16 * ((2 * h + 1) ^ (l16 & 7)));
                // rows l16 (block 0) and 16 + l16 (block 1)
                uint32_t aw[RB][16];
                uint4 bsr[RB];
                float dv[RB][4];
#pragma unroll
                for (int blk = 0; blk < RB; ++blk) {
                    const int rr = 16 * blk + l16;
                    const uint8_t *arow = base + G::ACT + 1024 * SB * (rr >> 2) + 1024 * gsb + 256 * (rr & 3);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint4 v = *reinterpret_cast<const uint4 *>(arow + 16 * ((4 * h + i) ^ l16));
                        aw[blk][4 * i] = v.x;
                        aw[blk][4 * i + 1] = v.y;
                        aw[blk][4 * i + 2] = v.z;
                        aw[blk][4 * i + 3] = v.w;
                    }
                    bsr[blk] = *reinterpret_cast<const uint4 *>(base + G::BSM + 1024 * (rr / G::RPB) +
                                                                16 * (2 * G::RPB * gsb + 2 * (rr % G::RPB) + (h & 1)));
                    const int rd = 16 * blk + 4 * h;  // d_a of rows rd .. rd + 3
                    const float4 d4 = *reinterpret_cast<const float4 *>(base + G::DA + 256 * (rd / G::RPD) +
                                                                        4 * (G::RPD * gsb + rd % G::RPD));
                    dv[blk][0] = d4.x;  // d_a of rows 16 blk + 4h .. + 3
                    dv[blk][1] = d4.y;
                    dv[blk][2] = d4.z;
                    dv[blk][3] = d4.w;
                }
                const uint32_t pw[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
                const float dcol = f16_bits_to_f32(hd.x & 0xffff);
                const float dmcol = f16_bits_to_f32(hd.x >> 16);
                const Q4KScales sc = unpack_scales(hd.y, hd.z, hd.w);
                // this lane's sub-blocks 2h (low nibbles) and 2h + 1 (high nibbles)
                const uint32_t sw = h < 2 ? sc.s_lo : sc.s_hi;
                const uint32_t sa = (sw >> (16 * (h & 1))) & 0xff, sb = (sw >> (16 * (h & 1) + 8)) & 0xff;
                const uint32_t ha = (sa >> 3) * 0x00010001u, la = (sa & 7) * 0x00010001u;
                const uint32_t hb = (sb >> 3) * 0x00010001u, lb = (sb & 7) * 0x00010001u;
                const v4i32r zero = {0, 0, 0, 0};
                v4i32r ah0 = zero, al0 = zero, ah1 = zero, al1 = zero;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const uint32_t w0 = pw[2 * t], w1 = pw[2 * t + 1];
                    const uint32_t q0 = w0 & 0x0f0f0f0fu, q1 = w1 & 0x0f0f0f0fu;
                    const uint32_t q2 = (w0 >> 4) & 0x0f0f0f0fu, q3 = (w1 >> 4) & 0x0f0f0f0fu;
                    const v4i32r bh = {plane(q0, ha), plane(q1, ha), plane(q2, hb), plane(q3, hb)};
                    const v4i32r bl = {plane(q0, la), plane(q1, la), plane(q2, lb), plane(q3, lb)};
                    const v4i32r a0 = {(int)aw[0][2 * t], (int)aw[0][2 * t + 1], (int)aw[0][8 + 2 * t],
                                       (int)aw[0][9 + 2 * t]};
                    ah0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, bh, ah0, 0, 0, 0);
                    al0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, bl, al0, 0, 0, 0);
                    if constexpr (RB == 2) {
                        const v4i32r a1 = {(int)aw[RB - 1][2 * t], (int)aw[RB - 1][2 * t + 1],
                                           (int)aw[RB - 1][8 + 2 * t], (int)aw[RB - 1][9 + 2 * t]};
                        ah1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, bh, ah1, 0, 0, 0);
                        al1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, bl, al1, 0, 0, 0);
                    }
                }
                // min term: bsums 8 (h & 1) .. + 7 of the row against the hi (h < 2)
                // or lo part of -dmin * m_j of sub-blocks 4 (h & 1) .. + 3
                v8h32r b_m;
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
                const v4f32r zf = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int blk = 0; blk < RB; ++blk) {
                    v8h32r a_bs;
                    {
                        const uint4 bv = bsr[blk];
                        const uint4 hv = make_uint4(h2_bits((int16_t)(bv.x & 0xffff), (int16_t)(bv.x >> 16)),
                                                    h2_bits((int16_t)(bv.y & 0xffff), (int16_t)(bv.y >> 16)),
                                                    h2_bits((int16_t)(bv.z & 0xffff), (int16_t)(bv.z >> 16)),
                                                    h2_bits((int16_t)(bv.w & 0xffff), (int16_t)(bv.w >> 16)));
                        __builtin_memcpy(&a_bs, &hv, 16);
                    }
                    const v4f32r mn = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_bs, b_m, zf, 0, 0, 0);
                    const v4i32r &ah = blk == 0 ? ah0 : ah1;
                    const v4i32r &al = blk == 0 ? al0 : al1;
                    v4f32r &acc = blk == 0 ? acc0 : acc1;
                    // epilogue: acc += d_a * (d * S - dmin * Mn) for rows 16 blk + 4h .. + 3
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int Sv = (ah[r] << 3) + al[r];
                        const float u = fmaf(dcol, (float)Sv, mn[r]);
                        acc[r] = fmaf(dv[blk][r], u, acc[r]);
                    }
                }
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this slot's reads are done
        }
        r32_barrier();  // every consumer is done with the ring: its start takes the partial tiles
        float *red = reinterpret_cast<float *>(lds);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            red[((c * RB + 0) * 4 + r) * 64 + lane] = acc0[r];
            if constexpr (RB == 2) red[((c * RB + 1) * 4 + r) * 64 + lane] = acc1[r];
        }
    }
    __syncthreads();
    // output (m, col): column group cg = col / 16, block m / 16, register m % 4 of
    // lane col % 16 + 16 ((m % 16) / 4) of consumers SB cg .. SB cg + SB - 1
    const float *red = reinterpret_cast<const float *>(lds);
    for (int o = tid; o < kRows * COLS; o += kThreads) {
        const int m = o / COLS, col = o % COLS;
        const int cg = col >> 4, blk = m >> 4, mm = m & 15;
        const int r = mm & 3, l = (col & 15) + 16 * (mm >> 2);
        auto at = [&](int cons) { return red[((cons * RB + blk) * 4 + r) * 64 + l]; };
        float v = at(SB * cg);
#pragma unroll
        for (int k = 1; k < SB; ++k) v += at(SB * cg + k);
        if (m < Mc && n_base + col < N) out[(int64_t)m * N + n_base + col] = v;
    }
}

template <int COLS, int D, int RB>
hipError_t launch_r32(const uint8_t *w, const uint8_t *y, float *out, int64_t M, int64_t N, int64_t K,
                      hipStream_t s) {
    static std::atomic<uint64_t> lds_set{0};  // the LDS budget above 64 KiB, per device
    const int bytes = R32Ring<COLS, D, RB>::BYTES;
    if (bytes > 64 * 1024) {
        const hipError_t e = ensure_lds_bytes((const void *)k_skinny32r_q4_K<COLS, D, RB>, bytes, lds_set);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((k_skinny32r_q4_K<COLS, D, RB>), dim3((unsigned)((N + COLS - 1) / COLS)),
                       dim3(r32_threads<RB>()), (unsigned)bytes, s, w, y, out, M, N, K);
    return hipGetLastError();
}

template <int RB>
hipError_t launch_rb(const uint8_t *w, const uint8_t *y, float *out, int64_t M, int64_t N, int64_t K,
                     hipStream_t s) {
    // 32 columns per workgroup once every CU gets one, and one stage in flight
    // once the grid gives two workgroups per CU (their rings share the LDS)
    const int64_t cus = cu_count();
#ifdef R32_COLS
    return launch_r32<R32_COLS, R32_DEPTH, RB>(w, y, out, M, N, K, s);
#endif
    if (N < 32 * cus) return launch_r32<16, 2, RB>(w, y, out, M, N, K, s);
    return (N + 31) / 32 >= 2 * cus ? launch_r32<32, 1, RB>(w, y, out, M, N, K, s)
                                    : launch_r32<32, 2, RB>(w, y, out, M, N, K, s);
}

}  // namespace

hipError_t launch_skinny32r_q4_K(const uint8_t *w, const uint8_t *y, float *out, int64_t M, int64_t N,
                                 int64_t K, hipStream_t s) {
    if (M < 1 || M > 32) return hipErrorInvalidValue;
    return M <= 16 ? launch_rb<1>(w, y, out, M, N, K, s) : launch_rb<2>(w, y, out, M, N, K, s);
}

}  // namespace qmm
