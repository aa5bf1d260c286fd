// skinny16r.hip -- Q4_K weights (repacked layout) x Q8_K activations for
// batches of up to 8 rows, gfx950: one producer wavefront streams the
// workgroup's 16 weight columns and the batch's activation blocks into an
// LDS ring, four consumer wavefronts contract them on v_mfma_i32_16x16x64_i8.
//
// A small batch reads every weight once, so the weight stream bounds it
// (BitBLAS page, "调度与自动调优": small-M shapes sit on the memory side of the
// roofline).  In skinny16.hip each wavefront both loads and computes: with one
// super-block requested ahead every step waits a full round trip, and a
// wavefront that requests several at once stalls on issuing them (the memory
// pipeline takes requests at the rate it delivers), so the arithmetic on the
// blocks that have landed waits behind the last request.  Here only the
// producer issues loads: direct global->LDS loads (buffer_load ... lds), a
// stage of four super-blocks per load batch, up to D stages requested ahead.
// It waits for the oldest stage (loads complete in issue order) and releases
// it with one workgroup barrier; consumer c then contracts super-block 4S + c
// of stage S (all of its K-slices), so a barrier covers four super-blocks and
// the four SIMDs work on them at once.  The best D is what keeps about three
// to four stages in flight per CU (measured): D = 3 with one workgroup per
// CU, 2 with two, 1 from three on.
//
// Arithmetic, per super-block and output (m, n), as in skinny16.hip (ggml-cpu
// mul_mat page, "正确性:缩放系数可以提到求和号外面" and "min 项与最终归约"):
// S = sum_j s_j P_j on two int8 digit planes of the sub-block scales
// (s = 8 hi + lo), the min term -dmin * sum_j m_j bsums_j on one fp16 MFMA
// (bsums exact in fp16, -dmin m_j the exact sum of two fp16 parts), then
// acc += d_a (d S - dmin Mn).  Operand layout of v_mfma_i32_16x16x64_i8: lane
// l supplies row (A) or column (B) l % 16 and K-values 16 (l / 16) .. + 15;
// result register r of lane l holds row 4 (l / 16) + r, column l % 16.  In
// MFMA t of a super-block, quarter h = l / 16 takes elements 64h + 8t + i (low
// nibbles of payload bytes 32h + 8t + i, sub-block 2h) and 64h + 32 + 8t + i
// (high nibbles, sub-block 2h + 1).  Consumer c accumulates the super-blocks
// c, c + 4, ... -- the same split and order as the four wavefronts of
// skinny16.hip's wide-matrix configuration, so both give identical bits --
// and the four partial tiles are summed through LDS at the end.
//
// Ring slot (16 columns, super-blocks 4S .. 4S + 3, 4*RG activation rows;
// every region a whole number of 64-lane load instructions):
//   HDR  1 KB      header of super-block l / 16, column l % 16 at 16 l
//   PAY  8 KB      super-block b, payload piece p of column c at 16 (128 b + 8 c + (p ^ (c & 7)))
//                  (each load instruction fetches eight whole 128-byte payloads; the
//                  XOR spreads the reads down 8 columns over distinct banks)
//   ACT  4 KB x RG row group g, super-block b, row r: code piece q at
//                  4096 g + 1024 b + 16 (16 (r & 3) + (q ^ r))   (XOR: rows read
//                  down 16 lanes hit distinct banks)
//   BSM  1 KB      super-block b, row r (< 8), bsums half e at 16 (16 b + 2 r + e)
//   DA   256 B     super-block b, row r at 4 (16 b + r)
// Rows past M, columns past N and super-blocks past K load the last valid
// one (every load in bounds, none predicated); their results are dropped.
#include "mfma_common.h"
#include "qmm_device.h"
#include "qmm_launch.h"

namespace qmm {
namespace {

typedef _Float16 v8h16 __attribute__((ext_vector_type(8)));
typedef int v4i16 __attribute__((ext_vector_type(4)));
typedef float v4f16 __attribute__((ext_vector_type(4)));

constexpr int kRingConsumers = 4;
constexpr int kRingThreads = 64 * (kRingConsumers + 1);

template <int RG, int D>
struct Ring {
    static_assert(RG == 1 || RG == 2, "up to 8 activation rows");
    static constexpr int HDR = 0, PAY = 1024, ACT = PAY + 8192, BSM = ACT + 4096 * RG, DA = BSM + 1024;
    static constexpr int STAGE = DA + 256;
    static constexpr int L = 1 + 8 + 4 * RG + 1 + 1;  // load instructions per stage
    static_assert(D >= 1 && D * L <= 63, "the wait counter holds 63 loads");
    static constexpr int R = D + 1;  // slots: D in flight, one being contracted
    static constexpr int BYTES = R * STAGE;
};

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// wait until at most n * L loads are outstanding (0 <= n, wave-uniform)
template <int L, int D>
__device__ __forceinline__ void wait_stages(int n) {
    if constexpr (D >= 0) {
        if (n >= D) {
            wait_vmcnt<D * L>();
            return;
        }
        wait_stages<L, D - 1>(n);
    }
}
// a workgroup barrier that the compiler does not move memory operations across
__device__ __forceinline__ void ring_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
__device__ __forceinline__ void dma4(rsrc_t r, uint32_t voff, uint32_t soff, uint8_t *lds_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds_base, 4, voff, soff, 0, 0);
}

template <int RG, int D>
__global__ __launch_bounds__(kRingThreads, 1) void k_skinny16r_q4_K(const uint8_t *__restrict__ W,
                                                                   const uint8_t *__restrict__ Y,
                                                                   float *__restrict__ out, int64_t M,
                                                                   int64_t N, int64_t K) {
    using RS = Ring<RG, D>;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int Mc = (int)M;  // 1 <= M <= 4 RG
    const int nb = (int)(K / QK_K), nst = (nb + 3) / 4;
    const int64_t n_base = (int64_t)blockIdx.x * 16;

    if (wave == kRingConsumers) {
        // ---------------- producer
        const int64_t w_bytes = N * (int64_t)nb * kQ4_KBytes, y_bytes = (int64_t)Mc * nb * kQ8_KBytes;
        const int64_t col = n_base + (lane & 15) < N ? n_base + (lane & 15) : N - 1;
        const uint32_t rowb = (uint32_t)(nb * kQ8_KBytes);
        const int g = lane >> 4;  // the super-block of a stage this lane's header, bsums and d_a come from
        const int rbs = ((lane >> 1) & 7) < Mc ? ((lane >> 1) & 7) : Mc - 1;
        const int rd = (lane & 15) < Mc ? (lane & 15) : Mc - 1;
        auto clamp_b = [&](int b) { return b < nb ? b : nb - 1; };
        auto issue = [&](int S) {
            uint8_t *base = lds + (S % RS::R) * RS::STAGE;
            const rsrc_t rw = make_rsrc(W, w_bytes);
            const rsrc_t ra = make_rsrc(Y, y_bytes);
            dma16(rw, (uint32_t)(16 * (col * nb + clamp_b(4 * S + g))), 0, base + RS::HDR);
#pragma unroll
            for (int k = 0; k < 8; ++k) {  // super-block k / 2, columns 8 (k % 2) .. + 7
                const int cc = 8 * (k & 1) + (lane >> 3);
                const int64_t ck = n_base + cc < N ? n_base + cc : N - 1;
                const int p = (lane & 7) ^ (cc & 7);  // the piece stored at position lane
                dma16(rw, (uint32_t)(16 * N * nb + 128 * (ck * nb + clamp_b(4 * S + (k >> 1))) + 16 * p), 0,
                      base + RS::PAY + 1024 * k);
            }
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                const uint32_t sb = (uint32_t)clamp_b(4 * S + bb) * kQ8_KBytes;
#pragma unroll
                for (int gg = 0; gg < RG; ++gg) {
                    const int r = 4 * gg + (lane >> 4);
                    const int rr = r < Mc ? r : Mc - 1;
                    const int q = (lane & 15) ^ r;  // the code piece stored at position lane % 16
                    dma16(ra, (uint32_t)rr * rowb + sb + 4 + 16 * q, 0, base + RS::ACT + 4096 * gg + 1024 * bb);
                }
            }
            const uint32_t sg = (uint32_t)clamp_b(4 * S + g) * kQ8_KBytes;
            dma16(ra, (uint32_t)rbs * rowb + sg + 260 + 16 * (lane & 1), 0, base + RS::BSM);
            dma4(ra, (uint32_t)rd * rowb + sg, 0, base + RS::DA);
        };
        const int first = nst < D ? nst : D;
        for (int S = 0; S < first; ++S) issue(S);
        for (int S = 0; S < nst; ++S) {
            // stage S has landed once no more than the later stages' loads are outstanding
            const int later = nst - 1 - S < D - 1 ? nst - 1 - S : D - 1;
            wait_stages<RS::L, D - 1>(later);
            ring_barrier();
            // into the slot of stage S - 1, which every consumer finished before this barrier
            if (S + D < nst) issue(S + D);
        }
    } else {
        // ---------------- consumer c: super-block 4S + c of every stage S
        const int c = wave, l16 = lane & 15, h = lane >> 4;
        const int rr = l16 < 4 * RG ? l16 : 4 * RG - 1;  // staged row this lane reads (rows past M: dropped)
        v4f16 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int S = 0; S < nst; ++S) {
            ring_barrier();
            if (4 * S + c < nb) {  // wavefront-uniform
                const uint8_t *base = lds + (S % RS::R) * RS::STAGE;
                const uint4 hd = *reinterpret_cast<const uint4 *>(base + RS::HDR + 16 * (16 * c + l16));
                const int pb = RS::PAY + 16 * (128 * c + 8 * l16);
                const uint4 p0 = *reinterpret_cast<const uint4 *>(base + pb + 16 * ((2 * h) ^ (l16 & 7)));
                const uint4 p1 = *reinterpret_cast<const uint4 *>(base + pb + 16 * ((2 * h + 1) ^ (l16 & 7)));
                const uint8_t *arow = base + RS::ACT + 4096 * (rr >> 2) + 1024 * c + 256 * (rr & 3);
                uint4 av[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) av[i] = *reinterpret_cast<const uint4 *>(arow + 16 * ((4 * h + i) ^ rr));
                const uint4 bsr = *reinterpret_cast<const uint4 *>(base + RS::BSM + 16 * (16 * c + 2 * rr + (h & 1)));
                const float4 d4 = *reinterpret_cast<const float4 *>(base + RS::DA + 4 * (16 * c + 4 * h));
                const float dv[4] = {d4.x, d4.y, d4.z, d4.w};  // d_a of rows 4h .. 4h + 3

                const uint32_t aw[16] = {av[0].x, av[0].y, av[0].z, av[0].w, av[1].x, av[1].y, av[1].z, av[1].w,
                                         av[2].x, av[2].y, av[2].z, av[2].w, av[3].x, av[3].y, av[3].z, av[3].w};
                const uint32_t pw[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
                const float dcol = f16_bits_to_f32(hd.x & 0xffff);
                const float dmcol = f16_bits_to_f32(hd.x >> 16);
                const Q4KScales sc = unpack_scales(hd.y, hd.z, hd.w);
                // this lane's sub-blocks 2h (low nibbles) and 2h + 1 (high nibbles)
                const uint32_t sw = h < 2 ? sc.s_lo : sc.s_hi;
                const uint32_t sa = (sw >> (16 * (h & 1))) & 0xff, sb = (sw >> (16 * (h & 1) + 8)) & 0xff;
                const uint32_t ha = (sa >> 3) * 0x00010001u, la = (sa & 7) * 0x00010001u;
                const uint32_t hb = (sb >> 3) * 0x00010001u, lb = (sb & 7) * 0x00010001u;
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
                // min term: bsums 8 (h & 1) .. + 7 of the row against the hi (h < 2)
                // or lo part of -dmin * m_j of sub-blocks 4 (h & 1) .. + 3
                v8h16 a_bs;
                {
                    const uint4 hv = make_uint4(h2_bits((int16_t)(bsr.x & 0xffff), (int16_t)(bsr.x >> 16)),
                                                h2_bits((int16_t)(bsr.y & 0xffff), (int16_t)(bsr.y >> 16)),
                                                h2_bits((int16_t)(bsr.z & 0xffff), (int16_t)(bsr.z >> 16)),
                                                h2_bits((int16_t)(bsr.w & 0xffff), (int16_t)(bsr.w >> 16)));
                    __builtin_memcpy(&a_bs, &hv, 16);
                }
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
                    const int Sv = (ah[r] << 3) + al[r];
                    const float u = fmaf(dcol, (float)Sv, mn[r]);
                    acc[r] = fmaf(dv[r], u, acc[r]);
                }
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this slot's reads are done
        }
        ring_barrier();  // every consumer is done with the ring: its start takes the partial tiles
        float *red = reinterpret_cast<float *>(lds);
#pragma unroll
        for (int r = 0; r < 4; ++r) red[(c * 4 + r) * 64 + lane] = acc[r];
    }
    if (wave == kRingConsumers) ring_barrier();  // the producer's side of the barrier above
    __syncthreads();
    // output (m, cc) sits in register m % 4 of lane cc + 16 (m / 4) of every consumer
    const float *red = reinterpret_cast<const float *>(lds);
    for (int o = tid; o < 256; o += kRingThreads) {
        const int m = o >> 4, cc = o & 15;
        const int r = m & 3, l = cc + 16 * (m >> 2);
        const float v = ((red[(0 * 4 + r) * 64 + l] + red[(1 * 4 + r) * 64 + l]) + red[(2 * 4 + r) * 64 + l]) +
                        red[(3 * 4 + r) * 64 + l];
        if (m < Mc && n_base + cc < N) out[(int64_t)m * N + n_base + cc] = v;
    }
}

template <int RG, int D>
hipError_t launch_rd(const uint8_t *w, const uint8_t *y, float *out, int64_t M, int64_t N, int64_t K,
                     hipStream_t s) {
    static std::atomic<uint64_t> lds_set{0};  // the LDS budget above 64 KiB, per device
    const int bytes = Ring<RG, D>::BYTES;
    if (bytes > 64 * 1024) {
        const hipError_t e = ensure_lds_bytes((const void *)k_skinny16r_q4_K<RG, D>, bytes, lds_set);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((k_skinny16r_q4_K<RG, D>), dim3((unsigned)((N + 15) / 16)), dim3(kRingThreads),
                       (unsigned)bytes, s, w, y, out, M, N, K);
    return hipGetLastError();
}

template <int RG>
hipError_t launch_rg(const uint8_t *w, const uint8_t *y, float *out, int64_t M, int64_t N, int64_t K,
                     hipStream_t s) {
    // stages in flight per workgroup from the workgroups each CU holds:
    // measured best with D = 3 / 2 / 1 at one / two / three or more per CU
    const int64_t per_cu = ((N + 15) / 16 + cu_count() - 1) / cu_count();
    if (per_cu <= 1) return launch_rd<RG, 3>(w, y, out, M, N, K, s);
    if (per_cu == 2) return launch_rd<RG, 2>(w, y, out, M, N, K, s);
    return launch_rd<RG, 1>(w, y, out, M, N, K, s);
}

}  // namespace

hipError_t launch_skinny16r_q4_K(const uint8_t *w, const uint8_t *y, float *out, int64_t M, int64_t N,
                                 int64_t K, hipStream_t s) {
    if (M < 1 || M > 8) return hipErrorInvalidValue;
    return M <= 4 ? launch_rg<1>(w, y, out, M, N, K, s) : launch_rg<2>(w, y, out, M, N, K, s);
}

}  // namespace qmm
