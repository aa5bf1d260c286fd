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
// Workgroup: 256 threads = 4 wavefronts; tile 128 (M) x 128 (N); wavefront w
// owns columns 32w..32w+31 for all 128 rows (4 MFMA tiles of 32 x 32), so each
// weight column is decoded by exactly one wavefront.  One super-block per K
// step is staged through LDS:
//   sA  int8 codes   [128][256 + 16]  row stride 272 B: conflict-free 16-byte reads
//   sB  Q4_K blocks  [128][144]       header + payload, stride 144 B: conflict-free
//   sBs bsums, fp16  [128][24]        stride 48 B
//   sDa d_a          [128]
//
// MFMA operand convention (v_mfma_*_32x32xK): lane l supplies row (A) or
// column (B) l % 32 and the K-slice selected by l / 32; A and B use the same
// slice assignment, so the sum over a sub-block is complete whatever the
// hardware order inside the slice.  Result register r of lane l holds row
// 8*(r/4) + 4*(l/32) + r%4, column l % 32.
#include "qmm_device.h"
#include "qmm_launch.h"

namespace qmm {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));

constexpr int BM = 128, BN = 128, MT = BM / 32;
constexpr int SA_STRIDE = 272;
constexpr int SB_STRIDE = 144;
constexpr int SBS_STRIDE = 48;
constexpr int SA_BYTES = BM * SA_STRIDE;
constexpr int SB_BYTES = BN * SB_STRIDE;
constexpr int SBS_BYTES = BM * SBS_STRIDE;
constexpr int SDA_BYTES = BM * 4;
constexpr int LDS_BYTES = SA_BYTES + SB_BYTES + SBS_BYTES + SDA_BYTES;

__device__ __forceinline__ uint32_t h2_bits(int lo, int hi) {
    return f32_to_f16_bits((float)lo) | (f32_to_f16_bits((float)hi) << 16);
}

// packed per-byte product of four codes (each <= 15) with a scale digit (<= 7)
__device__ __forceinline__ int plane(uint32_t q4, uint32_t digit_pair) {
    const us2 p = __builtin_bit_cast(us2, q4) * __builtin_bit_cast(us2, digit_pair);
    return (int)__builtin_bit_cast(uint32_t, p);
}

template <bool REPACKED>
__global__ __launch_bounds__(256, 2) void k_gemm_q4_K(const uint8_t *__restrict__ W,
                                                      const uint8_t *__restrict__ Y,
                                                      float *__restrict__ out, int64_t M, int64_t N,
                                                      int64_t K, int tiles_m, int tiles_n) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    uint8_t *sA = lds;
    uint8_t *sB = lds + SA_BYTES;
    uint8_t *sBs = sB + SB_BYTES;
    float *sDa = reinterpret_cast<float *>(sBs + SBS_BYTES);

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hh = lane >> 5;

    // XCD-aware tile order: workgroups are dealt round-robin to the 8 XCDs; give
    // each XCD a contiguous range of tiles (M-tile fastest) so the tiles that
    // share weight columns and activation rows meet in the same L2.
    const int nwg = tiles_m * tiles_n;
    const int bid = blockIdx.x;
    const int v = (nwg % 8 == 0) ? (bid % 8) * (nwg / 8) + bid / 8 : bid;
    const int tile_m = v % tiles_m, tile_n = v / tiles_m;
    const int64_t m_base = (int64_t)tile_m * BM, n_base = (int64_t)tile_n * BN;
    const int64_t nb = K / QK_K;

    // ---- staging sources.  Rows past M and columns past N are clamped to the
    // last valid one (their results are never stored), so no load is predicated.
    // Workgroup bases are uniform; per-thread offsets fit in 32 bits.
    const int m_last = (int)(M - 1 - m_base < BM - 1 ? M - 1 - m_base : BM - 1);
    const int n_last = (int)(N - 1 - n_base < BN - 1 ? N - 1 - n_base : BN - 1);
    const uint32_t a_rowstride = (uint32_t)(nb * kQ8_KBytes);
    const uint8_t *a_base = Y + m_base * nb * kQ8_KBytes;
    // activation codes: rows (tid>>4) + 16 i, 16-byte piece tid & 15
    const int a_p = tid & 15, a_r0 = tid >> 4;
    uint32_t a_off[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = a_r0 + 16 * i < m_last ? a_r0 + 16 * i : m_last;
        a_off[i] = (uint32_t)r * a_rowstride + 4 + 16 * a_p;
    }
    // weights: headers by threads 0..127, payload pieces (tid>>3) + 32 i, piece tid & 7
    const uint32_t hdr_step = REPACKED ? 16 : kQ4_KBytes, pay_step = REPACKED ? 128 : kQ4_KBytes;
    const uint8_t *h_base = W + (REPACKED ? 16 : kQ4_KBytes) * (n_base * nb);
    const uint8_t *p_base = REPACKED ? W + 16 * N * nb + 128 * (n_base * nb)
                                     : W + kQ4_KBytes * (n_base * nb) + 16;
    const int h_row = tid < BN ? (tid < n_last ? tid : n_last) : 0;
    const uint32_t h_off = (uint32_t)h_row * (uint32_t)nb * hdr_step;
    const int p_c = tid & 7, p_r0 = tid >> 3;
    uint32_t p_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = p_r0 + 32 * i < n_last ? p_r0 + 32 * i : n_last;
        p_off[i] = (uint32_t)r * (uint32_t)nb * pay_step + 16 * p_c;
    }
    // bsums and d_a: row tid>>1, half tid&1
    const int s_row = tid >> 1, s_half = tid & 1;
    const uint32_t s_off = (uint32_t)(s_row < m_last ? s_row : m_last) * a_rowstride;

    float acc[MT][16];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;

    const int col = wave * 32 + l32;  // this lane's column within the tile

    for (int64_t b = 0; b < nb; ++b) {
        // ---------------- stage super-block b
        __syncthreads();
        {
            const uint8_t *ab = a_base + b * kQ8_KBytes;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint4 val = ld_align4<uint4>(ab + a_off[i]);
                *reinterpret_cast<uint4 *>(sA + (a_r0 + 16 * i) * SA_STRIDE + 16 * a_p) = val;
            }
            const uint8_t *pb = p_base + b * pay_step;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint4 val = ld16(pb + p_off[i]);
                *reinterpret_cast<uint4 *>(sB + (p_r0 + 32 * i) * SB_STRIDE + 16 + 16 * p_c) = val;
            }
            if (tid < BN) {
                const uint4 val = ld16(h_base + b * hdr_step + h_off);
                *reinterpret_cast<uint4 *>(sB + tid * SB_STRIDE) = val;
            }
            const uint8_t *yb = ab + s_off;  // block start of this row
            const uint4 raw = ld_align4<uint4>(yb + 260 + 16 * s_half);
            const uint4 hv = make_uint4(h2_bits((int16_t)(raw.x & 0xffff), (int16_t)(raw.x >> 16)),
                                        h2_bits((int16_t)(raw.y & 0xffff), (int16_t)(raw.y >> 16)),
                                        h2_bits((int16_t)(raw.z & 0xffff), (int16_t)(raw.z >> 16)),
                                        h2_bits((int16_t)(raw.w & 0xffff), (int16_t)(raw.w >> 16)));
            *reinterpret_cast<uint4 *>(sBs + s_row * SBS_STRIDE + 16 * s_half) = hv;
            if (s_half == 0) sDa[s_row] = ld_align4<float>(yb);
        }
        __syncthreads();

        // ---------------- this lane's column: header
        const uint4 hdr = *reinterpret_cast<const uint4 *>(sB + col * SB_STRIDE);
        const float dcol = f16_bits_to_f32(hdr.x & 0xffff);
        const float dmcol = f16_bits_to_f32(hdr.x >> 16);
        const Q4KScales sc = unpack_scales(hdr.y, hdr.z, hdr.w);

        v16i acc_hi[MT], acc_lo[MT];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const uint4 pw = *reinterpret_cast<const uint4 *>(sB + col * SB_STRIDE + 16 + 32 * g + 16 * hh);
            const uint32_t sw = g < 2 ? sc.s_lo : sc.s_hi;
#pragma unroll
            for (int t = 0; t < 2; ++t) {  // t = 0: low nibbles (sub-block 2g), 1: high (2g+1)
                const int j = 2 * g + t;
                const int shift = t * 4;
                const uint32_t q0 = (pw.x >> shift) & 0x0f0f0f0fu, q1 = (pw.y >> shift) & 0x0f0f0f0fu;
                const uint32_t q2 = (pw.z >> shift) & 0x0f0f0f0fu, q3 = (pw.w >> shift) & 0x0f0f0f0fu;
                const uint32_t s = (sw >> (8 * (j & 3))) & 0xff;
                const uint32_t hi2 = (s >> 3) * 0x00010001u, lo2 = (s & 7) * 0x00010001u;
                const v4i bhi = v4i{plane(q0, hi2), plane(q1, hi2), plane(q2, hi2), plane(q3, hi2)};
                const v4i blo = v4i{plane(q0, lo2), plane(q1, lo2), plane(q2, lo2), plane(q3, lo2)};
#pragma unroll
                for (int i = 0; i < MT; ++i) {
                    const uint4 a = *reinterpret_cast<const uint4 *>(sA + (i * 32 + l32) * SA_STRIDE + 32 * j + 16 * hh);
                    const v4i va = v4i{(int)a.x, (int)a.y, (int)a.z, (int)a.w};
                    if (j == 0) {
                        const v16i zero = {};
                        acc_hi[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(va, bhi, zero, 0, 0, 0);
                        acc_lo[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(va, blo, zero, 0, 0, 0);
                    } else {
                        acc_hi[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(va, bhi, acc_hi[i], 0, 0, 0);
                        acc_lo[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(va, blo, acc_lo[i], 0, 0, 0);
                    }
                }
            }
        }

        // ---------------- min term and the fp32 block-scale epilogue.
        // -dmin*m_j has at most 17 significant bits: it is the exact sum of two
        // fp16 values (hi = fp16(-dmin*m), lo = remainder), so two fp16 MFMAs
        // against the exact fp16 bsums give -dmin*Mn with fp32 rounding only.
        const uint32_t mw = hh == 0 ? sc.m_lo : sc.m_hi;  // m_{4hh .. 4hh+3}
        uint32_t bh[4], bl[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float v = -dmcol * (float)((mw >> (8 * e)) & 0xff);  // exact in fp32
            const uint32_t hb = f32_to_f16_bits(v);
            const uint32_t lb = f32_to_f16_bits(v - f16_bits_to_f32(hb));
            bh[e] = hb | (hb << 16);
            bl[e] = lb | (lb << 16);
        }
        v8h bmh, bml;
        __builtin_memcpy(&bmh, bh, 16);
        __builtin_memcpy(&bml, bl, 16);
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            const uint4 au = *reinterpret_cast<const uint4 *>(sBs + (i * 32 + l32) * SBS_STRIDE + 16 * hh);
            v8h abs_;
            __builtin_memcpy(&abs_, &au, 16);
            const v16f zf = {};
            v16f mn = __builtin_amdgcn_mfma_f32_32x32x16_f16(abs_, bmh, zf, 0, 0, 0);
            mn = __builtin_amdgcn_mfma_f32_32x32x16_f16(abs_, bml, mn, 0, 0, 0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 da4 = *reinterpret_cast<const float4 *>(sDa + i * 32 + 8 * q + 4 * hh);
                const float dav[4] = {da4.x, da4.y, da4.z, da4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * q + e;
                    const int S = (acc_hi[i][r] << 3) + acc_lo[i][r];
                    const float t = fmaf(dcol, (float)S, mn[r]);
                    acc[i][r] = fmaf(dav[e], t, acc[i][r]);
                }
            }
        }
    }

    // ---- store: register r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32
    const int64_t n = n_base + col;
    if (n < N) {
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = m_base + i * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
                if (m < M) out[m * N + n] = acc[i][r];
            }
    }
}

}  // namespace

hipError_t launch_gemm_q4_K(const uint8_t *w, bool repacked, const uint8_t *y, float *out,
                            int64_t M, int64_t N, int64_t K, hipStream_t s) {
    const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
    const dim3 grid((unsigned)(tiles_m * tiles_n));
    if (repacked)
        hipLaunchKernelGGL(k_gemm_q4_K<true>, grid, dim3(256), LDS_BYTES, s, w, y, out, M, N, K,
                           tiles_m, tiles_n);
    else
        hipLaunchKernelGGL(k_gemm_q4_K<false>, grid, dim3(256), LDS_BYTES, s, w, y, out, M, N, K,
                           tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace qmm
