// gemm.hip -- compute-bound quantized GEMM (prefill-sized M) on int8 MFMA, gfx950.
//
// Long prefill is bound by matrix-core throughput (BitBLAS page, "调度与自动调优"
// shape table; "性能判断" roofline), so the weight tile is decoded once per
// workgroup step and contracted on v_mfma_i32_32x32x32_i8, whose K of 32 is one
// Q4_K sub-block.  Block scales are applied outside the integer sum (ggml-cpu
// mul_mat page, "正确性:缩放系数可以提到求和号外面"):
//   per sub-block j :  P_j  = sum_{k in j} q_k * y_k              (int8 MFMA, C = 0)
//                      S   += s_j * P_j                            (24-bit integer MAD)
//   per super-block :  Mn   = sum_g m_{g/2} * bsums[g]             (fp16 MFMA, exact:
//                            |bsums| <= 2032 and m <= 63 are exact fp16, the
//                            sum < 2^24 is exact fp32)
//                      acc += d_a * (d * S - dmin * Mn)            (fp32)
//
// Workgroup: 256 threads (4 wavefronts, 2 x 2), tile 128 (M) x 128 (N), one
// 256-element super-block per K step staged through LDS:
//   sA  int8 codes      [128][256 + 16]  (row stride 272 B: conflict-free b128 reads)
//   sB  Q4_K block      [128][144]       (header + payload, stride 144 B: conflict-free)
//   sBs bsums as fp16   [128][16 + 8]    (stride 48 B)
//   sDa d_a             [128]
// Each wavefront owns a 64 x 64 output tile = 2 x 2 MFMA tiles of 32 x 32.
//
// MFMA operand convention (v_mfma_*_32x32xK): lane l supplies row (A) or
// column (B) l % 32 and the K-slice selected by l / 32; both operands use the
// same slice assignment, so the sum over a sub-block is complete whatever the
// hardware order inside the slice.  Result register r of lane l holds
// row 8*(r/4) + 4*(l/32) + r%4, column l % 32.
#include "qmm_device.h"
#include "qmm_launch.h"

namespace qmm {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int BM = 128, BN = 128;
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

template <bool REPACKED>
__global__ __launch_bounds__(256, 1) void k_gemm_q4_K(const uint8_t *__restrict__ W,
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
    const int wm = wave >> 1, wn = wave & 1;

    // XCD-aware tile order: workgroups are dealt round-robin to the 8 XCDs;
    // give each XCD a contiguous range of tiles (M-tile fastest) so tiles that
    // share weight columns run on the same L2.
    const int nwg = tiles_m * tiles_n;
    const int bid = blockIdx.x;
    const int v = (nwg % 8 == 0) ? (bid % 8) * (nwg / 8) + bid / 8 : bid;
    const int tile_m = v % tiles_m, tile_n = v / tiles_m;
    const int64_t m_base = (int64_t)tile_m * BM, n_base = (int64_t)tile_n * BN;
    const int64_t nb = K / QK_K;

    float acc[2][2][16];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    for (int64_t b = 0; b < nb; ++b) {
        // ---- stage super-block b into LDS
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 8; ++i) {  // activation codes: 2048 pieces of 16 B
            const int piece = tid + 256 * i;
            const int row = piece >> 4, p = piece & 15;
            const int64_t m = m_base + row;
            uint4 val = make_uint4(0, 0, 0, 0);
            if (m < M) val = ld_align4<uint4>(Y + (m * nb + b) * kQ8_KBytes + 4 + 16 * p);
            *reinterpret_cast<uint4 *>(sA + row * SA_STRIDE + 16 * p) = val;
        }
#pragma unroll
        for (int i = 0; i < 5; ++i) {  // weight blocks: 1152 pieces of 16 B
            const int piece = tid + 256 * i;
            if (piece < BN * 9) {
                const int row = piece / 9, p = piece - row * 9;
                const int64_t n = n_base + row;
                uint4 val = make_uint4(0, 0, 0, 0);
                if (n < N) {
                    const uint8_t *src;
                    if (REPACKED)
                        src = p == 0 ? W + 16 * (n * nb + b)
                                     : W + 16 * N * nb + 128 * (n * nb + b) + 16 * (p - 1);
                    else
                        src = W + kQ4_KBytes * (n * nb + b) + 16 * p;
                    val = ld16(src);
                }
                *reinterpret_cast<uint4 *>(sB + row * SB_STRIDE + 16 * p) = val;
            }
        }
        {  // bsums -> fp16 (exact), and d_a
            const int row = tid >> 1, half = tid & 1;
            const int64_t m = m_base + row;
            uint4 hv = make_uint4(0, 0, 0, 0);
            float da = 0.0f;
            if (m < M) {
                const uint8_t *yb = Y + (m * nb + b) * kQ8_KBytes;
                const uint4 raw = ld_align4<uint4>(yb + 260 + 16 * half);
                const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
                uint32_t o4[4];
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    o4[t] = h2_bits((int16_t)(w4[t] & 0xffff), (int16_t)(w4[t] >> 16));
                hv = make_uint4(o4[0], o4[1], o4[2], o4[3]);
                da = ld_align4<float>(yb);
            }
            *reinterpret_cast<uint4 *>(sBs + row * SBS_STRIDE + 16 * half) = hv;
            if (half == 0) sDa[row] = da;
        }
        __syncthreads();

        // ---- per n-tile: this lane's column header (d, dmin, 6-bit scales/mins)
        float dcol[2], dmcol[2];
        Q4KScales scol[2];
        uint4 bmin[2];  // fp16 m_{k/2} for k = 8*hh .. 8*hh+7 (min-term B operand)
#pragma unroll
        for (int jn = 0; jn < 2; ++jn) {
            const int col = wn * 64 + jn * 32 + l32;
            const uint4 hdr = *reinterpret_cast<const uint4 *>(sB + col * SB_STRIDE);
            dcol[jn] = f16_bits_to_f32(hdr.x & 0xffff);
            dmcol[jn] = f16_bits_to_f32(hdr.x >> 16);
            scol[jn] = unpack_scales(hdr.y, hdr.z, hdr.w);
            const uint32_t mw = hh == 0 ? scol[jn].m_lo : scol[jn].m_hi;  // m_{4hh..4hh+3}
            bmin[jn] = make_uint4(h2_bits(mw & 0xff, mw & 0xff), h2_bits((mw >> 8) & 0xff, (mw >> 8) & 0xff),
                                  h2_bits((mw >> 16) & 0xff, (mw >> 16) & 0xff),
                                  h2_bits(mw >> 24, mw >> 24));
        }

        int S[2][2][16];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) S[i][j][r] = 0;

#pragma unroll
        for (int g = 0; g < 4; ++g) {
            v4i blo[2], bhi[2];
            int slo[2], shi[2];
#pragma unroll
            for (int jn = 0; jn < 2; ++jn) {
                const int col = wn * 64 + jn * 32 + l32;
                const uint4 pw =
                    *reinterpret_cast<const uint4 *>(sB + col * SB_STRIDE + 16 + 32 * g + 16 * hh);
                blo[jn] = v4i{(int)(pw.x & 0x0f0f0f0fu), (int)(pw.y & 0x0f0f0f0fu),
                              (int)(pw.z & 0x0f0f0f0fu), (int)(pw.w & 0x0f0f0f0fu)};
                bhi[jn] = v4i{(int)((pw.x >> 4) & 0x0f0f0f0fu), (int)((pw.y >> 4) & 0x0f0f0f0fu),
                              (int)((pw.z >> 4) & 0x0f0f0f0fu), (int)((pw.w >> 4) & 0x0f0f0f0fu)};
                const uint32_t sw = g < 2 ? scol[jn].s_lo : scol[jn].s_hi;
                const int sh = (g & 1) * 16;
                slo[jn] = (sw >> sh) & 0xff;
                shi[jn] = (sw >> (sh + 8)) & 0xff;
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = wm * 64 + i * 32 + l32;
                const uint4 alo = *reinterpret_cast<const uint4 *>(sA + row * SA_STRIDE + 64 * g + 16 * hh);
                const uint4 ahi =
                    *reinterpret_cast<const uint4 *>(sA + row * SA_STRIDE + 64 * g + 32 + 16 * hh);
                const v4i va_lo = v4i{(int)alo.x, (int)alo.y, (int)alo.z, (int)alo.w};
                const v4i va_hi = v4i{(int)ahi.x, (int)ahi.y, (int)ahi.z, (int)ahi.w};
#pragma unroll
                for (int jn = 0; jn < 2; ++jn) {
                    const v16i zero = {};
                    const v16i p0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(va_lo, blo[jn], zero, 0, 0, 0);
                    const v16i p1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(va_hi, bhi[jn], zero, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        S[i][jn][r] += __mul24(slo[jn], p0[r]) + __mul24(shi[jn], p1[r]);
                }
            }
        }

        // ---- min term on fp16 MFMA and the fp32 block-scale epilogue
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int row = wm * 64 + i * 32 + l32;
            const uint4 abs_ = *reinterpret_cast<const uint4 *>(sBs + row * SBS_STRIDE + 16 * hh);
            v8h a_bs;
            __builtin_memcpy(&a_bs, &abs_, 16);
            float dav[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 t = *reinterpret_cast<const float4 *>(sDa + wm * 64 + i * 32 + 8 * q + 4 * hh);
                dav[4 * q + 0] = t.x; dav[4 * q + 1] = t.y; dav[4 * q + 2] = t.z; dav[4 * q + 3] = t.w;
            }
#pragma unroll
            for (int jn = 0; jn < 2; ++jn) {
                v8h b_m;
                __builtin_memcpy(&b_m, &bmin[jn], 16);
                const v16f zf = {};
                const v16f mn = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_bs, b_m, zf, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float t = fmaf(dcol[jn], (float)S[i][jn][r], -dmcol[jn] * mn[r]);
                    acc[i][jn][r] = fmaf(dav[r], t, acc[i][jn][r]);
                }
            }
        }
    }

    // ---- store: register r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jn = 0; jn < 2; ++jn) {
            const int64_t n = n_base + wn * 64 + jn * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = m_base + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
                if (m < M && n < N) out[m * N + n] = acc[i][jn][r];
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
