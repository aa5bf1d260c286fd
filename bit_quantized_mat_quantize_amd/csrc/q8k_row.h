// q8k_row.h -- one Q8_K activation row staged in LDS for the GEMVs whose
// weights use 16-element groups (Q6_K, Q2_K): one Q8_K bsum per group.
//
// LDS layout: qs[K] | d[nb] (padded to 16 B) | bsums[nb][16] | 16-byte trash
// slot.  The row must fit the 64 KiB a workgroup gets by default.
#pragma once

#include "qmm_device.h"

namespace qmm {

__host__ __device__ constexpr int64_t q8k_row_lds_bytes(int64_t K) {
    return K + ((K / QK_K) * 4 + 15) / 16 * 16 + (K / QK_K) * 32 + 16;
}

// Largest K (a multiple of 256) whose staged row fits 60 KiB.
inline int64_t q8k_row_max_k() {
    int64_t k = 0;
    while (q8k_row_lds_bytes(k + QK_K) <= 60 * 1024) k += QK_K;
    return k;
}

struct Q8KRowLds {
    const uint8_t *qs;
    const float *d;
    const int16_t *bsums;
};

// The first part of a row for 256 threads, held in registers between the
// two halves of a staging: with these loads issued ahead of a wavefront's
// weight loads, the wait that precedes the LDS stores covers only them (loads
// complete in issue order), not the weights as well.
struct Q8KRowHead {
    uint4 q;   // code piece tid (16 codes)
    uint4 bs;  // bsums piece tid (8 sums)
    float d;   // d of block tid
};
__device__ __forceinline__ Q8KRowHead load_q8k_row_head(const uint8_t *__restrict__ Yrow, int64_t K) {
    const int64_t nb = K / QK_K;
    const int nq = (int)(K / 16), nbs = (int)(nb * 2);
    const int tid = threadIdx.x;
    const int pc = tid < nq ? tid : nq - 1, qb = tid < nbs ? tid : nbs - 1, qd = tid < nb ? tid : (int)nb - 1;
    Q8KRowHead h;
    h.q = ld_align4<uint4>(Yrow + (pc >> 4) * kQ8_KBytes + 4 + 16 * (pc & 15));
    h.bs = ld_align4<uint4>(Yrow + (qb >> 1) * kQ8_KBytes + 260 + 16 * (qb & 1));
    h.d = ld_align4<float>(Yrow + qd * kQ8_KBytes);
    return h;
}
// Store the head (threads past the row's pieces write the trash slot), stage
// the rest of the row, then barrier.  256 threads.
__device__ __forceinline__ Q8KRowLds commit_q8k_row(const Q8KRowHead &h, const uint8_t *__restrict__ Yrow,
                                                    int64_t K, uint8_t *ys) {
    const int64_t nb = K / QK_K;
    const int nq = (int)(K / 16), nbs = (int)(nb * 2);
    uint8_t *s_qs = ys;
    uint8_t *s_d = ys + K;
    uint8_t *s_bs = ys + K + (nb * 4 + 15) / 16 * 16;
    uint8_t *trash = s_bs + nb * 32;
    const int tid = threadIdx.x;
    *reinterpret_cast<uint4 *>(tid < nq ? s_qs + 16 * tid : trash) = h.q;
    *reinterpret_cast<uint4 *>(tid < nbs ? s_bs + 16 * tid : trash) = h.bs;
    *reinterpret_cast<float *>(tid < nb ? s_d + 4 * tid : trash) = h.d;
    for (int pc = tid + 256; pc < nq; pc += 256)
        *reinterpret_cast<uint4 *>(s_qs + 16 * pc) =
            ld_align4<uint4>(Yrow + (pc >> 4) * kQ8_KBytes + 4 + 16 * (pc & 15));
    for (int q = tid + 256; q < nbs; q += 256)
        *reinterpret_cast<uint4 *>(s_bs + 16 * q) = ld_align4<uint4>(Yrow + (q >> 1) * kQ8_KBytes + 260 + 16 * (q & 1));
    for (int q = tid + 256; q < nb; q += 256)
        *reinterpret_cast<float *>(s_d + 4 * q) = ld_align4<float>(Yrow + q * kQ8_KBytes);
    __syncthreads();
    return Q8KRowLds{s_qs, reinterpret_cast<const float *>(s_d), reinterpret_cast<const int16_t *>(s_bs)};
}

// Stage activation row Yrow into ys with `nthreads` threads (branch-free
// loads, 16 bytes per thread and trip), then barrier.
template <int kThreads>
__device__ __forceinline__ Q8KRowLds stage_q8k_row(const uint8_t *__restrict__ Yrow, int64_t K,
                                                   uint8_t *ys) {
    const int64_t nb = K / QK_K;
    const int nq = (int)(K / 16), nbs = (int)(nb * 2);
    uint8_t *s_qs = ys;
    uint8_t *s_d = ys + K;
    uint8_t *s_bs = ys + K + (nb * 4 + 15) / 16 * 16;
    const int tid = threadIdx.x;
    for (int pc = tid; pc < nq; pc += kThreads)
        *reinterpret_cast<uint4 *>(s_qs + 16 * pc) =
            ld_align4<uint4>(Yrow + (pc >> 4) * kQ8_KBytes + 4 + 16 * (pc & 15));
    for (int q = tid; q < nbs; q += kThreads)
        *reinterpret_cast<uint4 *>(s_bs + 16 * q) =
            ld_align4<uint4>(Yrow + (q >> 1) * kQ8_KBytes + 260 + 16 * (q & 1));
    for (int q = tid; q < nb; q += kThreads)
        *reinterpret_cast<float *>(s_d + 4 * q) = ld_align4<float>(Yrow + q * kQ8_KBytes);
    __syncthreads();
    return Q8KRowLds{s_qs, reinterpret_cast<const float *>(s_d), reinterpret_cast<const int16_t *>(s_bs)};
}

// ---- Fused quantize + GEMV kernels: the fp32 row quantized to Q8_K straight
// into the staged layout above, one 256-value block per wavefront call (four
// consecutive values per lane, the stand-alone quantizer's routine).  A block
// index past the row (b >= nb) is quantized too and stored to the trash slot,
// so the call stays branch-free.
__device__ __forceinline__ void q8k_quantize_block_lds(const float4 v, int b, int64_t K, uint8_t *ys, int lane) {
    const int64_t nb = K / QK_K;
    uint8_t *s_qs = ys;
    uint8_t *s_d = ys + K;
    uint8_t *s_bs = ys + K + (nb * 4 + 15) / 16 * 16;
    uint8_t *trash = s_bs + nb * 32;
    const bool valid = b < nb;
    const Q8KLane r = q8K_quantize_lane(v);
    const uint32_t packed = pack4_i8(r.q[0], r.q[1], r.q[2], r.q[3]);
    *reinterpret_cast<uint32_t *>(valid ? s_qs + b * QK_K + 4 * lane : trash) = packed;
    if ((lane & 3) == 0)
        *reinterpret_cast<int16_t *>(valid ? s_bs + 32 * b + 2 * (lane >> 2) : trash) = (int16_t)r.bsum;
    if (lane == 0) *reinterpret_cast<float *>(valid ? s_d + 4 * b : trash) = r.d;
}
// Copy the staged row to Yq in the Q8_K byte layout (d | 256 codes | 16 bsums
// per block), byte-identical to the stand-alone quantizer; kThreads threads.
template <int kThreads>
__device__ __forceinline__ void q8k_store_row(uint8_t *__restrict__ Yq, const uint8_t *ys, int64_t K) {
    const int64_t nb = K / QK_K;
    const uint8_t *s_qs = ys;
    const float *s_d = reinterpret_cast<const float *>(ys + K);
    const int16_t *s_bs = reinterpret_cast<const int16_t *>(ys + K + (nb * 4 + 15) / 16 * 16);
    for (int i = threadIdx.x; i < nb * (kQ8_KBytes / 4); i += kThreads) {
        const int b = i / (kQ8_KBytes / 4), w = i - b * (kQ8_KBytes / 4);  // dword w of block b
        const uint32_t v = w == 0 ? __float_as_uint(s_d[b])
                         : w <= QK_K / 4 ? *reinterpret_cast<const uint32_t *>(s_qs + b * QK_K + 4 * (w - 1))
                                         : *reinterpret_cast<const uint32_t *>(s_bs + 16 * b + 2 * (w - 1 - QK_K / 4));
        *reinterpret_cast<uint32_t *>(Yq + (int64_t)b * kQ8_KBytes + 4 * w) = v;
    }
}

}  // namespace qmm
