// repack.hip -- load-time permutation of canonical weight blocks into the
// GPU layout (BitBLAS page, "Ladder Permutation": static weights are permuted
// once, offline, into the order the kernel consumes; the canonical bytes stay
// the source of truth).
//
//   Q4_K: [N*nb 16-byte headers (d, dmin, scales)] [N*nb 128-byte payloads]
//   Q4_0: [N*nb fp16 scales, zero-padded to 256 B]  [N*nb 16-byte payloads]
//
// The split puts every payload on a 16-byte boundary, so the GEMV reads its
// weight stream with aligned, fully coalesced 16-byte loads.
#include "qmm_device.h"
#include "qmm_launch.h"

namespace qmm {
namespace {

// one thread per 16-byte piece of a Q4_K block (9 pieces: header + 8 payload)
__global__ __launch_bounds__(256) void k_repack_q4_K(const uint8_t *__restrict__ in,
                                                     uint8_t *__restrict__ out, int64_t nblocks) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= nblocks * 9) return;
    const int64_t blk = t / 9;
    const int piece = (int)(t - blk * 9);
    const uint4 v = ld16(in + blk * kQ4_KBytes + 16 * piece);
    uint8_t *dst = piece == 0 ? out + 16 * blk : out + 16 * nblocks + 128 * blk + 16 * (piece - 1);
    *reinterpret_cast<uint4 *>(dst) = v;
}

// one thread per Q4_0 block (18 bytes, 2-byte aligned in the canonical stream)
__global__ __launch_bounds__(256) void k_repack_q4_0(const uint8_t *__restrict__ in,
                                                     uint8_t *__restrict__ out, int64_t nblocks,
                                                     int64_t dsec) {
    const int64_t blk = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (blk < nblocks) {
        const uint16_t *src = reinterpret_cast<const uint16_t *>(in + blk * kQ4_0Bytes);
        reinterpret_cast<uint16_t *>(out)[blk] = src[0];
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = (uint32_t)src[1 + 2 * i] | ((uint32_t)src[2 + 2 * i] << 16);
        *reinterpret_cast<uint4 *>(out + dsec + 16 * blk) = make_uint4(w[0], w[1], w[2], w[3]);
    }
    // zero the padding of the scale section
    const int64_t pad0 = 2 * nblocks;
    for (int64_t i = pad0 + blk; i < dsec; i += (int64_t)gridDim.x * 256) out[i] = 0;
}

}  // namespace

int64_t repacked_bytes_q4_0(int64_t N, int64_t K) {
    const int64_t nblk = N * (K / QK4_0);
    return (2 * nblk + 255) / 256 * 256 + 16 * nblk;
}

hipError_t launch_repack_q4_K(const uint8_t *in, uint8_t *out, int64_t N, int64_t K, hipStream_t s) {
    const int64_t nblocks = N * (K / QK_K);
    const int64_t threads = nblocks * 9;
    hipLaunchKernelGGL(k_repack_q4_K, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, in,
                       out, nblocks);
    return hipGetLastError();
}

hipError_t launch_repack_q4_0(const uint8_t *in, uint8_t *out, int64_t N, int64_t K, hipStream_t s) {
    const int64_t nblocks = N * (K / QK4_0);
    const int64_t dsec = (2 * nblocks + 255) / 256 * 256;
    const int64_t grid = (nblocks + 255) / 256;
    hipLaunchKernelGGL(k_repack_q4_0, dim3((unsigned)(grid > 0 ? grid : 1)), dim3(256), 0, s, in,
                       out, nblocks, dsec);
    return hipGetLastError();
}

}  // namespace qmm
