// probe.hip -- calibration kernels for the roofline figures (libqmm_probe.so,
// declared in include/qmm_probe.h).  They compute nothing of the method; they
// measure what one kernel on this part can do, so that a kernel's rate can be
// read against a floor measured on the same box as well as against the spec
// (BitBLAS page, "6. 用 profiler 验证瓶颈": confirm the bound with a
// measurement, not with the datasheet alone).
//
//   k_probe_read   streams a buffer once with 16-byte loads, every load of a
//                  thread issued before any is used, and stores nothing unless
//                  the XOR of everything it read hits a fixed 128-bit value
//                  (it never does for the zero-filled buffers the benchmark
//                  passes; the branch keeps the loads alive).
//   k_probe_mfma   four independent chains of v_mfma_i32_32x32x32_i8 per
//                  wavefront, 8 wavefronts per SIMD; each thread writes one
//                  int of the chains' final state, so nothing is dead code.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qmm_probe.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kReadThreads = 256;

template <int LOADS>
__global__ __launch_bounds__(kReadThreads) void k_probe_read(const uint4 *__restrict__ p, int64_t n16,
                                                             uint32_t *__restrict__ sink) {
    const int64_t base = (int64_t)blockIdx.x * (kReadThreads * LOADS) + threadIdx.x;
    uint4 v[LOADS];
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        const int64_t i = base + (int64_t)j * kReadThreads;
        v[j] = i < n16 ? p[i] : make_uint4(0, 0, 0, 0);
    }
    uint4 x = v[0];
#pragma unroll
    for (int j = 1; j < LOADS; ++j) {
        x.x ^= v[j].x;
        x.y ^= v[j].y;
        x.z ^= v[j].z;
        x.w ^= v[j].w;
    }
    if (x.x == 0x9e3779b9u && x.y == 0x7f4a7c15u && x.z == 0x85ebca6bu && x.w == 0xc2b2ae35u)
        sink[0] = x.x ^ x.y ^ x.z ^ x.w;
}

constexpr int kMfmaThreads = 256;
constexpr int kMfmaBlocksPerCu = 8;      // 32 wavefronts per CU, 8 per SIMD
constexpr int kCus = 256;
constexpr int kMfmaBlocks = kCus * kMfmaBlocksPerCu;

__global__ __launch_bounds__(kMfmaThreads) void k_probe_mfma(int *__restrict__ out, int iters, int seed) {
    const int lane = threadIdx.x & 63;
    const v4i a = {lane + seed, lane * 3, lane ^ 5, 7};
    const v4i b = {lane, seed, 1, lane * 2};
    v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, b, c3, 0, 0, 0);
    }
    int s = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c0[r] ^ c1[r] ^ c2[r] ^ c3[r];
    out[(int64_t)blockIdx.x * kMfmaThreads + threadIdx.x] = s;
}

}  // namespace

extern "C" {

int qmm_probe_read(const void *buf, size_t bytes, int loads_per_thread, void *sink16, void *stream) {
    if (!buf || !sink16 || bytes == 0 || bytes % 16 != 0) return 1;
    if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0 || (reinterpret_cast<uintptr_t>(sink16) & 15u) != 0)
        return 1;
    const int64_t n16 = (int64_t)(bytes / 16);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint4 *p = static_cast<const uint4 *>(buf);
    uint32_t *sink = static_cast<uint32_t *>(sink16);
    auto grid = [&](int loads) { return dim3((unsigned)((n16 + kReadThreads * loads - 1) / (kReadThreads * loads))); };
    switch (loads_per_thread) {
        case 1: hipLaunchKernelGGL(k_probe_read<1>, grid(1), dim3(kReadThreads), 0, s, p, n16, sink); break;
        case 2: hipLaunchKernelGGL(k_probe_read<2>, grid(2), dim3(kReadThreads), 0, s, p, n16, sink); break;
        case 4: hipLaunchKernelGGL(k_probe_read<4>, grid(4), dim3(kReadThreads), 0, s, p, n16, sink); break;
        case 8: hipLaunchKernelGGL(k_probe_read<8>, grid(8), dim3(kReadThreads), 0, s, p, n16, sink); break;
        default: return 1;
    }
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

size_t qmm_probe_mfma_sink_bytes(void) { return (size_t)kMfmaBlocks * kMfmaThreads * sizeof(int); }

double qmm_probe_mfma_ops(int iters) {
    // wavefronts x iterations x 4 chains x 2*32*32*32 int8 operations
    return (double)kMfmaBlocks * (kMfmaThreads / 64) * (double)iters * 4.0 * 2.0 * 32 * 32 * 32;
}

int qmm_probe_mfma_i8(void *sink, size_t sink_bytes, int iters, int seed, void *stream) {
    if (!sink || sink_bytes < qmm_probe_mfma_sink_bytes() || iters < 1) return 1;
    hipLaunchKernelGGL(k_probe_mfma, dim3(kMfmaBlocks), dim3(kMfmaThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<int *>(sink), iters, seed);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
