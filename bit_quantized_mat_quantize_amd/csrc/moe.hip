// moe.hip -- expert grouping for mul_mat_id on gfx950.
//
// mul_mat_id is mul_mat with one more level, the grouping by expert id
// (ggml-cpu mul_mat page, "本篇没有覆盖的部分", the list of follow-up topics
// that names the expert-routed matrix product of MoE models).  For prefill-sized batches the (token, slot) pairs routed to
// the same expert become the rows of one GEMM against that expert's matrix,
// so the pairs are sorted by expert on the device (the ids come from a router
// kernel and never visit the host) and cut into row tiles of the GEMM.
//
// One workgroup of 1024 threads: LDS counters per expert (atomic adds), a
// block-wide exclusive scan of the counts and of the per-expert tile counts
// (thread t owns experts 4t..4t+3, so E <= 4096), the tile table, and a
// scatter of the pair indices to their expert's range.  The order of pairs
// inside an expert's range is whatever the atomics give: every output row is
// computed from its own pair alone, so the results do not depend on it.
//
// The grouping tables normally live in a workspace the caller passes.  For
// callers that cannot allocate device memory, the library also keeps one
// grouping area of its own per GPU: the file-scope array `scratch` below
// (kNoAllocScratchBytes, held by each GPU the library runs on until the
// process ends).  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol): noalloc_scratch() looks up its
// device address once per device with hipGetSymbolAddress, with that device
// current, and every use goes through that address.  The grouping kernel
// writes every word the GEMMs read (start, the tile table, the tile count and
// the sorted pairs), so nothing has to be cleared between calls.
#include <mutex>

#include "qmm_device.h"
#include "qmm_launch.h"

namespace qmm {
namespace {

static __device__ __align__(256) int32_t scratch[kNoAllocScratchBytes / sizeof(int32_t)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t *g_scratch_ptr[kMaxDevices] = {};

constexpr int kGroupThreads = 1024;

// inclusive scan of v over the workgroup (Hillis-Steele in LDS); all threads
__device__ __forceinline__ int block_inclusive_scan(int v, int *buf) {
    const int tid = threadIdx.x;
    buf[tid] = v;
    __syncthreads();
    for (int off = 1; off < kGroupThreads; off <<= 1) {
        const int add = tid >= off ? buf[tid - off] : 0;
        __syncthreads();
        buf[tid] += add;
        __syncthreads();
    }
    return buf[tid];
}

__global__ __launch_bounds__(kGroupThreads) void k_moe_group_ids(const int32_t *__restrict__ ids, int64_t P,
                                                                  int E, int bm, MoeGroupLayout L,
                                                                  int32_t *__restrict__ ws,
                                                                  float *__restrict__ out, int64_t N) {
    __shared__ int s_cnt[kMoeMaxExperts];    // counts, then scatter cursors
    __shared__ int s_start[kMoeMaxExperts];  // first sorted slot of each expert
    __shared__ int s_scan[kGroupThreads];
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += kGroupThreads) s_cnt[e] = 0;
    __syncthreads();
    for (int64_t p = tid; p < P; p += kGroupThreads) {
        const int e = ids[p];
        if (e >= 0 && e < E) {
            atomicAdd(&s_cnt[e], 1);
        } else {
            for (int64_t n = 0; n < N; ++n) out[p * N + n] = __builtin_nanf("");
        }
    }
    __syncthreads();

    // exclusive scans of the counts and of the tile counts over experts 4t..4t+3
    int c[4], tl[4], sc = 0, st = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = 4 * tid + j;
        c[j] = e < E ? s_cnt[e] : 0;
        tl[j] = (c[j] + bm - 1) / bm;
        sc += c[j];
        st += tl[j];
    }
    const int base_c = block_inclusive_scan(sc, s_scan) - sc;
    __syncthreads();
    const int base_t = block_inclusive_scan(st, s_scan) - st;
    int32_t *start = ws + L.start, *tile_e = ws + L.tile_e, *tile_r0 = ws + L.tile_r0;
    int rc = base_c, rt = base_t;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = 4 * tid + j;
        if (e < E) {
            s_start[e] = rc;
            start[e] = rc;
            for (int k = 0; k < tl[j]; ++k) {
                tile_e[rt + k] = e;
                tile_r0[rt + k] = rc + k * bm;
            }
        }
        rc += c[j];
        rt += tl[j];
    }
    if (tid == kGroupThreads - 1) {  // the last thread's running sums are the totals
        start[E] = rc;
        ws[L.ntiles] = rt;
    }
    __syncthreads();
    for (int e = tid; e < E; e += kGroupThreads) s_cnt[e] = 0;
    __syncthreads();
    int32_t *sorted = ws + L.sorted;
    for (int64_t p = tid; p < P; p += kGroupThreads) {
        const int e = ids[p];
        if (e >= 0 && e < E) sorted[s_start[e] + atomicAdd(&s_cnt[e], 1)] = (int32_t)p;
    }
}

}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, int32_t **ptr) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    int dev = cur;
    if (stream != nullptr) {
        hipDevice_t sd = 0;
        e = hipStreamGetDevice(stream, &sd);
        if (e != hipSuccess) return e;
        dev = (int)sd;
    }
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        // the symbol's address on `dev`, looked up with `dev` current
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = static_cast<int32_t *>(p);
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_moe_group_ids(const int32_t *ids, int64_t P, int64_t E, int32_t *ws, float *out,
                                int64_t N, hipStream_t s) {
    const int bm = gemm_tile_rows();
    const MoeGroupLayout L = moe_group_layout(P, E, bm);
    hipLaunchKernelGGL(k_moe_group_ids, dim3(1), dim3(kGroupThreads), 0, s, ids, P, (int)E, bm, L, ws,
                       out, N);
    return hipGetLastError();
}

}  // namespace qmm
