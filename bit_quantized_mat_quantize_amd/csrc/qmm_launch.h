// qmm_launch.h -- internal host launchers (called by api.hip after validation).
// Arguments are already checked: sizes in range, K a multiple of the block,
// pointers non-null and 16-byte aligned.  Each returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace qmm {

// Opts kernel `func` into `bytes` of dynamic LDS (past the default 64 KiB)
// once per device: `done` holds one bit per device id below 64 (higher ids
// set the attribute on every call).  The attribute call is idempotent and the
// mask atomic, so concurrent first calls from several threads are safe.
inline hipError_t ensure_lds_bytes(const void *func, int bytes, std::atomic<uint64_t> &done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev >= 0 && dev < 64 ? uint64_t(1) << dev : 0;
    if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
    e = hipFuncSetAttribute(func, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_acq_rel);
    return e;
}

hipError_t launch_quantize_q8_0(const float *x, uint8_t *y, int64_t M, int64_t K, hipStream_t s);
hipError_t launch_quantize_q8_K(const float *x, uint8_t *y, int64_t M, int64_t K, hipStream_t s);
hipError_t launch_encode_q4_0(const float *w, uint8_t *out, int64_t N, int64_t K, hipStream_t s);
hipError_t launch_encode_q4_K(const float *w, uint8_t *out, int64_t N, int64_t K, hipStream_t s);

int64_t repacked_bytes_q4_0(int64_t N, int64_t K);
int64_t repacked_bytes_q6_K(int64_t N, int64_t K);
hipError_t launch_repack_q4_0(const uint8_t *in, uint8_t *out, int64_t N, int64_t K, hipStream_t s);
hipError_t launch_repack_q4_K(const uint8_t *in, uint8_t *out, int64_t N, int64_t K, hipStream_t s);

// GEMV family: M <= 8.  `repacked` selects the weight layout.
hipError_t launch_gemv_q4_0(const uint8_t *w, bool repacked, const uint8_t *y, float *out,
                            int64_t M, int64_t N, int64_t K, hipStream_t s);
hipError_t launch_gemv_q4_K(const uint8_t *w, bool repacked, const uint8_t *y, float *out,
                            int64_t M, int64_t N, int64_t K, hipStream_t s);
// Fused M = 1 quantize + GEMV: x is one fp32 row of K values; yq receives its
// Q8_K bytes.  Valid for K <= gemv1_fused_max_k().
int64_t gemv1_fused_max_k();
hipError_t launch_gemv1_fused_q4_K(const uint8_t *w, bool repacked, const float *x, uint8_t *yq,
                                   float *out, int64_t N, int64_t K, hipStream_t s);
// int32 per-(sub-)block sums with the GEMV decode path (verification aid).
hipError_t launch_block_sums_q4_0(const uint8_t *w, bool repacked, const uint8_t *y, int32_t *P,
                                  int64_t M, int64_t N, int64_t K, hipStream_t s);
hipError_t launch_block_sums_q4_K(const uint8_t *w, bool repacked, const uint8_t *y, int32_t *P,
                                  int64_t M, int64_t N, int64_t K, hipStream_t s);

// Small-batch MFMA family: M <= skinny_max_m(), weight and activation
// matrices below 4 GiB (32-bit buffer offsets).
int64_t skinny_max_m();
hipError_t launch_skinny_q4_K(const uint8_t *w, bool repacked, const uint8_t *y, float *out,
                              int64_t M, int64_t N, int64_t K, hipStream_t s);
// The same on 16 x 16 MFMA tiles (workgroups of 16 rows and 16 or 32
// columns): M <= skinny16_max_m(), matrices below 4 GiB.
int64_t skinny16_max_m();
// compute units of the current device (queried once per device)
int cu_count();
// Q4_K small batch, repacked layout, 1 <= M <= 8 (skinny16r.hip): producer
// wavefront streaming through an LDS ring, four consumer wavefronts.
hipError_t launch_skinny16r_q4_K(const uint8_t *w, const uint8_t *y, float *out, int64_t M, int64_t N,
                                 int64_t K, hipStream_t s);
// Q4_K small batch, repacked layout, 1 <= M <= 32 (skinny32r.hip): two or three
// producer wavefronts streaming through an LDS ring, four consumer wavefronts.
hipError_t launch_skinny32r_q4_K(const uint8_t *w, const uint8_t *y, float *out, int64_t M, int64_t N,
                                 int64_t K, hipStream_t s);
hipError_t launch_skinny16_q4_K(const uint8_t *w, bool repacked, const uint8_t *y, float *out,
                                int64_t M, int64_t N, int64_t K, hipStream_t s);
// Q4_0, M = 1, small matrices (gemv_fused_q4_0_ok): quantize + GEMV in one launch
bool gemv_fused_q4_0_ok(int64_t N, int64_t K);
hipError_t launch_gemv_fused_q4_0(const uint8_t *w, bool repacked, const float *x, uint8_t *yq, float *out,
                                  int64_t N, int64_t K, hipStream_t s);
// Q6_K, M = 1, K <= 8192, N <= 32 * CUs (gemv_fused_q6_K_ok): quantize + GEMV in one launch
bool gemv_fused_q6_K_ok(int64_t N, int64_t K);
hipError_t launch_gemv_fused_q6_K(const uint8_t *w, bool repacked, const float *x, uint8_t *yq, float *out,
                                  int64_t N, int64_t K, hipStream_t s);
// Q2_K, M = 1, K <= 16384, N <= 32 * CUs (gemv_fused_q2_K_ok): quantize + GEMV in one launch
bool gemv_fused_q2_K_ok(int64_t N, int64_t K);
hipError_t launch_gemv_fused_q2_K(const uint8_t *w, bool repacked, const float *x, uint8_t *yq, float *out,
                                  int64_t N, int64_t K, hipStream_t s);
// Q4_0 GEMV with the M activation rows staged in LDS: K % 64 == 0 and
// M * K * 5/4 bytes <= 60 KiB (other shapes read the rows per lane).
bool gemv_q4_0s_fits(int64_t M, int64_t K);
// Q4_0 small batch: repacked layout, K % 256 == 0, M <= skinny_q4_0_max_m(),
// matrices below 4 GiB; w_bytes is the repacked matrix size.
int64_t skinny_q4_0_max_m();
hipError_t launch_skinny_q4_0(const uint8_t *w, int64_t w_bytes, const uint8_t *y, float *out, int64_t M,
                              int64_t N, int64_t K, hipStream_t s);

// Q6_K (encoder, load-time repack, GEMV for any M with K <= q6_K_max_k(),
// int32 group sums P[m][n][K/16] of the same decode path).
int64_t q6_K_max_k();
hipError_t launch_encode_q6_K(const float *w, uint8_t *out, int64_t N, int64_t K, hipStream_t s);
hipError_t launch_repack_q6_K(const uint8_t *in, uint8_t *out, int64_t N, int64_t K, hipStream_t s);
hipError_t launch_gemv_q6_K(const uint8_t *w, bool repacked, const uint8_t *y, float *out,
                            int64_t M, int64_t N, int64_t K, hipStream_t s);
hipError_t launch_group_sums_q6_K(const uint8_t *w, bool repacked, const uint8_t *y, int32_t *P,
                                  int64_t M, int64_t N, int64_t K, hipStream_t s);

// Q2_K (encoder, load-time repack, GEMV for any M with K <= q2_K_max_k(),
// int32 group sums P[m][n][K/16] of the same decode path).
int64_t repacked_bytes_q2_K(int64_t N, int64_t K);
int64_t q2_K_max_k();
hipError_t launch_encode_q2_K(const float *w, uint8_t *out, int64_t N, int64_t K, hipStream_t s);
hipError_t launch_repack_q2_K(const uint8_t *in, uint8_t *out, int64_t N, int64_t K, hipStream_t s);
hipError_t launch_gemv_q2_K(const uint8_t *w, bool repacked, const uint8_t *y, float *out,
                            int64_t M, int64_t N, int64_t K, hipStream_t s);
hipError_t launch_group_sums_q2_K(const uint8_t *w, bool repacked, const uint8_t *y, int32_t *P,
                                  int64_t M, int64_t N, int64_t K, hipStream_t s);
// both group-sum paths stage one activation row in LDS
inline int64_t q8k_group_max_k() { return q6_K_max_k() < q2_K_max_k() ? q6_K_max_k() : q2_K_max_k(); }

// MFMA GEMM family (any M >= 1; weight and activation matrices below 4 GiB:
// 32-bit buffer offsets).  The Q6_K and Q2_K GEMMs take the repacked layout
// of w_bytes bytes.
hipError_t launch_gemm_q4_K(const uint8_t *w, bool repacked, const uint8_t *y, float *out,
                            int64_t M, int64_t N, int64_t K, hipStream_t s);
// Q6_K small batch: repacked layout, M <= skinny_q6_K_max_m(), matrices below
// 4 GiB; w_bytes is the repacked matrix size.
int64_t skinny_q6_K_max_m();
hipError_t launch_skinny_q6_K(const uint8_t *w, int64_t w_bytes, const uint8_t *y, float *out, int64_t M,
                              int64_t N, int64_t K, hipStream_t s);
hipError_t launch_gemm_q6_K(const uint8_t *w, int64_t w_bytes, const uint8_t *y, float *out,
                            int64_t M, int64_t N, int64_t K, hipStream_t s);
hipError_t launch_gemm_q2_K(const uint8_t *w, int64_t w_bytes, const uint8_t *y, float *out,
                            int64_t M, int64_t N, int64_t K, hipStream_t s);
// Q2_K small batch: repacked layout, M <= skinny_q2_K_max_m(), matrices below
// 4 GiB; w_bytes is the repacked matrix size.
int64_t skinny_q2_K_max_m();
hipError_t launch_skinny_q2_K(const uint8_t *w, int64_t w_bytes, const uint8_t *y, float *out, int64_t M,
                              int64_t N, int64_t K, hipStream_t s);
// Q4_0 x Q8_0, repacked layout, K a multiple of 256.
hipError_t launch_gemm_q4_0(const uint8_t *w, int64_t w_bytes, const uint8_t *y, float *out,
                            int64_t M, int64_t N, int64_t K, hipStream_t s);

constexpr int kGemvMaxM = 8;

// ---- mul_mat_id (Q4_K).  The expert grouping lives in a caller workspace of
// int32 words: start[E+1] (first sorted slot of each expert), tile_e and
// tile_r0 [max_tiles] (expert and first sorted slot of each GEMM row tile),
// ntiles[1], sorted[P] (pair index per sorted slot), each section aligned to
// 16 bytes.  Each expert adds at most one partial tile, so max_tiles =
// ceil(P / bm) + E.
struct MoeGroupLayout {
    int64_t start, tile_e, tile_r0, ntiles, sorted, max_tiles, words;
};
inline MoeGroupLayout moe_group_layout(int64_t P, int64_t E, int64_t bm) {
    auto up4 = [](int64_t v) { return (v + 3) / 4 * 4; };
    MoeGroupLayout L;
    L.max_tiles = (P + bm - 1) / bm + E;
    L.start = 0;
    L.tile_e = L.start + up4(E + 1);
    L.tile_r0 = L.tile_e + up4(L.max_tiles);
    L.ntiles = L.tile_r0 + up4(L.max_tiles);
    L.sorted = L.ntiles + 4;
    L.words = L.sorted + up4(P);
    return L;
}
constexpr int kMoeMaxExperts = 4096;
int gemm_tile_rows();  // BM of the Q4_K GEMM
int64_t gemv1_max_k();
// The library's own grouping area for callers that cannot allocate: device
// address of a static array of kNoAllocScratchBytes on the device of `stream`
// (the current device for the null stream), looked up once per device.
constexpr size_t kNoAllocScratchBytes = size_t(2) << 20;
hipError_t noalloc_scratch(hipStream_t stream, int32_t **ptr);
// Build the grouping for pairs p < P with expert ids[p] (ids outside [0, E)
// are left out, and their output rows are filled with NaN).
hipError_t launch_moe_group_ids(const int32_t *ids, int64_t P, int64_t E, int32_t *ws, float *out,
                                int64_t N, hipStream_t s);
// M = 1 GEMV per (token, slot) pair; w_stride = bytes per expert matrix.
hipError_t launch_gemv_id_q4_K(const uint8_t *w, bool repacked, int64_t w_stride, const uint8_t *y,
                               int y_per_slot, const int32_t *ids, int64_t P, int64_t U, int64_t E,
                               float *out, int64_t N, int64_t K, hipStream_t s);
hipError_t launch_gemv_id_q6_K(const uint8_t *w, bool repacked, int64_t w_stride, const uint8_t *y,
                               int y_per_slot, const int32_t *ids, int64_t P, int64_t U, int64_t E,
                               float *out, int64_t N, int64_t K, hipStream_t s);
hipError_t launch_gemv_id_q2_K(const uint8_t *w, bool repacked, int64_t w_stride, const uint8_t *y,
                               int y_per_slot, const int32_t *ids, int64_t P, int64_t U, int64_t E,
                               float *out, int64_t N, int64_t K, hipStream_t s);
hipError_t launch_gemv_id_q4_0(const uint8_t *w, bool repacked, int64_t w_stride, const uint8_t *y,
                               int y_per_slot, const int32_t *ids, int64_t P, int64_t U, int64_t E,
                               float *out, int64_t N, int64_t K, hipStream_t s);
// The GEMMs over the grouped tiles (after launch_moe_group_ids on ws); the
// Q6_K, Q2_K and Q4_0 ones take the repacked layout, w_bytes = one expert.
hipError_t launch_gemm_id_q6_K(const uint8_t *w, int64_t w_bytes, const uint8_t *y, int64_t y_rows,
                               int y_per_slot, int64_t U, const int32_t *group_ws, int64_t E, int64_t P,
                               float *out, int64_t N, int64_t K, hipStream_t s);
hipError_t launch_gemm_id_q2_K(const uint8_t *w, int64_t w_bytes, const uint8_t *y, int64_t y_rows,
                               int y_per_slot, int64_t U, const int32_t *group_ws, int64_t E, int64_t P,
                               float *out, int64_t N, int64_t K, hipStream_t s);
hipError_t launch_gemm_id_q4_0(const uint8_t *w, int64_t w_bytes, const uint8_t *y, int64_t y_rows,
                               int y_per_slot, int64_t U, const int32_t *group_ws, int64_t E, int64_t P,
                               float *out, int64_t N, int64_t K, hipStream_t s);
hipError_t launch_gemm_id_q4_K(const uint8_t *w, bool repacked, int64_t w_stride, const uint8_t *y,
                               int64_t y_rows, int y_per_slot, int64_t U, const int32_t *group_ws,
                               int64_t E, int64_t P, float *out, int64_t N, int64_t K, hipStream_t s);

}  // namespace qmm
