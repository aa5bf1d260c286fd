/*
 * qmm.h -- C ABI of libqmm: quantized mul_mat (Q4_0 / Q4_K / Q6_K / Q2_K weights
 * times Q8_0 / Q8_K activations) on AMD Instinct MI355X (gfx950).
 *
 * Operation (BitBLAS page, "从数学表达式到真实存储:混合精度 GEMM 的计算对象";
 * ggml-cpu mul_mat page, "mul_mat:一次矩阵乘被切成什么样"):
 *     out[m*N + n] = sum_k  deq(A)[m,k] * deq(W)[n,k]
 * with W an [N, K] matrix of packed 4-bit weight blocks (row n = output channel,
 * K contiguous) and A an [M, K] matrix of int8 activation blocks, computed
 * without expanding W: per block, integer dot products of the codes with the
 * block scales pulled out of the sum (ggml-cpu mul_mat page,
 * "正确性:缩放系数可以提到求和号外面").
 *
 * Byte formats (little-endian), as the ggml-cpu mul_mat page defines them:
 *   Q4_0  18 B / 32:  fp16 d; qs[16], byte l = element l (low nibble) |
 *                     element l+16 (high nibble); w = d*(q-8)
 *   Q8_0  34 B / 32:  fp16 d; int8 qs[32]; a = d*y
 *   Q4_K 144 B / 256: fp16 d; fp16 dmin; scales[12]; qs[128]
 *                     w = d*s_j*q - dmin*m_j for element k in sub-block j = k/32;
 *                     qs byte 32g+l = element 64g+l (low) | element 64g+32+l (high)
 *                     scales[12] bit layout (section "6-bit 参数是怎么塞进 12 字节的"):
 *                       j<4 : s_j = byte j & 63,  m_j = byte j+4 & 63
 *                       j>=4: s_j = (byte j+4 & 15) | (byte j-4 >> 6) << 4
 *                             m_j = (byte j+4 >> 4) | (byte j   >> 6) << 4
 *   Q6_K 210 B / 256: ql[128] (low 4 bits) | qh[64] (high 2 bits) | int8 scales[16] |
 *                     fp16 d (section "更低的比特:Q6_K 与 Q2_K 的取舍"); w = d*s_j*q,
 *                     q in [-32, 31], j = element / 16, no min term.  Bit placement
 *                     (this library's reading): element k = 64g + r keeps its low
 *                     4 bits in ql byte 32g + r%32 (low nibble for r < 32, else
 *                     high) and its high 2 bits in qh byte r, bits 2g..2g+1; the
 *                     stored code is q + 32
 *   Q2_K  84 B / 256: scales[16] | qs[64] | fp16 d | fp16 dmin (same section: 2-bit
 *                     codes, a 4-bit scale and a 4-bit min per 16-element group);
 *                     w = d*s_j*q - dmin*m_j, q in [0, 3], j = element / 16.
 *                     Placement (this library's reading): scale byte j = s_j (low
 *                     nibble) | m_j << 4; element k = 128h + 32s + l sits in qs
 *                     byte 32h + l, bits 2s..2s+1
 *   Q8_K 292 B / 256: fp32 d; int8 qs[256]; int16 bsums[16] (sum of qs[16g..16g+15])
 *   Rows are arrays of blocks: row r of a [R, K] matrix starts at r * (K/QK) * bytes.
 *
 * Load-time layout QMM_LAYOUT_REPACKED (a lossless byte permutation of the
 * canonical matrix, BitBLAS page "Ladder Permutation"; produced by
 * qmm_repack_weights):
 *   Q4_K: [N*nb headers of 16 B: d, dmin, scales[12]] then
 *         [N*nb payloads of 128 B: qs], block (n,b) at index n*nb+b
 *   Q4_0: [N*nb fp16 d, zero-padded to a multiple of 256 B] then
 *         [N*nb payloads of 16 B: qs]
 *   Q6_K: [N*nb fp16 d, zero-padded to a multiple of 256 B] then [N*nb scales of
 *         16 B] then [N*nb ql of 128 B] then [N*nb qh of 64 B]
 *   Q2_K: [N*nb (d, dmin) pairs of 4 B, zero-padded to a multiple of 256 B] then
 *         [N*nb scales of 16 B] then [N*nb qs of 64 B]
 *   (nb = blocks per row).  The payload stream is 16-byte aligned, which lets a
 *   wavefront read weights with coalesced 16-byte loads.
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers (hipMalloc / torch CUDA tensors)
 *     owned by the caller and 16-byte aligned; the library never allocates,
 *     frees or synchronizes; work is enqueued on `stream` (a hipStream_t; NULL
 *     is the legacy default stream) and runs asynchronously.
 *   - Arguments are validated on the host before any HIP call; on failure the
 *     call returns a non-zero qmm_status, enqueues nothing and leaves a
 *     message for qmm_last_error().  M or N equal to 0 is a valid empty call.
 *   - K must be a positive multiple of the block length (32 for Q4_0/Q8_0,
 *     256 for Q4_K/Q6_K/Q8_K), else QMM_EUNSUPPORTED.  Sizes are limited to
 *     M, N <= 2^24 and K <= 2^20 (QMM_EUNSUPPORTED beyond).
 *   - `*_bytes` arguments give the size of the caller's buffer; a buffer
 *     smaller than the corresponding qmm_*_bytes() value gives QMM_EINVAL.
 *   - A failed kernel launch gives QMM_EDEVICE.
 *   - Functions are thread-safe (the error message is thread-local).
 */
#ifndef QMM_H
#define QMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QMM_OK = 0,
    QMM_EINVAL = 1,        /* bad argument (null pointer, negative size, small buffer) */
    QMM_EALIGN = 2,        /* pointer not 16-byte aligned */
    QMM_EUNSUPPORTED = 3,  /* K not a multiple of the block, size limit, unknown enum */
    QMM_EDEVICE = 4        /* HIP runtime error while enqueueing */
} qmm_status;

typedef enum { QMM_Q8_0 = 0, QMM_Q8_K = 1 } qmm_act_type;
typedef enum { QMM_Q4_0 = 0, QMM_Q4_K = 1, QMM_Q6_K = 2, QMM_Q2_K = 3 } qmm_weight_type;
typedef enum { QMM_LAYOUT_CANONICAL = 0, QMM_LAYOUT_REPACKED = 1 } qmm_layout;

/* Kernel family for a mul_mat call:
 *   GEMV    vector int8 dot products, one wavefront per output row (Q4_0 and
 *           Q4_K: M <= 8 per launch; Q6_K and Q2_K: any M, K <= 53760)
 *   SKINNY  small-batch int8 MFMA, one 32-column x 32-row tile per workgroup,
 *           K split over its wavefronts (Q4_K; Q6_K and Q2_K in the repacked
 *           layout; Q4_0 in the repacked layout with K % 256 == 0;
 *           M <= 65535*32).  For Q4_K up to 16 rows the tiles are 16 x 16,
 *           and up to 8 rows of the repacked layout one wavefront per
 *           workgroup streams the weights into LDS for four that compute;
 *           from 9 to 32 rows of the repacked layout two or three wavefronts
 *           stream weights and activation rows for four that compute
 *   MFMA    prefill GEMM on int8 MFMA, 128 x 256 output tiles (any M; Q6_K,
 *           Q2_K and Q4_0 need the repacked layout, Q4_0 also K % 256 == 0)
 * SKINNY and MFMA address the weight and activation matrices with 32-bit
 * offsets, so both must be below 4 GiB.  AUTO follows measured crossovers:
 * for Q4_K it takes GEMV for M = 1, SKINNY for the other M <= 32 and while
 * ceil(M/32)*N <= 9*8192, MFMA above (GEMV in groups of 8 rows where the
 * size limit rules the MFMA kernels out); for Q4_0 it takes GEMV for M = 1, for
 * M <= 4 or M*N <= 36864 when K % 64 == 0 and M*K*5/4 <= 61440 (the rows fit
 * the GEMV's LDS staging) and for M = 2 with N < 8192, SKINNY while
 * ceil(M/32)*N <= 16*8192, MFMA above, GEMV where the MFMA kernels are ruled
 * out; for Q6_K in the repacked layout it takes GEMV for M = 1 and for M = 2
 * with N < 8192, SKINNY while ceil(M/32)*N <= 8*8192, MFMA above; for Q2_K in
 * the repacked layout it takes GEMV for M = 1 and for M = 2 with N < 8192, SKINNY while
 * ceil(M/32)*N <= 6*8192, MFMA above.  For Q6_K and Q2_K, a K above the
 * GEMV's limit (53760) sends M = 1 and M = 2 to SKINNY or MFMA by the same
 * ceil(M/32)*N rule.  The canonical layout of Q6_K and Q2_K, and a matrix of
 * 4 GiB or more, have only the GEMV: AUTO takes it for every M. */
typedef enum {
    QMM_ALGO_AUTO = 0,
    QMM_ALGO_GEMV = 1,
    QMM_ALGO_MFMA = 2,
    QMM_ALGO_SKINNY = 3
} qmm_algo;

/* Bytes of an [M, K] activation matrix in format t: M*K/32*34 or M*K/256*292.
 * Returns 0 for invalid arguments. */
size_t qmm_act_bytes(qmm_act_type t, int64_t M, int64_t K);

/* Bytes of an [N, K] weight matrix in format t and layout l.  Canonical:
 * N*K/32*18, N*K/256*144, N*K/256*210 (Q6_K) or N*K/256*84 (Q2_K).  Repacked
 * Q4_0, Q6_K and Q2_K add the padding of their d section (at most 252 B).  Returns 0 for invalid
 * arguments. */
size_t qmm_weight_bytes(qmm_weight_type t, qmm_layout l, int64_t N, int64_t K);

/* Quantize fp32 activations x [M, K] (row-major) to int8 blocks y [M, K/QK]
 * (ggml-cpu mul_mat page, "第一步:激活得先变成 Q8_K": activations are
 * converted once per mul_mat and shared by all output tiles).
 * Per block: amax = max|x|, d = amax/127, y = rint(x * (1/d)) (ties to even),
 * d = 0 and y = 0 for an all-zero block; Q8_0 stores fp16(d), Q8_K stores the
 * fp32 d and the 16 bsums.  The result is bit-identical to the reference
 * encoder.  x: device fp32, M*K elements; y: device, y_bytes >= qmm_act_bytes. */
qmm_status qmm_quantize_row_q8(qmm_act_type t, const float *x, int64_t M, int64_t K,
                               void *y, size_t y_bytes, void *stream);

/* Encode fp32 weights w [N, K] into canonical blocks (offline; the pages give
 * the decoded form, the scale search is this library's reading):
 *   Q4_0: d = -xmax/8 (xmax = signed element of largest |x|, first wins),
 *         q = clamp(rint(x*(1/d)) + 8, 0, 15)
 *   Q4_K: per sub-block lo = min(0, min x), sc = (max x - lo)/15, mn = -lo;
 *         d = max sc/63, dmin = max mn/63; s_j = rint(sc/d), m_j = rint(mn/dmin)
 *         (clamped to 63); q = clamp(rint((x + f16(dmin)*m_j)/(f16(d)*s_j)), 0, 15)
 *   Q6_K: per 16-element group xm = signed element of largest |x| (first
 *         wins), sc = xm/-32; d = max |sc|/127; s_j = rint(sc/d) in [-127, 127];
 *         q = clamp(rint(x/(f16(d)*s_j)), -32, 31), 0 where f16(d)*s_j = 0
 *   Q2_K: the Q4_K rule per 16-element group with 2-bit codes and 4-bit
 *         scales: sc = (max x - lo)/3, d = max sc/15, dmin = max mn/15,
 *         s_j, m_j clamped to 15, q clamped to [0, 3]
 * out: device, out_bytes >= qmm_weight_bytes(t, CANONICAL, N, K). */
qmm_status qmm_quantize_weights(qmm_weight_type t, const float *w, int64_t N, int64_t K,
                                void *out, size_t out_bytes, void *stream);

/* Permute canonical weight blocks into QMM_LAYOUT_REPACKED (BitBLAS page,
 * "Ladder Permutation": an offline, lossless reordering of static weights into
 * the order the kernel reads them; same page, "4. 权重变换只做一次": the
 * transform runs once at load time and the original quantized blocks stay the
 * source of truth; GGML memory/quantization page, "量化:热路径是点积,不是反量化":
 * a load-time layout change that leaves the file's blocks untouched).  The byte map of each format is given at the top of this header.
 * w_canon: device, qmm_weight_bytes(t, CANONICAL, N, K) bytes; w_repacked:
 * device, out_bytes >= qmm_weight_bytes(t, REPACKED, N, K), fully written
 * (padding zeroed).  The two must not overlap (QMM_EINVAL). */
qmm_status qmm_repack_weights(qmm_weight_type t, const void *w_canon, int64_t N, int64_t K,
                              void *w_repacked, size_t out_bytes, void *stream);

/* out[m*N+n] = sum over blocks b of d_w*d_a*sum_i (q_i-8)*y_i  (ggml-cpu
 * mul_mat page, "最基础的两块:Q4_0 与 Q8_0": a Q4_0 block decodes to
 * d*(q-8) and a Q8_0 block to d*y, so a block pair's dot product is the int32
 * sum of (q-8)*y scaled once by both fp16 d's; "正确性:缩放系数可以提到求和号外面"
 * for pulling the scales out of the sum).  fp32 output, overwritten.
 * w: Q4_0 [N,K] in layout l; y: Q8_0 [M,K] from qmm_quantize_row_q8.
 * Kernel choice as QMM_ALGO_AUTO describes. */
qmm_status qmm_mul_mat_q4_0(const void *w, size_t w_bytes, qmm_layout l,
                            const void *y, size_t y_bytes,
                            float *out, size_t out_bytes,
                            int64_t M, int64_t N, int64_t K, void *stream);

/* Same as qmm_mul_mat_q4_0 with an explicit kernel family: QMM_ALGO_GEMV (any
 * M, launched in groups of 8 rows), QMM_ALGO_SKINNY (repacked layout, K a
 * multiple of 256, M <= 65535*32, both matrices below 4 GiB) or QMM_ALGO_MFMA
 * (repacked layout, K a multiple of 256, both matrices below 4 GiB); a family
 * whose limits the call exceeds, or an unknown one, gives QMM_EUNSUPPORTED. */
qmm_status qmm_mul_mat_q4_0_ex(const void *w, size_t w_bytes, qmm_layout l,
                               const void *y, size_t y_bytes,
                               float *out, size_t out_bytes,
                               int64_t M, int64_t N, int64_t K, qmm_algo algo,
                               void *stream);

/* out[m*N+n] = sum over super-blocks b of d_a*(d*S - dmin*Mn) with
 * S = sum_j s_j*P_j, P_j = sum_{i in j} q_i*y_i, Mn = sum_j m_j*(bsums[2j]+bsums[2j+1])
 * (ggml-cpu mul_mat page, "正确性" and "min 项与最终归约").  fp32 output,
 * overwritten.  w: Q4_K [N,K] in layout l; y: Q8_K [M,K]. */
qmm_status qmm_mul_mat_q4_K(const void *w, size_t w_bytes, qmm_layout l,
                            const void *y, size_t y_bytes,
                            float *out, size_t out_bytes,
                            int64_t M, int64_t N, int64_t K, void *stream);

/* out[m*N+n] = sum over super-blocks b of d_a*d*S with S = sum_j s_j*P_j,
 * P_j = sum_{i in j} q_i*y_i over the 16-element groups j (ggml-cpu mul_mat page,
 * "更低的比特:Q6_K 与 Q2_K 的取舍": no min term, so no bsums path; and
 * "正确性:缩放系数可以提到求和号外面").  fp32 output, overwritten.  w: Q6_K [N,K]
 * in layout l; y: Q8_K [M,K].  Kernel choice as QMM_ALGO_AUTO describes; a
 * call that no Q6_K kernel takes (K > 53760 with the canonical layout or with
 * a matrix of 4 GiB or more) gives QMM_EUNSUPPORTED. */
qmm_status qmm_mul_mat_q6_K(const void *w, size_t w_bytes, qmm_layout l,
                            const void *y, size_t y_bytes,
                            float *out, size_t out_bytes,
                            int64_t M, int64_t N, int64_t K, void *stream);

/* Same as qmm_mul_mat_q6_K with an explicit kernel family: QMM_ALGO_GEMV
 * (K <= 53760), QMM_ALGO_SKINNY (repacked layout, M <= 65535*32, both matrices
 * below 4 GiB) or QMM_ALGO_MFMA (repacked layout, both matrices below 4 GiB);
 * a family whose limits the call exceeds gives QMM_EUNSUPPORTED. */
qmm_status qmm_mul_mat_q6_K_ex(const void *w, size_t w_bytes, qmm_layout l,
                               const void *y, size_t y_bytes,
                               float *out, size_t out_bytes,
                               int64_t M, int64_t N, int64_t K, qmm_algo algo,
                               void *stream);

/* Same as qmm_mul_mat_q4_K with an explicit kernel family (for measuring the
 * GEMV / GEMM crossover).  QMM_ALGO_GEMV requires M <= 8; QMM_ALGO_SKINNY
 * requires M <= 65535*32; SKINNY and MFMA require both matrices below 4 GiB (else
 * QMM_EUNSUPPORTED). */
qmm_status qmm_mul_mat_q4_K_ex(const void *w, size_t w_bytes, qmm_layout l,
                               const void *y, size_t y_bytes,
                               float *out, size_t out_bytes,
                               int64_t M, int64_t N, int64_t K, qmm_algo algo,
                               void *stream);

/* out[m*N+n] = sum over super-blocks b of d_a*(d*S - dmin*Mn) with
 * S = sum_j s_j*P_j, P_j = sum_{i in j} q_i*y_i and Mn = sum_j m_j*bsums[j] over
 * the 16-element groups j (ggml-cpu mul_mat page, "更低的比特:Q6_K 与 Q2_K 的取舍",
 * "正确性:缩放系数可以提到求和号外面", "min 项与最终归约").  fp32 output,
 * overwritten.  w: Q2_K [N,K] in layout l; y: Q8_K [M,K].  Kernel choice as
 * qmm_algo states; limits as for qmm_mul_mat_q6_K. */
qmm_status qmm_mul_mat_q2_K(const void *w, size_t w_bytes, qmm_layout l,
                            const void *y, size_t y_bytes,
                            float *out, size_t out_bytes,
                            int64_t M, int64_t N, int64_t K, void *stream);

/* Same as qmm_mul_mat_q2_K with an explicit kernel family, with the rules of
 * qmm_mul_mat_q6_K_ex. */
qmm_status qmm_mul_mat_q2_K_ex(const void *w, size_t w_bytes, qmm_layout l,
                               const void *y, size_t y_bytes,
                               float *out, size_t out_bytes,
                               int64_t M, int64_t N, int64_t K, qmm_algo algo,
                               void *stream);

/* Bytes of the workspace qmm_mul_mat_id (and qmm_mul_mat_id_q4_K) needs for
 * its MFMA path (T tokens, U slots per token, E experts, any weight format):
 * int32 tables of the expert grouping.
 * Returns 0 for invalid arguments (U < 1, E outside [1, 4096], T*U >= 2^31). */
size_t qmm_mul_mat_id_workspace_bytes(int64_t T, int64_t U, int64_t E);

/* mul_mat_id (ggml-cpu mul_mat page, "本篇没有覆盖的部分", the follow-up
 * topics: mul_mat with one more level, the grouping by expert id).  For every token t < T and slot
 * u < U, with e = ids[t*U + u]:
 *     out[(t*U + u)*N + n] = mul_mat_q4_K(W_e, y_row)[n]
 * where W_e is expert e's Q4_K [N,K] matrix -- w holds the E matrices one
 * after another, each qmm_weight_bytes(QMM_Q4_K, l, N, K) bytes in layout l --
 * and y_row is Q8_K activation row t (y_per_slot = 0: every slot of a token
 * reads its row) or row t*U + u (y_per_slot = 1).  ids: device int32 [T*U].
 * Kernels: QMM_ALGO_GEMV runs one M = 1 GEMV per (token, slot) (K <= 53760);
 * QMM_ALGO_MFMA sorts the pairs by expert on the device into `workspace`
 * (device, at least qmm_mul_mat_id_workspace_bytes(T, U, E) bytes, contents
 * overwritten; not needed by the GEMV path, may be NULL there) and runs the
 * Q4_K GEMM over each expert's rows (one expert matrix and the activations
 * below 4 GiB); AUTO takes the GEMV for T*U <= 4*E, the GEMM above.  An id
 * outside [0, E) cannot be checked on the host: that pair's output row is
 * filled with NaN and nothing is read out of bounds.  Requires 1 <= E <= 4096,
 * 1 <= U <= E.  Equal to qmm_mul_mat_id(QMM_Q4_K, ...). */
qmm_status qmm_mul_mat_id_q4_K(const void *w, size_t w_bytes, int64_t E, qmm_layout l,
                               const void *y, size_t y_bytes, int y_per_slot,
                               const int32_t *ids, int64_t T, int64_t U,
                               float *out, size_t out_bytes, int64_t N, int64_t K,
                               void *workspace, size_t ws_bytes, qmm_algo algo,
                               void *stream);

/* mul_mat_id for any weight format t: the same contract as
 * qmm_mul_mat_id_q4_K with W_e in format t (Q8_0 activations for Q4_0, Q8_K
 * otherwise).  Kernels: QMM_ALGO_GEMV -- one GEMV per (token, slot) (K <=
 * 53760 for Q4_K, Q6_K and Q2_K, K <= 2^20 for Q4_0); QMM_ALGO_MFMA -- the expert grouping into
 * `workspace`, then the format's MFMA GEMM over each expert's rows (Q6_K, Q2_K
 * and Q4_0 need the repacked layout, and K % 256 == 0); AUTO takes the GEMV
 * for T*U <= 4*E and the GEMM above, whichever the call allows otherwise. */
qmm_status qmm_mul_mat_id(qmm_weight_type t, const void *w, size_t w_bytes, int64_t E, qmm_layout l,
                          const void *y, size_t y_bytes, int y_per_slot,
                          const int32_t *ids, int64_t T, int64_t U,
                          float *out, size_t out_bytes, int64_t N, int64_t K,
                          void *workspace, size_t ws_bytes, qmm_algo algo,
                          void *stream);

/* qmm_mul_mat_id without the workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same contract, kernels and results as
 * qmm_mul_mat_id; its MFMA path keeps the expert grouping in a scratch array
 * the library holds in device memory: 2 MiB per GPU, kept until the process
 * ends.  A call that may take the grouped path (algo AUTO or MFMA) and whose
 * grouping needs more than that (qmm_mul_mat_id_workspace_bytes(T, U, E) >
 * 2097152) gives QMM_EUNSUPPORTED before any HIP call.  Every call on one GPU
 * shares that GPU's array and leaves its tables in it (each call rewrites all
 * it reads, so nothing needs clearing): calls that overlap on one GPU (on
 * different streams, or from different threads without ordering) race and must
 * be serialized by the caller.  Allocates nothing. */
qmm_status qmm_mul_mat_id_noalloc(qmm_weight_type t, const void *w, size_t w_bytes, int64_t E,
                                  qmm_layout l, const void *y, size_t y_bytes, int y_per_slot,
                                  const int32_t *ids, int64_t T, int64_t U,
                                  float *out, size_t out_bytes, int64_t N, int64_t K,
                                  qmm_algo algo, void *stream);

/* Quantize-and-multiply in one call: y = quantize_row_q8(x) (Q8_0 for t = Q4_0,
 * Q8_K for t = Q4_K, Q6_K and Q2_K), then out = mul_mat(w, y).  The ggml-cpu mul_mat page
 * ("激活量化重复与融合") notes that quantizing the activations once at the
 * start of a fused node saves both the launch and the repeated conversion;
 * here, for Q4_K with M == 1 and K <= 16384 (for Q4_0 with M == 1, K % 64 ==
 * 0, K <= 4096 and N*K <= 2^22; for Q6_K with M == 1 and either K <= 4096 and
 * N at most 32 rows per compute unit or K <= 8192 and N at most 16 rows per
 * compute unit; for Q2_K with M == 1, K <= 16384 and N at most 32 rows per
 * compute unit), the quantization runs inside the
 * GEMV launch itself (one kernel), otherwise the two steps are enqueued back to
 * back.  Projections that share one input are handled by concatenating their
 * canonical weight rows along N before the repack (gate||up: N = 2*14336),
 * or by passing the returned y to qmm_mul_mat_q4_* for the other projections.
 * x: device fp32 [M, K]; y: device, y_bytes >= qmm_act_bytes(t's activation
 * type, M, K), always fully written (byte-identical to qmm_quantize_row_q8);
 * w, out as in qmm_mul_mat_q4_*.  x, y, w and out must not overlap.  N == 0
 * quantizes only (w and out are not read).  Results are identical to
 * qmm_quantize_row_q8 followed by qmm_mul_mat_q4_* (same rounding). */
qmm_status qmm_quantize_mul_mat(qmm_weight_type t, const void *w, size_t w_bytes,
                                qmm_layout l, const float *x, void *y, size_t y_bytes,
                                float *out, size_t out_bytes,
                                int64_t M, int64_t N, int64_t K, void *stream);

/* Verification aid: the int32 per-sub-block (Q4_K) or per-block (Q4_0) sums
 * P[m][n][K/32] = sum_{i in block} q_i*y_i  (Q4_0: (q_i-8)*y_i), or for Q6_K
 * and Q2_K the per-group sums P[m][n][K/16] of their codes (Q6_K: signed),
 * computed by the same decode and int8 dot-product code the GEMV kernels use.
 * P: device int32, p_bytes >= M*N*(K/32)*4 (Q6_K, Q2_K: M*N*(K/16)*4 and
 * K <= 53760). */
qmm_status qmm_debug_block_sums(qmm_weight_type t, const void *w, size_t w_bytes,
                                qmm_layout l, const void *y, size_t y_bytes,
                                int32_t *P, size_t p_bytes,
                                int64_t M, int64_t N, int64_t K, void *stream);

/* Static description of a status code. */
const char *qmm_status_string(qmm_status s);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char *qmm_last_error(void);

/* Library version string. */
const char *qmm_version(void);

#ifdef __cplusplus
}
#endif
#endif /* QMM_H */
