/*
 * qmm_oracle.h -- plain, slow CPU oracle for the quantized mul_mat.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
 * its Python binding) may include, link or call this code; only the tests, the
 * smoke check and the CPU-baseline leg of the benchmark use it.  It shares no
 * header, helper, table or constant with the GPU implementation.
 *
 * Sources (the pages):
 *   [P1] "llama.cpp 源码完全拆解(十三): ggml-cpu 的一次 mul_mat" (one mul_mat in
 *        ggml-cpu: quantized dot products, task split, thread pool)
 *   [P3] "BitBLAS 完全拆解" (BitBLAS teardown: mixed-precision GEMM)
 *
 * Block formats (all little-endian, byte offsets):
 *   Q4_0  (18 B / 32 weights)   [P1 "最基础的两块:Q4_0 与 Q8_0"]
 *         +0  fp16 d
 *         +2  qs[16]: byte l holds element l (low nibble) and l+16 (high nibble)
 *         weight w_i = d * (q_i - 8)
 *   Q8_0  (34 B / 32 values)    [P1 same section]
 *         +0  fp16 d, +2 int8 qs[32];  value a_i = d * y_i
 *   Q4_K  (144 B / 256 weights) [P1 "K-quant:为什么需要超级块",
 *                                   "6-bit 参数是怎么塞进 12 字节的",
 *                                   "正确性:缩放系数可以提到求和号外面"]
 *         +0 fp16 d, +2 fp16 dmin, +4 scales[12] (8 six-bit s_j + 8 six-bit m_j),
 *         +16 qs[128]: byte 32g+l holds element 64g+l (low) and 64g+32+l (high)
 *         weight w = d*s_j*q - dmin*m_j, j = element / 32
 *   Q6_K  (210 B / 256 weights) [P1 "更低的比特:Q6_K 与 Q2_K 的取舍"]
 *         +0 ql[128] (low 4 bits), +128 qh[64] (high 2 bits), +192 int8 scales[16],
 *         +208 fp16 d;  weight w = d * s_j * q, q in [-32, 31], j = element / 16
 *   Q2_K  ( 84 B / 256 weights) [P1 "更低的比特:Q6_K 与 Q2_K 的取舍"]
 *         +0 scales[16] (s_j low nibble, m_j high), +16 qs[64] (2-bit codes),
 *         +80 fp16 d, +82 fp16 dmin;  weight w = d*s_j*q - dmin*m_j, q in [0, 3],
 *         j = element / 16
 *   Q8_K  (292 B / 256 values)  [P1 "更低的比特:Q6_K 与 Q2_K 的取舍"]
 *         +0 fp32 d, +4 int8 qs[256], +260 int16 bsums[16] (sum of each 16 qs)
 *
 * Parity status of every function is stated next to it and in the design notes.
 */
#ifndef QMM_ORACLE_H
#define QMM_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_Q4_0_BYTES 18
#define ORC_Q8_0_BYTES 34
#define ORC_Q4_K_BYTES 144
#define ORC_Q8_K_BYTES 292
#define ORC_Q6_K_BYTES 210
#define ORC_Q2_K_BYTES 84

/* ---- IEEE binary16 <-> binary32 (definition of the format; RNE) ---- */
uint16_t orc_f32_to_f16(float x);
float    orc_f16_to_f32(uint16_t h);

/* ---- Q4_K 12-byte scale/min field ---- */
void orc_q4_K_get_scale_min(const uint8_t *scales12, int j, uint8_t *s, uint8_t *m);
void orc_q4_K_pack_scales(const uint8_t s[8], const uint8_t m[8], uint8_t out12[12]);

/* ---- weight encoders (input generators; rows of K floats) ---- */
void orc_quantize_q4_0(const float *x, int64_t rows, int64_t K, uint8_t *out);
void orc_quantize_q4_K(const float *x, int64_t rows, int64_t K, uint8_t *out);

/* ---- activation encoders (the GPU must reproduce these bytes exactly) ---- */
void orc_quantize_q8_0(const float *x, int64_t rows, int64_t K, uint8_t *out);
void orc_quantize_q8_K(const float *x, int64_t rows, int64_t K, uint8_t *out);

/* ---- decoders to fp64 (exact: every value is representable) ---- */
void orc_dequantize_q4_0(const uint8_t *w, int64_t rows, int64_t K, double *out);
void orc_dequantize_q4_K(const uint8_t *w, int64_t rows, int64_t K, double *out);
void orc_dequantize_q8_0(const uint8_t *y, int64_t rows, int64_t K, double *out);
void orc_dequantize_q8_K(const uint8_t *y, int64_t rows, int64_t K, double *out);

/* ---- fp64 brute force on dequantized operands (tiny shapes) ----
 * out[m*N+n] = sum_k w[n*K+k]*a[m*K+k];  terms[m*N+n] = sum_k |w*a|            */
void orc_brute_force(const double *w, const double *a, int64_t M, int64_t N,
                     int64_t K, double *out, double *terms);

/* ---- integer path: block dot products with the scales pulled out ----
 * out is fp64, out[m*N+n].  nthreads <= 0 means "all available".          */
void orc_mul_mat_q4_0_q8_0(const uint8_t *w, const uint8_t *y, int64_t M,
                           int64_t N, int64_t K, double *out, int nthreads);
void orc_mul_mat_q4_K_q8_K(const uint8_t *w, const uint8_t *y, int64_t M,
                           int64_t N, int64_t K, double *out, int nthreads);

/* per-sub-block int32 sums P[m][n][K/32] = sum_{i in sub-block} q_i*y_i   */
void orc_q4_K_subblock_sums(const uint8_t *w, const uint8_t *y, int64_t M,
                            int64_t N, int64_t K, int32_t *P);
/* per-block int32 sums P[m][n][K/32] = sum_i (q_i-8)*y_i                  */
void orc_q4_0_block_sums(const uint8_t *w, const uint8_t *y, int64_t M,
                         int64_t N, int64_t K, int32_t *P);

/* sampled outputs: only the listed (m,n) pairs, plus sum|terms| for each  */
void orc_sample_q4_K_q8_K(const uint8_t *w, const uint8_t *y, int64_t M,
                          int64_t N, int64_t K, const int64_t *ms,
                          const int64_t *ns, int64_t count, double *out,
                          double *terms);
void orc_sample_q4_0_q8_0(const uint8_t *w, const uint8_t *y, int64_t M,
                          int64_t N, int64_t K, const int64_t *ms,
                          const int64_t *ns, int64_t count, double *out,
                          double *terms);

/* ---- the documented load-time layouts (byte permutations) ----
 * Q4_K repacked: [N*nb headers of 16 B (d, dmin, scales[12])]
 *                [N*nb payloads of 128 B (qs, same nibble order)]
 *                header of (n,b) at 16*(n*nb+b); payload at 16*N*nb + 128*(n*nb+b)
 * Q4_0 repacked: [N*nb fp16 d, zero-padded to a multiple of 256 B]
 *                [N*nb payloads of 16 B (qs, same nibble order)]            */
int64_t orc_repacked_bytes_q4_0(int64_t N, int64_t K);
int64_t orc_repacked_bytes_q4_K(int64_t N, int64_t K);
void orc_repack_q4_0(const uint8_t *canon, int64_t N, int64_t K, uint8_t *out);
void orc_repack_q4_K(const uint8_t *canon, int64_t N, int64_t K, uint8_t *out);

/* ---- Q6_K (ql[128] | qh[64] | int8 scales[16] | fp16 d; w = d*s_j*q,
 * q in [-32, 31], 16-element groups j).  Bit placement, encoder and layout
 * are readings stated in qmm_oracle.c. ---- */
void orc_q6_K_pack_codes(const int8_t q[256], uint8_t ql_qh[192]);
void orc_quantize_q6_K(const float *x, int64_t rows, int64_t K, uint8_t *out);
void orc_dequantize_q6_K(const uint8_t *w, int64_t rows, int64_t K, double *out);
void orc_mul_mat_q6_K_q8_K(const uint8_t *w, const uint8_t *y, int64_t M,
                           int64_t N, int64_t K, double *out, int nthreads);
/* per-group int32 sums P[m][n][K/16] = sum_{i in group} q_i*y_i          */
void orc_q6_K_group_sums(const uint8_t *w, const uint8_t *y, int64_t M,
                         int64_t N, int64_t K, int32_t *P);
void orc_sample_q6_K_q8_K(const uint8_t *w, const uint8_t *y, int64_t M,
                          int64_t N, int64_t K, const int64_t *ms,
                          const int64_t *ns, int64_t count, double *out,
                          double *terms);
int64_t orc_repacked_bytes_q6_K(int64_t N, int64_t K);
void orc_repack_q6_K(const uint8_t *canon, int64_t N, int64_t K, uint8_t *out);

/* ---- Q2_K (scales[16] (s_j low nibble, m_j high) | qs[64] | fp16 d | fp16 dmin;
 * w = d*s_j*q - dmin*m_j, q in [0, 3], 16-element groups j).  Byte order,
 * code placement, encoder and layout are readings stated in qmm_oracle.c. ---- */
void orc_q2_K_pack_codes(const uint8_t q[256], uint8_t qs[64]);
void orc_quantize_q2_K(const float *x, int64_t rows, int64_t K, uint8_t *out);
void orc_dequantize_q2_K(const uint8_t *w, int64_t rows, int64_t K, double *out);
void orc_mul_mat_q2_K_q8_K(const uint8_t *w, const uint8_t *y, int64_t M,
                           int64_t N, int64_t K, double *out, int nthreads);
/* per-group int32 sums P[m][n][K/16] = sum_{i in group} q_i*y_i          */
void orc_q2_K_group_sums(const uint8_t *w, const uint8_t *y, int64_t M,
                         int64_t N, int64_t K, int32_t *P);
void orc_sample_q2_K_q8_K(const uint8_t *w, const uint8_t *y, int64_t M,
                          int64_t N, int64_t K, const int64_t *ms,
                          const int64_t *ns, int64_t count, double *out,
                          double *terms);
int64_t orc_repacked_bytes_q2_K(int64_t N, int64_t K);
void orc_repack_q2_K(const uint8_t *canon, int64_t N, int64_t K, uint8_t *out);

/* ---- mul_mat_id: out[(t*U+u)*N + n] = mul_mat(W[ids[t*U+u]], y_row)[n] with
 * W a stack [E][N][K] of canonical matrices in format wfmt (0 Q4_0, 1 Q4_K,
 * 2 Q6_K, 3 Q2_K) and y_row = row t (y_per_slot = 0) or t*U+u (1).  Returns
 * -1 for an id outside [0, E) or an unknown format, 0 otherwise.  terms may
 * be NULL. ---- */
int orc_mul_mat_id(int wfmt, const uint8_t *w, int64_t E, int64_t N, int64_t K,
                   const uint8_t *y, const int32_t *ids, int64_t T, int64_t U,
                   int y_per_slot, double *out, double *terms);

int orc_max_threads(void);

#ifdef __cplusplus
}
#endif
#endif /* QMM_ORACLE_H */
