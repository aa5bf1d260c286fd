/*
 * qmm_oracle.c -- plain, slow CPU oracle for the quantized mul_mat.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * CPU-baseline leg of the benchmark; never by the product path.  It includes no
 * header of the GPU library and the GPU library includes nothing from here.
 *
 * Every function follows a passage of the pages (cited per function).  Where
 * the pages leave a step open, the reading taken is stated at the function.
 * Floating point: single IEEE binary32 operations where the encoders fix the
 * precision (no contraction: built with -ffp-contract=off), fp64 for results.
 */
#include "qmm_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define QK4_0 32
#define QK8_0 32
#define QK_K 256

int orc_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static int pick_threads(int nthreads) {
    int mx = orc_max_threads();
    if (nthreads <= 0 || nthreads > mx) return mx;
    return nthreads;
}

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16.  Written from the format's definition: 1 sign bit,     */
/* 5 exponent bits (bias 15), 10 fraction bits, subnormals below 2^-14.      */
/* Rounding is to nearest, ties to even.  (The pages only say "ggml_half",   */
/* i.e. FP16: P1 "最基础的两块:Q4_0 与 Q8_0".)                               */
/* ------------------------------------------------------------------------ */
uint16_t orc_f32_to_f16(float x) {
    uint32_t bits;
    memcpy(&bits, &x, 4);
    uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
    if (isnan(x)) return (uint16_t)(sign | 0x7e00u);
    double a = fabs((double)x);
    if (isinf(x) || a >= 65520.0) return (uint16_t)(sign | 0x7c00u); /* rounds past 65504 */
    if (a == 0.0) return sign;
    /* quantum of the binade that a falls in (subnormal quantum 2^-24) */
    int e;
    frexp(a, &e);              /* a = f * 2^e, f in [0.5, 1) -> binade exponent e-1 */
    int E = e - 1;
    if (E < -14) E = -14;      /* subnormal range shares the quantum of 2^-14's binade */
    double quantum = ldexp(1.0, E - 10);
    double n = nearbyint(a / quantum);   /* exact division by a power of two; RNE */
    double v = n * quantum;
    if (v >= 65536.0) return (uint16_t)(sign | 0x7c00u);
    if (v < ldexp(1.0, -14)) {           /* subnormal: fraction = v / 2^-24 */
        return (uint16_t)(sign | (uint16_t)(v / ldexp(1.0, -24)));
    }
    frexp(v, &e);
    int Ev = e - 1;                      /* v = (1 + frac/1024) * 2^Ev */
    double frac = (v / ldexp(1.0, Ev) - 1.0) * 1024.0;
    return (uint16_t)(sign | (uint16_t)((Ev + 15) << 10) | (uint16_t)frac);
}

float orc_f16_to_f32(uint16_t h) {
    int sign = (h >> 15) & 1;
    int E = (h >> 10) & 0x1f;
    int F = h & 0x3ff;
    double v;
    if (E == 0)
        v = ldexp((double)F, -24);
    else if (E == 31)
        v = F ? NAN : INFINITY;
    else
        v = ldexp(1.0 + F / 1024.0, E - 15);
    return (float)(sign ? -v : v);
}

static float rd_f16(const uint8_t *p) {
    return orc_f16_to_f32((uint16_t)(p[0] | (p[1] << 8)));
}
static void wr_f16(uint8_t *p, uint16_t h) {
    p[0] = (uint8_t)(h & 0xff);
    p[1] = (uint8_t)(h >> 8);
}
static float rd_f32(const uint8_t *p) {
    float f;
    memcpy(&f, p, 4);
    return f;
}
static int16_t rd_i16(const uint8_t *p) {
    return (int16_t)(uint16_t)(p[0] | (p[1] << 8));
}

/* ------------------------------------------------------------------------ */
/* Q4_K 12-byte scale field.  P1 "6-bit 参数是怎么塞进 12 字节的": the decode  */
/* rule there fixes all 96 bits.  This project's statement of that layout,   */
/* as bit pieces (byte, first bit, width), low piece first:                  */
/*                                                                          */
/*   field        low piece            high piece                           */
/*   s_j, j<4     byte j,   bit 0, 6   -                                    */
/*   m_j, j<4     byte j+4, bit 0, 6   -                                    */
/*   s_j, j>=4    byte j+4, bit 0, 4   byte j-4, bit 6, 2                    */
/*   m_j, j>=4    byte j+4, bit 4, 4   byte j,   bit 6, 2                    */
/*                                                                          */
/* (The prose of that section puts the two nibbles of bytes 8..11 the other  */
/* way round; the decode rule is followed.)  Decoding reads the pieces and   */
/* joins them; packing writes them.  Every one of the 96 bits belongs to     */
/* exactly one piece, which the exhaustive round-trip test relies on.        */
/* ------------------------------------------------------------------------ */
typedef struct { int byte, bit, width; } bit_piece;

/* the pieces of field `which` (0 = scale s_j, 1 = min m_j) of sub-block j;  */
/* returns the number of pieces (1 or 2), low piece first                    */
static int scale_field_pieces(int j, int which, bit_piece pc[2]) {
    if (j < 4) {
        pc[0] = (bit_piece){ j + 4 * which, 0, 6 };
        return 1;
    }
    pc[0] = (bit_piece){ j + 4, 4 * which, 4 };
    pc[1] = (bit_piece){ which ? j : j - 4, 6, 2 };
    return 2;
}

static uint8_t read_field(const uint8_t *q, int j, int which) {
    bit_piece pc[2];
    int n = scale_field_pieces(j, which, pc), v = 0, at = 0;
    for (int i = 0; i < n; ++i) {
        v |= ((q[pc[i].byte] >> pc[i].bit) & ((1 << pc[i].width) - 1)) << at;
        at += pc[i].width;
    }
    return (uint8_t)v;
}

static void write_field(uint8_t *q, int j, int which, int v) {
    bit_piece pc[2];
    int n = scale_field_pieces(j, which, pc);
    for (int i = 0; i < n; ++i) {
        int mask = (1 << pc[i].width) - 1;
        q[pc[i].byte] = (uint8_t)((q[pc[i].byte] & ~(mask << pc[i].bit)) | ((v & mask) << pc[i].bit));
        v >>= pc[i].width;
    }
}

void orc_q4_K_get_scale_min(const uint8_t *q, int j, uint8_t *s, uint8_t *m) {
    *s = read_field(q, j, 0);
    *m = read_field(q, j, 1);
}

void orc_q4_K_pack_scales(const uint8_t s[8], const uint8_t m[8], uint8_t out[12]) {
    memset(out, 0, 12);
    for (int j = 0; j < 8; ++j) {
        write_field(out, j, 0, s[j] & 63);
        write_field(out, j, 1, m[j] & 63);
    }
}

static int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

/* ------------------------------------------------------------------------ */
/* Q4_0 encoder (input generator).  P1 "最基础的两块:Q4_0 与 Q8_0": per 32    */
/* weights, d = -xmax/8 with xmax the signed element of largest magnitude,   */
/* w ~ d*(q-8).  Readings: first index wins a tie in |x|; q = rint(x/d)+8    */
/* computed as x*(1/d) in fp32, ties to even, clamped to [0,15]; the high   */
/* nibble of byte l holds element l+16 (the split-half order the K-quant     */
/* section uses).                                                           */
/* ------------------------------------------------------------------------ */
void orc_quantize_q4_0(const float *x, int64_t rows, int64_t K, uint8_t *out) {
    const int64_t nb = K / QK4_0;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const float *xb = x + r * K + b * QK4_0;
            uint8_t *blk = out + (r * nb + b) * ORC_Q4_0_BYTES;
            float amax = 0.0f, xmax = 0.0f;
            for (int i = 0; i < QK4_0; ++i) {
                float a = fabsf(xb[i]);
                if (a > amax) { amax = a; xmax = xb[i]; }
            }
            float d = 0.0f - xmax / 8.0f;   /* +0 for an all-zero block */
            float id = d != 0.0f ? 1.0f / d : 0.0f;
            uint8_t q[QK4_0];
            for (int i = 0; i < QK4_0; ++i) {
                float t = xb[i] * id;
                q[i] = (uint8_t)clampi((int)rintf(t) + 8, 0, 15);
            }
            wr_f16(blk, orc_f32_to_f16(d));
            for (int l = 0; l < 16; ++l)
                blk[2 + l] = (uint8_t)(q[l] | (q[l + 16] << 4));
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Q4_K encoder (input generator).  P1 "K-quant:为什么需要超级块" fixes the   */
/* decoded value w = d*s_j*q - dmin*m_j with q in [0,15] and 6-bit s_j, m_j; */
/* the nibble order comes from "正确性:缩放系数可以提到求和号外面" (byte l of  */
/* 64-element group g holds element l low, element l+32 high).  The pages do */
/* not give the scale search; the plain min/max reading is taken:            */
/*   lo_j = min(0, min x), hi_j = max x, sc_j = (hi_j - lo_j)/15, mn_j = -lo_j */
/*   d = max sc_j / 63, dmin = max mn_j / 63                                 */
/*   s_j = rint(sc_j/d), m_j = rint(mn_j/dmin), clamped to [0,63]             */
/*   with D_j = f16(d)*s_j, M_j = f16(dmin)*m_j: q = rint((x+M_j)/D_j) in [0,15] */
/* ------------------------------------------------------------------------ */
void orc_quantize_q4_K(const float *x, int64_t rows, int64_t K, uint8_t *out) {
    const int64_t nb = K / QK_K;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const float *xb = x + r * K + b * QK_K;
            uint8_t *blk = out + (r * nb + b) * ORC_Q4_K_BYTES;
            float sc[8], mn[8];
            float maxsc = 0.0f, maxmn = 0.0f;
            for (int j = 0; j < 8; ++j) {
                const float *xs = xb + 32 * j;
                float lo = xs[0], hi = xs[0];
                for (int i = 1; i < 32; ++i) {
                    if (xs[i] < lo) lo = xs[i];
                    if (xs[i] > hi) hi = xs[i];
                }
                if (!(lo < 0.0f)) lo = 0.0f;
                sc[j] = (hi - lo) / 15.0f;
                mn[j] = 0.0f - lo;
                if (sc[j] > maxsc) maxsc = sc[j];
                if (mn[j] > maxmn) maxmn = mn[j];
            }
            float d = maxsc / 63.0f;
            float dmin = maxmn / 63.0f;
            uint8_t s[8], m[8];
            for (int j = 0; j < 8; ++j) {
                s[j] = (uint8_t)(d > 0.0f ? clampi((int)rintf(sc[j] / d), 0, 63) : 0);
                m[j] = (uint8_t)(dmin > 0.0f ? clampi((int)rintf(mn[j] / dmin), 0, 63) : 0);
            }
            uint16_t dh = orc_f32_to_f16(d), dmh = orc_f32_to_f16(dmin);
            float df = orc_f16_to_f32(dh), dmf = orc_f16_to_f32(dmh);
            uint8_t q[QK_K];
            for (int j = 0; j < 8; ++j) {
                float Dj = df * (float)s[j];
                float Mj = dmf * (float)m[j];
                for (int i = 0; i < 32; ++i) {
                    int k = 32 * j + i;
                    q[k] = (uint8_t)(Dj > 0.0f ? clampi((int)rintf((xb[k] + Mj) / Dj), 0, 15) : 0);
                }
            }
            wr_f16(blk, dh);
            wr_f16(blk + 2, dmh);
            orc_q4_K_pack_scales(s, m, blk + 4);
            for (int g = 0; g < 4; ++g)
                for (int l = 0; l < 32; ++l)
                    blk[16 + 32 * g + l] = (uint8_t)(q[64 * g + l] | (q[64 * g + 32 + l] << 4));
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Activation encoders.  P1 "最基础的两块:Q4_0 与 Q8_0" (Q8_0: symmetric      */
/* int8, fp16 d, 32 values) and "更低的比特" (Q8_K: fp32 d, 256 int8 and      */
/* int16 bsums, each the sum of 16 consecutive values; also "正确性" where   */
/* bsums are said to be filled while quantizing).  The formula is not on the */
/* pages; reading: amax = max|x|, d = amax/127, id = d ? 1/d : 0,            */
/* y = rint(x*id) (one fp32 multiply, ties to even) clamped to [-127,127].   */
/* Q8_0 computes y from the fp32 d and stores f16(d).                        */
/* ------------------------------------------------------------------------ */
static void q8_block(const float *xb, int n, float *d_out, int8_t *q) {
    float amax = 0.0f;
    for (int i = 0; i < n; ++i) {
        float a = fabsf(xb[i]);
        if (a > amax) amax = a;
    }
    float d = amax / 127.0f;
    float id = d != 0.0f ? 1.0f / d : 0.0f;
    for (int i = 0; i < n; ++i) {
        float t = xb[i] * id;
        q[i] = (int8_t)clampi((int)rintf(t), -127, 127);
    }
    *d_out = d;
}

void orc_quantize_q8_0(const float *x, int64_t rows, int64_t K, uint8_t *out) {
    const int64_t nb = K / QK8_0;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            uint8_t *blk = out + (r * nb + b) * ORC_Q8_0_BYTES;
            float d;
            int8_t q[QK8_0];
            q8_block(x + r * K + b * QK8_0, QK8_0, &d, q);
            wr_f16(blk, orc_f32_to_f16(d));
            memcpy(blk + 2, q, QK8_0);
        }
}

void orc_quantize_q8_K(const float *x, int64_t rows, int64_t K, uint8_t *out) {
    const int64_t nb = K / QK_K;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            uint8_t *blk = out + (r * nb + b) * ORC_Q8_K_BYTES;
            float d;
            int8_t q[QK_K];
            q8_block(x + r * K + b * QK_K, QK_K, &d, q);
            memcpy(blk, &d, 4);
            memcpy(blk + 4, q, QK_K);
            for (int g = 0; g < 16; ++g) {
                int s = 0;
                for (int i = 0; i < 16; ++i) s += q[16 * g + i];
                uint16_t u = (uint16_t)(int16_t)s;
                blk[260 + 2 * g] = (uint8_t)(u & 0xff);
                blk[260 + 2 * g + 1] = (uint8_t)(u >> 8);
            }
        }
}

/* ------------------------------------------------------------------------ */
/* Decoders.  Q4_0: w = d*(q-8); Q4_K: w = d*s_j*q - dmin*m_j; Q8: a = d*y.   */
/* (P1 "最基础的两块" and "K-quant:为什么需要超级块".)  All products are exact  */
/* in fp64 (at most 11+6+4 significant bits).                                */
/* ------------------------------------------------------------------------ */
static int q4_0_nibble(const uint8_t *qs, int i) {
    return i < 16 ? (qs[i] & 0x0f) : (qs[i - 16] >> 4);
}
static int q4_K_nibble(const uint8_t *qs, int k) {
    int g = k / 64, r = k % 64;
    uint8_t byte = qs[32 * g + (r % 32)];
    return r < 32 ? (byte & 0x0f) : (byte >> 4);
}

void orc_dequantize_q4_0(const uint8_t *w, int64_t rows, int64_t K, double *out) {
    const int64_t nb = K / QK4_0;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *blk = w + (r * nb + b) * ORC_Q4_0_BYTES;
            double d = rd_f16(blk);
            for (int i = 0; i < QK4_0; ++i)
                out[r * K + b * QK4_0 + i] = d * (q4_0_nibble(blk + 2, i) - 8);
        }
}

void orc_dequantize_q4_K(const uint8_t *w, int64_t rows, int64_t K, double *out) {
    const int64_t nb = K / QK_K;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *blk = w + (r * nb + b) * ORC_Q4_K_BYTES;
            double d = rd_f16(blk), dmin = rd_f16(blk + 2);
            for (int k = 0; k < QK_K; ++k) {
                uint8_t s, m;
                orc_q4_K_get_scale_min(blk + 4, k / 32, &s, &m);
                out[r * K + b * QK_K + k] = d * s * q4_K_nibble(blk + 16, k) - dmin * m;
            }
        }
}

void orc_dequantize_q8_0(const uint8_t *y, int64_t rows, int64_t K, double *out) {
    const int64_t nb = K / QK8_0;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *blk = y + (r * nb + b) * ORC_Q8_0_BYTES;
            double d = rd_f16(blk);
            for (int i = 0; i < QK8_0; ++i)
                out[r * K + b * QK8_0 + i] = d * (int8_t)blk[2 + i];
        }
}

void orc_dequantize_q8_K(const uint8_t *y, int64_t rows, int64_t K, double *out) {
    const int64_t nb = K / QK_K;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *blk = y + (r * nb + b) * ORC_Q8_K_BYTES;
            double d = rd_f32(blk);
            for (int i = 0; i < QK_K; ++i)
                out[r * K + b * QK_K + i] = d * (int8_t)blk[4 + i];
        }
}

/* ------------------------------------------------------------------------ */
/* The plain definition C[m,n] = sum_k A[m,k] W[n,k] (P3 "从数学表达式到真实 */
/* 存储:混合精度 GEMM 的计算对象"), in fp64 on decoded values.                */
/* ------------------------------------------------------------------------ */
void orc_brute_force(const double *w, const double *a, int64_t M, int64_t N,
                     int64_t K, double *out, double *terms) {
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0, t = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = w[n * K + k] * a[m * K + k];
                s += p;
                t += fabs(p);
            }
            out[m * N + n] = s;
            if (terms) terms[m * N + n] = t;
        }
}

/* ------------------------------------------------------------------------ */
/* Integer path.  P1 "正确性:缩放系数可以提到求和号外面": for one sub-block,    */
/* sum w_i a_i = d*d_a*s*sum q_i y_i - dmin*d_a*m*sum y_i, with sum y_i taken */
/* from bsums (two 16-element sums per 32-element sub-block, "min 项与最终归 */
/* 约").  Per super-block: P_j (int32), S = sum_j s_j P_j, Mn = sum_j m_j Y_j,*/
/* contribution d_a*(d*S - dmin*Mn); accumulated in fp64.                    */
/* Q4_0 x Q8_0: P_b = sum (q_i-8) y_i, contribution d_w*d_a*P_b.             */
/* ------------------------------------------------------------------------ */
static double q4_K_row_dot(const uint8_t *wrow, const uint8_t *yrow, int64_t nb,
                           int32_t *P_out, double *terms) {
    double acc = 0.0, tacc = 0.0;
    for (int64_t b = 0; b < nb; ++b) {
        const uint8_t *wb = wrow + b * ORC_Q4_K_BYTES;
        const uint8_t *yb = yrow + b * ORC_Q8_K_BYTES;
        float d = rd_f16(wb), dmin = rd_f16(wb + 2), da = rd_f32(yb);
        int32_t S = 0, Mn = 0;
        for (int j = 0; j < 8; ++j) {
            uint8_t s, m;
            orc_q4_K_get_scale_min(wb + 4, j, &s, &m);
            int32_t P = 0;
            for (int i = 0; i < 32; ++i) {
                int k = 32 * j + i;
                int q = q4_K_nibble(wb + 16, k);
                int y = (int8_t)yb[4 + k];
                P += q * y;
                if (terms) tacc += fabs(((double)d * s * q - (double)dmin * m) * ((double)da * y));
            }
            if (P_out) P_out[b * 8 + j] = P;
            int32_t Y = rd_i16(yb + 260 + 4 * j) + rd_i16(yb + 260 + 4 * j + 2);
            S += (int32_t)s * P;
            Mn += (int32_t)m * Y;
        }
        acc += (double)da * ((double)d * S - (double)dmin * Mn);
    }
    if (terms) *terms = tacc;
    return acc;
}

static double q4_0_row_dot(const uint8_t *wrow, const uint8_t *yrow, int64_t nb,
                           int32_t *P_out, double *terms) {
    double acc = 0.0, tacc = 0.0;
    for (int64_t b = 0; b < nb; ++b) {
        const uint8_t *wb = wrow + b * ORC_Q4_0_BYTES;
        const uint8_t *yb = yrow + b * ORC_Q8_0_BYTES;
        double dw = rd_f16(wb), da = rd_f16(yb);
        int32_t P = 0;
        for (int i = 0; i < QK4_0; ++i) {
            int q = q4_0_nibble(wb + 2, i) - 8;
            int y = (int8_t)yb[2 + i];
            P += q * y;
            if (terms) tacc += fabs(dw * q * da * y);
        }
        if (P_out) P_out[b] = P;
        acc += dw * da * P;
    }
    if (terms) *terms = tacc;
    return acc;
}

void orc_mul_mat_q4_K_q8_K(const uint8_t *w, const uint8_t *y, int64_t M,
                           int64_t N, int64_t K, double *out, int nthreads) {
    const int64_t nb = K / QK_K;
    const int nt = pick_threads(nthreads);
    (void)nt;
#pragma omp parallel for collapse(2) schedule(static) num_threads(nt)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            out[m * N + n] = q4_K_row_dot(w + n * nb * ORC_Q4_K_BYTES,
                                          y + m * nb * ORC_Q8_K_BYTES, nb, NULL, NULL);
}

void orc_mul_mat_q4_0_q8_0(const uint8_t *w, const uint8_t *y, int64_t M,
                           int64_t N, int64_t K, double *out, int nthreads) {
    const int64_t nb = K / QK4_0;
    const int nt = pick_threads(nthreads);
    (void)nt;
#pragma omp parallel for collapse(2) schedule(static) num_threads(nt)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            out[m * N + n] = q4_0_row_dot(w + n * nb * ORC_Q4_0_BYTES,
                                          y + m * nb * ORC_Q8_0_BYTES, nb, NULL, NULL);
}

void orc_q4_K_subblock_sums(const uint8_t *w, const uint8_t *y, int64_t M,
                            int64_t N, int64_t K, int32_t *P) {
    const int64_t nb = K / QK_K;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            (void)q4_K_row_dot(w + n * nb * ORC_Q4_K_BYTES, y + m * nb * ORC_Q8_K_BYTES,
                               nb, P + (m * N + n) * (K / 32), NULL);
}

void orc_q4_0_block_sums(const uint8_t *w, const uint8_t *y, int64_t M,
                         int64_t N, int64_t K, int32_t *P) {
    const int64_t nb = K / QK4_0;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            (void)q4_0_row_dot(w + n * nb * ORC_Q4_0_BYTES, y + m * nb * ORC_Q8_0_BYTES,
                               nb, P + (m * N + n) * nb, NULL);
}

void orc_sample_q4_K_q8_K(const uint8_t *w, const uint8_t *y, int64_t M,
                          int64_t N, int64_t K, const int64_t *ms,
                          const int64_t *ns, int64_t count, double *out,
                          double *terms) {
    const int64_t nb = K / QK_K;
    (void)M; (void)N;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < count; ++i)
        out[i] = q4_K_row_dot(w + ns[i] * nb * ORC_Q4_K_BYTES,
                              y + ms[i] * nb * ORC_Q8_K_BYTES, nb, NULL, &terms[i]);
}

void orc_sample_q4_0_q8_0(const uint8_t *w, const uint8_t *y, int64_t M,
                          int64_t N, int64_t K, const int64_t *ms,
                          const int64_t *ns, int64_t count, double *out,
                          double *terms) {
    const int64_t nb = K / QK4_0;
    (void)M; (void)N;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < count; ++i)
        out[i] = q4_0_row_dot(w + ns[i] * nb * ORC_Q4_0_BYTES,
                              y + ms[i] * nb * ORC_Q8_0_BYTES, nb, NULL, &terms[i]);
}

/* ------------------------------------------------------------------------ */
/* Load-time layouts.  P3 "Ladder Permutation" describes an offline,        */
/* lossless permutation of static weights into the order the kernel reads.   */
/* The layouts below are this project's own; this is their definition as an */
/* index map, written independently of the GPU repack kernels.               */
/* ------------------------------------------------------------------------ */
int64_t orc_repacked_bytes_q4_K(int64_t N, int64_t K) {
    return N * (K / QK_K) * ORC_Q4_K_BYTES;
}

int64_t orc_repacked_bytes_q4_0(int64_t N, int64_t K) {
    int64_t nblk = N * (K / QK4_0);
    int64_t dsec = (2 * nblk + 255) / 256 * 256;
    return dsec + 16 * nblk;
}

void orc_repack_q4_K(const uint8_t *canon, int64_t N, int64_t K, uint8_t *out) {
    const int64_t nb = K / QK_K;
    const int64_t pay0 = 16 * N * nb;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *src = canon + (n * nb + b) * ORC_Q4_K_BYTES;
            memcpy(out + 16 * (n * nb + b), src, 16);
            memcpy(out + pay0 + 128 * (n * nb + b), src + 16, 128);
        }
}

void orc_repack_q4_0(const uint8_t *canon, int64_t N, int64_t K, uint8_t *out) {
    const int64_t nblk = N * (K / QK4_0);
    const int64_t dsec = (2 * nblk + 255) / 256 * 256;
    memset(out, 0, (size_t)dsec);
    for (int64_t i = 0; i < nblk; ++i) {
        const uint8_t *src = canon + i * ORC_Q4_0_BYTES;
        memcpy(out + 2 * i, src, 2);
        memcpy(out + dsec + 16 * i, src + 2, 16);
    }
}

/* ======================================================================== */
/* Q6_K (210 B / 256 weights).  P1 "更低的比特:Q6_K 与 Q2_K 的取舍": ql[128]  */
/* holds the low 4 bits of each 6-bit value, qh[64] the high 2 bits,         */
/* scales[16] are plain int8 (one per 16-element group), d is fp16; the      */
/* 6-bit value is a signed integer q in [-32, 31] with no min term:          */
/*   w = d * s_j * q,  j = element / 16.                                     */
/* Readings (the pages list the fields but not the bit placement):           */
/*   byte order   ql @0, qh @128, scales @192, d @208 (the order listed);    */
/*   low 4 bits   of element k sit in ql byte 32*(k/64) + (k%64)%32, low     */
/*                nibble for (k%64) < 32, high nibble otherwise (the split-  */
/*                half order of the Q4_K codes);                             */
/*   high 2 bits  of element k sit in qh byte k%64, bits 2*(k/64)+1..2*(k/64);*/
/*   stored code  u = q + 32 in [0, 63].                                     */
/* Parity with llama.cpp's own Q6_K files is unpinned (no vectors here).     */
/* ======================================================================== */
static int q6_K_code(const uint8_t *blk, int k) {
    int g = k / 64, r = k % 64;
    uint8_t lb = blk[32 * g + (r % 32)];
    int lo = r < 32 ? (lb & 0x0f) : (lb >> 4);
    int hi = (blk[128 + r] >> (2 * g)) & 3;
    return (lo | (hi << 4)) - 32;
}

void orc_q6_K_pack_codes(const int8_t q[256], uint8_t ql_qh[192]) {
    memset(ql_qh, 0, 192);
    for (int k = 0; k < 256; ++k) {
        int u = q[k] + 32, g = k / 64, r = k % 64;
        uint8_t *lb = ql_qh + 32 * g + (r % 32);
        *lb |= (uint8_t)(r < 32 ? (u & 0x0f) : ((u & 0x0f) << 4));
        ql_qh[128 + r] |= (uint8_t)(((u >> 4) & 3) << (2 * g));
    }
}

/* Q6_K encoder (input generator).  Plain symmetric reading, as for Q4_0:    */
/* per 16-element group, xm_j = signed element of largest |x| (first wins),  */
/* sc_j = xm_j / -32 (so xm_j maps to q = -32); d = max |sc_j| / 127;        */
/* s_j = rint(sc_j / d) clamped to [-127, 127]; with D_j = f16(d) * s_j:     */
/* q = rint(x / D_j) clamped to [-32, 31], or 0 where D_j = 0.               */
void orc_quantize_q6_K(const float *x, int64_t rows, int64_t K, uint8_t *out) {
    const int64_t nb = K / QK_K;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const float *xb = x + r * K + b * QK_K;
            uint8_t *blk = out + (r * nb + b) * ORC_Q6_K_BYTES;
            float sc[16], maxsc = 0.0f;
            for (int j = 0; j < 16; ++j) {
                float amax = 0.0f, xm = 0.0f;
                for (int i = 0; i < 16; ++i) {
                    float a = fabsf(xb[16 * j + i]);
                    if (a > amax) { amax = a; xm = xb[16 * j + i]; }
                }
                sc[j] = xm / -32.0f;
                if (fabsf(sc[j]) > maxsc) maxsc = fabsf(sc[j]);
            }
            float d = maxsc / 127.0f;
            uint16_t dh = orc_f32_to_f16(d);
            float df = orc_f16_to_f32(dh);
            int8_t s[16], q[256];
            for (int j = 0; j < 16; ++j) {
                s[j] = (int8_t)(d > 0.0f ? clampi((int)rintf(sc[j] / d), -127, 127) : 0);
                float Dj = df * (float)s[j];
                for (int i = 0; i < 16; ++i) {
                    int k = 16 * j + i;
                    q[k] = (int8_t)(Dj != 0.0f ? clampi((int)rintf(xb[k] / Dj), -32, 31) : 0);
                }
            }
            orc_q6_K_pack_codes(q, blk);
            for (int j = 0; j < 16; ++j) blk[192 + j] = (uint8_t)s[j];
            wr_f16(blk + 208, dh);
        }
}

void orc_dequantize_q6_K(const uint8_t *w, int64_t rows, int64_t K, double *out) {
    const int64_t nb = K / QK_K;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *blk = w + (r * nb + b) * ORC_Q6_K_BYTES;
            double d = rd_f16(blk + 208);
            for (int k = 0; k < QK_K; ++k)
                out[r * K + b * QK_K + k] = d * (int8_t)blk[192 + k / 16] * q6_K_code(blk, k);
        }
}

/* Integer path, the same factorization as Q4_K without the min term:        */
/* P_j = sum_{i in j} q_i y_i over the 16-element group j (int32),           */
/* S = sum_j s_j P_j (int32), contribution d_a * d * S (fp64).               */
static double q6_K_row_dot(const uint8_t *wrow, const uint8_t *yrow, int64_t nb,
                           int32_t *P_out, double *terms) {
    double acc = 0.0, tacc = 0.0;
    for (int64_t b = 0; b < nb; ++b) {
        const uint8_t *wb = wrow + b * ORC_Q6_K_BYTES;
        const uint8_t *yb = yrow + b * ORC_Q8_K_BYTES;
        double d = rd_f16(wb + 208), da = rd_f32(yb);
        int32_t S = 0;
        for (int j = 0; j < 16; ++j) {
            int s = (int8_t)wb[192 + j];
            int32_t P = 0;
            for (int i = 0; i < 16; ++i) {
                int k = 16 * j + i;
                int q = q6_K_code(wb, k);
                int yv = (int8_t)yb[4 + k];
                P += q * yv;
                if (terms) tacc += fabs(d * s * q * da * yv);
            }
            if (P_out) P_out[b * 16 + j] = P;
            S += s * P;
        }
        acc += da * (d * (double)S);
    }
    if (terms) *terms = tacc;
    return acc;
}

void orc_mul_mat_q6_K_q8_K(const uint8_t *w, const uint8_t *y, int64_t M,
                           int64_t N, int64_t K, double *out, int nthreads) {
    const int64_t nb = K / QK_K;
    const int nt = pick_threads(nthreads);
    (void)nt;
#pragma omp parallel for collapse(2) schedule(static) num_threads(nt)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            out[m * N + n] = q6_K_row_dot(w + n * nb * ORC_Q6_K_BYTES,
                                          y + m * nb * ORC_Q8_K_BYTES, nb, NULL, NULL);
}

void orc_q6_K_group_sums(const uint8_t *w, const uint8_t *y, int64_t M,
                         int64_t N, int64_t K, int32_t *P) {
    const int64_t nb = K / QK_K;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            q6_K_row_dot(w + n * nb * ORC_Q6_K_BYTES, y + m * nb * ORC_Q8_K_BYTES, nb,
                         P + (m * N + n) * (K / 16), NULL);
}

void orc_sample_q6_K_q8_K(const uint8_t *w, const uint8_t *y, int64_t M,
                          int64_t N, int64_t K, const int64_t *ms,
                          const int64_t *ns, int64_t count, double *out,
                          double *terms) {
    const int64_t nb = K / QK_K;
    (void)M; (void)N;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < count; ++i)
        out[i] = q6_K_row_dot(w + ns[i] * nb * ORC_Q6_K_BYTES,
                              y + ms[i] * nb * ORC_Q8_K_BYTES, nb, NULL, &terms[i]);
}

/* Q6_K load-time layout (this library's own byte permutation):               */
/*   [N*nb fp16 d, zero-padded to a multiple of 256 B][N*nb scales of 16 B]   */
/*   [N*nb ql of 128 B][N*nb qh of 64 B], block (n,b) at index n*nb+b.        */
int64_t orc_repacked_bytes_q6_K(int64_t N, int64_t K) {
    int64_t nblk = N * (K / QK_K);
    return (2 * nblk + 255) / 256 * 256 + 208 * nblk;
}

void orc_repack_q6_K(const uint8_t *canon, int64_t N, int64_t K, uint8_t *out) {
    const int64_t nblk = N * (K / QK_K);
    const int64_t dsec = (2 * nblk + 255) / 256 * 256;
    const int64_t s0 = dsec, l0 = s0 + 16 * nblk, h0 = l0 + 128 * nblk;
    memset(out, 0, (size_t)dsec);
    for (int64_t i = 0; i < nblk; ++i) {
        const uint8_t *src = canon + i * ORC_Q6_K_BYTES;
        memcpy(out + 2 * i, src + 208, 2);
        memcpy(out + s0 + 16 * i, src + 192, 16);
        memcpy(out + l0 + 128 * i, src, 128);
        memcpy(out + h0 + 64 * i, src + 128, 64);
    }
}

/* ======================================================================== */
/* Q2_K.  P1 "更低的比特:Q6_K 与 Q2_K 的取舍": 256 2-bit values in 64 bytes,  */
/* 16 sub-blocks (16 elements each) with a 4-bit scale and a 4-bit min,     */
/* fp16 d and dmin: 84 B / 256 = 2.625 bpw, asymmetric like Q4_K:           */
/*   w = d * s_j * q - dmin * m_j,  q in [0, 3],  j = element / 16.         */
/* Readings (the page gives the fields and sizes, not the placement):      */
/*   byte order   scales[16] @0, qs[64] @16, d @80, dmin @82;               */
/*   scale byte j s_j in the low nibble, m_j in the high nibble (the order */
/*                the Q4_K decode rule uses for its packed 4-bit pairs);    */
/*   codes        element k = 128h + 32s + l sits in qs byte 32h + l,       */
/*                bits 2s..2s+1 (BitBLAS page, "位级打包": field i of a word */
/*                is (u >> b*i) & (2^b - 1), here with b = 2 on bytes, over */
/*                split halves of 128 elements as the Q4_K codes use).      */
/* Parity with llama.cpp's own Q2_K files is unpinned (no vectors here).    */
/* ======================================================================== */
static int q2_K_code(const uint8_t *blk, int k) {
    int h = k / 128, sh = (k % 128) / 32, l = k % 32;
    return (blk[16 + 32 * h + l] >> (2 * sh)) & 3;
}

void orc_q2_K_pack_codes(const uint8_t q[256], uint8_t qs[64]) {
    memset(qs, 0, 64);
    for (int k = 0; k < 256; ++k) {
        int h = k / 128, sh = (k % 128) / 32, l = k % 32;
        qs[32 * h + l] |= (uint8_t)((q[k] & 3) << (2 * sh));
    }
}

/* Q2_K encoder (input generator), the Q4_K reading with 2-bit codes and     */
/* 4-bit scales: per 16-element group lo = min(0, min x), hi = max x,        */
/* sc = (hi - lo)/3, mn = -lo; d = max sc/15, dmin = max mn/15;              */
/* s_j = rint(sc/d), m_j = rint(mn/dmin), both clamped to [0, 15]; with      */
/* D_j = f16(d)*s_j and M_j = f16(dmin)*m_j: q = rint((x + M_j)/D_j)         */
/* clamped to [0, 3], or 0 where D_j = 0.                                    */
void orc_quantize_q2_K(const float *x, int64_t rows, int64_t K, uint8_t *out) {
    const int64_t nb = K / QK_K;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const float *xb = x + r * K + b * QK_K;
            uint8_t *blk = out + (r * nb + b) * ORC_Q2_K_BYTES;
            float sc[16], mn[16], maxsc = 0.0f, maxmn = 0.0f;
            for (int j = 0; j < 16; ++j) {
                const float *xs = xb + 16 * j;
                float lo = xs[0], hi = xs[0];
                for (int i = 1; i < 16; ++i) {
                    if (xs[i] < lo) lo = xs[i];
                    if (xs[i] > hi) hi = xs[i];
                }
                if (!(lo < 0.0f)) lo = 0.0f;
                sc[j] = (hi - lo) / 3.0f;
                mn[j] = 0.0f - lo;
                if (sc[j] > maxsc) maxsc = sc[j];
                if (mn[j] > maxmn) maxmn = mn[j];
            }
            float d = maxsc / 15.0f, dmin = maxmn / 15.0f;
            uint8_t s[16], m[16], q[QK_K];
            for (int j = 0; j < 16; ++j) {
                s[j] = (uint8_t)(d > 0.0f ? clampi((int)rintf(sc[j] / d), 0, 15) : 0);
                m[j] = (uint8_t)(dmin > 0.0f ? clampi((int)rintf(mn[j] / dmin), 0, 15) : 0);
            }
            uint16_t dh = orc_f32_to_f16(d), dmh = orc_f32_to_f16(dmin);
            float df = orc_f16_to_f32(dh), dmf = orc_f16_to_f32(dmh);
            for (int j = 0; j < 16; ++j) {
                float Dj = df * (float)s[j], Mj = dmf * (float)m[j];
                for (int i = 0; i < 16; ++i) {
                    int k = 16 * j + i;
                    q[k] = (uint8_t)(Dj > 0.0f ? clampi((int)rintf((xb[k] + Mj) / Dj), 0, 3) : 0);
                }
                blk[j] = (uint8_t)(s[j] | (m[j] << 4));
            }
            orc_q2_K_pack_codes(q, blk + 16);
            wr_f16(blk + 80, dh);
            wr_f16(blk + 82, dmh);
        }
}

void orc_dequantize_q2_K(const uint8_t *w, int64_t rows, int64_t K, double *out) {
    const int64_t nb = K / QK_K;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *blk = w + (r * nb + b) * ORC_Q2_K_BYTES;
            double d = rd_f16(blk + 80), dmin = rd_f16(blk + 82);
            for (int k = 0; k < QK_K; ++k) {
                int sj = blk[k / 16] & 15, mj = blk[k / 16] >> 4;
                out[r * K + b * QK_K + k] = d * sj * q2_K_code(blk, k) - dmin * mj;
            }
        }
}

/* Integer path, the Q4_K factorization over 16-element groups (one Q8_K    */
/* bsum per group): P_j = sum_{i in j} q_i y_i, S = sum_j s_j P_j,           */
/* Mn = sum_j m_j bsums[j], contribution d_a * (d*S - dmin*Mn).              */
static double q2_K_row_dot(const uint8_t *wrow, const uint8_t *yrow, int64_t nb,
                           int32_t *P_out, double *terms) {
    double acc = 0.0, tacc = 0.0;
    for (int64_t b = 0; b < nb; ++b) {
        const uint8_t *wb = wrow + b * ORC_Q2_K_BYTES;
        const uint8_t *yb = yrow + b * ORC_Q8_K_BYTES;
        double d = rd_f16(wb + 80), dmin = rd_f16(wb + 82), da = rd_f32(yb);
        int32_t S = 0, Mn = 0;
        for (int j = 0; j < 16; ++j) {
            int sj = wb[j] & 15, mj = wb[j] >> 4;
            int32_t P = 0;
            for (int i = 0; i < 16; ++i) {
                int k = 16 * j + i;
                int q = q2_K_code(wb, k);
                int yv = (int8_t)yb[4 + k];
                P += q * yv;
                if (terms) tacc += fabs((d * sj * q - dmin * mj) * da * yv);
            }
            if (P_out) P_out[b * 16 + j] = P;
            S += sj * P;
            Mn += mj * (int32_t)rd_i16(yb + 260 + 2 * j);
        }
        acc += da * (d * (double)S - dmin * (double)Mn);
    }
    if (terms) *terms = tacc;
    return acc;
}

void orc_mul_mat_q2_K_q8_K(const uint8_t *w, const uint8_t *y, int64_t M,
                           int64_t N, int64_t K, double *out, int nthreads) {
    const int64_t nb = K / QK_K;
    const int nt = pick_threads(nthreads);
    (void)nt;
#pragma omp parallel for collapse(2) schedule(static) num_threads(nt)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            out[m * N + n] = q2_K_row_dot(w + n * nb * ORC_Q2_K_BYTES,
                                          y + m * nb * ORC_Q8_K_BYTES, nb, NULL, NULL);
}

void orc_q2_K_group_sums(const uint8_t *w, const uint8_t *y, int64_t M,
                         int64_t N, int64_t K, int32_t *P) {
    const int64_t nb = K / QK_K;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            q2_K_row_dot(w + n * nb * ORC_Q2_K_BYTES, y + m * nb * ORC_Q8_K_BYTES, nb,
                         P + (m * N + n) * (K / 16), NULL);
}

void orc_sample_q2_K_q8_K(const uint8_t *w, const uint8_t *y, int64_t M,
                          int64_t N, int64_t K, const int64_t *ms,
                          const int64_t *ns, int64_t count, double *out,
                          double *terms) {
    const int64_t nb = K / QK_K;
    (void)M; (void)N;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < count; ++i)
        out[i] = q2_K_row_dot(w + ns[i] * nb * ORC_Q2_K_BYTES,
                              y + ms[i] * nb * ORC_Q8_K_BYTES, nb, NULL, &terms[i]);
}

/* Q2_K load-time layout (this library's own byte permutation):              */
/*   [N*nb (d, dmin) pairs of 4 B, zero-padded to a multiple of 256 B]       */
/*   [N*nb scales of 16 B][N*nb qs of 64 B], block (n,b) at index n*nb+b.    */
int64_t orc_repacked_bytes_q2_K(int64_t N, int64_t K) {
    int64_t nblk = N * (K / QK_K);
    return (4 * nblk + 255) / 256 * 256 + 80 * nblk;
}

void orc_repack_q2_K(const uint8_t *canon, int64_t N, int64_t K, uint8_t *out) {
    const int64_t nblk = N * (K / QK_K);
    const int64_t dsec = (4 * nblk + 255) / 256 * 256;
    const int64_t s0 = dsec, q0 = s0 + 16 * nblk;
    memset(out, 0, (size_t)dsec);
    for (int64_t i = 0; i < nblk; ++i) {
        const uint8_t *src = canon + i * ORC_Q2_K_BYTES;
        memcpy(out + 4 * i, src + 80, 4);
        memcpy(out + s0 + 16 * i, src, 16);
        memcpy(out + q0 + 64 * i, src + 16, 64);
    }
}

/* ======================================================================== */
/* mul_mat_id.  P1 "本篇没有覆盖的部分" (its list of follow-up topics names   */
/* the expert-routed product of MoE models): mul_mat with one more level,    */
/* the grouping by expert id.                                                */
/* Reading: a stack of E weight matrices [E][N][K] (expert e's rows start at */
/* e*N rows), a token-by-slot table ids[T][U] of expert ids, and activation  */
/* rows either one per token (y_per_slot = 0: row t serves every slot of     */
/* token t) or one per (token, slot) (y_per_slot = 1: row t*U + u);          */
/*   out[(t*U + u)*N + n] = mul_mat(W[ids[t][u]], y_row)[n].                 */
/* Each (t, u) is the plain integer path of its format; an id outside        */
/* [0, E) makes the call fail (returns -1, out untouched).                   */
/* wfmt: 0 Q4_0, 1 Q4_K, 2 Q6_K, 3 Q2_K (the activation format follows).     */
/* ======================================================================== */
int orc_mul_mat_id(int wfmt, const uint8_t *w, int64_t E, int64_t N, int64_t K,
                   const uint8_t *y, const int32_t *ids, int64_t T, int64_t U,
                   int y_per_slot, double *out, double *terms) {
    int64_t nb, wblk, yblk;
    double (*dot)(const uint8_t *, const uint8_t *, int64_t, int32_t *, double *);
    switch (wfmt) {
        case 0: nb = K / QK4_0; wblk = ORC_Q4_0_BYTES; yblk = ORC_Q8_0_BYTES; dot = q4_0_row_dot; break;
        case 1: nb = K / QK_K; wblk = ORC_Q4_K_BYTES; yblk = ORC_Q8_K_BYTES; dot = q4_K_row_dot; break;
        case 2: nb = K / QK_K; wblk = ORC_Q6_K_BYTES; yblk = ORC_Q8_K_BYTES; dot = q6_K_row_dot; break;
        case 3: nb = K / QK_K; wblk = ORC_Q2_K_BYTES; yblk = ORC_Q8_K_BYTES; dot = q2_K_row_dot; break;
        default: return -1;
    }
    for (int64_t p = 0; p < T * U; ++p)
        if (ids[p] < 0 || ids[p] >= E) return -1;
    const int64_t wrow = nb * wblk, yrow = nb * yblk;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t p = 0; p < T * U; ++p)
        for (int64_t n = 0; n < N; ++n) {
            const int64_t e = ids[p];
            const int64_t r = y_per_slot ? p : p / U;
            double tm = 0.0;
            out[p * N + n] = dot(w + (e * N + n) * wrow, y + r * yrow, nb, NULL, terms ? &tm : NULL);
            if (terms) terms[p * N + n] = tm;
        }
    return 0;
}
