// q6k.hip -- Q6_K weights x Q8_K activations on gfx950: encoder, load-time
// repack, GEMV and the int32 group sums of its decode path.
//
// Format (ggml-cpu mul_mat page, "更低的比特:Q6_K 与 Q2_K 的取舍"): 210 bytes
// per 256 weights, ql[128] (low 4 bits of each code) | qh[64] (high 2 bits) |
// int8 scales[16] | fp16 d, with w = d * s_j * q for the signed 6-bit code q in
// [-32, 31] and the 16-element group j.  No min term.  Placement of the bits
// (this library's reading; the page lists the fields only):
//   element k = 64g + r:  low 4 bits in ql byte 32g + r%32 (low nibble for
//   r < 32, high nibble otherwise), high 2 bits in qh byte r, bits 2g..2g+1;
//   the stored code is u = q + 32 in [0, 63].
//
// Integer path (same page, "正确性:缩放系数可以提到求和号外面", without the min
// term): P_j = sum_{i in j} q_i y_i (int32), S = sum_j s_j P_j, and
// out += d_a * d * S.  The GEMV forms u = q + 32 as bytes (a nibble and a
// 2-bit field merged per byte), takes sum u*y with v_dot4_i32_i8 and removes
// the offset with the activation bsums: P_j = sum u*y - 32 * bsums[j] (a
// Q8_K bsum covers exactly one 16-element group).
//
// Load-time layout (QMM_LAYOUT_REPACKED), block (n, b) at index i = n*nb + b:
//   [fp16 d of every block, zero-padded to a multiple of 256 B]
//   [scales, 16 B each][ql, 128 B each][qh, 64 B each]
// so every 16-byte piece a lane loads is aligned.
#include <type_traits>

#include "q8k_row.h"
#include "qmm_device.h"
#include "qmm_launch.h"

namespace qmm {
namespace {

constexpr int kQ6_KBytes = 210;

__device__ __forceinline__ int clampi6(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// ---------------------------------------------------------------------------
// Encoder (input generator; the same reading as the oracle): per 16-element
// group the signed element of largest |x| (first index wins) gives
// sc_j = xm_j / -32; d = max |sc_j| / 127; s_j = rint(sc_j / d) in [-127, 127];
// with D_j = f16(d) * s_j, q = rint(x / D_j) in [-32, 31] (0 where D_j = 0).
// One wavefront per block; lane l holds elements 4l..4l+3 (group l/4).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_encode_q6_K(const float *__restrict__ w,
                                                     uint8_t *__restrict__ out, int64_t nblocks,
                                                     int64_t nb_row, int64_t K) {
    __shared__ __attribute__((aligned(16))) uint8_t su[4][256];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t blk0 = (int64_t)blockIdx.x * 4 + wave;
    const bool valid = blk0 < nblocks;  // a spare wavefront encodes the last block, stores nothing
    const int64_t blk = valid ? blk0 : nblocks - 1;
    const int64_t row = blk / nb_row, b = blk - row * nb_row;
    const float4 v = *reinterpret_cast<const float4 *>(w + row * K + b * QK_K + lane * 4);
    const float xv[4] = {v.x, v.y, v.z, v.w};

    // signed element of largest magnitude in the group, first index on ties
    float best = 0.0f, xm = 0.0f;
    int idx = 1 << 30;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float a = fabsf(xv[e]);
        if (a > best) { best = a; xm = xv[e]; idx = 4 * lane + e; }
    }
#pragma unroll
    for (int o = 1; o <= 2; o <<= 1) {
        const float ob = __shfl_xor(best, o, kWave), ox = __shfl_xor(xm, o, kWave);
        const int oi = __shfl_xor(idx, o, kWave);
        if (ob > best || (ob == best && oi < idx)) { best = ob; xm = ox; idx = oi; }
    }
    const float sc = xm / -32.0f;
    const float d = wave_max(fabsf(sc)) / 127.0f;
    const int s = d > 0.0f ? clampi6((int)rintf(sc / d), -127, 127) : 0;
    const uint32_t dh = f32_to_f16_bits(d);
    const float Dj = f16_bits_to_f32(dh) * (float)s;
    uint32_t mine = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int q = Dj != 0.0f ? clampi6((int)rintf(xv[e] / Dj), -32, 31) : 0;
        mine |= (uint32_t)(q + 32) << (8 * e);
    }
    *reinterpret_cast<uint32_t *>(&su[wave][4 * lane]) = mine;
    __syncthreads();

    // the block is only 2-byte aligned: 16-bit stores
    uint16_t *o = reinterpret_cast<uint16_t *>(out + blk * kQ6_KBytes);
    const uint8_t *u = su[wave];
    if (lane < 32) {          // ql bytes 4l..4l+3
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int B = 4 * lane + i, g = B >> 5, c = B & 31;
            word |= (uint32_t)((u[64 * g + c] & 15) | ((u[64 * g + 32 + c] & 15) << 4)) << (8 * i);
        }
        if (valid) { o[2 * lane] = (uint16_t)word; o[2 * lane + 1] = (uint16_t)(word >> 16); }
    } else if (lane < 48) {   // qh bytes 4(l-32)..+3
        const int l = lane - 32;
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * l + i;
            word |= (uint32_t)((u[r] >> 4) | ((u[r + 64] >> 4) << 2) | ((u[r + 128] >> 4) << 4) |
                               ((u[r + 192] >> 4) << 6)) << (8 * i);
        }
        if (valid) { o[64 + 2 * l] = (uint16_t)word; o[64 + 2 * l + 1] = (uint16_t)(word >> 16); }
    }
    // scales: byte j = s of group j (held by lane 4j); d at byte 208
    const int t = lane & 7;  // lanes 48..55 write scale bytes 2t, 2t+1
    const int s_lo = __shfl(s, 8 * t, kWave) & 0xff;
    const int s_hi = __shfl(s, 8 * t + 4, kWave) & 0xff;
    if (valid && lane >= 48 && lane < 56) o[96 + (lane - 48)] = (uint16_t)(s_lo | (s_hi << 8));
    if (valid && lane == 0) o[104] = (uint16_t)dh;
}

// ---------------------------------------------------------------------------
// Repack: one thread per block copies its 210 bytes into the four sections
// (2-byte loads: canonical blocks are only 2-byte aligned); threads past the
// last block zero the padding of the d section.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_repack_q6_K(const uint8_t *__restrict__ in,
                                                     uint8_t *__restrict__ out, int64_t nblk,
                                                     int64_t dsec) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= nblk) {
        if (2 * i < dsec) *reinterpret_cast<uint16_t *>(out + 2 * i) = 0;
        return;
    }
    const uint16_t *src = reinterpret_cast<const uint16_t *>(in + i * kQ6_KBytes);
    uint16_t *ql = reinterpret_cast<uint16_t *>(out + dsec + 16 * nblk + 128 * i);
    uint16_t *qh = reinterpret_cast<uint16_t *>(out + dsec + 144 * nblk + 64 * i);
    uint16_t *sc = reinterpret_cast<uint16_t *>(out + dsec + 16 * i);
    for (int k = 0; k < 64; ++k) ql[k] = src[k];
    for (int k = 0; k < 32; ++k) qh[k] = src[64 + k];
    for (int k = 0; k < 8; ++k) sc[k] = src[96 + k];
    *reinterpret_cast<uint16_t *>(out + 2 * i) = src[104];
}

// ---------------------------------------------------------------------------
// GEMV, rows of at most four units per lane (K <= 8192).  The unit of work is
// one 16-byte ql piece: unit u = 8b + p (p = 2g + h)
// holds the low nibbles of group 4g + h and the high nibbles of group
// 4g + 2 + h of super-block b; their 2-bit high parts sit in bits 2g..2g+1 of
// the qh pieces h and h + 2, their scales in bytes h and 2 + h of scale dword
// g.  One wavefront per output row, lane l takes units l, l + 64, ...: the
// wavefront's ql loads cover a contiguous 1 KB (eight blocks) and its qh loads
// 512 bytes (each qh piece is read by the four lanes of its half of the block),
// so every load touches few cache lines.  Longer rows use half a super-block
// per unit (Q6KHalf below): per element it needs fewer loads and less
// scale work, which outweighs its less contiguous loads once a lane holds
// more than four piece units.  The activation row is staged in LDS
// (q8k_row.h).
// ---------------------------------------------------------------------------
template <bool REPACKED>
struct Q6KAddr {
    const uint8_t *W;
    int64_t NB, dsec;  // blocks in the matrix, bytes of the d section
    __device__ __forceinline__ int64_t blk_off(int64_t i) const { return i * kQ6_KBytes; }
    __device__ __forceinline__ const uint8_t *ql(int64_t i) const {
        return REPACKED ? W + dsec + 16 * NB + 128 * i : W + blk_off(i);
    }
    __device__ __forceinline__ const uint8_t *qh(int64_t i) const {
        return REPACKED ? W + dsec + 144 * NB + 64 * i : W + blk_off(i) + 128;
    }
    __device__ __forceinline__ const uint8_t *sc(int64_t i) const {
        return REPACKED ? W + dsec + 16 * i : W + blk_off(i) + 192;
    }
    __device__ __forceinline__ const uint8_t *d(int64_t i) const {
        return REPACKED ? W + 2 * i : W + blk_off(i) + 208;
    }
};

// 16 bytes at an address that is 16-byte aligned (repacked) or only 2-byte
// aligned (canonical blocks)
template <bool ALIGNED>
__device__ __forceinline__ uint4 ld16a(const uint8_t *p) {
    if constexpr (ALIGNED) {
        return *reinterpret_cast<const uint4 *>(p);
    } else {
        uint4 v;
        __builtin_memcpy(&v, __builtin_assume_aligned(p, 2), 16);
        return v;
    }
}

struct Q6KUnit {
    uint4 ql;      // ql piece p
    uint4 qa, qb;  // qh pieces h and h + 2
    uint32_t sc;   // scale dword g (scales of groups 4g .. 4g + 3)
    uint32_t d;    // fp16 d bits
};

// 4 bytes at an address that is 4-byte aligned (repacked) or only 2-byte
// aligned (canonical blocks)
template <bool ALIGNED>
__device__ __forceinline__ uint32_t ld4a(const uint8_t *p) {
    if constexpr (ALIGNED) {
        return *reinterpret_cast<const uint32_t *>(p);
    } else {
        return ld_u16(p) | (ld_u16(p + 2) << 16);
    }
}

template <bool REPACKED>
__device__ __forceinline__ void q6k_load(const Q6KAddr<REPACKED> &A, int64_t n, int64_t nb, int u,
                                         Q6KUnit &x) {
    const int64_t i = n * nb + (u >> 3);
    const int p = u & 7, g = p >> 1, h = p & 1;
    x.ql = ld16a<REPACKED>(A.ql(i) + 16 * p);
    x.qa = ld16a<REPACKED>(A.qh(i) + 16 * h);
    x.qb = ld16a<REPACKED>(A.qh(i) + 32 + 16 * h);
    x.sc = ld4a<REPACKED>(A.sc(i) + 4 * g);
    x.d = ld_u16(A.d(i));
}

// The two group sums of a unit: group 4g + h -> P[0], group 4g + 2 + h -> P[1].
__device__ __forceinline__ void q6k_group_sums(const Q6KUnit &x, int u, const uint8_t *s_qs,
                                               const int16_t *s_bs, int P[2]) {
    const int b = u >> 3, p = u & 7, g = p >> 1, h = p & 1;
    const uint8_t *yrow = s_qs + b * QK_K;
    const uint32_t qa[4] = {x.qa.x, x.qa.y, x.qa.z, x.qa.w};
    const uint32_t qb[4] = {x.qb.x, x.qb.y, x.qb.z, x.qb.w};
    const uint32_t ql[4] = {x.ql.x, x.ql.y, x.ql.z, x.ql.w};
    const uint4 ylo = *reinterpret_cast<const uint4 *>(yrow + 64 * g + 16 * h);
    const uint4 yhi = *reinterpret_cast<const uint4 *>(yrow + 64 * g + 32 + 16 * h);
    const uint32_t yl[4] = {ylo.x, ylo.y, ylo.z, ylo.w};
    const uint32_t yh[4] = {yhi.x, yhi.y, yhi.z, yhi.w};
    int plo = 0, phi = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t ulo = (ql[w] & 0x0f0f0f0fu) | (((qa[w] >> (2 * g)) & 0x03030303u) << 4);
        const uint32_t uhi = ((ql[w] >> 4) & 0x0f0f0f0fu) | (((qb[w] >> (2 * g)) & 0x03030303u) << 4);
        plo = dot4(ulo, yl[w], plo);
        phi = dot4(uhi, yh[w], phi);
    }
    P[0] = plo - 32 * s_bs[16 * b + 4 * g + h];
    P[1] = phi - 32 * s_bs[16 * b + 4 * g + 2 + h];
}

// Half a super-block: unit u = 2b + h owns the ql pieces 2g + h (g = 0..3,
// both nibbles) and the qh pieces h and h + 2 -- 96 bytes no other unit reads
// -- i.e. the 16-element groups 4g + h (low nibbles) and 4g + 2 + h (high).
struct Q6KHalf {
    uint4 ql[4];   // ql pieces 2g + h
    uint4 qa, qb;  // qh pieces h and h + 2
    uint4 sc;      // the block's 16 scales
    uint32_t d;    // fp16 d bits
};

template <bool REPACKED>
__device__ __forceinline__ void q6k_load_half(const Q6KAddr<REPACKED> &A, int64_t n, int64_t nb, int u,
                                         Q6KHalf &x) {
    const int64_t i = n * nb + (u >> 1);
    const int h = u & 1;
#pragma unroll
    for (int g = 0; g < 4; ++g) x.ql[g] = ld16a<REPACKED>(A.ql(i) + 32 * g + 16 * h);
    x.qa = ld16a<REPACKED>(A.qh(i) + 16 * h);
    x.qb = ld16a<REPACKED>(A.qh(i) + 32 + 16 * h);
    x.sc = ld16a<REPACKED>(A.sc(i));
    x.d = ld_u16(A.d(i));
}

// The eight group sums P of a unit (groups 4g + h -> P[2g], 4g + 2 + h -> P[2g+1]).
__device__ __forceinline__ void q6k_group_sums_half(const Q6KHalf &x, int u, const uint8_t *s_qs,
                                               const int16_t *s_bs, int P[8]) {
    const int b = u >> 1, h = u & 1;
    const uint8_t *yrow = s_qs + b * QK_K;
    const uint32_t qa[4] = {x.qa.x, x.qa.y, x.qa.z, x.qa.w};
    const uint32_t qb[4] = {x.qb.x, x.qb.y, x.qb.z, x.qb.w};
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const uint32_t ql[4] = {x.ql[g].x, x.ql[g].y, x.ql[g].z, x.ql[g].w};
        const uint4 ylo = *reinterpret_cast<const uint4 *>(yrow + 64 * g + 16 * h);
        const uint4 yhi = *reinterpret_cast<const uint4 *>(yrow + 64 * g + 32 + 16 * h);
        const uint32_t yl[4] = {ylo.x, ylo.y, ylo.z, ylo.w};
        const uint32_t yh[4] = {yhi.x, yhi.y, yhi.z, yhi.w};
        int plo = 0, phi = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t ulo = (ql[w] & 0x0f0f0f0fu) | (((qa[w] >> (2 * g)) & 0x03030303u) << 4);
            const uint32_t uhi = ((ql[w] >> 4) & 0x0f0f0f0fu) | (((qb[w] >> (2 * g)) & 0x03030303u) << 4);
            plo = dot4(ulo, yl[w], plo);
            phi = dot4(uhi, yh[w], phi);
        }
        P[2 * g] = plo - 32 * s_bs[16 * b + 4 * g + h];
        P[2 * g + 1] = phi - 32 * s_bs[16 * b + 4 * g + 2 + h];
    }
}

constexpr int kQ6Waves = 4;

// MODE 0: out[m*N + n] (fp32).  MODE 1: P[m][n][K/16] (int32 group sums).
// ID = true (MODE 0): mul_mat_id, one (token, slot) pair per blockIdx.y.
template <bool REPACKED, int kNit, int MODE, bool ID = false, bool PIECE = true>
__global__ __launch_bounds__(256) void k_gemv_q6_K(const uint8_t *__restrict__ W,
                                                   const uint8_t *__restrict__ Y,
                                                   void *__restrict__ dst, int64_t N, int64_t K,
                                                   IdRoute route = {}) {
    extern __shared__ __attribute__((aligned(16))) uint8_t ys[];
    const int64_t nb = K / QK_K;
    int64_t m = blockIdx.y, m_out = blockIdx.y;  // activation row, output row
    bool valid = true;
    if constexpr (ID) {
        const IdPair ip = id_route(route);
        valid = ip.valid;
        W += ip.w_off;
        Y += ip.y_off;
        m_out = ip.out_row;
        m = 0;
    }
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int64_t n = (int64_t)blockIdx.x * kQ6Waves + wave;
    const int64_t nn = n < N ? n : N - 1;  // a tail wavefront loads a valid row, stores nothing
    const int nunits = (int)((PIECE ? 8 : 2) * nb);
    const Q6KAddr<REPACKED> A{W, N * nb, REPACKED ? (2 * N * nb + 255) / 256 * 256 : 0};
    using Unit = std::conditional_t<PIECE, Q6KUnit, Q6KHalf>;
    auto load = [&](int u, Unit &x) {
        if constexpr (PIECE) q6k_load<REPACKED>(A, nn, nb, u, x);
        else q6k_load_half<REPACKED>(A, nn, nb, u, x);
    };

    // the activation row's first pieces, then this row's first units, then
    // the activations into LDS (the wait before the stores covers only them)
    const uint8_t *yrow = Y + m * nb * kQ8_KBytes;
    const Q8KRowHead yh = load_q8k_row_head(yrow, K);
    __builtin_amdgcn_sched_barrier(0);
    Unit x[kNit];
#pragma unroll
    for (int it = 0; it < kNit; ++it) {
        const int u = lane + 64 * it;
        load(u < nunits ? u : nunits - 1, x[it]);
    }
    const Q8KRowLds row = commit_q8k_row(yh, yrow, K, ys);
    const uint8_t *s_qs = row.qs;
    const float *s_d = row.d;
    const int16_t *s_bs = row.bsums;

    float acc = 0.0f;
    for (int base = 0; base < nunits; base += 64 * kNit) {
        if (base > 0) {
#pragma unroll
            for (int it = 0; it < kNit; ++it) {
                const int u = base + lane + 64 * it;
                load(u < nunits ? u : nunits - 1, x[it]);
            }
        }
#pragma unroll
        for (int it = 0; it < kNit; ++it) {
            const int u = base + lane + 64 * it;
            if (u >= nunits) continue;
            if constexpr (!PIECE) {
                int P[8];
                q6k_group_sums_half(x[it], u, s_qs, s_bs, P);
                const int b = u >> 1, h = u & 1;
                if (MODE == 0) {
                    const uint32_t sw[4] = {x[it].sc.x, x[it].sc.y, x[it].sc.z, x[it].sc.w};
                    int S = 0;
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int s_lo = (int)(int8_t)(sw[g] >> (8 * h));
                        const int s_hi = (int)(int8_t)(sw[g] >> (8 * (2 + h)));
                        S += s_lo * P[2 * g] + s_hi * P[2 * g + 1];
                    }
                    acc = fmaf(s_d[b], f16_bits_to_f32(x[it].d) * (float)S, acc);
                } else if (n < N) {
                    int32_t *Pout = reinterpret_cast<int32_t *>(dst) + (m * N + n) * (K / 16) + 16 * b;
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        Pout[4 * g + h] = P[2 * g];
                        Pout[4 * g + 2 + h] = P[2 * g + 1];
                    }
                }
            } else {
                int P[2];
                q6k_group_sums(x[it], u, s_qs, s_bs, P);
                const int b = u >> 3, p = u & 7, g = p >> 1, h = p & 1;
                if (MODE == 0) {
                    const int s_lo = (int)(int8_t)(x[it].sc >> (8 * h));
                    const int s_hi = (int)(int8_t)(x[it].sc >> (8 * (2 + h)));
                    const int S = s_lo * P[0] + s_hi * P[1];
                    acc = fmaf(s_d[b], f16_bits_to_f32(x[it].d) * (float)S, acc);
                } else if (n < N) {
                    int32_t *Pout = reinterpret_cast<int32_t *>(dst) + (m * N + n) * (K / 16) + 16 * b;
                    Pout[4 * g + h] = P[0];
                    Pout[4 * g + 2 + h] = P[1];
                }
            }
        }
    }
    if (MODE == 0) {
        acc = wave_sum(acc);
        if (lane == 0 && n < N) reinterpret_cast<float *>(dst)[m_out * N + n] = valid ? acc : __builtin_nanf("");
    }
}

// ---------------------------------------------------------------------------
// Fused M = 1 path for Q6_K (rows of up to four piece units per lane; two rows
// per wavefront at most, one where a row takes four units per lane, as two
// rows of four would not fit the 128 VGPRs of a 1024-thread workgroup without
// spills): the fp32 row is quantized to Q8_K inside the GEMV,
// straight into LDS, so one launch covers quantize + mul_mat.  As in the Q4_K
// fused kernel every workgroup quantizes the whole row, so the grid holds one
// 16-wavefront workgroup per CU and wavefront w of workgroup g takes rows
// g*16 + w and (kRows = 2) g*16 + w + 16*gridDim.x.  A wavefront first loads
// its fp32 activation blocks (b = wave + 16i), issues its first row's units
// (below four units per lane only once the activation blocks have arrived)
// and quantizes while they are in flight; its second row (if any) is
// requested after the barrier, before the first is reduced.  Workgroup 0 also
// stores the Q8_K bytes to Yq.  Per row the same integer sums and fp32
// operations, in the same order, as k_gemv_q6_K.
// ---------------------------------------------------------------------------
constexpr int kQ6FusedWaves = 16;

template <bool REPACKED, int kNit, int kXB, int kRows>
__global__ __launch_bounds__(kQ6FusedWaves * 64) void k_gemv_fused_q6_K(
    const uint8_t *__restrict__ W, const float *__restrict__ X, uint8_t *__restrict__ Yq,
    float *__restrict__ out, int64_t N, int64_t K) {
    extern __shared__ __attribute__((aligned(16))) uint8_t ys[];
    const int64_t nb = K / QK_K;
    const int nunits = (int)(8 * nb);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int64_t stride = (int64_t)gridDim.x * kQ6FusedWaves;
    const int64_t row = (int64_t)blockIdx.x * kQ6FusedWaves + wave, row2 = row + stride;  // uniform
    const Q6KAddr<REPACKED> A{W, N * nb, REPACKED ? (2 * N * nb + 255) / 256 * 256 : 0};
    auto load_row = [&](int64_t r, Q6KUnit (&x)[kNit]) {
        const int64_t rr = r < N ? r : N - 1;  // past the last row: a valid row, never stored
#pragma unroll
        for (int it = 0; it < kNit; ++it) {
            const int u = lane + 64 * it;
            q6k_load<REPACKED>(A, rr, nb, u < nunits ? u : nunits - 1, x[it]);
        }
    };
    float4 xv[kXB];
#pragma unroll
    for (int i = 0; i < kXB; ++i) {  // block indices past the row load the last block again
        const int b0 = wave + kQ6FusedWaves * i;
        const int b = b0 < nb ? b0 : (int)nb - 1;
        xv[i] = *reinterpret_cast<const float4 *>(X + (int64_t)b * QK_K + 4 * lane);
    }
    // up to two units per lane the activation loads complete before any weight
    // load is issued (queued behind the chip's weight stream they would arrive
    // late); at four, the quantization waits only for them, with the row's
    // units already requested (0.1-0.2 us faster there, 0.1-0.4 us slower below)
    if constexpr (kNit < 4) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    Q6KUnit x[kNit], x2[kRows == 2 ? kNit : 1];
    load_row(row, x);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kXB; ++i) q8k_quantize_block_lds(xv[i], wave + kQ6FusedWaves * i, K, ys, lane);
    __syncthreads();
    const uint8_t *s_qs = ys;
    const float *s_d = reinterpret_cast<const float *>(ys + K);
    const int16_t *s_bs = reinterpret_cast<const int16_t *>(ys + K + (nb * 4 + 15) / 16 * 16);
    const bool two = kRows == 2 && row2 < N;  // wavefront-uniform
    if constexpr (kRows == 2)
        if (two) load_row(row2, x2);
    auto reduce = [&](int64_t r, const Q6KUnit (&xx)[kNit]) {
        float acc = 0.0f;
#pragma unroll
        for (int it = 0; it < kNit; ++it) {
            const int u = lane + 64 * it;
            if (u >= nunits) continue;
            int P[2];
            q6k_group_sums(xx[it], u, s_qs, s_bs, P);
            const int b = u >> 3, p = u & 7, h = p & 1;
            const int s_lo = (int)(int8_t)(xx[it].sc >> (8 * h));
            const int s_hi = (int)(int8_t)(xx[it].sc >> (8 * (2 + h)));
            const int S = s_lo * P[0] + s_hi * P[1];
            acc = fmaf(s_d[b], f16_bits_to_f32(xx[it].d) * (float)S, acc);
        }
        acc = wave_sum(acc);
        if (lane == 0 && r < N) out[r] = acc;
    };
    reduce(row, x);
    if constexpr (kRows == 2)
        if (two) reduce(row2, x2);
    // workgroup 0 copies the Q8_K row to Yq last (stores issued earlier would
    // sit in the in-order counter ahead of the weight loads)
    if (blockIdx.x == 0) q8k_store_row<kQ6FusedWaves * 64>(Yq, ys, K);
}

template <int MODE>
hipError_t dispatch_q6_K(const uint8_t *w, bool repacked, const uint8_t *y, void *dst, int64_t M,
                         int64_t N, int64_t K, hipStream_t s) {
    const int64_t nit = (8 * (K / QK_K) + 63) / 64;       // piece units per lane
    const int64_t nit_half = (2 * (K / QK_K) + 63) / 64;  // half-block units per lane
    const dim3 grid((unsigned)((N + kQ6Waves - 1) / kQ6Waves), (unsigned)M);  // M <= 65535
    const unsigned lds = (unsigned)q8k_row_lds_bytes(K);
#define QMM_Q6(NIT, PC)                                                                                    \
    do {                                                                                                   \
        if (repacked)                                                                                      \
            hipLaunchKernelGGL((k_gemv_q6_K<true, NIT, MODE, false, PC>), grid, dim3(256), lds, s, w, y, dst, N, K, \
                               IdRoute{});                                                                 \
        else                                                                                               \
            hipLaunchKernelGGL((k_gemv_q6_K<false, NIT, MODE, false, PC>), grid, dim3(256), lds, s, w, y, dst, N, \
                               K, IdRoute{});                                                              \
    } while (0)
    if (nit <= 1) QMM_Q6(1, true);
    else if (nit <= 2) QMM_Q6(2, true);
    else if (nit <= 4) QMM_Q6(4, true);
    else if (nit_half <= 2) QMM_Q6(2, false);
    else QMM_Q6(4, false);
#undef QMM_Q6
    return hipGetLastError();
}

}  // namespace

int64_t repacked_bytes_q6_K(int64_t N, int64_t K) {
    const int64_t nblk = N * (K / QK_K);
    return (2 * nblk + 255) / 256 * 256 + 208 * nblk;
}

int64_t q6_K_max_k() { return q8k_row_max_k(); }  // the staged activation row fits LDS

hipError_t launch_encode_q6_K(const float *w, uint8_t *out, int64_t N, int64_t K, hipStream_t s) {
    const int64_t nb = K / QK_K, total = N * nb;
    hipLaunchKernelGGL(k_encode_q6_K, dim3((unsigned)((total + 3) / 4)), dim3(256), 0, s, w, out,
                       total, nb, K);
    return hipGetLastError();
}

hipError_t launch_repack_q6_K(const uint8_t *in, uint8_t *out, int64_t N, int64_t K, hipStream_t s) {
    const int64_t nblk = N * (K / QK_K);
    const int64_t dsec = (2 * nblk + 255) / 256 * 256;
    const int64_t threads = nblk > dsec / 2 ? nblk : dsec / 2;
    hipLaunchKernelGGL(k_repack_q6_K, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, in,
                       out, nblk, dsec);
    return hipGetLastError();
}

// activation rows go to grid.y, in chunks of at most 65535 rows
hipError_t launch_gemv_q6_K(const uint8_t *w, bool repacked, const uint8_t *y, float *out,
                            int64_t M, int64_t N, int64_t K, hipStream_t s) {
    const int64_t rowb = (K / QK_K) * kQ8_KBytes;
    for (int64_t m0 = 0; m0 < M; m0 += 65535) {
        const int64_t mm = M - m0 < 65535 ? M - m0 : 65535;
        const hipError_t e = dispatch_q6_K<0>(w, repacked, y + m0 * rowb, out + m0 * N, mm, N, K, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

bool gemv_fused_q6_K_ok(int64_t N, int64_t K) {
    // rows of up to four piece units per lane (K <= 8192); two rows per
    // wavefront at most, one at four units; each workgroup repeats the
    // quantization
    const int64_t rows = K <= 4096 ? 2 : 1;
    return K <= 8192 && N <= rows * kQ6FusedWaves * cu_count() && q8k_row_lds_bytes(K) <= 60 * 1024;
}

hipError_t launch_gemv_fused_q6_K(const uint8_t *w, bool repacked, const float *x, uint8_t *yq, float *out,
                                  int64_t N, int64_t K, hipStream_t s) {
    if (!gemv_fused_q6_K_ok(N, K)) return hipErrorInvalidValue;
    const int64_t nit = (8 * (K / QK_K) + 63) / 64;
    const int64_t groups = (N + kQ6FusedWaves - 1) / kQ6FusedWaves, cus = cu_count();
    const dim3 grid((unsigned)(groups < cus ? groups : cus)), block(kQ6FusedWaves * 64);
    const unsigned lds = (unsigned)q8k_row_lds_bytes(K);
#define QMM_Q6F(NIT, XB, ROWS)                                                                                  \
    do {                                                                                                        \
        if (repacked)                                                                                           \
            hipLaunchKernelGGL((k_gemv_fused_q6_K<true, NIT, XB, ROWS>), grid, block, lds, s, w, x, yq, out, N, K);  \
        else                                                                                                    \
            hipLaunchKernelGGL((k_gemv_fused_q6_K<false, NIT, XB, ROWS>), grid, block, lds, s, w, x, yq, out, N, K); \
    } while (0)
    // kXB = activation blocks per wavefront: ceil(nb / 16) (nb <= 8 * kNit <= 16 * kXB)
    if (nit <= 1) QMM_Q6F(1, 1, 2);
    else if (nit <= 2) QMM_Q6F(2, 1, 2);
    else QMM_Q6F(4, 2, 1);
#undef QMM_Q6F
    return hipGetLastError();
}

hipError_t launch_gemv_id_q6_K(const uint8_t *w, bool repacked, int64_t w_stride, const uint8_t *y,
                               int y_per_slot, const int32_t *ids, int64_t P, int64_t U, int64_t E,
                               float *out, int64_t N, int64_t K, hipStream_t s) {
    const int64_t nit = (8 * (K / QK_K) + 63) / 64, nit_half = (2 * (K / QK_K) + 63) / 64;
    const unsigned lds = (unsigned)q8k_row_lds_bytes(K);
    for (int64_t p0 = 0; p0 < P; p0 += 65535) {
        const int64_t pp = P - p0 < 65535 ? P - p0 : 65535;
        const dim3 grid((unsigned)((N + kQ6Waves - 1) / kQ6Waves), (unsigned)pp);
        const IdRoute r{ids, p0, U, E, w_stride, (K / QK_K) * kQ8_KBytes, y_per_slot};
#define QMM_ID(NIT, PC)                                                                                 \
    do {                                                                                                \
        if (repacked)                                                                                   \
            hipLaunchKernelGGL((k_gemv_q6_K<true, NIT, 0, true, PC>), grid, dim3(256), lds, s, w, y, (void *)out, N, \
                               K, r);                                                                   \
        else                                                                                            \
            hipLaunchKernelGGL((k_gemv_q6_K<false, NIT, 0, true, PC>), grid, dim3(256), lds, s, w, y, (void *)out, \
                               N, K, r);                                                                \
    } while (0)
        if (nit <= 1) QMM_ID(1, true);
        else if (nit <= 2) QMM_ID(2, true);
        else if (nit <= 4) QMM_ID(4, true);
        else if (nit_half <= 2) QMM_ID(2, false);
        else QMM_ID(4, false);
#undef QMM_ID
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_group_sums_q6_K(const uint8_t *w, bool repacked, const uint8_t *y, int32_t *P,
                                  int64_t M, int64_t N, int64_t K, hipStream_t s) {
    const int64_t rowb = (K / QK_K) * kQ8_KBytes;
    for (int64_t m0 = 0; m0 < M; m0 += 65535) {
        const int64_t mm = M - m0 < 65535 ? M - m0 : 65535;
        const hipError_t e =
            dispatch_q6_K<1>(w, repacked, y + m0 * rowb, P + m0 * N * (K / 16), mm, N, K, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace qmm
