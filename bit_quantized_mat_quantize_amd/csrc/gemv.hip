// gemv.hip -- memory-bound quantized GEMV (M <= 8) for gfx950.
//
// Decode is bound by the weight stream (ggml-cpu mul_mat page, "先把账算清楚":
// at M = 1 the time per token is the weight bytes over the bandwidth), so the
// kernel is shaped around HBM: one wavefront per R output rows, each lane owns
// one 16-byte piece of a block payload per step, consecutive lanes read
// consecutive pieces (a wavefront step reads 1 KiB per row, coalesced), and the
// nibbles are unpacked in registers with two masks and a shift, never written
// back to memory (same section; "正确性:缩放系数可以提到求和号外面" for the
// byte order).  The int8 products use v_dot4_i32_i8 (4 MACs per lane per
// instruction), the block scales are applied once per 16-element piece, and
// the per-lane fp32 partials are reduced across the wavefront at the end.
//
// Q4_K piece c of block b (c = 2g + h, g = 64-element group, h = half):
//   payload bytes 32g+16h .. +15 -> low nibbles  = elements 64g+16h+i    (sub-block 2g)
//                                   high nibbles = elements 64g+32+16h+i (sub-block 2g+1)
//   activation codes qs[64g+16h ..], qs[64g+32+16h ..], bsums[4g+h], bsums[4g+2+h]
//   partial = d_a * (d * (s_2g*P_lo + s_2g+1*P_hi) - dmin * (m_2g*B_lo + m_2g+1*B_hi))
// Summed over the 8 pieces of a block this is d_a*(d*S - dmin*Mn) of the
// ggml-cpu page ("正确性" and "min 项与最终归约").
#include "q8k_row.h"
#include "qmm_device.h"
#include "qmm_launch.h"

namespace qmm {
namespace {

constexpr int kWavesPerBlock = 4;

template <bool REPACKED>
struct Q4KAddr {
    const uint8_t *W;
    int64_t N, nb;
    __device__ __forceinline__ const uint8_t *header(int64_t n, int64_t b) const {
        return REPACKED ? W + 16 * (n * nb + b) : W + kQ4_KBytes * (n * nb + b);
    }
    __device__ __forceinline__ const uint8_t *piece(int64_t n, int64_t b, int c) const {
        return REPACKED ? W + 16 * N * nb + 128 * (n * nb + b) + 16 * c
                        : W + kQ4_KBytes * (n * nb + b) + 16 + 16 * c;
    }
};

// MODE 0: out[m*N+n] fp32.  MODE 1: int32 sub-block sums P[m][n][K/32].
template <int M, int R, bool REPACKED, int MODE>
__global__ __launch_bounds__(256) void k_gemv_q4_K(const uint8_t *__restrict__ W,
                                                   const uint8_t *__restrict__ Y,
                                                   void *__restrict__ dst, int64_t N, int64_t K) {
    const int64_t nb = K / QK_K;
    const int nchunk = (int)(nb * 8);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t n0 = ((int64_t)blockIdx.x * kWavesPerBlock + wave) * R;
    if (n0 >= N) return;  // uniform per wavefront
    const Q4KAddr<REPACKED> A{W, N, nb};

    float acc[R][M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

    for (int c = lane; c < nchunk; c += kWave) {
        const int b = c >> 3, cc = c & 7, g = cc >> 1, h = cc & 1;
        uint4 pw[R], hw[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t n = n0 + r < N ? n0 + r : N - 1;
            hw[r] = ld16(A.header(n, b));
            pw[r] = ld16(A.piece(n, b, cc));
        }
        uint4 ylo[M], yhi[M];
        float da[M];
        int bs_lo[M], bs_hi[M];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const uint8_t *yb = Y + ((int64_t)m * nb + b) * kQ8_KBytes;
            ylo[m] = ld_align4<uint4>(yb + 4 + 64 * g + 16 * h);
            yhi[m] = ld_align4<uint4>(yb + 4 + 64 * g + 32 + 16 * h);
            da[m] = ld_align4<float>(yb);
            bs_lo[m] = *reinterpret_cast<const int16_t *>(yb + 260 + 2 * (4 * g + h));
            bs_hi[m] = *reinterpret_cast<const int16_t *>(yb + 260 + 2 * (4 * g + 2 + h));
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const Q4KScales sc = unpack_scales(hw[r].y, hw[r].z, hw[r].w);
            const uint32_t sw = g < 2 ? sc.s_lo : sc.s_hi;
            const uint32_t mw = g < 2 ? sc.m_lo : sc.m_hi;
            const int sh = (g & 1) * 16;
            const int s0 = (sw >> sh) & 0xff, s1 = (sw >> (sh + 8)) & 0xff;
            const int m0 = (mw >> sh) & 0xff, m1 = (mw >> (sh + 8)) & 0xff;
            const float d = f16_bits_to_f32(hw[r].x & 0xffff);
            const float dmin = f16_bits_to_f32(hw[r].x >> 16);
            const uint32_t l0 = pw[r].x & 0x0f0f0f0fu, l1 = pw[r].y & 0x0f0f0f0fu;
            const uint32_t l2 = pw[r].z & 0x0f0f0f0fu, l3 = pw[r].w & 0x0f0f0f0fu;
            const uint32_t h0 = (pw[r].x >> 4) & 0x0f0f0f0fu, h1 = (pw[r].y >> 4) & 0x0f0f0f0fu;
            const uint32_t h2 = (pw[r].z >> 4) & 0x0f0f0f0fu, h3 = (pw[r].w >> 4) & 0x0f0f0f0fu;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                int plo = dot4(l0, ylo[m].x, 0);
                plo = dot4(l1, ylo[m].y, plo);
                plo = dot4(l2, ylo[m].z, plo);
                plo = dot4(l3, ylo[m].w, plo);
                int phi = dot4(h0, yhi[m].x, 0);
                phi = dot4(h1, yhi[m].y, phi);
                phi = dot4(h2, yhi[m].z, phi);
                phi = dot4(h3, yhi[m].w, phi);
                if (MODE == 0) {
                    const int S = s0 * plo + s1 * phi;
                    const int Mn = m0 * bs_lo[m] + m1 * bs_hi[m];
                    const float t = fmaf(d, (float)S, -dmin * (float)Mn);
                    acc[r][m] = fmaf(da[m], t, acc[r][m]);
                } else {
                    // full sub-block sums: the two halves sit in lanes c and c^1
                    const int plo_all = plo + __shfl_xor(plo, 1, kWave);
                    const int phi_all = phi + __shfl_xor(phi, 1, kWave);
                    if (h == 0 && n0 + r < N) {
                        int32_t *P = reinterpret_cast<int32_t *>(dst) +
                                     ((int64_t)m * N + n0 + r) * (K / 32) + 8 * b + 2 * g;
                        P[0] = plo_all;
                        P[1] = phi_all;
                    }
                }
            }
        }
    }
    if (MODE == 0) {
        float *out = reinterpret_cast<float *>(dst);
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const float v = wave_sum(acc[r][m]);
                if (lane == 0 && n0 + r < N) out[(int64_t)m * N + n0 + r] = v;
            }
    }
}

// ---------------------------------------------------------------------------
// M = 1 variant: one wavefront per output row.  Every lane first issues the
// loads of all its weight pieces of the row (up to kNit per pass) together
// with the workgroup's share of the activation row, so one memory round trip
// covers the whole row; the activation row (shared by the 4 rows of the
// workgroup) is staged in LDS with its 16-byte pieces aligned:
//   qs [K] int8 | d [nb] fp32 (padded to 16 B) | bsums [nb][16] int16 | 16 B
// The last 16 bytes take the stores of threads without a piece to stage, so
// loads and stores need no branches (a load whose only use sits in a branch
// is sunk past the weight loads by the compiler, which then has to wait for
// every weight before staging the activations).
// ---------------------------------------------------------------------------

__host__ __device__ constexpr int64_t gemv1_lds_bytes(int64_t K) {
    return K + ((K / QK_K) * 4 + 15) / 16 * 16 + (K / QK_K) * 32 + 16;
}

// A pass moves kNit 16-byte pieces per lane, in kNit / kP sub-passes of kP =
// min(kNit, 2) consecutive pieces: in sub-pass s, lane l owns the pieces
// c = base + 64*kP*s + kP*l + i (i < kP) of row nn.  The kP pieces of a
// sub-pass lie in one super-block, so one header serves them, and pieces 2g,
// 2g+1 (the two halves of the 32-byte group g) share their sub-block scales.
// The wavefront's pieces of one sub-pass are contiguous (64 * kP * 16 bytes),
// so each load touches few cache lines whatever the row length.  A lane past
// the row end loads the last group again and leaves it unused; the loads stay
// branch-free, so the compiler can wait for older loads (the activations)
// while these are still in flight.
template <int kNit>
constexpr int gemv1_kp() { return kNit >= 2 ? 2 : 1; }
template <int kNit>
constexpr int gemv1_subs() { return kNit / gemv1_kp<kNit>(); }

// Sub-passes SP0 .. SP1 - 1 only (the fused kernel splits a row's requests).
template <bool REPACKED, int kNit, int SP0 = 0, int SP1 = gemv1_subs<kNit>()>
__device__ __forceinline__ void gemv1_load(const Q4KAddr<REPACKED> &A, int64_t nn, int base,
                                           int nchunk, int lane, uint4 (&hw)[gemv1_subs<kNit>()],
                                           uint4 (&pw)[kNit]) {
    constexpr int kP = gemv1_kp<kNit>();
#pragma unroll
    for (int sp = SP0; sp < SP1; ++sp) {
        const int c0 = base + 64 * kP * sp + kP * lane;
        const int c = c0 < nchunk ? c0 : nchunk - kP;
        const int b = c >> 3, cc = c & 7;
        hw[sp] = ld16(A.header(nn, b));
#pragma unroll
        for (int i = 0; i < kP; ++i) pw[kP * sp + i] = ld16(A.piece(nn, b, cc + i));
    }
}

// Integer dot products of the loaded pieces with the activation row in LDS.
// Piece cc = 2g + h of super-block b holds bytes 16h..16h+15 of the 32-byte
// group g: elements 64g+16h.. (low nibbles, sub-block 2g) and 64g+32+16h..
// (high nibbles, sub-block 2g+1).  With P the dot products and Y the matching
// 16-element activation sums (bsums), the lane's pieces give
//   S  = sum_g (s_2g * P_lo,g + s_2g+1 * P_hi,g),  Mn = sum_g (m_2g * Y_lo,g + m_2g+1 * Y_hi,g)
//   acc += d_a * (d * S - dmin * Mn)
// for the kNit (at most 2) pieces of one sub-pass.  S stays an exact int32 and
// its conversion to fp32 exact (|S| < 2^24).
template <int kNit>
__device__ __forceinline__ float gemv1_acc_sub(const uint4 &hw, const uint4 *pw, int base, int nchunk,
                                               int lane, const uint8_t *s_qs, const int16_t *s_bs,
                                               const float *s_d, float acc) {
    constexpr int kH = kNit >= 2 ? 2 : 1;  // pieces per 32-byte group
    constexpr int kG = kNit / kH;          // groups per lane
    const int c = base + kNit * lane;
    if (c < nchunk) {
        const int b = c >> 3, cc0 = c & 7;
        const Q4KScales sc = unpack_scales(hw.y, hw.z, hw.w);
        const float d = f16_bits_to_f32(hw.x & 0xffff);
        const float dmin = f16_bits_to_f32(hw.x >> 16);
        const uint8_t *yrow = s_qs + b * QK_K;
        float t = 0.0f;
        int S = 0, Mn = 0;
#pragma unroll
        for (int gi = 0; gi < kG; ++gi) {
            const int g = (cc0 >> 1) + gi;
            const uint32_t sw = g < 2 ? sc.s_lo : sc.s_hi;
            const uint32_t mw = g < 2 ? sc.m_lo : sc.m_hi;
            const int sh = (g & 1) * 16;
            const int s0 = (sw >> sh) & 0xff, s1 = (sw >> (sh + 8)) & 0xff;
            const int m0 = (mw >> sh) & 0xff, m1 = (mw >> (sh + 8)) & 0xff;
            int plo = 0, phi = 0, ylo_sum = 0, yhi_sum = 0;
#pragma unroll
            for (int hi = 0; hi < kH; ++hi) {
                const int h = kH == 2 ? hi : (cc0 & 1);
                const uint4 q = pw[gi * kH + hi];
                const uint4 ylo = *reinterpret_cast<const uint4 *>(yrow + 64 * g + 16 * h);
                const uint4 yhi = *reinterpret_cast<const uint4 *>(yrow + 64 * g + 32 + 16 * h);
                plo = dot4(q.x & 0x0f0f0f0fu, ylo.x, plo);
                plo = dot4(q.y & 0x0f0f0f0fu, ylo.y, plo);
                plo = dot4(q.z & 0x0f0f0f0fu, ylo.z, plo);
                plo = dot4(q.w & 0x0f0f0f0fu, ylo.w, plo);
                phi = dot4((q.x >> 4) & 0x0f0f0f0fu, yhi.x, phi);
                phi = dot4((q.y >> 4) & 0x0f0f0f0fu, yhi.y, phi);
                phi = dot4((q.z >> 4) & 0x0f0f0f0fu, yhi.z, phi);
                phi = dot4((q.w >> 4) & 0x0f0f0f0fu, yhi.w, phi);
                ylo_sum += s_bs[16 * b + 4 * g + h];
                yhi_sum += s_bs[16 * b + 4 * g + 2 + h];
            }
            S += s0 * plo + s1 * phi;
            Mn += m0 * ylo_sum + m1 * yhi_sum;
            if (kG == 4 && gi == 1) {  // first half of an eight-piece lane
                t = fmaf(d, (float)S, -dmin * (float)Mn);
                S = 0;
                Mn = 0;
            }
        }
        t += fmaf(d, (float)S, -dmin * (float)Mn);
        acc = fmaf(s_d[b], t, acc);
    }
    return acc;
}

template <int kNit>
__device__ __forceinline__ float gemv1_accumulate(const uint4 (&hw)[gemv1_subs<kNit>()],
                                                  const uint4 (&pw)[kNit], int base, int nchunk,
                                                  int lane, const uint8_t *s_qs, const int16_t *s_bs,
                                                  const float *s_d, float acc) {
    constexpr int kP = gemv1_kp<kNit>();
#pragma unroll
    for (int sp = 0; sp < gemv1_subs<kNit>(); ++sp)
        acc = gemv1_acc_sub<kP>(hw[sp], pw + kP * sp, base + 64 * kP * sp, nchunk, lane, s_qs, s_bs, s_d, acc);
    return acc;
}

// ID = true: mul_mat_id, one (token, slot) pair per blockIdx.y (id_route).
template <bool REPACKED, int kNit, bool ID>
__global__ __launch_bounds__(256) void k_gemv1_q4_K(const uint8_t *__restrict__ W,
                                                    const uint8_t *__restrict__ Y,
                                                    float *__restrict__ out, int64_t N, int64_t K,
                                                    IdRoute route) {
    bool valid = true;
    if constexpr (ID) {
        const IdPair ip = id_route(route);
        valid = ip.valid;
        W += ip.w_off;
        Y += ip.y_off;
        out += ip.out_row * N;
    }
    // 16-byte activation pieces per thread loaded up front (K <= 4096 * kYT)
    constexpr int kYT = kNit >= 8 ? 4 : (kNit + 1) / 2;
    extern __shared__ __attribute__((aligned(16))) uint8_t ys[];
    const int64_t nb = K / QK_K;
    const int nchunk = (int)(nb * 8);
    uint8_t *s_qs = ys;
    float *s_d = reinterpret_cast<float *>(ys + K);
    int16_t *s_bs = reinterpret_cast<int16_t *>(ys + K + (nb * 4 + 15) / 16 * 16);
    uint8_t *s_trash = ys + K + (nb * 4 + 15) / 16 * 16 + nb * 32;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int64_t n = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    const int64_t nn = n < N ? n : N - 1;  // a tail wavefront loads a valid row, stores nothing
    const Q4KAddr<REPACKED> A{W, N, nb};
    const int nq = (int)(K / 16), nbs = (int)(nb * 2);

    // activation row -> registers (indices clamped: branch-free loads), then
    // the first pass of this row's weights, then the row -> LDS
    uint4 yq[kYT];
#pragma unroll
    for (int t = 0; t < kYT; ++t) {
        const int pc = tid + 256 * t < nq ? tid + 256 * t : nq - 1;
        yq[t] = ld_align4<uint4>(Y + (pc >> 4) * kQ8_KBytes + 4 + 16 * (pc & 15));
    }
    const int qb = tid < nbs ? tid : nbs - 1, qd = tid < nb ? tid : (int)nb - 1;
    const uint4 yb = ld_align4<uint4>(Y + (qb >> 1) * kQ8_KBytes + 260 + 16 * (qb & 1));
    const float yd = ld_align4<float>(Y + qd * kQ8_KBytes);
    __builtin_amdgcn_sched_barrier(0);  // keep the activation loads ahead of the weights
    uint4 pw[kNit], hw[gemv1_subs<kNit>()];
    gemv1_load<REPACKED, kNit>(A, nn, 0, nchunk, lane, hw, pw);
#pragma unroll
    for (int t = 0; t < kYT; ++t) {
        const int pc = tid + 256 * t;
        *reinterpret_cast<uint4 *>(pc < nq ? s_qs + 16 * pc : s_trash) = yq[t];
    }
    *reinterpret_cast<uint4 *>(tid < nbs ? reinterpret_cast<uint8_t *>(s_bs + 8 * tid) : s_trash) = yb;
    *reinterpret_cast<float *>(tid < nb ? reinterpret_cast<uint8_t *>(s_d + tid) : s_trash) = yd;
    // rows longer than 256 * kYT pieces: the rest of the activation row
    for (int pc = tid + 256 * kYT; pc < nq; pc += 256)
        *reinterpret_cast<uint4 *>(s_qs + 16 * pc) =
            ld_align4<uint4>(Y + (pc >> 4) * kQ8_KBytes + 4 + 16 * (pc & 15));
    for (int q = tid + 256; q < nbs; q += 256)
        *reinterpret_cast<uint4 *>(s_bs + 8 * q) =
            ld_align4<uint4>(Y + (q >> 1) * kQ8_KBytes + 260 + 16 * (q & 1));
    for (int q = tid + 256; q < nb; q += 256) s_d[q] = ld_align4<float>(Y + q * kQ8_KBytes);
    __syncthreads();

    float acc = gemv1_accumulate<kNit>(hw, pw, 0, nchunk, lane, s_qs, s_bs, s_d, 0.0f);
    for (int base = 64 * kNit; base < nchunk; base += 64 * kNit) {
        gemv1_load<REPACKED, kNit>(A, nn, base, nchunk, lane, hw, pw);
        acc = gemv1_accumulate<kNit>(hw, pw, base, nchunk, lane, s_qs, s_bs, s_d, acc);
    }
    acc = wave_sum(acc);
    if (lane == 0 && n < N) out[n] = valid ? acc : __builtin_nanf("");
}

// ---------------------------------------------------------------------------
// Fused M = 1 path: the fp32 activation row is quantized to Q8_K inside the
// GEMV, straight into LDS, so one launch covers quantize + mul_mat.
// Quantization costs vector-ALU work that every workgroup repeats, so the
// grid holds one 16-wavefront workgroup per CU and each workgroup loops over
// rows (wavefront w of workgroup g takes rows g*16 + w, then + 16*gridDim.x,
// ...).  A wavefront first loads up to kXB of its fp32 activation blocks
// (b = wave + 16i), then issues the loads of its first row and quantizes
// while the weights are in flight; in the row loop the next row's
// pieces are loaded before the current row is reduced when the row takes at
// most two pieces per lane (longer rows load it right after).  Rows are one
// pass: K <= 16384, at most eight pieces per lane.  With eight pieces a
// wavefront requests only the first two of its four sub-passes before
// quantizing and the other two after the barrier: the memory pipeline takes
// requests at the rate it delivers, so a wavefront issuing all twelve loads
// first reached its quantization, and the whole workgroup its barrier, late,
// and every row was then reduced at once after the barrier (N = 4096,
// K = 14336: 9.35 against 10.6 us for this kernel with all requests first, or
// for the two launches).  Workgroup 0 also stores
// the Q8_K bytes to Yq, byte-identical to the stand-alone quantizer (same
// device routine), so another projection of the same input can reuse them.
// ---------------------------------------------------------------------------
constexpr int kFusedWaves = 16;

template <bool REPACKED, int kNit, int kXB>
__global__ __launch_bounds__(kFusedWaves * 64) void k_gemv1_fused_q4_K(
    const uint8_t *__restrict__ W, const float *__restrict__ X, uint8_t *__restrict__ Yq,
    float *__restrict__ out, int64_t N, int64_t K) {
    extern __shared__ __attribute__((aligned(16))) uint8_t ys[];
    const int64_t nb = K / QK_K;
    const int nchunk = (int)(nb * 8);
    uint8_t *s_qs = ys;
    float *s_d = reinterpret_cast<float *>(ys + K);
    int16_t *s_bs = reinterpret_cast<int16_t *>(ys + K + (nb * 4 + 15) / 16 * 16);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int64_t stride = (int64_t)gridDim.x * kFusedWaves;
    int64_t row = (int64_t)blockIdx.x * kFusedWaves + wave;  // uniform per wavefront
    const Q4KAddr<REPACKED> A{W, N, nb};
    const bool store_q = blockIdx.x == 0;

    // one 256-value block per wavefront and step: quantize, write LDS (a block
    // past the row goes to the trash slot)
    auto quantize_block = [&](const float4 v, int b) { q8k_quantize_block_lds(v, b, K, ys, lane); };

    // the launcher guarantees nb <= 16 * kXB; block indices past the row end
    // load the last block again (branch-free loads)
    float4 xv[kXB];
#pragma unroll
    for (int i = 0; i < kXB; ++i) {
        const int b0 = wave + kFusedWaves * i;  // uniform per wavefront
        const int b = b0 < nb ? b0 : (int)nb - 1;
        xv[i] = *reinterpret_cast<const float4 *>(X + (int64_t)b * QK_K + 4 * lane);
    }
    // With at most two rows per wavefront the activation loads complete before
    // any weight load is issued: queued behind the weight stream of the whole
    // chip they would arrive late, and the quantization, the barrier and every
    // reduction would wait for them (measured: N = K = 4096 4.2 against
    // 4.7 us; N = 4096, K = 8192 6.3 against 6.8 us).  With more rows the
    // first rows' weights are better requested at once (N = 28672, K = 4096:
    // 13.5 against 13.8 us).
    // Rows of eight pieces issue only part of the row first (below), so there
    // the x loads need no head start (9.35 against 9.45 us at N = 4096,
    // K = 14336).
    if (kNit < 8 && N <= 2 * stride) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // uniform
    __builtin_amdgcn_sched_barrier(0);
    uint4 pw[kNit], hw[gemv1_subs<kNit>()];
    // sub-passes of the first row requested before quantizing: all, or two of
    // four for rows of eight pieces (one or three measured slower: 9.7 and
    // 10.0 us at N = 4096, K = 14336)
    constexpr int kFirst = kNit >= 8 ? 2 : gemv1_subs<kNit>();
    // a wavefront without rows loads a valid row and stores nothing
    gemv1_load<REPACKED, kNit, 0, kFirst>(A, row < N ? row : N - 1, 0, nchunk, lane, hw, pw);
    // and every weight load ahead of the quantization: left to itself the
    // scheduler issues part of them after the first block's arithmetic
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kXB; ++i) quantize_block(xv[i], wave + kFusedWaves * i);
    __syncthreads();
    // the rest of the first row, requested once the activation row is in LDS
    gemv1_load<REPACKED, kNit, kFirst>(A, row < N ? row : N - 1, 0, nchunk, lane, hw, pw);

    auto finish = [&](int64_t r, float acc) {
        acc = wave_sum(acc);
        if (lane == 0) out[r] = acc;
    };
    if constexpr (kNit <= 2) {
        // Rows of one pass, two register stages: the next row's pieces are
        // requested before the current row is reduced.  Every load is
        // unconditional (past the last row it fetches row N - 1 again and
        // drops it), so the wait before a reduction covers only the older
        // stage; a conditional prefetch would make it wait for both.
        uint4 pn[kNit], hn[gemv1_subs<kNit>()];
        for (; row < N; row += 2 * stride) {
            const int64_t r1 = row + stride, r2 = r1 + stride;
            gemv1_load<REPACKED, kNit>(A, r1 < N ? r1 : N - 1, 0, nchunk, lane, hn, pn);
            finish(row, gemv1_accumulate<kNit>(hw, pw, 0, nchunk, lane, s_qs, s_bs, s_d, 0.0f));
            if (r1 >= N) break;
            gemv1_load<REPACKED, kNit>(A, r2 < N ? r2 : N - 1, 0, nchunk, lane, hw, pw);
            finish(r1, gemv1_accumulate<kNit>(hn, pn, 0, nchunk, lane, s_qs, s_bs, s_d, 0.0f));
        }
    } else {
        // longer rows: the first row's pieces are in flight already; it is
        // reduced outside the loop, so its waits follow the pieces in order
        if (row < N) finish(row, gemv1_accumulate<kNit>(hw, pw, 0, nchunk, lane, s_qs, s_bs, s_d, 0.0f));
        for (row += stride; row < N; row += stride) {
            gemv1_load<REPACKED, kNit>(A, row, 0, nchunk, lane, hw, pw);
            finish(row, gemv1_accumulate<kNit>(hw, pw, 0, nchunk, lane, s_qs, s_bs, s_d, 0.0f));
        }
    }
    // Workgroup 0 copies the Q8_K row to Yq last: stores issued before the
    // row loop would sit in the same in-order counter as the weight loads and
    // make the first reduction wait for all of them.
    if (store_q) q8k_store_row<kFusedWaves * 64>(Yq, ys, K);
}

// ---------------------------------------------------------------------------
// Q4_0 x Q8_0: one lane per 32-element block (16-byte payload).  Canonical
// blocks are 18 B and Q8_0 blocks 34 B, so both are read with 2-byte loads;
// the repacked weight payload is read with one aligned 16-byte load.
// P_b = sum (q-8)*y = sum q*y - 8*sum y; partial = d_w*d_a*P_b.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t ld_u32_a2(const uint8_t *p) {
    const uint16_t *q = reinterpret_cast<const uint16_t *>(p);
    return (uint32_t)q[0] | ((uint32_t)q[1] << 16);
}

// ID = true (M = 1, MODE 0): mul_mat_id, one (token, slot) pair per blockIdx.y.
template <int M, bool REPACKED, int MODE, bool ID = false>
__global__ __launch_bounds__(256) void k_gemv_q4_0(const uint8_t *__restrict__ W,
                                                   const uint8_t *__restrict__ Y,
                                                   void *__restrict__ dst, int64_t N, int64_t K,
                                                   int64_t dsec, IdRoute route = {}) {
    bool valid = true;
    if constexpr (ID) {
        const IdPair ip = id_route(route);
        valid = ip.valid;
        W += ip.w_off;
        Y += ip.y_off;
        dst = reinterpret_cast<float *>(dst) + ip.out_row * N;
    }
    const int64_t nb = K / QK4_0;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t n = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    if (n >= N) return;  // uniform per wavefront
    float acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = 0.0f;
    for (int64_t b = lane; b < nb; b += kWave) {
        uint32_t w[4];
        float dw;
        if (REPACKED) {
            const uint4 v = ld16(W + dsec + 16 * (n * nb + b));
            w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
            dw = f16_bits_to_f32(ld_u16(W + 2 * (n * nb + b)));
        } else {
            const uint8_t *blk = W + kQ4_0Bytes * (n * nb + b);
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = ld_u32_a2(blk + 2 + 4 * i);
            dw = f16_bits_to_f32(ld_u16(blk));
        }
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const uint8_t *yb = Y + ((int64_t)m * nb + b) * kQ8_0Bytes;
            const float da = f16_bits_to_f32(ld_u16(yb));
            int p = 0, ys = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t ya = ld_u32_a2(yb + 2 + 4 * i);        // elements 4i..4i+3
                const uint32_t yc = ld_u32_a2(yb + 2 + 16 + 4 * i);   // elements 16+4i..
                p = dot4(w[i] & 0x0f0f0f0fu, ya, p);
                p = dot4((w[i] >> 4) & 0x0f0f0f0fu, yc, p);
                ys = dot4(0x01010101u, ya, ys);
                ys = dot4(0x01010101u, yc, ys);
            }
            p -= 8 * ys;
            if (MODE == 0) {
                acc[m] = fmaf(dw * da, (float)p, acc[m]);
            } else {
                reinterpret_cast<int32_t *>(dst)[((int64_t)m * N + n) * nb + b] = p;
            }
        }
    }
    if (MODE == 0) {
        float *out = reinterpret_cast<float *>(dst);
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const float v = wave_sum(acc[m]);
            if (lane == 0) out[(int64_t)m * N + n] = valid ? v : __builtin_nanf("");
        }
    }
}

// ---------------------------------------------------------------------------
// Q4_0 x Q8_0 with the activation rows staged in LDS (K a multiple of 64 and
// M * K * 5/4 bytes within the LDS budget).  The workgroup first moves its M
// activation rows into LDS once, in 68-byte block pairs (dword-aligned because
// nb is even: four 16-byte loads and one 4-byte load per pair), realigns the
// first block's codes with v_alignbyte, and stores per block the 32 codes, d_a
// as fp32 and the code sum sum_i y_i (for the -8 of every weight).  Then each
// wavefront takes one output row as in k_gemv_q4_0, with the activation
// operands from LDS instead of 2-byte global loads.  The two 16-byte code reads
// of block b go in the order (b & 1, 1 - (b & 1)), so 16 consecutive lanes
// (consecutive blocks) read 16 distinct 16-byte slots; the weight nibbles are
// paired to match.  Same integer sums and the same fp32 operations, in the
// same order, as k_gemv_q4_0.
// ---------------------------------------------------------------------------
int64_t gemv_q4_0s_lds_bytes(int64_t M, int64_t K) { return M * (K / QK4_0) * (32 + 4 + 4); }

// Rows of a Q4_0 GEMV against activation rows staged in LDS (codes [M][nb][32],
// d_a [M][nb] as fp32, code sums [M][nb]): wavefront w of the workgroup takes
// output row blockIdx.x * 4 + w (the compute half of k_gemv_q4_0s, shared with
// the fused quantize + GEMV kernel).
template <int M, bool REPACKED, int MODE>
__device__ __forceinline__ void gemv_q4_0_lds_rows(const uint8_t *__restrict__ W, void *__restrict__ dst,
                                                   int64_t N, int64_t nb, int64_t dsec, const uint8_t *s_q,
                                                   const float *s_d, const int *s_s, bool valid,
                                                   const uint32_t *pre_w = nullptr, float pre_dw = 0.f) {
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int64_t n = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    if (n >= N) return;  // uniform per wavefront; the caller's barrier is behind it
    float acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = 0.0f;
    for (int64_t b = lane; b < nb; b += kWave) {
        uint32_t w[4];
        float dw;
        if (pre_w != nullptr && b == lane) {
            w[0] = pre_w[0]; w[1] = pre_w[1]; w[2] = pre_w[2]; w[3] = pre_w[3];
            dw = pre_dw;
        } else if (REPACKED) {
            const uint4 v = ld16(W + dsec + 16 * (n * nb + b));
            w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
            dw = f16_bits_to_f32(ld_u16(W + 2 * (n * nb + b)));
        } else {
            const uint8_t *blk = W + kQ4_0Bytes * (n * nb + b);
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = ld_u32_a2(blk + 2 + 4 * i);
            dw = f16_bits_to_f32(ld_u16(blk));
        }
        // first read: elements 16*odd .. +15 (nibbles >> 4*odd), second: the other half
        const int odd = (int)(b & 1), sa = 4 * odd, sb = 4 - sa;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int64_t bi = (int64_t)m * nb + b;
            const uint8_t *cq = s_q + bi * 32;
            const uint4 ra = *reinterpret_cast<const uint4 *>(cq + 16 * odd);
            const uint4 rb = *reinterpret_cast<const uint4 *>(cq + 16 - 16 * odd);
            const uint32_t ya[4] = {ra.x, ra.y, ra.z, ra.w}, yb[4] = {rb.x, rb.y, rb.z, rb.w};
            int p = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p = dot4((w[i] >> sa) & 0x0f0f0f0fu, ya[i], p);
                p = dot4((w[i] >> sb) & 0x0f0f0f0fu, yb[i], p);
            }
            p -= 8 * s_s[bi];
            if (MODE == 0) {
                acc[m] = fmaf(dw * s_d[bi], (float)p, acc[m]);
            } else {
                reinterpret_cast<int32_t *>(dst)[((int64_t)m * N + n) * nb + b] = p;
            }
        }
    }
    if (MODE == 0) {
        float *out = reinterpret_cast<float *>(dst);
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const float v = wave_sum(acc[m]);
            if (lane == 0) out[(int64_t)m * N + n] = valid ? v : __builtin_nanf("");
        }
    }
}

template <int M, bool REPACKED, int MODE, bool ID = false>
__global__ __launch_bounds__(256) void k_gemv_q4_0s(const uint8_t *__restrict__ W,
                                                    const uint8_t *__restrict__ Y,
                                                    void *__restrict__ dst, int64_t N, int64_t K,
                                                    int64_t dsec, IdRoute route = {}) {
    bool valid = true;
    if constexpr (ID) {
        const IdPair ip = id_route(route);
        valid = ip.valid;
        W += ip.w_off;
        Y += ip.y_off;
        dst = reinterpret_cast<float *>(dst) + ip.out_row * N;
    }
    extern __shared__ __attribute__((aligned(16))) uint8_t ys[];
    const int64_t nb = K / QK4_0;
    const int nbi = (int)nb, half = nbi / 2;
    uint8_t *s_q = ys;                                             // codes [M][nb][32]
    float *s_d = reinterpret_cast<float *>(ys + (int64_t)M * nb * 32);  // d_a [M][nb]
    int *s_s = reinterpret_cast<int *>(s_d + M * nb);              // sum of codes [M][nb]
    const int tid = threadIdx.x;

    // ---- stage the M rows: pair pr of row m is [d0 | 32 codes | d1 | 32 codes]
    for (int q = tid; q < M * half; q += 256) {
        const int m = q / half, pr = q - m * half;
        const int blk = m * nbi + 2 * pr;
        const uint8_t *src = Y + (int64_t)blk * kQ8_0Bytes;
        uint4 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = ld_align4<uint4>(src + 16 * k);
        const uint32_t w[17] = {v[0].x, v[0].y, v[0].z, v[0].w, v[1].x, v[1].y, v[1].z, v[1].w, v[2].x,
                                v[2].y, v[2].z, v[2].w, v[3].x, v[3].y, v[3].z, v[3].w,
                                ld_align4<uint32_t>(src + 64)};
        uint32_t c0[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) c0[j] = __builtin_amdgcn_alignbyte(w[j + 1], w[j], 2);
        uint4 *dq = reinterpret_cast<uint4 *>(s_q + (int64_t)blk * 32);
        dq[0] = make_uint4(c0[0], c0[1], c0[2], c0[3]);
        dq[1] = make_uint4(c0[4], c0[5], c0[6], c0[7]);
        dq[2] = make_uint4(w[9], w[10], w[11], w[12]);
        dq[3] = make_uint4(w[13], w[14], w[15], w[16]);
        int s0 = 0, s1 = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            s0 = dot4(0x01010101u, c0[j], s0);
            s1 = dot4(0x01010101u, w[9 + j], s1);
        }
        s_d[blk] = f16_bits_to_f32(w[0] & 0xffff);
        s_d[blk + 1] = f16_bits_to_f32(w[8] >> 16);
        s_s[blk] = s0;
        s_s[blk + 1] = s1;
    }
    __syncthreads();
    gemv_q4_0_lds_rows<M, REPACKED, MODE>(W, dst, N, nb, dsec, s_q, s_d, s_s, valid);
}

// ---------------------------------------------------------------------------
// Fused M = 1 path for Q4_0 on small matrices, where a second launch costs
// more than the work: every workgroup quantizes the fp32 row into Q8_0 codes
// in LDS, in the staged layout above, with the stand-alone quantizer's block
// routine (8 lanes per 32-value block); workgroup 0 also stores the Q8_0
// bytes to Yq, byte-identical to quantize_row_q8.  Then each wavefront takes
// one output row (gemv_q4_0_lds_rows): the same integer sums and fp32
// operations, in the same order, as quantize_row_q8 followed by either Q4_0
// GEMV.  The first pass's activation values and each lane's first weight
// block are requested before the quantization, so the weight latency runs
// under it (N = 256, K = 1024: 2.98 -> 2.83 us).
// ---------------------------------------------------------------------------
template <bool REPACKED>
__global__ __launch_bounds__(256) void k_gemv_fused_q4_0(const uint8_t *__restrict__ W,
                                                         const float *__restrict__ X, uint8_t *__restrict__ Yq,
                                                         float *__restrict__ out, int64_t N, int64_t K,
                                                         int64_t dsec) {
    extern __shared__ __attribute__((aligned(16))) uint8_t ys[];
    const int64_t nb = K / QK4_0;
    uint8_t *s_q = ys;                                   // codes [nb][32]
    float *s_d = reinterpret_cast<float *>(ys + nb * 32);  // d_a [nb] (the fp16 value)
    int *s_s = reinterpret_cast<int *>(s_d + nb);         // sum of codes [nb]
    const int tid = threadIdx.x, sub = tid & 7;
    float4 xv0 = make_float4(0.f, 0.f, 0.f, 0.f);
    if ((tid >> 3) < nb) xv0 = *reinterpret_cast<const float4 *>(X + (tid >> 3) * QK4_0 + sub * 4);
    __builtin_amdgcn_sched_barrier(0);
    uint32_t pw[4] = {0, 0, 0, 0};
    float pdw = 0.f;
    {
        const int wave = tid >> 6, lane = tid & 63;
        const int64_t n = (int64_t)blockIdx.x * kWavesPerBlock + wave;
        if (n < N && lane < nb) {
            const int64_t b = lane;
            if (REPACKED) {
                const uint4 v = ld16(W + dsec + 16 * (n * nb + b));
                pw[0] = v.x; pw[1] = v.y; pw[2] = v.z; pw[3] = v.w;
                pdw = f16_bits_to_f32(ld_u16(W + 2 * (n * nb + b)));
            } else {
                const uint8_t *blk = W + kQ4_0Bytes * (n * nb + b);
#pragma unroll
                for (int i = 0; i < 4; ++i) pw[i] = ld_u32_a2(blk + 2 + 4 * i);
                pdw = f16_bits_to_f32(ld_u16(blk));
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    for (int64_t base = 0; base < nb; base += 32) {  // 32 blocks per pass, every lane in each pass
        const int64_t blk = base + (tid >> 3);
        const bool live = blk < nb;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (base == 0) v = xv0;
        else if (live) v = *reinterpret_cast<const float4 *>(X + blk * QK4_0 + sub * 4);
        const Q80Part r = q8_0_quantize_part(v);
        int cs = dot4(0x01010101u, r.q, 0);  // the block's code sum over its 8 lanes
#pragma unroll
        for (int o = 4; o > 0; o >>= 1) cs += __shfl_xor(cs, o, kWave);
        if (live) {
            const uint32_t d16 = f32_to_f16_bits(r.d);
            *reinterpret_cast<uint32_t *>(s_q + blk * 32 + 4 * sub) = r.q;
            if (sub == 0) {
                s_d[blk] = f16_bits_to_f32(d16);
                s_s[blk] = cs;
            }
            if (blockIdx.x == 0) {
                uint8_t *o = Yq + blk * kQ8_0Bytes;
                uint16_t *o16 = reinterpret_cast<uint16_t *>(o + 2 + sub * 4);
                o16[0] = (uint16_t)(r.q & 0xffff);
                o16[1] = (uint16_t)(r.q >> 16);
                if (sub == 0) *reinterpret_cast<uint16_t *>(o) = (uint16_t)d16;
            }
        }
    }
    __syncthreads();
    gemv_q4_0_lds_rows<1, REPACKED, 0>(W, out, N, nb, dsec, s_q, s_d, s_s, true, pw, pdw);
}

template <int MODE>
hipError_t dispatch_q4_K(const uint8_t *w, bool rep, const uint8_t *y, void *dst, int64_t M,
                         int64_t N, int64_t K, hipStream_t s) {
#define QMM_GEMV_K(MM, RR)                                                                       \
    do {                                                                                         \
        const int64_t rows_per_block = (int64_t)kWavesPerBlock * (RR);                           \
        const dim3 grid((unsigned)((N + rows_per_block - 1) / rows_per_block));                  \
        if (rep)                                                                                 \
            hipLaunchKernelGGL((k_gemv_q4_K<MM, RR, true, MODE>), grid, dim3(256), 0, s, w, y,    \
                               dst, N, K);                                                       \
        else                                                                                     \
            hipLaunchKernelGGL((k_gemv_q4_K<MM, RR, false, MODE>), grid, dim3(256), 0, s, w, y,   \
                               dst, N, K);                                                       \
    } while (0)
    switch (M) {
        case 1: QMM_GEMV_K(1, 1); break;
        case 2: QMM_GEMV_K(2, 2); break;
        case 3: QMM_GEMV_K(3, 2); break;
        case 4: QMM_GEMV_K(4, 2); break;
        case 5: QMM_GEMV_K(5, 2); break;
        case 6: QMM_GEMV_K(6, 2); break;
        case 7: QMM_GEMV_K(7, 2); break;
        case 8: QMM_GEMV_K(8, 2); break;
        default: return hipErrorInvalidValue;
    }
#undef QMM_GEMV_K
    return hipGetLastError();
}

template <int MODE>
hipError_t dispatch_q4_0(const uint8_t *w, bool rep, const uint8_t *y, void *dst, int64_t M,
                         int64_t N, int64_t K, hipStream_t s) {
    const int64_t dsec = repacked_bytes_q4_0(N, K) - 16 * N * (K / QK4_0);
    const dim3 grid((unsigned)((N + kWavesPerBlock - 1) / kWavesPerBlock));
    // activation rows staged in LDS where they fit and the matrix is large
    // enough for the staging latency to pay (N*K >= 2^22; at c1, 256 x 1024,
    // the per-lane kernel is 0.2 us faster), else read per lane
    const bool staged = gemv_q4_0s_fits(M, K) && N * K >= (int64_t(1) << 22);
    const unsigned lds = staged ? (unsigned)gemv_q4_0s_lds_bytes(M, K) : 0u;
#define QMM_GEMV_0(MM)                                                                                   \
    do {                                                                                                 \
        if (staged && rep)                                                                               \
            hipLaunchKernelGGL((k_gemv_q4_0s<MM, true, MODE>), grid, dim3(256), lds, s, w, y, dst, N, K,  \
                               dsec, IdRoute{});                                                         \
        else if (staged)                                                                                 \
            hipLaunchKernelGGL((k_gemv_q4_0s<MM, false, MODE>), grid, dim3(256), lds, s, w, y, dst, N, K, \
                               dsec, IdRoute{});                                                         \
        else if (rep)                                                                                    \
            hipLaunchKernelGGL((k_gemv_q4_0<MM, true, MODE>), grid, dim3(256), 0, s, w, y, dst, N, K,     \
                               dsec);                                                                    \
        else                                                                                             \
            hipLaunchKernelGGL((k_gemv_q4_0<MM, false, MODE>), grid, dim3(256), 0, s, w, y, dst, N, K,    \
                               dsec);                                                                    \
    } while (0)
    switch (M) {
        case 1: QMM_GEMV_0(1); break;
        case 2: QMM_GEMV_0(2); break;
        case 3: QMM_GEMV_0(3); break;
        case 4: QMM_GEMV_0(4); break;
        case 5: QMM_GEMV_0(5); break;
        case 6: QMM_GEMV_0(6); break;
        case 7: QMM_GEMV_0(7); break;
        case 8: QMM_GEMV_0(8); break;
        default: return hipErrorInvalidValue;
    }
#undef QMM_GEMV_0
    return hipGetLastError();
}

}  // namespace

bool gemv_q4_0s_fits(int64_t M, int64_t K) {
    return K % 64 == 0 && gemv_q4_0s_lds_bytes(M, K) <= 60 * 1024;
}

hipError_t launch_gemv_q4_K(const uint8_t *w, bool repacked, const uint8_t *y, float *out,
                            int64_t M, int64_t N, int64_t K, hipStream_t s) {
    const int64_t lds = gemv1_lds_bytes(K);
    const int64_t nit = (K / QK_K * 8 + 63) / 64;  // 16-byte pieces per lane for one row
    if (M == 1 && lds <= 60 * 1024) {
        const dim3 grid((unsigned)((N + kWavesPerBlock - 1) / kWavesPerBlock));
#define QMM_GEMV1(NIT)                                                                                     \
    do {                                                                                                   \
        if (repacked)                                                                                      \
            hipLaunchKernelGGL((k_gemv1_q4_K<true, NIT, false>), grid, dim3(256), (unsigned)lds, s, w, y, out,   \
                               N, K, IdRoute{});                                                           \
        else                                                                                               \
            hipLaunchKernelGGL((k_gemv1_q4_K<false, NIT, false>), grid, dim3(256), (unsigned)lds, s, w, y, out,  \
                               N, K, IdRoute{});                                                           \
    } while (0)
        if (nit <= 1) QMM_GEMV1(1);
        else if (nit <= 2) QMM_GEMV1(2);
        else if (nit <= 4) QMM_GEMV1(4);
        else QMM_GEMV1(8);
#undef QMM_GEMV1
        return hipGetLastError();
    }
    return dispatch_q4_K<0>(w, repacked, y, out, M, N, K, s);
}

int64_t gemv1_max_k() {
    int64_t k = 0;
    while (gemv1_lds_bytes(k + QK_K) <= 60 * 1024) k += QK_K;
    return k;
}

hipError_t launch_gemv_id_q4_K(const uint8_t *w, bool repacked, int64_t w_stride, const uint8_t *y,
                               int y_per_slot, const int32_t *ids, int64_t P, int64_t U, int64_t E,
                               float *out, int64_t N, int64_t K, hipStream_t s) {
    const int64_t lds = gemv1_lds_bytes(K);
    const int64_t nit = (K / QK_K * 8 + 63) / 64;
    for (int64_t p0 = 0; p0 < P; p0 += 65535) {
        const int64_t pp = P - p0 < 65535 ? P - p0 : 65535;
        const dim3 grid((unsigned)((N + kWavesPerBlock - 1) / kWavesPerBlock), (unsigned)pp);
        const IdRoute r{ids, p0, U, E, w_stride, (K / QK_K) * kQ8_KBytes, y_per_slot};
#define QMM_GEMV_ID(NIT)                                                                                   \
    do {                                                                                                   \
        if (repacked)                                                                                      \
            hipLaunchKernelGGL((k_gemv1_q4_K<true, NIT, true>), grid, dim3(256), (unsigned)lds, s, w, y, out,    \
                               N, K, r);                                                                   \
        else                                                                                               \
            hipLaunchKernelGGL((k_gemv1_q4_K<false, NIT, true>), grid, dim3(256), (unsigned)lds, s, w, y, out,   \
                               N, K, r);                                                                   \
    } while (0)
        if (nit <= 1) QMM_GEMV_ID(1);
        else if (nit <= 2) QMM_GEMV_ID(2);
        else if (nit <= 4) QMM_GEMV_ID(4);
        else QMM_GEMV_ID(8);
#undef QMM_GEMV_ID
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

int64_t gemv1_fused_max_k() {
    // rows of up to eight 16-byte pieces per lane (K <= 16384, 104-117
    // registers); longer rows take two launches (quantize, then the GEMV)
    return 8 * 64 / 8 * QK_K;
}

int cu_count() {
    static int cached[64];  // per device; 0 = not queried yet
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = __atomic_load_n(&cached[dev], __ATOMIC_RELAXED);
    if (v == 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
            v = 256;
        __atomic_store_n(&cached[dev], v, __ATOMIC_RELAXED);
    }
    return v;
}

hipError_t launch_gemv1_fused_q4_K(const uint8_t *w, bool repacked, const float *x, uint8_t *yq,
                                   float *out, int64_t N, int64_t K, hipStream_t s) {
    const int64_t lds = gemv1_lds_bytes(K);
    const int64_t nit = (K / QK_K * 8 + 63) / 64;
    // at most one workgroup per CU: every extra workgroup repeats the
    // quantization, and 16 wavefronts per CU, each with two rows in flight,
    // keep the weight stream full (measured: a second 16-wavefront workgroup
    // per CU, or a third register stage, made N = 28672, K = 4096 slower)
    const int64_t groups = (N + kFusedWaves - 1) / kFusedWaves;
    const int64_t cus = cu_count();
    const dim3 grid((unsigned)(groups < cus ? groups : cus)), block(kFusedWaves * 64);
#define QMM_FUSED1(NIT, XB)                                                                        \
    do {                                                                                           \
        if (repacked)                                                                              \
            hipLaunchKernelGGL((k_gemv1_fused_q4_K<true, NIT, XB>), grid, block, (unsigned)lds, s, \
                               w, x, yq, out, N, K);                                               \
        else                                                                                       \
            hipLaunchKernelGGL((k_gemv1_fused_q4_K<false, NIT, XB>), grid, block, (unsigned)lds,   \
                               s, w, x, yq, out, N, K);                                            \
    } while (0)
    // kXB = activation blocks per wavefront: ceil(nb / 16) (nb <= 8 * kNit <= 16 * kXB)
    if (nit <= 1) QMM_FUSED1(1, 1);
    else if (nit <= 2) QMM_FUSED1(2, 1);
    else if (nit <= 4) QMM_FUSED1(4, 2);
    else QMM_FUSED1(8, 4);
#undef QMM_FUSED1
    return hipGetLastError();
}

hipError_t launch_block_sums_q4_K(const uint8_t *w, bool repacked, const uint8_t *y, int32_t *P,
                                  int64_t M, int64_t N, int64_t K, hipStream_t s) {
    // the sums path is launched per group of up to 8 activation rows
    for (int64_t m0 = 0; m0 < M; m0 += kGemvMaxM) {
        const int64_t mm = M - m0 < kGemvMaxM ? M - m0 : kGemvMaxM;
        hipError_t e = dispatch_q4_K<1>(w, repacked, y + m0 * (K / QK_K) * kQ8_KBytes,
                                        P + m0 * N * (K / 32), mm, N, K, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_gemv_q4_0(const uint8_t *w, bool repacked, const uint8_t *y, float *out,
                            int64_t M, int64_t N, int64_t K, hipStream_t s) {
    return dispatch_q4_0<0>(w, repacked, y, out, M, N, K, s);
}

bool gemv_fused_q4_0_ok(int64_t N, int64_t K) {
    // small matrices only: each of the N/4 workgroups repeats the quantization,
    // one pass of 32 blocks after another (N = 256, K = 16384 took 14.5 us
    // against 9.4 us for the two launches; N = 1024, K = 4096: 5.3 against
    // 5.7 us)
    constexpr int64_t kFusedQ40MaxK = 4096, kFusedQ40MaxNK = int64_t(1) << 22;
    return K % 64 == 0 && K <= kFusedQ40MaxK && N * K <= kFusedQ40MaxNK;
}

hipError_t launch_gemv_fused_q4_0(const uint8_t *w, bool repacked, const float *x, uint8_t *yq, float *out,
                                  int64_t N, int64_t K, hipStream_t s) {
    if (!gemv_fused_q4_0_ok(N, K)) return hipErrorInvalidValue;
    const int64_t dsec = repacked_bytes_q4_0(N, K) - 16 * N * (K / QK4_0);
    const dim3 grid((unsigned)((N + kWavesPerBlock - 1) / kWavesPerBlock));
    const unsigned lds = (unsigned)gemv_q4_0s_lds_bytes(1, K);
    if (repacked)
        hipLaunchKernelGGL((k_gemv_fused_q4_0<true>), grid, dim3(256), lds, s, w, x, yq, out, N, K, dsec);
    else
        hipLaunchKernelGGL((k_gemv_fused_q4_0<false>), grid, dim3(256), lds, s, w, x, yq, out, N, K, dsec);
    return hipGetLastError();
}

hipError_t launch_gemv_id_q4_0(const uint8_t *w, bool repacked, int64_t w_stride, const uint8_t *y,
                               int y_per_slot, const int32_t *ids, int64_t P, int64_t U, int64_t E,
                               float *out, int64_t N, int64_t K, hipStream_t s) {
    const int64_t dsec = repacked ? (2 * N * (K / QK4_0) + 255) / 256 * 256 : 0;
    for (int64_t p0 = 0; p0 < P; p0 += 65535) {
        const int64_t pp = P - p0 < 65535 ? P - p0 : 65535;
        const dim3 grid((unsigned)((N + kWavesPerBlock - 1) / kWavesPerBlock), (unsigned)pp);
        const IdRoute r{ids, p0, U, E, w_stride, (K / QK4_0) * kQ8_0Bytes, y_per_slot};
        if (gemv_q4_0s_fits(1, K) && N * K >= (int64_t(1) << 22)) {
            const unsigned lds = (unsigned)gemv_q4_0s_lds_bytes(1, K);
            if (repacked)
                hipLaunchKernelGGL((k_gemv_q4_0s<1, true, 0, true>), grid, dim3(256), lds, s, w, y, (void *)out, N,
                                   K, dsec, r);
            else
                hipLaunchKernelGGL((k_gemv_q4_0s<1, false, 0, true>), grid, dim3(256), lds, s, w, y, (void *)out, N,
                                   K, dsec, r);
        } else if (repacked) {
            hipLaunchKernelGGL((k_gemv_q4_0<1, true, 0, true>), grid, dim3(256), 0, s, w, y, (void *)out, N, K,
                               dsec, r);
        } else {
            hipLaunchKernelGGL((k_gemv_q4_0<1, false, 0, true>), grid, dim3(256), 0, s, w, y, (void *)out, N, K,
                               dsec, r);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_block_sums_q4_0(const uint8_t *w, bool repacked, const uint8_t *y, int32_t *P,
                                  int64_t M, int64_t N, int64_t K, hipStream_t s) {
    for (int64_t m0 = 0; m0 < M; m0 += kGemvMaxM) {
        const int64_t mm = M - m0 < kGemvMaxM ? M - m0 : kGemvMaxM;
        hipError_t e = dispatch_q4_0<1>(w, repacked, y + m0 * (K / QK4_0) * kQ8_0Bytes,
                                        P + m0 * N * (K / 32), mm, N, K, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace qmm
