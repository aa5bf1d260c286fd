// q2k.hip -- Q2_K weights x Q8_K activations on gfx950: encoder, load-time
// repack, GEMV and the int32 group sums of its decode path.
//
// Format (ggml-cpu mul_mat page, "更低的比特:Q6_K 与 Q2_K 的取舍"): 84 bytes per
// 256 weights -- 2-bit codes in 64 bytes, 16 groups of 16 elements with a
// 4-bit scale and a 4-bit min each, fp16 d and dmin -- and the asymmetric
// value w = d * s_j * q - dmin * m_j, q in [0, 3].  This library's reading of
// the placement: scales[16] @0 (s_j low nibble, m_j high), qs[64] @16, d @80,
// dmin @82; element k = 128h + 32s + l sits in qs byte 32h + l, bits 2s..2s+1.
//
// Integer path (same page, "正确性:缩放系数可以提到求和号外面" and "min 项与最终
// 归约", over 16-element groups, one Q8_K bsum per group):
//   P_j = sum_{i in j} q_i y_i,  S = sum_j s_j P_j,  Mn = sum_j m_j bsums_j,
//   out += d_a * (d * S - dmin * Mn).
//
// Load-time layout (QMM_LAYOUT_REPACKED), block (n, b) at index i = n*nb + b:
//   [(d, dmin) of every block, 4 B each, zero-padded to a multiple of 256 B]
//   [scales, 16 B each][qs, 64 B each]
// so every 16-byte piece a lane loads is aligned.  Canonical blocks are
// 4-byte aligned (84 = 4 * 21).
#include "q8k_row.h"
#include "qmm_device.h"
#include "qmm_launch.h"

namespace qmm {
namespace {

constexpr int kQ2_KBytes = 84;

__device__ __forceinline__ int clampi2(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// ---------------------------------------------------------------------------
// Encoder (input generator; the oracle's reading): per 16-element group
// lo = min(0, min x), hi = max x, sc = (hi - lo)/3, mn = -lo; d = max sc/15,
// dmin = max mn/15; s_j = rint(sc/d), m_j = rint(mn/dmin) in [0, 15]; with
// D_j = f16(d) s_j and M_j = f16(dmin) m_j, q = rint((x + M_j)/D_j) in [0, 3]
// (0 where D_j = 0).  One wavefront per block; lane l holds elements
// 4l..4l+3, so a group is four consecutive lanes.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_encode_q2_K(const float *__restrict__ w,
                                                     uint8_t *__restrict__ out, int64_t nblocks,
                                                     int64_t nb_row, int64_t K) {
    __shared__ __attribute__((aligned(16))) uint8_t sq[4][256];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t blk0 = (int64_t)blockIdx.x * 4 + wave;
    const bool valid = blk0 < nblocks;  // a spare wavefront encodes the last block, stores nothing
    const int64_t blk = valid ? blk0 : nblocks - 1;
    const int64_t row = blk / nb_row, b = blk - row * nb_row;
    const float4 v = *reinterpret_cast<const float4 *>(w + row * K + b * QK_K + lane * 4);
    const float xv[4] = {v.x, v.y, v.z, v.w};

    float lo = fminf(fminf(xv[0], xv[1]), fminf(xv[2], xv[3]));
    float hi = fmaxf(fmaxf(xv[0], xv[1]), fmaxf(xv[2], xv[3]));
#pragma unroll
    for (int o = 1; o <= 2; o <<= 1) {
        lo = fminf(lo, __shfl_xor(lo, o, kWave));
        hi = fmaxf(hi, __shfl_xor(hi, o, kWave));
    }
    if (!(lo < 0.0f)) lo = 0.0f;
    const float sc = (hi - lo) / 3.0f;
    const float mn = 0.0f - lo;
    const float d = wave_max(sc) / 15.0f;
    const float dmin = wave_max(mn) / 15.0f;
    const int s = d > 0.0f ? clampi2((int)rintf(sc / d), 0, 15) : 0;
    const int m = dmin > 0.0f ? clampi2((int)rintf(mn / dmin), 0, 15) : 0;
    const uint32_t dh = f32_to_f16_bits(d), dmh = f32_to_f16_bits(dmin);
    const float Dj = f16_bits_to_f32(dh) * (float)s;
    const float Mj = f16_bits_to_f32(dmh) * (float)m;
    uint32_t mine = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int q = Dj > 0.0f ? clampi2((int)rintf((xv[e] + Mj) / Dj), 0, 3) : 0;
        mine |= (uint32_t)q << (8 * e);
    }
    *reinterpret_cast<uint32_t *>(&sq[wave][4 * lane]) = mine;
    __syncthreads();

    // 4-byte stores: the block base 84 * blk is 4-byte aligned
    uint32_t *o = reinterpret_cast<uint32_t *>(out + blk * kQ2_KBytes);
    const uint8_t *q = sq[wave];
    const int sm = s | (m << 4);  // scale byte of this lane's group
    // scale dword t holds groups 4t..4t+3 (lanes 16t, 16t+4, 16t+8, 16t+12)
    const int t = lane & 3;
    const uint32_t sw = (uint32_t)(__shfl(sm, 16 * t, kWave) | (__shfl(sm, 16 * t + 4, kWave) << 8) |
                                   (__shfl(sm, 16 * t + 8, kWave) << 16) |
                                   (__shfl(sm, 16 * t + 12, kWave) << 24));
    if (valid && lane < 4) o[lane] = sw;
    if (lane >= 16 && lane < 32) {  // qs dword lane-16: bytes B = 4(lane-16)+i
        const int l4 = lane - 16;
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int B = 4 * l4 + i, h = B >> 5, l = B & 31;
            word |= (uint32_t)(q[128 * h + l] | (q[128 * h + 32 + l] << 2) | (q[128 * h + 64 + l] << 4) |
                               (q[128 * h + 96 + l] << 6)) << (8 * i);
        }
        if (valid) o[4 + l4] = word;
    }
    if (valid && lane == 32) o[20] = dh | (dmh << 16);
}

// ---------------------------------------------------------------------------
// Repack: one thread per block copies its 84 bytes (4-byte loads) into the
// three sections; threads past the last block zero the padding of the
// (d, dmin) section.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_repack_q2_K(const uint8_t *__restrict__ in,
                                                     uint8_t *__restrict__ out, int64_t nblk,
                                                     int64_t dsec) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= nblk) {
        if (4 * i < dsec) *reinterpret_cast<uint32_t *>(out + 4 * i) = 0;
        return;
    }
    const uint32_t *src = reinterpret_cast<const uint32_t *>(in + i * kQ2_KBytes);
    uint32_t *sc = reinterpret_cast<uint32_t *>(out + dsec + 16 * i);
    uint32_t *qs = reinterpret_cast<uint32_t *>(out + dsec + 16 * nblk + 64 * i);
    for (int k = 0; k < 4; ++k) sc[k] = src[k];
    for (int k = 0; k < 16; ++k) qs[k] = src[4 + k];
    *reinterpret_cast<uint32_t *>(out + 4 * i) = src[20];
}

// ---------------------------------------------------------------------------
// GEMV.  The unit of work is a quarter of a super-block: unit u = 4b + p owns
// qs piece p (bytes 16p..16p+15), whose four 2-bit fields are the groups
// G = 8(p/2) + 2s + (p%2), s = 0..3 (elements 128(p/2) + 32s + 16(p%2) + i).
// One wavefront per output row, lane l takes units l, l + 64, ...; the
// activation row is staged in LDS (q8k_row.h).
// ---------------------------------------------------------------------------
template <bool REPACKED>
struct Q2KAddr {
    const uint8_t *W;
    int64_t NB, dsec;  // blocks in the matrix, bytes of the (d, dmin) section
    __device__ __forceinline__ const uint8_t *qs(int64_t i) const {
        return REPACKED ? W + dsec + 16 * NB + 64 * i : W + i * kQ2_KBytes + 16;
    }
    __device__ __forceinline__ const uint8_t *sc(int64_t i) const {
        return REPACKED ? W + dsec + 16 * i : W + i * kQ2_KBytes;
    }
    __device__ __forceinline__ const uint8_t *dm(int64_t i) const {
        return REPACKED ? W + 4 * i : W + i * kQ2_KBytes + 80;
    }
};

struct Q2KUnit {
    uint4 qs;      // qs piece p
    uint2 sc;      // scale bytes 8(p/2)..8(p/2)+7
    uint32_t dm;   // fp16 d | fp16 dmin << 16
};

template <bool REPACKED>
__device__ __forceinline__ void q2k_load(const Q2KAddr<REPACKED> &A, int64_t n, int64_t nb, int u,
                                         Q2KUnit &x) {
    const int64_t i = n * nb + (u >> 2);
    const int p = u & 3;
    if constexpr (REPACKED) {
        x.qs = *reinterpret_cast<const uint4 *>(A.qs(i) + 16 * p);
        x.sc = *reinterpret_cast<const uint2 *>(A.sc(i) + 8 * (p >> 1));
    } else {
        x.qs = ld_align4<uint4>(A.qs(i) + 16 * p);
        x.sc = ld_align4<uint2>(A.sc(i) + 8 * (p >> 1));
    }
    x.dm = ld_align4<uint32_t>(A.dm(i));
}

// The four group sums of a unit: P[s] for group 8(p/2) + 2s + (p%2).
__device__ __forceinline__ void q2k_group_sums(const Q2KUnit &x, int u, const uint8_t *s_qs, int P[4]) {
    const int b = u >> 2, p = u & 3;
    const uint8_t *yb = s_qs + b * QK_K + 128 * (p >> 1) + 16 * (p & 1);
    const uint32_t qw[4] = {x.qs.x, x.qs.y, x.qs.z, x.qs.w};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const uint4 yv = *reinterpret_cast<const uint4 *>(yb + 32 * s);
        const uint32_t yw[4] = {yv.x, yv.y, yv.z, yv.w};
        int acc = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) acc = dot4((qw[w] >> (2 * s)) & 0x03030303u, yw[w], acc);
        P[s] = acc;
    }
}

// acc + d_a * (d * S - dmin * Mn) for one unit (the Q4_K-style min term, over
// the unit's four groups).
__device__ __forceinline__ float q2k_unit_accum(const Q2KUnit &x, int u, const uint8_t *s_qs,
                                                const float *s_d, const int16_t *s_bs, float acc) {
    int P[4];
    q2k_group_sums(x, u, s_qs, P);
    const int b = u >> 2, p = u & 3;
    // scale bytes of groups 8(p/2) + 2s + (p%2): byte 2s + (p%2) of x.sc
    const uint32_t sw[2] = {x.sc.x, x.sc.y};
    const int16_t *bs = s_bs + 16 * b + 8 * (p >> 1) + (p & 1);
    int S = 0, Mn = 0;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const uint32_t byte = (sw[s >> 1] >> (16 * (s & 1) + 8 * (p & 1))) & 0xff;
        S += (int)(byte & 15) * P[s];
        Mn += (int)(byte >> 4) * (int)bs[2 * s];
    }
    const float d = f16_bits_to_f32(x.dm & 0xffff);
    const float dmin = f16_bits_to_f32(x.dm >> 16);
    return fmaf(s_d[b], d * (float)S - dmin * (float)Mn, acc);
}

constexpr int kQ2Waves = 4;

// MODE 0: out[m*N + n] (fp32).  MODE 1: P[m][n][K/16] (int32 group sums).
// ID = true (MODE 0): mul_mat_id, one (token, slot) pair per blockIdx.y.
template <bool REPACKED, int kNit, int MODE, bool ID = false>
__global__ __launch_bounds__(256) void k_gemv_q2_K(const uint8_t *__restrict__ W,
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
    const int64_t n = (int64_t)blockIdx.x * kQ2Waves + wave;
    const int64_t nn = n < N ? n : N - 1;  // a tail wavefront loads a valid row, stores nothing
    const int nunits = (int)(4 * nb);
    const Q2KAddr<REPACKED> A{W, N * nb, REPACKED ? (4 * N * nb + 255) / 256 * 256 : 0};

    // the activation row's first pieces, then this row's first units, then
    // the activations into LDS (the wait before the stores covers only them)
    const uint8_t *yrow = Y + m * nb * kQ8_KBytes;
    const Q8KRowHead yh = load_q8k_row_head(yrow, K);
    __builtin_amdgcn_sched_barrier(0);
    Q2KUnit x[kNit];
#pragma unroll
    for (int it = 0; it < kNit; ++it) {
        const int u = lane + 64 * it;
        q2k_load<REPACKED>(A, nn, nb, u < nunits ? u : nunits - 1, x[it]);
    }
    const Q8KRowLds row = commit_q8k_row(yh, yrow, K, ys);

    float acc = 0.0f;
    for (int base = 0; base < nunits; base += 64 * kNit) {
        if (base > 0) {
#pragma unroll
            for (int it = 0; it < kNit; ++it) {
                const int u = base + lane + 64 * it;
                q2k_load<REPACKED>(A, nn, nb, u < nunits ? u : nunits - 1, x[it]);
            }
        }
#pragma unroll
        for (int it = 0; it < kNit; ++it) {
            const int u = base + lane + 64 * it;
            if (u < nunits) {
                if (MODE == 0) {
                    acc = q2k_unit_accum(x[it], u, row.qs, row.d, row.bsums, acc);
                } else if (n < N) {
                    int P[4];
                    q2k_group_sums(x[it], u, row.qs, P);
                    const int b = u >> 2, p = u & 3;
                    int32_t *Pout = reinterpret_cast<int32_t *>(dst) + (m * N + n) * (K / 16) + 16 * b;
#pragma unroll
                    for (int s = 0; s < 4; ++s) Pout[8 * (p >> 1) + 2 * s + (p & 1)] = P[s];
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
// Fused M = 1 path (rows of up to four units per lane, K <= 16384, at most two
// rows per wavefront): the fp32 row is quantized to Q8_K inside the GEMV,
// straight into LDS, so one launch covers quantize + mul_mat.  Every
// workgroup quantizes the whole row, so the grid holds one 16-wavefront
// workgroup per CU; wavefront w of workgroup g takes rows g*16 + w and
// g*16 + w + 16*gridDim.x.  A wavefront loads its fp32 activation blocks
// (b = wave + 16i), requests its first row's units (below four units per lane
// only once the activation blocks have arrived), quantizes while they are in
// flight, and requests its second row (if any)
// after the barrier.  Workgroup 0 also stores the Q8_K bytes to Yq.  Per row
// the same integer sums and fp32 operations, in the same order, as
// k_gemv_q2_K.
// ---------------------------------------------------------------------------
constexpr int kQ2FusedWaves = 16;

template <bool REPACKED, int kNit, int kXB>
__global__ __launch_bounds__(kQ2FusedWaves * 64) void k_gemv_fused_q2_K(
    const uint8_t *__restrict__ W, const float *__restrict__ X, uint8_t *__restrict__ Yq,
    float *__restrict__ out, int64_t N, int64_t K) {
    extern __shared__ __attribute__((aligned(16))) uint8_t ys[];
    const int64_t nb = K / QK_K;
    const int nunits = (int)(4 * nb);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int64_t stride = (int64_t)gridDim.x * kQ2FusedWaves;
    const int64_t row = (int64_t)blockIdx.x * kQ2FusedWaves + wave, row2 = row + stride;  // uniform
    const Q2KAddr<REPACKED> A{W, N * nb, REPACKED ? (4 * N * nb + 255) / 256 * 256 : 0};
    auto load_row = [&](int64_t r, Q2KUnit (&x)[kNit]) {
        const int64_t rr = r < N ? r : N - 1;  // past the last row: a valid row, never stored
#pragma unroll
        for (int it = 0; it < kNit; ++it) {
            const int u = lane + 64 * it;
            q2k_load<REPACKED>(A, rr, nb, u < nunits ? u : nunits - 1, x[it]);
        }
    };
    float4 xv[kXB];
#pragma unroll
    for (int i = 0; i < kXB; ++i) {  // block indices past the row load the last block again
        const int b0 = wave + kQ2FusedWaves * i;
        const int b = b0 < nb ? b0 : (int)nb - 1;
        xv[i] = *reinterpret_cast<const float4 *>(X + (int64_t)b * QK_K + 4 * lane);
    }
    // up to two units per lane the activation loads complete before any weight
    // load is issued (queued behind the chip's weight stream they would arrive
    // late); at four, the quantization waits only for them, with the row's
    // units already requested (0.1-0.2 us faster there, 0.1-0.4 us slower below)
    if constexpr (kNit < 4) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    Q2KUnit x[kNit], x2[kNit];
    load_row(row, x);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kXB; ++i) q8k_quantize_block_lds(xv[i], wave + kQ2FusedWaves * i, K, ys, lane);
    __syncthreads();
    const uint8_t *s_qs = ys;
    const float *s_d = reinterpret_cast<const float *>(ys + K);
    const int16_t *s_bs = reinterpret_cast<const int16_t *>(ys + K + (nb * 4 + 15) / 16 * 16);
    const bool two = row2 < N;  // wavefront-uniform
    if (two) load_row(row2, x2);
    auto reduce = [&](int64_t r, const Q2KUnit (&xx)[kNit]) {
        float acc = 0.0f;
#pragma unroll
        for (int it = 0; it < kNit; ++it) {
            const int u = lane + 64 * it;
            if (u < nunits) acc = q2k_unit_accum(xx[it], u, s_qs, s_d, s_bs, acc);
        }
        acc = wave_sum(acc);
        if (lane == 0 && r < N) out[r] = acc;
    };
    reduce(row, x);
    if (two) reduce(row2, x2);
    // workgroup 0 copies the Q8_K row to Yq last (stores issued earlier would
    // sit in the in-order counter ahead of the weight loads)
    if (blockIdx.x == 0) q8k_store_row<kQ2FusedWaves * 64>(Yq, ys, K);
}

template <int MODE>
hipError_t dispatch_q2_K(const uint8_t *w, bool repacked, const uint8_t *y, void *dst, int64_t M,
                         int64_t N, int64_t K, hipStream_t s) {
    const int64_t nunits = 4 * (K / QK_K);
    const int64_t nit = (nunits + 63) / 64;
    const dim3 grid((unsigned)((N + kQ2Waves - 1) / kQ2Waves), (unsigned)M);  // M <= 65535
    const unsigned lds = (unsigned)q8k_row_lds_bytes(K);
#define QMM_Q2(NIT)                                                                                \
    do {                                                                                           \
        if (repacked)                                                                              \
            hipLaunchKernelGGL((k_gemv_q2_K<true, NIT, MODE>), grid, dim3(256), lds, s, w, y, dst, N, K); \
        else                                                                                       \
            hipLaunchKernelGGL((k_gemv_q2_K<false, NIT, MODE>), grid, dim3(256), lds, s, w, y, dst, N, K); \
    } while (0)
    if (nit <= 1) QMM_Q2(1);
    else if (nit <= 2) QMM_Q2(2);
    else QMM_Q2(4);
#undef QMM_Q2
    return hipGetLastError();
}

}  // namespace

int64_t repacked_bytes_q2_K(int64_t N, int64_t K) {
    const int64_t nblk = N * (K / QK_K);
    return (4 * nblk + 255) / 256 * 256 + 80 * nblk;
}

int64_t q2_K_max_k() { return q8k_row_max_k(); }  // the staged activation row fits LDS

hipError_t launch_encode_q2_K(const float *w, uint8_t *out, int64_t N, int64_t K, hipStream_t s) {
    const int64_t nb = K / QK_K, total = N * nb;
    hipLaunchKernelGGL(k_encode_q2_K, dim3((unsigned)((total + 3) / 4)), dim3(256), 0, s, w, out,
                       total, nb, K);
    return hipGetLastError();
}

hipError_t launch_repack_q2_K(const uint8_t *in, uint8_t *out, int64_t N, int64_t K, hipStream_t s) {
    const int64_t nblk = N * (K / QK_K);
    const int64_t dsec = (4 * nblk + 255) / 256 * 256;
    const int64_t threads = nblk > dsec / 4 ? nblk : dsec / 4;
    hipLaunchKernelGGL(k_repack_q2_K, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, in,
                       out, nblk, dsec);
    return hipGetLastError();
}

// activation rows go to grid.y, in chunks of at most 65535 rows
hipError_t launch_gemv_q2_K(const uint8_t *w, bool repacked, const uint8_t *y, float *out,
                            int64_t M, int64_t N, int64_t K, hipStream_t s) {
    const int64_t rowb = (K / QK_K) * kQ8_KBytes;
    for (int64_t m0 = 0; m0 < M; m0 += 65535) {
        const int64_t mm = M - m0 < 65535 ? M - m0 : 65535;
        const hipError_t e = dispatch_q2_K<0>(w, repacked, y + m0 * rowb, out + m0 * N, mm, N, K, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

bool gemv_fused_q2_K_ok(int64_t N, int64_t K) {
    // rows of up to four units per lane (K <= 16384) and at most two rows per
    // wavefront; each workgroup repeats the quantization
    return K <= 16384 && N <= 2 * (int64_t)kQ2FusedWaves * cu_count();
}

hipError_t launch_gemv_fused_q2_K(const uint8_t *w, bool repacked, const float *x, uint8_t *yq, float *out,
                                  int64_t N, int64_t K, hipStream_t s) {
    if (!gemv_fused_q2_K_ok(N, K)) return hipErrorInvalidValue;
    const int64_t nit = (4 * (K / QK_K) + 63) / 64;
    const int64_t groups = (N + kQ2FusedWaves - 1) / kQ2FusedWaves, cus = cu_count();
    const dim3 grid((unsigned)(groups < cus ? groups : cus)), block(kQ2FusedWaves * 64);
    const unsigned lds = (unsigned)q8k_row_lds_bytes(K);
#define QMM_Q2F(NIT, XB)                                                                                  \
    do {                                                                                                  \
        if (repacked)                                                                                     \
            hipLaunchKernelGGL((k_gemv_fused_q2_K<true, NIT, XB>), grid, block, lds, s, w, x, yq, out, N, K);  \
        else                                                                                              \
            hipLaunchKernelGGL((k_gemv_fused_q2_K<false, NIT, XB>), grid, block, lds, s, w, x, yq, out, N, K); \
    } while (0)
    // kXB = activation blocks per wavefront: ceil(nb / 16) (nb <= 16 * kNit = 16 * kXB)
    if (nit <= 1) QMM_Q2F(1, 1);
    else if (nit <= 2) QMM_Q2F(2, 2);
    else QMM_Q2F(4, 4);
#undef QMM_Q2F
    return hipGetLastError();
}

hipError_t launch_gemv_id_q2_K(const uint8_t *w, bool repacked, int64_t w_stride, const uint8_t *y,
                               int y_per_slot, const int32_t *ids, int64_t P, int64_t U, int64_t E,
                               float *out, int64_t N, int64_t K, hipStream_t s) {
    const int64_t nit = (4 * (K / QK_K) + 63) / 64;
    const unsigned lds = (unsigned)q8k_row_lds_bytes(K);
    for (int64_t p0 = 0; p0 < P; p0 += 65535) {
        const int64_t pp = P - p0 < 65535 ? P - p0 : 65535;
        const dim3 grid((unsigned)((N + kQ2Waves - 1) / kQ2Waves), (unsigned)pp);
        const IdRoute r{ids, p0, U, E, w_stride, (K / QK_K) * kQ8_KBytes, y_per_slot};
#define QMM_ID(NIT)                                                                                   \
    do {                                                                                              \
        if (repacked)                                                                                 \
            hipLaunchKernelGGL((k_gemv_q2_K<true, NIT, 0, true>), grid, dim3(256), lds, s, w, y, (void *)out, N, K, r);  \
        else                                                                                          \
            hipLaunchKernelGGL((k_gemv_q2_K<false, NIT, 0, true>), grid, dim3(256), lds, s, w, y, (void *)out, N, K, r); \
    } while (0)
        if (nit <= 1) QMM_ID(1);
        else if (nit <= 2) QMM_ID(2);
        else QMM_ID(4);
#undef QMM_ID
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_group_sums_q2_K(const uint8_t *w, bool repacked, const uint8_t *y, int32_t *P,
                                  int64_t M, int64_t N, int64_t K, hipStream_t s) {
    const int64_t rowb = (K / QK_K) * kQ8_KBytes;
    for (int64_t m0 = 0; m0 < M; m0 += 65535) {
        const int64_t mm = M - m0 < 65535 ? M - m0 : 65535;
        const hipError_t e =
            dispatch_q2_K<1>(w, repacked, y + m0 * rowb, P + m0 * N * (K / 16), mm, N, K, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace qmm
