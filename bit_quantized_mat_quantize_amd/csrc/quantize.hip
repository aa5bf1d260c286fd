// quantize.hip -- activation quantizers (Q8_0, Q8_K) and offline weight
// encoders (Q4_0, Q4_K) for gfx950.
//
// Activation quantization happens once per mul_mat call and is shared by all
// output tiles (ggml-cpu mul_mat page, "第一步:激活得先变成 Q8_K").  The
// encoders reproduce the reference byte-for-byte, so every floating-point step
// is a single IEEE binary32 operation in a fixed order (the library is built
// with -ffp-contract=off and correctly rounded division); max/min reductions
// are exact in any order.
#include "qmm_device.h"
#include "qmm_launch.h"

namespace qmm {
namespace {

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// ---------------------------------------------------------------------------
// Q8_K: one wavefront per 256-value block, 4 consecutive values per lane
// (one 16-byte load).  Block bytes: fp32 d | int8 qs[256] | int16 bsums[16]
// (ggml-cpu mul_mat page, "更低的比特"): bsums[g] is the sum of the 16 codes
// held by lanes 4g..4g+3.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_quantize_q8_K(const float *__restrict__ x,
                                                       uint8_t *__restrict__ y, int64_t nblocks,
                                                       int64_t nb_row, int64_t K) {
    const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (blk >= nblocks) return;  // uniform per wavefront
    const int lane = threadIdx.x & 63;
    const int64_t row = blk / nb_row, b = blk - row * nb_row;
    const float4 v = *reinterpret_cast<const float4 *>(x + row * K + b * QK_K + lane * 4);
    const Q8KLane r = q8K_quantize_lane(v);
    uint8_t *out = y + blk * kQ8_KBytes;
    *reinterpret_cast<uint32_t *>(out + 4 + lane * 4) = pack4_i8(r.q[0], r.q[1], r.q[2], r.q[3]);
    if ((lane & 3) == 0) *reinterpret_cast<int16_t *>(out + 260 + (lane >> 2) * 2) = (int16_t)r.bsum;
    if (lane == 0) *reinterpret_cast<float *>(out) = r.d;
}

// ---------------------------------------------------------------------------
// Q8_0: 8 lanes per 32-value block (8 blocks per wavefront).  Block bytes:
// fp16 d | int8 qs[32]; blocks are 34 B, so only 2-byte stores are aligned.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_quantize_q8_0(const float *__restrict__ x,
                                                       uint8_t *__restrict__ y, int64_t nblocks,
                                                       int64_t nb_row, int64_t K) {
    const int64_t blk = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
    const int sub = threadIdx.x & 7;
    const bool live = blk < nblocks;
    const int64_t bb = live ? blk : 0;
    const int64_t row = bb / nb_row, b = bb - row * nb_row;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (live) v = *reinterpret_cast<const float4 *>(x + row * K + b * QK4_0 + sub * 4);
    const Q80Part r = q8_0_quantize_part(v);  // all lanes: they exchange their maxima
    if (!live) return;
    uint8_t *out = y + blk * kQ8_0Bytes;
    uint16_t *o16 = reinterpret_cast<uint16_t *>(out + 2 + sub * 4);
    o16[0] = (uint16_t)(r.q & 0xffff);
    o16[1] = (uint16_t)(r.q >> 16);
    if (sub == 0) *reinterpret_cast<uint16_t *>(out) = (uint16_t)f32_to_f16_bits(r.d);
}

// ---------------------------------------------------------------------------
// Q4_0 encoder: 8 lanes per 32-weight block.  d = -xmax/8 where xmax is the
// signed element of largest magnitude (lowest index wins a tie); q = rint(x/d)+8
// computed as x*(1/d), clamped to [0,15] (ggml-cpu mul_mat page, "最基础的两块").
// Byte l of qs = q[l] | q[l+16] << 4; lanes 0..3 hold elements 0..15.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_encode_q4_0(const float *__restrict__ w,
                                                     uint8_t *__restrict__ out, int64_t nblocks,
                                                     int64_t nb_row, int64_t K) {
    const int64_t blk = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
    const int sub = threadIdx.x & 7;
    const bool live = blk < nblocks;
    const int64_t bb = live ? blk : 0;
    const int64_t row = bb / nb_row, b = bb - row * nb_row;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (live) v = *reinterpret_cast<const float4 *>(w + row * K + b * QK4_0 + sub * 4);
    // first element of largest magnitude within the lane, then across 8 lanes
    float amax = fabsf(v.x), xmax = v.x;
    int idx = sub * 4;
    if (fabsf(v.y) > amax) { amax = fabsf(v.y); xmax = v.y; idx = sub * 4 + 1; }
    if (fabsf(v.z) > amax) { amax = fabsf(v.z); xmax = v.z; idx = sub * 4 + 2; }
    if (fabsf(v.w) > amax) { amax = fabsf(v.w); xmax = v.w; idx = sub * 4 + 3; }
#pragma unroll
    for (int o = 4; o > 0; o >>= 1) {
        const float oa = __shfl_xor(amax, o, kWave);
        const float ox = __shfl_xor(xmax, o, kWave);
        const int oi = __shfl_xor(idx, o, kWave);
        if (oa > amax || (oa == amax && oi < idx)) { amax = oa; xmax = ox; idx = oi; }
    }
    if (amax == 0.0f) xmax = 0.0f;  // all-zero block: d = +0
    const float d = 0.0f - xmax / 8.0f;
    const float id = d != 0.0f ? 1.0f / d : 0.0f;
    const int q0 = clampi((int)rintf(v.x * id) + 8, 0, 15);
    const int q1 = clampi((int)rintf(v.y * id) + 8, 0, 15);
    const int q2 = clampi((int)rintf(v.z * id) + 8, 0, 15);
    const int q3 = clampi((int)rintf(v.w * id) + 8, 0, 15);
    const uint32_t lo = (uint32_t)q0 | (q1 << 8) | (q2 << 16) | (q3 << 24);
    const uint32_t hi = __shfl_down(lo, 4, 8);  // lanes 0..3 take elements 16..31
    if (!live) return;
    uint8_t *o = out + blk * kQ4_0Bytes;
    if (sub < 4) {
        const uint32_t p = lo | (hi << 4);
        uint16_t *o16 = reinterpret_cast<uint16_t *>(o + 2 + sub * 4);
        o16[0] = (uint16_t)(p & 0xffff);
        o16[1] = (uint16_t)(p >> 16);
    }
    if (sub == 0) *reinterpret_cast<uint16_t *>(o) = (uint16_t)f32_to_f16_bits(d);
}

// ---------------------------------------------------------------------------
// Q4_K encoder: one wavefront per 256-weight super-block, 4 weights per lane;
// sub-block j is held by lanes 8j..8j+7.  Min/max reading of the scale search
// (the pages give only the decoded form w = d*s_j*q - dmin*m_j):
//   lo = min(0, min x), sc = (max x - lo)/15, mn = 0 - lo
//   d = max sc / 63, dmin = max mn / 63, s_j = rint(sc/d), m_j = rint(mn/dmin)
//   q = rint((x + f16(dmin)*m_j) / (f16(d)*s_j)), clamped to [0,15]
// Maxima start from +0 and only grow on a strictly larger value, so an
// all-non-positive super-block yields +0 scales.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float max_pos(float a, float b) { return b > a ? b : a; }

__global__ __launch_bounds__(256) void k_encode_q4_K(const float *__restrict__ w,
                                                     uint8_t *__restrict__ out, int64_t nblocks,
                                                     int64_t nb_row, int64_t K) {
    const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (blk >= nblocks) return;  // uniform per wavefront
    const int lane = threadIdx.x & 63;
    const int64_t row = blk / nb_row, b = blk - row * nb_row;
    const float4 v = *reinterpret_cast<const float4 *>(w + row * K + b * QK_K + lane * 4);
    float lo = v.x, hi = v.x;
    lo = v.y < lo ? v.y : lo; hi = v.y > hi ? v.y : hi;
    lo = v.z < lo ? v.z : lo; hi = v.z > hi ? v.z : hi;
    lo = v.w < lo ? v.w : lo; hi = v.w > hi ? v.w : hi;
#pragma unroll
    for (int o = 4; o > 0; o >>= 1) {
        const float olo = __shfl_xor(lo, o, kWave), ohi = __shfl_xor(hi, o, kWave);
        lo = olo < lo ? olo : lo;
        hi = ohi > hi ? ohi : hi;
    }
    if (!(lo < 0.0f)) lo = 0.0f;
    const float sc = (hi - lo) / 15.0f;
    const float mn = 0.0f - lo;
    float maxsc = max_pos(0.0f, sc), maxmn = max_pos(0.0f, mn);
#pragma unroll
    for (int o = 8; o < 64; o <<= 1) {
        maxsc = max_pos(maxsc, __shfl_xor(maxsc, o, kWave));
        maxmn = max_pos(maxmn, __shfl_xor(maxmn, o, kWave));
    }
    const float d = maxsc / 63.0f;
    const float dmin = maxmn / 63.0f;
    const int s = d > 0.0f ? clampi((int)rintf(sc / d), 0, 63) : 0;
    const int m = dmin > 0.0f ? clampi((int)rintf(mn / dmin), 0, 63) : 0;
    const uint32_t dh = f32_to_f16_bits(d), dmh = f32_to_f16_bits(dmin);
    const float Dj = f16_bits_to_f32(dh) * (float)s;
    const float Mj = f16_bits_to_f32(dmh) * (float)m;
    int q[4];
    const float xv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int t = 0; t < 4; ++t)
        q[t] = Dj > 0.0f ? clampi((int)rintf((xv[t] + Mj) / Dj), 0, 15) : 0;
    // nibbles: byte 32g+l = q[64g+l] | q[64g+32+l] << 4.  Lane 16g+i (i<8)
    // holds elements 64g+4i..+3; lane 16g+8+i holds 64g+32+4i..+3.
    const uint32_t mine = (uint32_t)q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
    const uint32_t upper = __shfl_down(mine, 8, 16);
    uint8_t *o = out + blk * kQ4_KBytes;
    const int g = lane >> 4, i = lane & 15;
    if (i < 8) *reinterpret_cast<uint32_t *>(o + 16 + 32 * g + 4 * i) = mine | (upper << 4);
    // scale field: gather s_j, m_j from the first lane of each sub-block
    int sj[8], mj[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        sj[j] = __shfl(s, 8 * j, kWave);
        mj[j] = __shfl(m, 8 * j, kWave);
    }
    if (lane == 0) {
        // bytes 0..3: s_j | top bits of s_{j+4};  4..7: m_j | top bits of m_{j+4};
        // 8..11: low nibbles of s_{j+4} (low) and m_{j+4} (high)
        uint32_t f0 = 0, f1 = 0, f2 = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f0 |= (uint32_t)(sj[j] | ((sj[j + 4] >> 4) << 6)) << (8 * j);
            f1 |= (uint32_t)(mj[j] | ((mj[j + 4] >> 4) << 6)) << (8 * j);
            f2 |= (uint32_t)((sj[j + 4] & 15) | ((mj[j + 4] & 15) << 4)) << (8 * j);
        }
        *reinterpret_cast<uint4 *>(o) = make_uint4(dh | (dmh << 16), f0, f1, f2);
    }
}

}  // namespace

hipError_t launch_quantize_q8_K(const float *x, uint8_t *y, int64_t M, int64_t K, hipStream_t s) {
    const int64_t nb = K / QK_K, total = M * nb;
    hipLaunchKernelGGL(k_quantize_q8_K, dim3((unsigned)((total + 3) / 4)), dim3(256), 0, s, x, y,
                       total, nb, K);
    return hipGetLastError();
}

hipError_t launch_quantize_q8_0(const float *x, uint8_t *y, int64_t M, int64_t K, hipStream_t s) {
    const int64_t nb = K / QK4_0, total = M * nb;
    hipLaunchKernelGGL(k_quantize_q8_0, dim3((unsigned)((total + 31) / 32)), dim3(256), 0, s, x, y,
                       total, nb, K);
    return hipGetLastError();
}

hipError_t launch_encode_q4_0(const float *w, uint8_t *out, int64_t N, int64_t K, hipStream_t s) {
    const int64_t nb = K / QK4_0, total = N * nb;
    hipLaunchKernelGGL(k_encode_q4_0, dim3((unsigned)((total + 31) / 32)), dim3(256), 0, s, w, out,
                       total, nb, K);
    return hipGetLastError();
}

hipError_t launch_encode_q4_K(const float *w, uint8_t *out, int64_t N, int64_t K, hipStream_t s) {
    const int64_t nb = K / QK_K, total = N * nb;
    hipLaunchKernelGGL(k_encode_q4_K, dim3((unsigned)((total + 3) / 4)), dim3(256), 0, s, w, out,
                       total, nb, K);
    return hipGetLastError();
}

}  // namespace qmm
