// qmm_device.h -- device-side helpers shared by the libqmm kernels (gfx950).
//
// Byte formats are those of include/qmm.h.  Everything here is written for
// CDNA4: 64-lane wavefronts, int8 dot products (v_dot4_i32_i8), MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {

constexpr int kWave = 64;
constexpr int QK4_0 = 32;
constexpr int QK_K = 256;
constexpr int kQ4_0Bytes = 18;
constexpr int kQ8_0Bytes = 34;
constexpr int kQ4_KBytes = 144;
constexpr int kQ8_KBytes = 292;

// ---- fp16 <-> fp32 (hardware conversions; fp32 -> fp16 rounds to nearest even)
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
    _Float16 v;
    uint16_t b = (uint16_t)h;
    __builtin_memcpy(&v, &b, 2);
    return (float)v;
}
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
    _Float16 v = (_Float16)f;
    uint16_t b;
    __builtin_memcpy(&b, &v, 2);
    return b;
}

// ---- loads with the alignment the formats guarantee
template <typename T>
__device__ __forceinline__ T ld_align4(const void *p) {
    T v;
    __builtin_memcpy(&v, __builtin_assume_aligned(p, 4), sizeof(T));
    return v;
}
__device__ __forceinline__ uint4 ld16(const void *p) {   // 16-byte aligned
    return *reinterpret_cast<const uint4 *>(p);
}
__device__ __forceinline__ uint32_t ld_u16(const void *p) {
    return *reinterpret_cast<const uint16_t *>(p);
}

// ---- cross-lane moves.  DPP moves within rows of 16 lanes (gfx9 DPP control
// codes: quad_perm [1,0,3,2] = 0xB1, quad_perm [2,3,0,1] = 0x4E,
// row_half_mirror = 0x141, row_mirror = 0x140), then v_readlane across the
// four rows: no LDS round trips.  All 64 lanes must be active.
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, false));
}
template <int kCtrl>
__device__ __forceinline__ int dpp_i32(int v) {
    return __builtin_amdgcn_update_dpp(0, v, kCtrl, 0xf, 0xf, false);
}
__device__ __forceinline__ float readlane_f32(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Sum over the 64 lanes (every lane gets the same value; a fixed tree order).
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f32<0xB1>(v);
    v += dpp_f32<0x4E>(v);
    v += dpp_f32<0x141>(v);
    v += dpp_f32<0x140>(v);
    return (readlane_f32(v, 0) + readlane_f32(v, 16)) + (readlane_f32(v, 32) + readlane_f32(v, 48));
}

// Max over the 64 lanes (exact; every lane gets the value).
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_f32<0xB1>(v));
    v = fmaxf(v, dpp_f32<0x4E>(v));
    v = fmaxf(v, dpp_f32<0x141>(v));
    v = fmaxf(v, dpp_f32<0x140>(v));
    return fmaxf(fmaxf(readlane_f32(v, 0), readlane_f32(v, 16)),
                 fmaxf(readlane_f32(v, 32), readlane_f32(v, 48)));
}

// Sum over each group of 4 consecutive lanes (lanes 4k..4k+3 all get it).
__device__ __forceinline__ int quad_sum(int v) {
    v += dpp_i32<0xB1>(v);
    v += dpp_i32<0x4E>(v);
    return v;
}

// ---- int8 dot product of 4 packed bytes, accumulated (v_dot4_i32_i8)
__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// ---- Q4_K 12-byte scale field, word-parallel: from the three little-endian
// words w1 = scales[0..3], w2 = scales[4..7], w3 = scales[8..11] build four
// words whose bytes are s_0..s_3, m_0..m_3, s_4..s_7, m_4..m_7.
struct Q4KScales {
    uint32_t s_lo, m_lo, s_hi, m_hi;
};
__device__ __forceinline__ Q4KScales unpack_scales(uint32_t w1, uint32_t w2, uint32_t w3) {
    Q4KScales r;
    r.s_lo = w1 & 0x3f3f3f3fu;
    r.m_lo = w2 & 0x3f3f3f3fu;
    r.s_hi = (w3 & 0x0f0f0f0fu) | ((w1 >> 2) & 0x30303030u);
    r.m_hi = ((w3 >> 4) & 0x0f0f0f0fu) | ((w2 >> 2) & 0x30303030u);
    return r;
}

// ---- Q8_K quantization of one 256-value block held by a wavefront, four
// consecutive values per lane (lane l holds elements 4l..4l+3).  Per block:
// amax = max|x|, d = amax/127, id = d ? 1/d : 0, y = rint(x*id) clamped to
// [-127, 127] (single IEEE fp32 operations; the library is built without FMA
// contraction), bsum of 16 values = sum over lanes 4k..4k+3.  All 64 lanes
// must be active.
// Every caller goes through this routine, so all paths produce identical bytes.
struct Q8KLane {
    int q[4];
    float d;
    int bsum;
};
__device__ __forceinline__ int clamp127(int v) { return v < -127 ? -127 : (v > 127 ? 127 : v); }
__device__ __forceinline__ Q8KLane q8K_quantize_lane(const float4 v) {
    const float a = wave_max(fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    Q8KLane r;
    r.d = a / 127.0f;
    const float id = r.d != 0.0f ? 1.0f / r.d : 0.0f;
    r.q[0] = clamp127((int)rintf(v.x * id));
    r.q[1] = clamp127((int)rintf(v.y * id));
    r.q[2] = clamp127((int)rintf(v.z * id));
    r.q[3] = clamp127((int)rintf(v.w * id));
    r.bsum = quad_sum(r.q[0] + r.q[1] + r.q[2] + r.q[3]);
    return r;
}
__device__ __forceinline__ uint32_t pack4_i8(int a, int b, int c, int d) {
    return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
           ((uint32_t)(d & 0xff) << 24);
}

// ---- Q8_0 quantization of one 32-value block held by 8 consecutive lanes,
// four consecutive values per lane (lane 8k + s holds elements 4s .. 4s + 3):
// amax over the 8 lanes, d = amax/127, id = d ? 1/d : 0, q = rint(x*id)
// clamped to [-127, 127] (ggml-cpu mul_mat page, "最基础的两块:Q4_0 与 Q8_0").
// Every lane of the wavefront must call it (the lanes exchange their maxima);
// d is returned in fp32, the block stores it as fp16.
struct Q80Part {
    uint32_t q;  // this lane's four codes, packed
    float d;
};
__device__ __forceinline__ Q80Part q8_0_quantize_part(const float4 v) {
    float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
#pragma unroll
    for (int o = 4; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, kWave));
    Q80Part r;
    r.d = a / 127.0f;
    const float id = r.d != 0.0f ? 1.0f / r.d : 0.0f;
    r.q = pack4_i8(clamp127((int)rintf(v.x * id)), clamp127((int)rintf(v.y * id)),
                   clamp127((int)rintf(v.z * id)), clamp127((int)rintf(v.w * id)));
    return r;
}

// ---- mul_mat_id routing for the per-pair GEMVs: blockIdx.y is the (token,
// slot) pair p0 + y; its expert id selects the weight matrix, its token (or the
// pair itself) the activation row, and the pair the output row.  An id outside
// [0, E) selects expert 0 (every load stays in bounds) and reports invalid;
// the caller then stores NaN.
struct IdRoute {
    const int32_t *ids;
    int64_t p0, U, E;
    int64_t w_stride;    // bytes per expert matrix
    int64_t y_rowbytes;  // bytes per activation row
    int y_per_slot;
};
struct IdPair {
    int64_t w_off, y_off, out_row;  // byte offsets into W and Y, output row
    bool valid;
};
__device__ __forceinline__ IdPair id_route(const IdRoute &r) {
    const int64_t p = r.p0 + blockIdx.y;
    const int e = r.ids[p];
    const bool valid = e >= 0 && e < r.E;
    return IdPair{(valid ? (int64_t)e : 0) * r.w_stride, (r.y_per_slot ? p : p / r.U) * r.y_rowbytes, p, valid};
}

}  // namespace qmm
