// mfma_common.h -- pieces shared by the int8 MFMA kernels (gfx950): operand
// vector types, buffer-resource loads and the per-byte digit-plane product.
//
// Staging goes through buffer resources: a scalar base and byte count per
// source and 32-bit per-lane offsets, with the K step in the scalar offset.
// Loads past the byte count return zero instead of faulting.  Plain global
// pointers would need 64-bit per-lane addresses, and a generic (flat) load
// would make the compiler wait for every outstanding global->LDS transfer.
// A resource must be built where it is used: one held across a lambda is
// treated as divergent and the loads that take it get waterfall loops.
#pragma once

#include "qmm_device.h"

namespace qmm {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ rsrc_t make_rsrc(const uint8_t *base, int64_t bytes) {
    const int64_t n = bytes < 0 ? 0 : (bytes > 0xffffffffll ? 0xffffffffll : bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(base), 0, (int)(uint32_t)n,
                                             0x00020000);  // raw dword access (gfx9 family)
}
__device__ __forceinline__ uint4 bld16(rsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}
// 16 bytes per lane into LDS at lds_base + 16 * lane (lds_base wavefront-uniform)
__device__ __forceinline__ void dma16(rsrc_t r, uint32_t voff, uint32_t soff, uint8_t *lds_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds_base, 16, voff, soff, 0, 0);
}

// packed per-byte product of four codes (each <= 15) with a scale digit (<= 7):
// every byte product is below 256, so no carry crosses a byte
__device__ __forceinline__ int plane(uint32_t q4, uint32_t digit_pair) {
    const us2 p = __builtin_bit_cast(us2, q4) * __builtin_bit_cast(us2, digit_pair);
    return (int)__builtin_bit_cast(uint32_t, p);
}
// Q6_K weight operands (the GEMM and the small-batch kernel):
// Four codes u (bytes in [0, 63]) with the pairs s2 = (s, s) and
// c2 = (128 - 32s, 128 - 32s) -> the digit bytes of t = s*(u - 32) = 256*hi + lo:
// t' = t + 128 = s*u + 128 - 32s (one packed 16-bit multiply-add per two codes;
// |t'| < 2^15), hi = the high byte of t' (floor(t'/256), signed), lo = the low
// byte of t' minus 128 (its top bit flipped), both in int8 range.
__device__ __forceinline__ void t_digits(uint32_t u, s16x2 s2, s16x2 c2, uint32_t &hi, uint32_t &lo) {
    const uint32_t e = __builtin_amdgcn_perm(u, u, 0x0c020c00u);  // u0, u2 in 16-bit lanes
    const uint32_t o = __builtin_amdgcn_perm(u, u, 0x0c030c01u);  // u1, u3
    const uint32_t te = __builtin_bit_cast(uint32_t, __builtin_bit_cast(s16x2, e) * s2 + c2);
    const uint32_t to = __builtin_bit_cast(uint32_t, __builtin_bit_cast(s16x2, o) * s2 + c2);
    // bytes 0-3 of the pair are the second operand, 4-7 the first
    hi = __builtin_amdgcn_perm(to, te, 0x07030501u);
    lo = __builtin_amdgcn_perm(to, te, 0x06020400u) ^ 0x80808080u;
}

// two int16 values as two fp16 (exact for |v| <= 2048)
__device__ __forceinline__ uint32_t h2_bits(int lo, int hi) {
    return f32_to_f16_bits((float)lo) | (f32_to_f16_bits((float)hi) << 16);
}

// mul_mat_id (GROUPED GEMMs): the expert-grouped tile table that
// k_moe_group_ids builds.  Tile g covers the sorted slots tile_r0[g] .. of
// expert tile_e[g] (at most 128 of them, up to start[e+1]); sorted[slot] is a
// (token, slot) pair p, whose activation row is p (y_per_slot) or p / U and
// whose output row is p.  The GEMM's M is then the number of activation rows.
struct Grouping {
    const int32_t *start, *tile_e, *tile_r0, *ntiles, *sorted;
    int64_t U, w_stride;
    int y_per_slot;
};
// Tile of workgroup bid (tiles_n column tiles per row tile): false when the
// routing produced fewer tiles (the whole workgroup then exits).
__device__ __forceinline__ bool grouped_tile(const Grouping &g, int bid, int tiles_n, int bm, int &tile_n,
                                             int &r0, int &m_last, int &e) {
    const int t = bid / tiles_n;
    tile_n = bid - t * tiles_n;
    if (t >= *g.ntiles) return false;
    e = g.tile_e[t];
    r0 = g.tile_r0[t];
    const int rows = g.start[e + 1] - r0;
    m_last = (rows < bm ? rows : bm) - 1;
    return true;
}
// activation row of tile row rr (0 <= rr <= m_last)
__device__ __forceinline__ int64_t grouped_row(const Grouping &g, int r0, int rr) {
    const int p = g.sorted[r0 + rr];
    return g.y_per_slot ? (int64_t)p : (int64_t)p / g.U;
}

}  // namespace
}  // namespace qmm
