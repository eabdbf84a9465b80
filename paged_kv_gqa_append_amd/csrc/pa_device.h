// pa_device.h -- small device helpers shared by the libpa kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kHQ = 32;       // query heads
constexpr int kHKV = 8;       // KV heads
constexpr int kGroup = 4;     // query heads per KV head
constexpr int kD = 64;        // head dim
constexpr int kPage = 16;     // tokens per page
constexpr int kTile = kPage * kD;          // elements of one (page, kv head) tile
constexpr int kPageElems = kHKV * kTile;   // elements of one page (all heads)
constexpr int kCuPerXcd = 32;  // gfx950: 8 XCDs x 32 CUs; workgroup ids are dealt to XCDs by id mod 8

constexpr uint32_t kDevErrContextLen = 0x1u;
constexpr uint32_t kDevErrPageId = 0x2u;
constexpr uint32_t kDevErrDispatchOrder = 0x4u;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __builtin_bit_cast(float, static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// <a, b> over the 8 bf16 elements held in two 16-byte words, fp32 accumulation.
// The words are reinterpreted whole and split with shufflevector: hipcc 7.2
// mis-lowers __builtin_bit_cast applied to a single vector element (a.x) into
// a reload of element 0, which would feed the same pair to all four dot2s.
__device__ __forceinline__ float dot8_bf16(u32x4 a, u32x4 b, float acc) {
    const bf16x8 x = __builtin_bit_cast(bf16x8, a);
    const bf16x8 y = __builtin_bit_cast(bf16x8, b);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 0, 1), __builtin_shufflevector(y, y, 0, 1), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 2, 3), __builtin_shufflevector(y, y, 2, 3), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 4, 5), __builtin_shufflevector(y, y, 4, 5), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 6, 7), __builtin_shufflevector(y, y, 6, 7), acc, false);
    return acc;
}

// Data-parallel-primitive lane permutes (DPP).  Control codes (GCN/CDNA):
//   quad_perm [1,0,3,2] = 0xB1, quad_perm [2,3,0,1] = 0x4E,
//   row_half_mirror = 0x141 (lane i <-> 7-i within each 8 lanes),
//   row_ror:8 = 0x128 (lane i <-> i^8 within each 16 lanes).
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, true));
}

// Sum over the 8 consecutive lanes of an aligned lane group; every lane gets it.
__device__ __forceinline__ float sum_lanes8(float v) {
    v += dpp_f32<0xB1>(v);
    v += dpp_f32<0x4E>(v);
    v += dpp_f32<0x141>(v);
    return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// The bf16 nearest to the double x, ties to even, in one rounding step: x's
// binade has bf16 spacing 2^(e-8) for 2^(e-1) <= |x| < 2^e (2^-133 below
// 2^-126); x is scaled by the spacing, rounded to an integer (ties to even) and
// scaled back, all exact in double, and the result is a binary32 whose low 16
// bits are zero.  Without branches: zeros and infinities pass through the
// scaling unchanged (their exponent reads as 0), a result of 2^128 or more
// converts to infinity, and NaN gives 0x7FC0.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
    const int e = __builtin_amdgcn_frexp_exp(x);
    const int qexp = max(e - 8, -133);
    const double y = __builtin_ldexp(__builtin_rint(__builtin_ldexp(x, -qexp)), qexp);
    const uint16_t b = static_cast<uint16_t>(__builtin_bit_cast(uint32_t, static_cast<float>(y)) >> 16);
    return __builtin_isnan(x) ? static_cast<uint16_t>(0x7FC0) : b;
}

// Rotate-half RoPE of the pair (x_i, x_{i+32}) by (c, s) = (cos, sin) of
// pos * theta^(-2i/64), both doubles from the table:
//     (x_i c - x_{i+32} s,  x_{i+32} c + x_i s),
// evaluated in double with every product and the sum rounded on its own (no
// fused multiply-add), then rounded once to bf16.  These are the operations of
// the plain fp64 definition, so the rotated rows are bitwise those of an exact
// evaluation rounded the same way, and every kernel that rotates uses this one
// function.
__device__ __forceinline__ void rope_pair_bf16(float x0, float x1, double c, double s, uint16_t &lo, uint16_t &hi) {
    const double a = x0, b = x1;
    double p0 = a * c, p1 = b * s, p2 = b * c, p3 = a * s;
    // The products leave through an empty asm, so the compiler (built with
    // contraction on) cannot fuse them into the sums.
    asm("" : "+v"(p0), "+v"(p1), "+v"(p2), "+v"(p3));
    lo = f64_to_bf16(p0 - p1);
    hi = f64_to_bf16(p2 + p3);
}

// Rotate-half pairs i0 .. i0+3 of a row held as a = elements i0 .. i0+3 and
// b = their partners i0+32 .. i0+35 (8 bytes each) by the (cos, sin) entries
// t[k] of pair i0 + k (rope_pair_bf16); the rotated halves, packed the same way.
__device__ __forceinline__ void rope4(uint2 a, uint2 b, const double2 (&t)[4], uint2 &lo_out, uint2 &hi_out) {
    uint16_t lo[4], hi[4];
    rope_pair_bf16(bf16_lo(a.x), bf16_lo(b.x), t[0].x, t[0].y, lo[0], hi[0]);
    rope_pair_bf16(bf16_hi(a.x), bf16_hi(b.x), t[1].x, t[1].y, lo[1], hi[1]);
    rope_pair_bf16(bf16_lo(a.y), bf16_lo(b.y), t[2].x, t[2].y, lo[2], hi[2]);
    rope_pair_bf16(bf16_hi(a.y), bf16_hi(b.y), t[3].x, t[3].y, lo[3], hi[3]);
    lo_out = uint2{lo[0] | (uint32_t(lo[1]) << 16), lo[2] | (uint32_t(lo[3]) << 16)};
    hi_out = uint2{hi[0] | (uint32_t(hi[1]) << 16), hi[2] | (uint32_t(hi[3]) << 16)};
}

}  // namespace pa
