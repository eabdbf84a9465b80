// pa_i8_core.h -- the INT8 tile format and the lane-level pieces its kernels
// share (pa_i8.hip: append, quantiser, decode; pa_prefill_i8.hip: chunked
// prefill).  The format (TinyLoop, "Lifecycle and Memory Model", section
// "Per-request / handle-owned memory", INT8 K/V mode): one symmetric fp32
// scale per (token, KV head) row of 64 values, code = round-half-even(x /
// scale) with scale = max|x| / 127, the value a code stands for code * scale;
// the tile layout is described at the top of pa_i8.hip.
#pragma once

#include <math.h>

#include "pa_decode_core.h"

namespace pa {

constexpr int kI8Tile = 2176;     // bytes per (page, KV head) tile
constexpr int kI8VOff = 1024;     // V block offset
constexpr int kI8KScOff = 2048;   // K scales
constexpr int kI8VScOff = 2112;   // V scales
constexpr int kPageBytesI8 = kHKV * kI8Tile;
constexpr float kOffsetF16 = 1152.0f;  // value of the f16 an INT8 code c becomes, minus c

// The P.V products take each weight (softmax weight x V scale) as an f16 hi
// half plus an f16 lo half (its rounding remainder).  With bf16 output the lo
// half is dropped for keys whose live V scales are all <= 1/8, i.e. every
// |v| <= 127/8: an f16 weight is within 2^-11 of its value relative, so the
// output (a weighted mean of the v) moves by at most 2^-11 * 16 < 8e-3, inside
// the bf16 output's 1e-2 bound, before its own rounding to bf16.
constexpr uint32_t kHiOnlyVScaleBits = 0x3E000000u;  // 0.125f, as bits

__device__ __forceinline__ int i8_kpos(int t, int d) { return (((d & 31) >> 3) * 16 + t) * 16 + (d >> 5) * 8 + (d & 7); }
__device__ __forceinline__ int i8_vpos(int t, int d) {
    return kI8VOff + ((t >> 2) * 16 + (d & 15)) * 16 + (d >> 4) * 4 + (t & 3);
}

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Quantise one value against a row scale (binary32 throughout, the decision
// the format defines): round-half-even(x / scale), clamped to [-127, 127].
__device__ __forceinline__ int quant_code(float x, float scale) {
    if (!(scale > 0.0f)) return 0;
    float c = rintf(x / scale);
    c = fminf(fmaxf(c, -127.0f), 127.0f);
    return static_cast<int>(c);
}

// Max over the 32 lanes of each half-wave (lanes 0-31 and 32-63 separately).
__device__ __forceinline__ float max_lanes32(float v) {
#pragma unroll
    for (int k = 1; k < 32; k <<= 1) v = fmaxf(v, __shfl_xor(v, k, 64));
    return v;
}
// Max over the 8 consecutive lanes of an aligned lane group.
__device__ __forceinline__ float max_lanes8(float v) {
    v = fmaxf(v, dpp_f32<0xB1>(v));
    v = fmaxf(v, dpp_f32<0x4E>(v));
    v = fmaxf(v, dpp_f32<0x141>(v));
    return v;
}

// 4 codes (two's complement bytes of w) -> the f16 values 1152 + code, as two
// packed pairs (bytes 0,1 and 2,3): code ^ 0x80 = code + 128 under the f16
// exponent byte 0x64 is 1024 + code + 128, exactly.
__device__ __forceinline__ void codes_to_f16x4(uint32_t w, uint32_t &p01, uint32_t &p23) {
    const uint32_t u = w ^ 0x80808080u;
    p01 = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
    p23 = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
}
__device__ __forceinline__ half8 codes8_to_f16(uint32_t w0, uint32_t w1) {
    uint32_t a, b, c, d;
    codes_to_f16x4(w0, a, b);
    codes_to_f16x4(w1, c, d);
    return __builtin_bit_cast(half8, u32x4{a, b, c, d});
}
// 4 codes -> the f16 values of the codes themselves (1152 + code, minus 1152
// in packed f16: exact, every integer in [-127, 127] being an f16).
__device__ __forceinline__ half4 codes4_to_f16_signed(uint32_t w) {
    uint32_t a, b;
    codes_to_f16x4(w, a, b);
    const half4 off = {static_cast<_Float16>(-kOffsetF16), static_cast<_Float16>(-kOffsetF16),
                       static_cast<_Float16>(-kOffsetF16), static_cast<_Float16>(-kOffsetF16)};
    return __builtin_bit_cast(half4, u32x2{a, b}) + off;
}

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, half2v));
}

struct I8Page {
    u32x4 k, v;   // the lane's K unit and V unit
    f32x4 ks, vs; // K and V scales of tokens 4(l/16) .. +3
};

// The value lane src (wave-uniform) holds, as a scalar.
__device__ __forceinline__ float lane_value(float v, int src) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), src));
}

// Sum (or max) over the four lanes l, l^16, l^32, l^48.
__device__ __forceinline__ float sum_quarters(float v) {
    float lo, hi;
    xor16_pair(v, lo, hi);
    v = lo + hi;
    xor32_pair(v, lo, hi);
    return lo + hi;
}
__device__ __forceinline__ float max_quarters(float v) {
    float lo, hi;
    xor16_pair(v, lo, hi);
    v = fmaxf(lo, hi);
    xor32_pair(v, lo, hi);
    return fmaxf(lo, hi);
}

}  // namespace pa
