// pa_i8.hip -- INT8 K/V pages: quantising append, bulk quantiser, and paged
// GQA decode over INT8 tiles (optionally fused with the append).
//
// TinyLoop ("Lifecycle and Memory Model", section "Per-request / handle-owned
// memory") names an INT8 K/V cache mode beside FP16 and gives no rule.  The
// format here: one symmetric fp32 scale per (token, KV head) row of 64 values,
//   scale = max|x| / 127,   code = round-half-even(x / scale), |code| <= 127,
// both evaluated in IEEE binary32 (a zero row has scale 0 and codes 0); the
// value a code stands for is code * scale.  K rows are quantised after RoPE
// from their bf16-rounded values (the same bf16 row the bf16 pool would hold),
// V rows from their bf16 input.
//
// Tile of (page, KV head), PA_I8_TILE_BYTES = 2176 bytes:
//   [0, 1024)     K codes, [1024, 2048) V codes,
//   2048 + 8t     K scale (fp32) of token t, 2052 + 8t its V scale.
//   Code of element d of token t at byte ((t & 7) * 8 + d / 8) * 16 + (t / 8) * 8 + d % 8
//   of its 1 KiB block, so 16-byte unit u = 8g + c holds the chunk c*8..c*8+7
//   of tokens g (bytes 0-7) and g+8 (bytes 8-15): exactly what lane u of the
//   bf16 decode kernel holds, read here with ONE 16-byte load per block.
//
// Decode arithmetic: codes enter as u = code + 128 (an XOR of the sign bit)
// converted exactly to fp32 and, for K, to bf16 pairs, so the bf16 kernel's
// dot-product and reduction machinery applies unchanged:
//   <q, code> = <q, u> - 128 * sum(q)            (per query head, fp32)
//   x_t = scale * K_scale_t * <q, code_t>
//   acc = sum_t w_t V_scale_t (u_t - 128) = sum_t (w_t V_scale_t) u_t - 128 * sum_t w_t V_scale_t
// Everything else (online softmax, lazy max, wave and partition merges) is the
// bf16 kernel's, from pa_decode_core.h.
#include <math.h>

#include "pa_decode_core.h"

namespace pa {

constexpr int kI8Tile = 2176;     // bytes per (page, KV head) tile
constexpr int kI8VOff = 1024;     // V block offset
constexpr int kI8ScOff = 2048;    // scales offset
constexpr int kPageBytesI8 = kHKV * kI8Tile;

__device__ __forceinline__ int i8_pos(int t, int d) { return (((t & 7) * 8 + (d >> 3)) * 16) + (t >> 3) * 8 + (d & 7); }

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

// 4 codes (two's complement bytes) -> u = code + 128 as two bf16 pairs (exact:
// every integer up to 256 is a bf16 value, whose fp32 pattern has a zero low half).
__device__ __forceinline__ void codes_to_bf16x4(uint32_t w, uint32_t &p01, uint32_t &p23) {
    const uint32_t u = w ^ 0x80808080u;
    const uint32_t f0 = __builtin_bit_cast(uint32_t, static_cast<float>(u & 0xFFu));
    const uint32_t f1 = __builtin_bit_cast(uint32_t, static_cast<float>((u >> 8) & 0xFFu));
    const uint32_t f2 = __builtin_bit_cast(uint32_t, static_cast<float>((u >> 16) & 0xFFu));
    const uint32_t f3 = __builtin_bit_cast(uint32_t, static_cast<float>(u >> 24));
    p01 = __builtin_amdgcn_perm(f1, f0, 0x07060302u);
    p23 = __builtin_amdgcn_perm(f3, f2, 0x07060302u);
}
// 8 codes (two words) -> 8 bf16 values of u = code + 128, in element order.
__device__ __forceinline__ u32x4 codes8_to_bf16(uint32_t w0, uint32_t w1) {
    u32x4 r;
    uint32_t a, b, c, d;
    codes_to_bf16x4(w0, a, b);
    codes_to_bf16x4(w1, c, d);
    r.x = a;
    r.y = b;
    r.z = c;
    r.w = d;
    return r;
}
// 8 codes (two words) -> 8 fp32 values of u = code + 128, in element order.
__device__ __forceinline__ void codes8_to_f32(uint32_t w0, uint32_t w1, float (&f)[8]) {
    const uint32_t u0 = w0 ^ 0x80808080u, u1 = w1 ^ 0x80808080u;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        f[k] = static_cast<float>((u0 >> (8 * k)) & 0xFFu);
        f[4 + k] = static_cast<float>((u1 >> (8 * k)) & 0xFFu);
    }
}

// ------------------------------------------------------------- append ------
// One workgroup (256 threads) per sequence: thread t serves KV head j = t/32,
// rotate-half pair p = t%32 of K and elements 2p, 2p+1 of V, plus 4 q pairs.
__global__ __launch_bounds__(256) void k_append_rope_i8(uint16_t *__restrict__ q, const uint16_t *__restrict__ k_new,
                                                        const uint16_t *__restrict__ v_new, uint8_t *__restrict__ pool,
                                                        const int32_t *__restrict__ bt, const int32_t *__restrict__ lens,
                                                        const float *__restrict__ rope, int max_blocks, int num_pages,
                                                        int max_pos, uint32_t *__restrict__ flags) {
    const int s = blockIdx.x;
    const int64_t len = lens[s];
    const int64_t pos = len - 1;
    if (len < 1 || pos >= static_cast<int64_t>(max_blocks) * kPage || pos >= max_pos) {
        if (threadIdx.x == 0 && flags) atomicOr(flags, kDevErrContextLen);
        return;
    }
    const int page = bt[static_cast<int64_t>(s) * max_blocks + (pos >> 4)];
    if (page < 0 || page >= num_pages) {
        if (threadIdx.x == 0 && flags) atomicOr(flags, kDevErrPageId);
        return;
    }
    const int slot = static_cast<int>(pos & (kPage - 1));
    const float *cs = rope + pos * kD;  // [32][2]
    const int t = threadIdx.x;
    const int j = t >> 5, p = t & 31;
    uint8_t *tile = pool + (static_cast<int64_t>(page) * kHKV + j) * kI8Tile;
    {
        // K: rotate the pair, round to bf16 (the stored row of the bf16 format), quantise the row
        const uint16_t *src = k_new + (static_cast<int64_t>(s) * kHKV + j) * kD;
        const float x0 = bf16_to_f32(src[p]), x1 = bf16_to_f32(src[p + 32]);
        const float c = cs[2 * p], sn = cs[2 * p + 1];
        const float y0 = bf16_to_f32(f32_to_bf16(rope_lo(x0, x1, c, sn)));
        const float y1 = bf16_to_f32(f32_to_bf16(rope_hi(x0, x1, c, sn)));
        const float sc = max_lanes32(fmaxf(fabsf(y0), fabsf(y1))) / 127.0f;
        tile[i8_pos(slot, p)] = static_cast<uint8_t>(quant_code(y0, sc));
        tile[i8_pos(slot, p + 32)] = static_cast<uint8_t>(quant_code(y1, sc));
        if (p == 0) *reinterpret_cast<float *>(tile + kI8ScOff + 8 * slot) = sc;
    }
    {
        // V: elements 2p, 2p+1 verbatim from bf16, quantised with the row's scale
        const uint32_t wv = reinterpret_cast<const uint32_t *>(v_new + (static_cast<int64_t>(s) * kHKV + j) * kD)[p];
        const float v0 = bf16_lo(wv), v1 = bf16_hi(wv);
        const float sc = max_lanes32(fmaxf(fabsf(v0), fabsf(v1))) / 127.0f;
        const uint32_t pair = (static_cast<uint32_t>(quant_code(v0, sc)) & 0xFFu) |
                              ((static_cast<uint32_t>(quant_code(v1, sc)) & 0xFFu) << 8);
        *reinterpret_cast<uint16_t *>(tile + kI8VOff + i8_pos(slot, 2 * p)) = static_cast<uint16_t>(pair);
        if (p == 0) *reinterpret_cast<float *>(tile + kI8ScOff + 8 * slot + 4) = sc;
    }
    if (q) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int idx = t + 256 * r;
            const int h = idx >> 5, pp = idx & 31;
            uint16_t *row = q + (static_cast<int64_t>(s) * kHQ + h) * kD;
            const float x0 = bf16_to_f32(row[pp]), x1 = bf16_to_f32(row[pp + 32]);
            const float c = cs[2 * pp], sn = cs[2 * pp + 1];
            row[pp] = f32_to_bf16(rope_lo(x0, x1, c, sn));
            row[pp + 32] = f32_to_bf16(rope_hi(x0, x1, c, sn));
        }
    }
}

// --------------------------------------------------------- bulk quantiser --
// One workgroup (256 threads) per (listed page, KV head): thread t quantises
// chunk c = t%8 of row r = t/8 (rows 0-15: K slots, 16-31: V slots).
__global__ __launch_bounds__(256) void k_quantize_pages_i8(uint8_t *__restrict__ pool, const uint16_t *__restrict__ k_pool,
                                                           const uint16_t *__restrict__ v_pool,
                                                           const int32_t *__restrict__ page_ids, int num_pages,
                                                           uint32_t *__restrict__ flags) {
    const int idx = blockIdx.x >> 3;
    const int j = blockIdx.x & 7;
    const int page = page_ids ? page_ids[idx] : idx;
    if (page < 0 || page >= num_pages) {
        if (threadIdx.x == 0 && j == 0 && flags) atomicOr(flags, kDevErrPageId);
        return;
    }
    const int t = threadIdx.x;
    const int r = t >> 3, c = t & 7;
    const int is_v = r >> 4, slot = r & 15;
    const uint16_t *src = (is_v ? v_pool : k_pool) + ((static_cast<int64_t>(page) * kHKV + j) * kPage + slot) * kD + c * 8;
    const u32x4 raw = *reinterpret_cast<const u32x4 *>(src);
    const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
    float x[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        x[2 * k] = bf16_lo(wd[k]);
        x[2 * k + 1] = bf16_hi(wd[k]);
    }
    float a = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) a = fmaxf(a, fabsf(x[k]));
    const float sc = max_lanes8(a) / 127.0f;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        lo |= (static_cast<uint32_t>(quant_code(x[k], sc)) & 0xFFu) << (8 * k);
        hi |= (static_cast<uint32_t>(quant_code(x[4 + k], sc)) & 0xFFu) << (8 * k);
    }
    uint8_t *tile = pool + (static_cast<int64_t>(page) * kHKV + j) * kI8Tile;
    *reinterpret_cast<uint2 *>(tile + is_v * kI8VOff + i8_pos(slot, c * 8)) = make_uint2(lo, hi);
    if (c == 0) *reinterpret_cast<float *>(tile + kI8ScOff + 8 * slot + 4 * is_v) = sc;
}

// ------------------------------------------------------------- decode ------
// The bf16 kernel's structure (see pa_decode.hip) over INT8 tiles.  The pool
// travels in DecodeParams::k_pool (v_pool is unused): K, V and scales of a
// (page, head) are one tile.
struct I8Regs {
    u32x4 k, v;   // K / V codes of tokens g (words 0,1) and g+8 (words 2,3), chunk c
    float2 sc;    // (K scale, V scale) of the lane's score token g + 8*t0
};

template <int kWaves, bool kFused>
__global__ __launch_bounds__(64 * kWaves, 4) void k_decode_paged_i8(DecodeParams P) {
    constexpr int kThreads = 64 * kWaves;
    static_assert(kMaxPartPages <= 64 * kWaves, "one page id per lane must cover a partition");
    const int part = blockIdx.x % P.num_parts;
    const int sj = blockIdx.x / P.num_parts;
    const int j = sj & (kHKV - 1);
    const int s = sj >> 3;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    __builtin_amdgcn_s_setprio(3);
    const uint8_t *pool = reinterpret_cast<const uint8_t *>(P.k_pool);

    __shared__ int s_app_page;
    __shared__ float s_m[kWaves][kGroup];
    __shared__ float s_l[kWaves][kGroup];
    __shared__ float s_l2[kWaves][kGroup];   // sum of w * V scale (the 128-offset correction)
    __shared__ float s_acc[kWaves][kGroup][kD];
    __shared__ __align__(16) uint16_t s_q[kGroup][kD];  // rotated q (fused)
    __shared__ __align__(16) int8_t s_nk[kD];           // appended K row codes (fused)
    __shared__ __align__(16) int8_t s_nv[kD];           // appended V row codes (fused)
    __shared__ float s_nsc[2];                          // appended row scales (K, V)

    const int g = lane >> 3;
    const int c = lane & 7;
    const int b0 = c & 1, b1 = (c >> 1) & 1, b2 = c >> 2;
    const int t0 = b0 ^ b2;
    const int hm = ((b1 ^ b2) << 1) | b2;
    const int tok_s = g + 8 * t0;  // the lane's score token in a page

    const int pg0 = part * P.part_pages;
    const int slice = min(P.part_pages, P.max_blocks - pg0);
    const int32_t *bt_row = P.bt + static_cast<int64_t>(s) * P.max_blocks;
    const int L = P.lens[s];
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const int first_id = wu < slice ? bt_row[pg0 + wu] : -1;
    const int my_idx = wu + kWaves * lane;
    const int my_id = bt_row[pg0 + min(my_idx, slice - 1)];
    const int64_t qrow0 = (static_cast<int64_t>(s) * kHQ + j * kGroup) * kD;
    const int64_t nrow = (static_cast<int64_t>(s) * kHKV + j) * kD;
    const int pos = L - 1;
    const int pr = tid & 31;
    float x0 = 0.0f, x1 = 0.0f;
    uint32_t vword = 0;
    if (kFused) {
        const uint16_t *src = tid < 128 ? P.q + qrow0 + ((tid >> 5) & 3) * kD : P.k_new + nrow;
        x0 = bf16_to_f32(src[pr]);
        x1 = bf16_to_f32(src[pr + 32]);
        vword = reinterpret_cast<const uint32_t *>(P.v_new + nrow)[pr];
    }
    u32x4 qv[kGroup];
    if (!kFused) {
#pragma unroll
        for (int m = 0; m < kGroup; ++m) qv[m] = *reinterpret_cast<const u32x4 *>(P.q + qrow0 + (m ^ hm) * kD + c * 8);
    }
    __builtin_amdgcn_sched_barrier(0);
    float co = 0.0f, si = 0.0f;
    if (kFused) {
        const int pos_c = min(max(pos, 0), P.max_pos - 1);
        const float *cs = P.rope + static_cast<int64_t>(pos_c) * kD + 2 * pr;
        co = cs[0];
        si = cs[1];
    }
    __builtin_amdgcn_sched_barrier(0);
    const int64_t tile_j = static_cast<int64_t>(j) * kI8Tile;
    auto load_tile = [&](int page_id) {
        const uint8_t *t = pool + static_cast<int64_t>(page_id) * kPageBytesI8 + tile_j;
        I8Regs r;
        r.k = *reinterpret_cast<const u32x4 *>(t + lane * 16);
        r.v = *reinterpret_cast<const u32x4 *>(t + kI8VOff + lane * 16);
        r.sc = *reinterpret_cast<const float2 *>(t + kI8ScOff + 8 * tok_s);
        return r;
    };
    I8Regs cur = load_tile(first_id >= 0 && first_id < P.num_pages ? first_id : 0);
    __builtin_amdgcn_sched_barrier(0);

    // fused: rotate q into LDS (threads 0..127); wave 2 rotates the new K row
    // (lanes 0-31, pair pr) and takes the new V row (lanes 32-63, elements
    // 2pr, 2pr+1), then quantises both rows exactly as k_append_rope_i8 does.
    if (kFused && tid < 192) {
        if (tid < 128) {
            s_q[tid >> 5][pr] = f32_to_bf16(rope_lo(x0, x1, co, si));
            s_q[tid >> 5][pr + 32] = f32_to_bf16(rope_hi(x0, x1, co, si));
        } else {
            const bool is_k = tid < 160;
            const float e0 = is_k ? bf16_to_f32(f32_to_bf16(rope_lo(x0, x1, co, si))) : bf16_lo(vword);
            const float e1 = is_k ? bf16_to_f32(f32_to_bf16(rope_hi(x0, x1, co, si))) : bf16_hi(vword);
            const float sc = max_lanes32(fmaxf(fabsf(e0), fabsf(e1))) / 127.0f;
            const int c0 = quant_code(e0, sc), c1 = quant_code(e1, sc);
            if (is_k) {
                s_nk[pr] = static_cast<int8_t>(c0);
                s_nk[pr + 32] = static_cast<int8_t>(c1);
            } else {
                s_nv[2 * pr] = static_cast<int8_t>(c0);
                s_nv[2 * pr + 1] = static_cast<int8_t>(c1);
            }
            if (pr == 0) s_nsc[is_k ? 0 : 1] = sc;
        }
    }

    bool len_ok = (L >= 1) && (L <= P.max_blocks * kPage);
    if (kFused) len_ok = len_ok && (L - 1 < P.max_pos);
    const int n_pages = len_ok ? (L + kPage - 1) / kPage : 0;
    const int n_parts_s = (n_pages + P.part_pages - 1) / P.part_pages;
    const int pg1 = min(pg0 + P.part_pages, n_pages);
    const int bad = (my_idx < slice) && (pg0 + my_idx < n_pages) && (my_id < 0 || my_id >= P.num_pages);
    if (kFused) {
        const int rel = (pos >> 4) - pg0;
        if (len_ok && rel >= 0 && rel == my_idx && rel < slice) s_app_page = my_id;
    }
    bool ok = len_ok && (__syncthreads_or(bad) == 0);
    if (ok && n_parts_s > 1) {
        int bad_row = 0;
        for (int b = tid; b < n_pages; b += kThreads) {
            const int pid = bt_row[b];
            bad_row |= (pid < 0) | (pid >= P.num_pages);
        }
        ok = __syncthreads_or(bad_row) == 0;
    }
    if (!ok) {
        if (part == 0 && tid < kGroup * kD) {
            const int64_t o = (static_cast<int64_t>(s) * kHQ + j * kGroup) * kD + tid;
            if (P.out_fp32) static_cast<float *>(P.out)[o] = 0.0f;
            else static_cast<uint16_t *>(P.out)[o] = 0;
            if (tid == 0 && P.flags) atomicOr(P.flags, len_ok ? kDevErrPageId : kDevErrContextLen);
        }
        return;
    }
    if (part >= n_parts_s) return;
    if (kFused) {
#pragma unroll
        for (int m = 0; m < kGroup; ++m) qv[m] = *reinterpret_cast<const u32x4 *>(&s_q[m ^ hm][c * 8]);
        if (tid < 9 && pg1 == n_pages) {  // append the quantised row (last partition only)
            const int sl = pos & (kPage - 1);
            uint8_t *tw = const_cast<uint8_t *>(pool) + static_cast<int64_t>(s_app_page) * kPageBytesI8 + tile_j;
            if (tid < 8) {
                *reinterpret_cast<uint2 *>(tw + i8_pos(sl, tid * 8)) = *reinterpret_cast<const uint2 *>(&s_nk[tid * 8]);
                *reinterpret_cast<uint2 *>(tw + kI8VOff + i8_pos(sl, tid * 8)) =
                    *reinterpret_cast<const uint2 *>(&s_nv[tid * 8]);
            } else {
                *reinterpret_cast<float2 *>(tw + kI8ScOff + 8 * sl) = make_float2(s_nsc[0], s_nsc[1]);
            }
        }
        if (P.write_q && n_parts_s == 1 && tid >= 64 && tid < 96)
            *reinterpret_cast<u32x4 *>(P.q + qrow0 + (tid - 64) * 8) =
                *reinterpret_cast<const u32x4 *>(&s_q[0][(tid - 64) * 8]);
    }
    // scale * log2(e) * <q, 128> of the lane's own score head: the offset the
    // u = code + 128 encoding adds to every K score.  It goes through the same
    // lane-permuted reduction as the scores (a key row of bf16 128.0s), so it
    // lands on the lane that owns that head's score.
    const u32x4 k128 = {0x43004300u, 0x43004300u, 0x43004300u, 0x43004300u};
    const float corr_k = page_score(qv, k128, k128, P.scale_log2);

    auto load_page = [&](int p) {
        return load_tile(__builtin_amdgcn_readlane(my_id, (p - pg0 - wu) / kWaves));
    };
    int p = pg0 + wu;

    float m_run = kNegBig;
    float l_run = 0.0f;   // sum of the lane's own weights
    float l2_run = 0.0f;  // sum of the lane's own weights times their V scales
    float acc[kGroup][8];
#pragma unroll
    for (int e = 0; e < kGroup; ++e)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[e][i] = 0.0f;

    // One page; `last` pages may be partly empty (dead slots hold anything:
    // their weight is forced to 0 before it meets a scale).
    auto process = [&](const I8Regs &r, bool last, int p) {
        const uint32_t kw0 = t0 ? r.k.z : r.k.x, kw1 = t0 ? r.k.w : r.k.y;
        const uint32_t kw2 = t0 ? r.k.x : r.k.z, kw3 = t0 ? r.k.y : r.k.w;
        const u32x4 ka = codes8_to_bf16(kw0, kw1);
        const u32x4 kb = codes8_to_bf16(kw2, kw3);
        float x = (page_score(qv, ka, kb, P.scale_log2) - corr_k) * r.sc.x;
        bool dead = false;
        if (last) {
            dead = p * kPage + tok_s >= L;
            if (dead) x = -INFINITY;
        }
        const float pw = softmax_step_t<true>(x, m_run, l_run, l2_run, acc);
        float pv = pw * r.sc.y;
        if (last && dead) pv = 0.0f;
        l2_run += pv;
        float va[8], vb[8];
        const uint32_t vw0 = b2 ? r.v.z : r.v.x, vw1 = b2 ? r.v.w : r.v.y;
        const uint32_t vw2 = b2 ? r.v.x : r.v.z, vw3 = b2 ? r.v.y : r.v.w;
        codes8_to_f32(vw0, vw1, va);
        codes8_to_f32(vw2, vw3, vb);
        accumulate(pv, va, vb, acc);
    };
    auto process_last = [&](I8Regs r, int p) {
        if (kFused) {  // patch the appended token's codes and scales into the registers
            const int sl = pos & (kPage - 1);
            if (g == (sl & 7)) {
                const uint2 nk = *reinterpret_cast<const uint2 *>(&s_nk[c * 8]);
                const uint2 nv = *reinterpret_cast<const uint2 *>(&s_nv[c * 8]);
                if (sl >> 3) {
                    r.k.z = nk.x; r.k.w = nk.y;
                    r.v.z = nv.x; r.v.w = nv.y;
                } else {
                    r.k.x = nk.x; r.k.y = nk.y;
                    r.v.x = nv.x; r.v.y = nv.y;
                }
            }
            if (tok_s == sl) r.sc = make_float2(s_nsc[0], s_nsc[1]);
        }
        process(r, true, p);
    };
    const int p_stop = (pg1 == n_pages) ? n_pages - 1 : pg1;
    I8Regs alt;
    bool last_in_alt = false;
    const int span = pg1 - pg0;
    auto level = [&]() {
        const int done16 = 16 * (p - pg0);
        if (done16 >= 15 * span) __builtin_amdgcn_s_setprio(0);
        else if (done16 >= 13 * span) __builtin_amdgcn_s_setprio(1);
        else if (done16 >= 10 * span) __builtin_amdgcn_s_setprio(2);
    };
    while (p < p_stop) {
        if (p + kWaves < pg1) alt = load_page(p + kWaves);
        process(cur, false, p);
        p += kWaves;
        level();
        if (p >= p_stop) { last_in_alt = true; break; }
        if (p + kWaves < pg1) cur = load_page(p + kWaves);
        process(alt, false, p);
        p += kWaves;
        level();
    }
    if (pg1 == n_pages && p == n_pages - 1) {
        if (last_in_alt) cur = alt;
        process_last(cur, p);
    }
    // ---- wave epilogue (as the bf16 kernel, plus the V offset sum) ---------
    float l_tot = l_run + dpp_f32<kXor1>(l_run);
    l_tot = sum_groups(l_tot);
    float l2_tot = l2_run + dpp_f32<kXor1>(l2_run);
    l2_tot = sum_groups(l2_tot);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float a01 = swap32_sum(acc[0][i], acc[2][i]);
        const float a11 = swap32_sum(acc[1][i], acc[3][i]);
        float t = swap16_sum(a01, a11);
        t += dpp_f32<kRowRor8>(t);
        acc[0][i] = t;
    }
    if ((g & 1) == 0) {
        const int h = (g >> 1) ^ (3 * b2);
        *reinterpret_cast<f32x4 *>(&s_acc[w][h][c * 8]) = f32x4{acc[0][0], acc[0][1], acc[0][2], acc[0][3]};
        *reinterpret_cast<f32x4 *>(&s_acc[w][h][c * 8 + 4]) = f32x4{acc[0][4], acc[0][5], acc[0][6], acc[0][7]};
    }
    if (g == 0 && b0 == 0) {
        s_m[w][hm] = m_run;
        s_l[w][hm] = l_tot;
        s_l2[w][hm] = l2_tot;
    }
    __syncthreads();

    if (tid < kGroup * kD) {
        const int h = tid >> 6;
        const int d = tid & 63;
        float M = kNegBig;
#pragma unroll
        for (int k = 0; k < kWaves; ++k) M = fmaxf(M, s_m[k][h]);
        float Ls = 0.0f, A = 0.0f;
#pragma unroll
        for (int k = 0; k < kWaves; ++k) {
            const float wgt = fast_exp2(s_m[k][h] - M);
            Ls = fmaf(wgt, s_l[k][h], Ls);
            A = fmaf(wgt, fmaf(-128.0f, s_l2[k][h], s_acc[k][h][d]), A);
        }
        const int qh = j * kGroup + h;
        if (n_parts_s == 1) {
            const int64_t o = (static_cast<int64_t>(s) * kHQ + qh) * kD + d;
            const float r = A / Ls;
            if (P.out_fp32) static_cast<float *>(P.out)[o] = r;
            else static_cast<uint16_t *>(P.out)[o] = f32_to_bf16(r);
        } else {
            const int64_t row = (static_cast<int64_t>(s) * kHQ + qh) * P.num_parts + part;
            P.ws_acc[row * kD + d] = A;
            if (d == 0) {
                P.ws_ml[row * 2] = M;
                P.ws_ml[row * 2 + 1] = Ls;
            }
        }
    }
}

constexpr int kDecodeWavesI8 = 8;

hipError_t launch_append_rope_i8(const AppendLaunch &a, hipStream_t stream) {
    if (a.num_seqs == 0) return hipSuccess;
    hipLaunchKernelGGL(k_append_rope_i8, dim3(static_cast<unsigned>(a.num_seqs)), dim3(256), 0, stream,
                       static_cast<uint16_t *>(a.q), static_cast<const uint16_t *>(a.k_new),
                       static_cast<const uint16_t *>(a.v_new), static_cast<uint8_t *>(a.k_pool), a.block_tables,
                       a.lens, a.rope, a.max_blocks, a.num_pages, a.max_pos, a.flags);
    return hipGetLastError();
}

hipError_t launch_quantize_pages_i8(void *pool, const void *k_pool, const void *v_pool, const int32_t *page_ids,
                                    int count, int num_pages, uint32_t *flags, hipStream_t stream) {
    if (count == 0) return hipSuccess;
    hipLaunchKernelGGL(k_quantize_pages_i8, dim3(static_cast<unsigned>(count) * kHKV), dim3(256), 0, stream,
                       static_cast<uint8_t *>(pool), static_cast<const uint16_t *>(k_pool),
                       static_cast<const uint16_t *>(v_pool), page_ids, num_pages, flags);
    return hipGetLastError();
}

hipError_t launch_decode_i8(const DecodeLaunch &d, hipStream_t stream) {
    if (d.num_seqs == 0) return hipSuccess;
    DecodeParams P{};
    P.out = d.out;
    P.q = static_cast<uint16_t *>(d.q);
    P.k_new = static_cast<const uint16_t *>(d.k_new);
    P.v_new = static_cast<const uint16_t *>(d.v_new);
    P.k_pool = static_cast<uint16_t *>(d.k_pool);  // the INT8 tile pool
    P.v_pool = nullptr;
    P.bt = d.block_tables;
    P.lens = d.context_lens;
    P.rope = d.rope;
    P.max_blocks = d.max_blocks;
    P.num_pages = d.num_pages;
    P.max_pos = d.max_pos;
    P.scale_log2 = d.scale * 1.4426950408889634f;
    P.out_fp32 = d.out_fp32;
    P.part_pages = d.part_pages;
    P.num_parts = d.num_parts;
    P.write_q = d.write_q;
    P.ws_ml = d.ws_ml;
    P.ws_acc = d.ws_acc;
    P.flags = d.flags;
    const int64_t blocks = static_cast<int64_t>(d.num_seqs) * kHKV * d.num_parts;
    if (d.fused)
        hipLaunchKernelGGL((k_decode_paged_i8<kDecodeWavesI8, true>), dim3(static_cast<unsigned>(blocks)),
                           dim3(64 * kDecodeWavesI8), 0, stream, P);
    else
        hipLaunchKernelGGL((k_decode_paged_i8<kDecodeWavesI8, false>), dim3(static_cast<unsigned>(blocks)),
                           dim3(64 * kDecodeWavesI8), 0, stream, P);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || d.num_parts == 1) return e;
    if (d.fused)
        hipLaunchKernelGGL((k_decode_merge<true>), dim3(static_cast<unsigned>(d.num_seqs * kHQ)), dim3(64), 0, stream,
                           P);
    else
        hipLaunchKernelGGL((k_decode_merge<false>), dim3(static_cast<unsigned>(d.num_seqs * kHQ)), dim3(64), 0, stream,
                           P);
    return hipGetLastError();
}

}  // namespace pa
