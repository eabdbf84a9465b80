// pa_i8.hip -- INT8 K/V pages: quantising append, bulk quantiser, and paged
// GQA decode over INT8 tiles on f16 MFMAs (optionally fused with the append).
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
//   [0, 1024)     K codes: 16-byte unit 16*((d%32)/8) + t holds dims
//                 8*((d%32)/8) .. +7 (bytes 0-7) and 32 + the same (bytes 8-15)
//                 of token t;
//   [1024, 2048)  V codes: 16-byte unit 16*(t/4) + d%16 holds tokens
//                 4*(t/4) .. +3 of dims d%16 + 16n at bytes 4n .. 4n+3;
//   2048 + 4t     K scale (fp32) of token t;  2112 + 4t  V scale of token t.
// One 16-byte K unit and one V unit are exactly the operands lane u of a wave
// feeds to the MFMAs below, so a page costs each lane two 16-byte loads (plus
// two 16-byte scale loads shared by 16 lanes).
//
// Decode per page and wave (16 tokens of one KV head, its 4 query heads):
//   S^T[16 tokens][16] = K[16 x 64] . Q^T[64 x 16]   two v_mfma_f32_16x16x32_f16,
//       columns 0-3 the 4 query heads, 4-15 zero (lane l holds tokens
//       4(l/16)..+3 of column l%16);
//   O[16][64] += P'[16][16 tokens] . V[16 tokens][64] four v_mfma_f32_16x16x16_f16,
//       whose A operand is exactly the lane's 4 weights from S^T (rows 0-3
//       are the 4 heads; rows 4-15 are never read).
// Codes become f16 values 1152 + code: the byte code ^ 0x80 (= code + 128)
// under an f16 exponent pattern 0x64 is 1024 + code + 128, built with one
// v_perm per pair, exactly.  K codes enter the MFMAs so; the score subtracts
// 1152 * <q, 1> (an MFMA over a key row of 1152s), which is exact up to the
// score's own fp32 rounding.  V codes lose the offset before the MFMA (one
// packed f16 subtraction per pair, exact: the result is the code itself), so
// the output sums carry no 1152 * weight terms: with them, a row of large
// values whose small elements quantise to code 0 would leave fp32 rounding
// noise of the large row's size in those elements.  q enters as f16 after a power-of-two
// scaling (exact) that puts its largest element in [2^14, 2^15).  Weights
// P' = 2^(x - m) * V scale * 2^-ve are fed as an f16 pair hi + lo (two MFMA
// passes, about 22 significant bits, so the weights' rounding stays ~2^-22 of
// |V|); the running sum uses the fp32 2^(x - m).  ve >= 0 is a wave-uniform
// exponent raised lazily, like the running max, whenever a live token's V
// scale exceeds 2^(ve + 7); with 2^(x - m) <= 2^8 the weights then stay below
// 2^15 and hi never overflows f16, for any finite bf16 V row.  Raising ve
// halves the accumulators exactly; the wave epilogue multiplies by 2^ve.
// Online softmax (log2 units, lazy max), wave and partition merges follow the
// bf16 kernel's.  The grid size chooses the cache hint on the code loads and
// whether wave priorities are levelled; neither changes the arithmetic.
#include <math.h>

#include "pa_decode_core.h"
#include "pa_i8_core.h"

namespace pa {

// ------------------------------------------------------------- append ------
// One workgroup (256 threads) per appended token; token = blockIdx.x =
// s * tokens_per_seq + i;
//   decode (prefix_mode == 0): pos = lens[s] - 1   (tokens_per_seq == 1)
//   prefill (prefix_mode == 1): pos = lens[s] + i  (lens holds prefix lengths)
__global__ __launch_bounds__(256) void k_append_rope_i8(uint16_t *__restrict__ q, const uint16_t *__restrict__ k_new,
                                                        const uint16_t *__restrict__ v_new, uint8_t *__restrict__ pool,
                                                        const int32_t *__restrict__ bt, const int32_t *__restrict__ lens,
                                                        const double *__restrict__ rope, int tokens_per_seq,
                                                        int prefix_mode, int max_blocks, int num_pages, int max_pos,
                                                        uint32_t *__restrict__ flags) {
    // Work in units of 4 pairs, as the bf16 append: K is 8 heads x 8 units
    // (threads 0..63), V 8 heads x 8 chunks of 8 dims (threads 64..127), q 32
    // heads x 8 units in place (one per thread).  The rows depend on the token
    // alone, so their loads go out first, beside the length's; the table row
    // waits for the length and the stores for the page id, and a token that
    // fails either check writes nothing.  A row's scale is the maximum |x| over
    // its 64 dims (the 8 lanes of its head) / 127.
    const int tok = blockIdx.x;
    const int s = tok / tokens_per_seq;
    const int i = tok - s * tokens_per_seq;
    const int t = threadIdx.x;
    const int u = t & 7;
    const int i0 = 4 * u;
    const int j = (t >> 3) & (kHKV - 1);
    const int64_t len = lens[s];
    uint2 qa{0u, 0u}, qb{0u, 0u}, ka{0u, 0u}, kb{0u, 0u};
    u32x4 vv{0u, 0u, 0u, 0u};
    uint16_t *qrow = q ? q + (static_cast<int64_t>(tok) * kHQ + (t >> 3)) * kD : nullptr;
    if (q) {
        qa = *reinterpret_cast<const uint2 *>(qrow + i0);
        qb = *reinterpret_cast<const uint2 *>(qrow + i0 + kD / 2);
    }
    const int64_t krow = (static_cast<int64_t>(tok) * kHKV + j) * kD;
    if (t < 64) {
        ka = *reinterpret_cast<const uint2 *>(k_new + krow + i0);
        kb = *reinterpret_cast<const uint2 *>(k_new + krow + i0 + kD / 2);
    } else if (t < 128) {
        vv = reinterpret_cast<const u32x4 *>(v_new + krow)[u];
    }
    const int64_t pos = prefix_mode ? len + i : len - 1;
    const bool bad_len = prefix_mode ? (len < 0) : (len < 1);
    if (bad_len || pos >= static_cast<int64_t>(max_blocks) * kPage || pos >= max_pos) {
        if (t == 0 && flags) atomicOr(flags, kDevErrContextLen);
        return;
    }
    const int page = bt[static_cast<int64_t>(s) * max_blocks + (pos >> 4)];
    const double *cs = rope + pos * kD + 2 * i0;  // pairs i0 .. i0+3 of [32][2]
    const double2 tb[4] = {reinterpret_cast<const double2 *>(cs)[0], reinterpret_cast<const double2 *>(cs)[1],
                           reinterpret_cast<const double2 *>(cs)[2], reinterpret_cast<const double2 *>(cs)[3]};
    if (page < 0 || page >= num_pages) {
        if (t == 0 && flags) atomicOr(flags, kDevErrPageId);
        return;
    }
    const int slot = static_cast<int>(pos & (kPage - 1));
    uint8_t *tile = pool + (static_cast<int64_t>(page) * kHKV + j) * kI8Tile;
    if (t < 64) {
        // K: rotate, round to bf16 (the stored row of the bf16 format), quantise
        uint2 lo, hi;
        rope4(ka, kb, tb, lo, hi);
        const float y[8] = {bf16_lo(lo.x), bf16_hi(lo.x), bf16_lo(lo.y), bf16_hi(lo.y),
                            bf16_lo(hi.x), bf16_hi(hi.x), bf16_lo(hi.y), bf16_hi(hi.y)};
        float a = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) a = fmaxf(a, fabsf(y[k]));
        const float sc = max_lanes8(a) / 127.0f;
        uint32_t w0 = 0, w1 = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            w0 |= (static_cast<uint32_t>(quant_code(y[k], sc)) & 0xFFu) << (8 * k);
            w1 |= (static_cast<uint32_t>(quant_code(y[4 + k], sc)) & 0xFFu) << (8 * k);
        }
        // dims i0 .. i0+3 and i0+32 .. i0+35 are 4 consecutive bytes each
        *reinterpret_cast<uint32_t *>(tile + i8_kpos(slot, i0)) = w0;
        *reinterpret_cast<uint32_t *>(tile + i8_kpos(slot, i0 + 32)) = w1;
        if (u == 0) *reinterpret_cast<float *>(tile + kI8KScOff + 4 * slot) = sc;
    } else if (t < 128) {
        // V: dims 8u .. 8u+7 verbatim from bf16, quantised with the row's scale
        const uint32_t wd[4] = {vv.x, vv.y, vv.z, vv.w};
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
#pragma unroll
        for (int k = 0; k < 8; ++k) tile[i8_vpos(slot, 8 * u + k)] = static_cast<uint8_t>(quant_code(x[k], sc));
        if (u == 0) *reinterpret_cast<float *>(tile + kI8VScOff + 4 * slot) = sc;
    }
    if (q) {
        uint2 lo, hi;
        rope4(qa, qb, tb, lo, hi);
        *reinterpret_cast<uint2 *>(qrow + i0) = lo;
        *reinterpret_cast<uint2 *>(qrow + i0 + kD / 2) = hi;
    }
}

// --------------------------------------------------------- bulk quantiser --
// One workgroup (256 threads) per (listed page, KV head): thread t quantises
// chunk c = t%8 (dims 8c..8c+7) of row r = t/8 (rows 0-15: K slots, 16-31: V slots).
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
    uint8_t *tile = pool + (static_cast<int64_t>(page) * kHKV + j) * kI8Tile;
    if (is_v) {
        // V: the 8 dims of this chunk lie in 8 different 16-byte units
#pragma unroll
        for (int k = 0; k < 8; ++k) tile[i8_vpos(slot, c * 8 + k)] = static_cast<uint8_t>(quant_code(x[k], sc));
    } else {
        // K: dims 8c..8c+7 are 8 consecutive bytes of one unit
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            lo |= (static_cast<uint32_t>(quant_code(x[k], sc)) & 0xFFu) << (8 * k);
            hi |= (static_cast<uint32_t>(quant_code(x[4 + k], sc)) & 0xFFu) << (8 * k);
        }
        *reinterpret_cast<uint2 *>(tile + i8_kpos(slot, c * 8)) = make_uint2(lo, hi);
    }
    if (c == 0) *reinterpret_cast<float *>(tile + (is_v ? kI8VScOff : kI8KScOff) + 4 * slot) = sc;
}

// ------------------------------------------------------------- decode ------
// Workgroups and page ids as in the bf16 kernel (pa_decode.hip): one
// workgroup of kWaves waves per (sequence, KV head, context partition), pages
// dealt round-robin to the waves, the next page's loads always in flight.
// The pool travels in DecodeParams::k_pool (v_pool is unused).

// kLevel: the wave priority starts high and steps down as the wave's pages run
// out (as in the bf16 kernel).  The s_setprio instructions also constrain how
// the compiler schedules the page loop, so the form without them is kept for
// grids where levelling does not pay (see launch_decode_i8).
template <int kWaves, bool kFused, bool kNt, bool kLevel, class Ord>
__global__ __launch_bounds__(64 * kWaves, 4) void k_decode_paged_i8(DecodeParams P, Ord order) {
    constexpr int kThreads = 64 * kWaves;
    static_assert(kMaxPartPages <= 64 * kWaves, "one page id per lane must cover a partition");
    const WgCoords wc = wg_coords(order, P.num_parts);
    const int part = wc.part;
    const int j = wc.j;
    // A device order entry outside the batch is never used as an index: the
    // workgroup reads sequence 0's rows instead (always valid to read) and
    // leaves at the validation below, having written nothing.
    const bool order_ok = order_entry_ok(order, wc.s);
    const int s = order_ok ? wc.s : 0;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    if (kLevel) __builtin_amdgcn_s_setprio(3);
    const uint8_t *pool = reinterpret_cast<const uint8_t *>(P.k_pool);

    __shared__ int s_app_page;
    __shared__ float s_m[kWaves][kGroup];
    __shared__ float s_l[kWaves][kGroup];
    __shared__ float s_acc[kWaves][kGroup][kD];
    __shared__ __align__(16) uint16_t s_q[kGroup][kD];  // rotated q (fused)
    __shared__ __align__(16) int8_t s_nk[kD];           // appended K row codes (fused)
    __shared__ __align__(16) int8_t s_nv[kD];           // appended V row codes (fused)
    __shared__ float s_nsc[2];                          // appended row scales (K, V)

    // ---- lane roles: column hh of the MFMAs (query head hh < 4, K token hh),
    // quarter qd (K dims 8qd..+7 and 32+8qd..+7; V tokens and scales 4qd..+3)
    const int hh = lane & 15;
    const int qd = lane >> 4;
    const bool head_lane = hh < kGroup;

    const int pg0 = part * P.part_pages;
    const int slice = min(P.part_pages, P.max_blocks - pg0);
    const int32_t *bt_row = P.bt + static_cast<int64_t>(s) * P.max_blocks;
    const int L = P.lens[s];
    const int wu = __builtin_amdgcn_readfirstlane(w);
    // The wave's first two pages are issued in the prologue: the prologue's
    // arithmetic (q rotation and scaling, quantising the appended rows, a
    // barrier) then runs under two pages of loads per wave instead of one.
    // An id past the table or outside the pool reads page 0 instead; such a
    // page is never used.
    const int first_id = wu < slice ? bt_row[pg0 + wu] : -1;
    const int second_id = wu + kWaves < slice ? bt_row[pg0 + wu + kWaves] : -1;
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
    // q chunks of this lane (non-fused: straight from q; head lanes only, the
    // other columns are zero): dims 8qd..8qd+7 and 32+8qd..+7 of head hh
    u32x4 qraw0 = {0u, 0u, 0u, 0u}, qraw1 = {0u, 0u, 0u, 0u};
    if (!kFused) {
        const uint16_t *qh = P.q + qrow0 + min(hh, kGroup - 1) * kD;
        const u32x4 a = *reinterpret_cast<const u32x4 *>(qh + 8 * qd);
        const u32x4 b = *reinterpret_cast<const u32x4 *>(qh + 32 + 8 * qd);
        qraw0 = head_lane ? a : qraw0;
        qraw1 = head_lane ? b : qraw1;
    }
    __builtin_amdgcn_sched_barrier(0);
    double co = 0.0, si = 0.0;
    if (kFused) {
        const int pos_c = min(max(pos, 0), P.max_pos - 1);
        const double *cs = P.rope + static_cast<int64_t>(pos_c) * kD + 2 * pr;
        co = cs[0];
        si = cs[1];
    }
    __builtin_amdgcn_sched_barrier(0);
    const int64_t tile_j = static_cast<int64_t>(j) * kI8Tile;
    auto load_tile = [&](int page_id) {
        const uint8_t *t = pool + static_cast<int64_t>(page_id) * kPageBytesI8 + tile_j;
        I8Page r;
        // kNt: the 2 KiB of codes are read with the non-temporal hint, the
        // scales without (the host picks it by grid size; see launch_decode_i8).
        if (kNt) {
            r.k = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(t + lane * 16));
            r.v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(t + kI8VOff + lane * 16));
        } else {
            r.k = *reinterpret_cast<const u32x4 *>(t + lane * 16);
            r.v = *reinterpret_cast<const u32x4 *>(t + kI8VOff + lane * 16);
        }
        r.ks = *reinterpret_cast<const f32x4 *>(t + kI8KScOff + qd * 16);
        r.vs = *reinterpret_cast<const f32x4 *>(t + kI8VScOff + qd * 16);
        return r;
    };
    I8Page cur = load_tile(first_id >= 0 && first_id < P.num_pages ? first_id : 0);
    I8Page alt = load_tile(second_id >= 0 && second_id < P.num_pages ? second_id : 0);
    __builtin_amdgcn_sched_barrier(0);

    // fused: rotate q into LDS (threads 0..127); wave 2 rotates the new K row
    // (lanes 0-31, pair pr) and takes the new V row (lanes 32-63, elements
    // 2pr, 2pr+1), then quantises both rows exactly as k_append_rope_i8 does.
    if (kFused && tid < 192) {
        uint16_t r0 = 0, r1 = 0;
        if (tid < 160) rope_pair_bf16(x0, x1, co, si, r0, r1);
        if (tid < 128) {
            s_q[tid >> 5][pr] = r0;
            s_q[tid >> 5][pr + 32] = r1;
        } else {
            const bool is_k = tid < 160;
            const float e0 = is_k ? bf16_to_f32(r0) : bf16_lo(vword);
            const float e1 = is_k ? bf16_to_f32(r1) : bf16_hi(vword);
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
    if (!order_ok) {  // uniform over the workgroup
        if (tid == 0 && P.flags) atomicOr(P.flags, kDevErrDispatchOrder);
        return;
    }
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
    const int sl = pos & (kPage - 1);  // slot of the appended token (fused)
    if (kFused) {
        if (head_lane) {
            qraw0 = *reinterpret_cast<const u32x4 *>(&s_q[hh][8 * qd]);
            qraw1 = *reinterpret_cast<const u32x4 *>(&s_q[hh][32 + 8 * qd]);
        }
    }

    // ---- q as the f16 B operand of Q.K^T, scaled by 2^(15 - e) so that its
    // largest element (over the 4 heads: every wave finds the same e) lies in
    // [2^14, 2^15); the score then carries 2^(e - 15), folded into the scale.
    float qf[16];
    {
        const uint32_t a[8] = {qraw0.x, qraw0.y, qraw0.z, qraw0.w, qraw1.x, qraw1.y, qraw1.z, qraw1.w};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            qf[2 * k] = bf16_lo(a[k]);
            qf[2 * k + 1] = bf16_hi(a[k]);
        }
    }
    float qmax = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) qmax = fmaxf(qmax, fabsf(qf[k]));
    qmax = max_groups(max_lanes8(qmax));
    int qe = 0;
    if (qmax > 0.0f) (void)frexpf(qmax, &qe);  // qmax in [2^(qe-1), 2^qe)
    const int qshift = min(15 - qe, 126);       // (kept a finite fp32 power of two)
    const float qscale = ldexpf(1.0f, qshift);
    half8 qb0, qb1;
    {
        uint32_t h[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) h[k] = pack_f16x2(qf[2 * k] * qscale, qf[2 * k + 1] * qscale);
        qb0 = __builtin_bit_cast(half8, u32x4{h[0], h[1], h[2], h[3]});
        qb1 = __builtin_bit_cast(half8, u32x4{h[4], h[5], h[6], h[7]});
    }
    // 1152 * <q', 1> for column hh: the offset the code encoding adds to a score
    float corr;
    {
        const uint32_t c1152 = 0x64806480u;  // f16 1152.0 twice
        const half8 k1152 = __builtin_bit_cast(half8, u32x4{c1152, c1152, c1152, c1152});
        f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
        z = __builtin_amdgcn_mfma_f32_16x16x32_f16(k1152, qb0, z, 0, 0, 0);
        z = __builtin_amdgcn_mfma_f32_16x16x32_f16(k1152, qb1, z, 0, 0, 0);
        corr = z[0];
    }
    const float sc_log2 = P.scale_log2 * ldexpf(1.0f, -qshift);

    int p = pg0 + wu;

    float m_run = kNegBig;  // running max (log2 units) of head hh
    float l_run = 0.0f;     // sum of 2^(x - m) over the lane's tokens
    // acc[n]: O[head 4qd + r][dim 16n + hh] (rows 0-3, lanes 0-15, are the heads)
    f32x4 acc[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // V scales enter the weights as vs * 2^-ve (wave-uniform ve >= 0, raised
    // lazily): every live scale seen so far is below vlim = 2^(ve + 7).
    int ve = 0;
    float vmul = 1.0f;                                       // 2^-ve
    uint32_t vlim_bits = __builtin_bit_cast(uint32_t, 128.0f);  // 2^(ve + 7), as bits

    auto process = [&](const I8Page &r, bool last, int p) {
        // scores of tokens 4qd + i (i < 4) for column hh
        f32x4 st = {0.0f, 0.0f, 0.0f, 0.0f};
        st = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes8_to_f16(r.k.x, r.k.y), qb0, st, 0, 0, 0);
        st = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes8_to_f16(r.k.z, r.k.w), qb1, st, 0, 0, 0);
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = (st[i] - corr) * (r.ks[i] * sc_log2);
        bool dead[4] = {false, false, false, false};
        if (last) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                dead[i] = p * kPage + 4 * qd + i >= L;
                if (dead[i]) x[i] = -INFINITY;
            }
        }
        // lazy running max of head hh (uniform over the 4 lanes of column hh)
        const float xm = max_quarters(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
        const bool need = (xm > m_run + kRescaleLog2) && head_lane;
        // V scales of the live tokens (a dead slot's scale may be anything);
        // vneed: one of them exceeds 2^(ve + 7).  The scales are >= 0, so
        // their bit patterns order as unsigned integers the way the values do
        // (an integer max needs no NaN-quieting of its loaded operands).
        float vsl[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) vsl[i] = (last && dead[i]) ? 0.0f : r.vs[i];
        const uint32_t vmx = max(max(__builtin_bit_cast(uint32_t, vsl[0]), __builtin_bit_cast(uint32_t, vsl[1])),
                                 max(__builtin_bit_cast(uint32_t, vsl[2]), __builtin_bit_cast(uint32_t, vsl[3])));
        const bool vneed = vmx > vlim_bits;
        // one ballot and one branch per page for both rare events
        if (__builtin_amdgcn_ballot_w64(need || vneed)) {
            if (__builtin_amdgcn_ballot_w64(need)) {
                const float mn = need ? xm : m_run;
                const float f = fast_exp2(m_run - mn);
                m_run = mn;
                l_run *= f;
                // accumulator row i of lanes 0-15 is head i: its factor is lane i's
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float fi = lane_value(f, i);
#pragma unroll
                    for (int n = 0; n < 4; ++n) acc[n][i] *= fi;
                }
            }
            if (__builtin_amdgcn_ballot_w64(vneed)) {
                // raise ve so that the page's largest scale times 2^-ve < 2^7
                // (every lane of a quarter holds the same 4 scales, so the max
                // over the quarters is the page's, the same in every lane)
                const float wmx = __builtin_bit_cast(
                    float, __builtin_amdgcn_readfirstlane(
                               __builtin_bit_cast(int, max_quarters(__builtin_bit_cast(float, vmx)))));
                int e = 0;
                (void)frexpf(wmx, &e);  // wmx in [2^(e-1), 2^e), e >= ve + 8
                const int ve_new = e - 7;
                if (ve_new > ve) {     // (not for a NaN scale, which the contract excludes)
                    const float f = ldexpf(1.0f, ve - ve_new);
#pragma unroll
                    for (int n = 0; n < 4; ++n)
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[n][i] *= f;
                    ve = ve_new;
                    vmul = ldexpf(1.0f, -ve);
                    vlim_bits = __builtin_bit_cast(uint32_t, ldexpf(1.0f, ve + 7));
                }
            }
        }
        float pw[4], pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pw[i] = fast_exp2(x[i] - m_run);
            pv[i] = (last && dead[i]) ? 0.0f : pw[i] * (vsl[i] * vmul);
        }
        l_run += (pw[0] + pw[1]) + (pw[2] + pw[3]);
        // weights as an f16 pair hi + lo (lo = the rounding remainder of hi);
        // the lo products only where the output needs them (kHiOnlyVScaleBits)
        const uint32_t h01 = pack_f16x2(pv[0], pv[1]);
        const uint32_t h23 = pack_f16x2(pv[2], pv[3]);
        const half4 ph = __builtin_bit_cast(half4, u32x2{h01, h23});
        const half4 vb[4] = {codes4_to_f16_signed(r.v.x), codes4_to_f16_signed(r.v.y),
                             codes4_to_f16_signed(r.v.z), codes4_to_f16_signed(r.v.w)};
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[n] = __builtin_amdgcn_mfma_f32_16x16x16f16(ph, vb[n], acc[n], 0, 0, 0);
        if (P.out_fp32 || __builtin_amdgcn_ballot_w64(vmx > kHiOnlyVScaleBits)) {
            const half2v e01 = __builtin_bit_cast(half2v, h01), e23 = __builtin_bit_cast(half2v, h23);
            const uint32_t l01 = pack_f16x2(pv[0] - static_cast<float>(e01[0]), pv[1] - static_cast<float>(e01[1]));
            const uint32_t l23 = pack_f16x2(pv[2] - static_cast<float>(e23[0]), pv[3] - static_cast<float>(e23[1]));
            const half4 pl = __builtin_bit_cast(half4, u32x2{l01, l23});
#pragma unroll
            for (int n = 0; n < 4; ++n) acc[n] = __builtin_amdgcn_mfma_f32_16x16x16f16(pl, vb[n], acc[n], 0, 0, 0);
        }
    };
    auto process_last = [&](I8Page r, int p) {
        if (kFused) {  // patch the appended token's codes and scales into the registers
            if (hh == sl) {
                const uint2 a = *reinterpret_cast<const uint2 *>(&s_nk[8 * qd]);
                const uint2 b = *reinterpret_cast<const uint2 *>(&s_nk[32 + 8 * qd]);
                r.k = u32x4{a.x, a.y, b.x, b.y};
            }
            if ((sl >> 2) == qd) {
                const int sh = 8 * (sl & 3);
                const uint32_t keep = ~(0xFFu << sh);
                r.v.x = (r.v.x & keep) | (static_cast<uint32_t>(static_cast<uint8_t>(s_nv[hh])) << sh);
                r.v.y = (r.v.y & keep) | (static_cast<uint32_t>(static_cast<uint8_t>(s_nv[16 + hh])) << sh);
                r.v.z = (r.v.z & keep) | (static_cast<uint32_t>(static_cast<uint8_t>(s_nv[32 + hh])) << sh);
                r.v.w = (r.v.w & keep) | (static_cast<uint32_t>(static_cast<uint8_t>(s_nv[48 + hh])) << sh);
                r.ks[sl & 3] = s_nsc[0];
                r.vs[sl & 3] = s_nsc[1];
            }
        }
        process(r, true, p);
    };
    auto load_page = [&](int p) {
        return load_tile(__builtin_amdgcn_readlane(my_id, (p - pg0 - wu) / kWaves));
    };
    const int p_stop = (pg1 == n_pages) ? n_pages - 1 : pg1;
    const int span = pg1 - pg0;
    auto level = [&]() {
        if (!kLevel) return;
        const int done16 = 16 * (p - pg0);
        if (done16 >= 15 * span) __builtin_amdgcn_s_setprio(0);
        else if (done16 >= 13 * span) __builtin_amdgcn_s_setprio(1);
        else if (done16 >= 10 * span) __builtin_amdgcn_s_setprio(2);
    };
    // At the top of each step cur holds page p and alt page p + kWaves, both
    // issued; a page is consumed before the one after next is issued, so one
    // page is in flight while another is processed, as in the bf16 kernel.
    // Steady state: both loads of a double step are known to be needed, so they
    // are issued unconditionally (a load under a branch makes the compiler's
    // wait counting drain every outstanding load each step).
    while (p + kWaves < p_stop && p + 3 * kWaves < pg1) {
        process(cur, false, p);
        p += kWaves;
        level();
        cur = load_page(p + kWaves);
        process(alt, false, p);
        p += kWaves;
        level();
        alt = load_page(p + kWaves);
    }
    // The wave's last full pages, one per step.
    while (p < p_stop) {
        process(cur, false, p);
        p += kWaves;
        level();
        cur = alt;
        if (p + kWaves < pg1) alt = load_page(p + kWaves);
    }
    if (pg1 == n_pages && p == n_pages - 1) process_last(cur, p);  // the sequence's last page
    // ---- wave epilogue ---------------------------------------------------------
    const float l_tot = sum_quarters(l_run);
    if (lane < 16) {  // O x 2^ve, per head
        const float vback = ldexpf(1.0f, ve);
#pragma unroll
        for (int n = 0; n < 4; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i) s_acc[w][i][16 * n + hh] = acc[n][i] * vback;
    }
    if (lane < kGroup) {
        s_m[w][lane] = m_run;
        s_l[w][lane] = l_tot;
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
            A = fmaf(wgt, s_acc[k][h][d], A);
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
    if (kFused) {
        // The appended row and the rotated q are stored last: nothing in this
        // kernel reads them back (the last page's registers were patched from
        // LDS), and stores issued ahead of the page loads would hold up the
        // wave's first wait for page data (vector memory completes in order).
        if (pg1 == n_pages) {  // append the quantised row (last partition only)
            uint8_t *tw = const_cast<uint8_t *>(pool) + static_cast<int64_t>(s_app_page) * kPageBytesI8 + tile_j;
            if (tid < 4) {  // K unit 16*tid + sl: dims 8tid..+7 and 32+8tid..+7
                const uint2 a = *reinterpret_cast<const uint2 *>(&s_nk[8 * tid]);
                const uint2 b = *reinterpret_cast<const uint2 *>(&s_nk[32 + 8 * tid]);
                *reinterpret_cast<u32x4 *>(tw + (16 * tid + sl) * 16) = u32x4{a.x, a.y, b.x, b.y};
            } else if (tid >= 64 && tid < 128) {
                const int d = tid - 64;
                tw[i8_vpos(sl, d)] = static_cast<uint8_t>(s_nv[d]);
            } else if (tid == 4) {
                *reinterpret_cast<float *>(tw + kI8KScOff + 4 * sl) = s_nsc[0];
                *reinterpret_cast<float *>(tw + kI8VScOff + 4 * sl) = s_nsc[1];
            }
        }
        if (P.write_q && n_parts_s == 1 && tid >= 192 && tid < 224)
            *reinterpret_cast<u32x4 *>(P.q + qrow0 + (tid - 192) * 8) =
                *reinterpret_cast<const u32x4 *>(&s_q[0][(tid - 192) * 8]);
    }
}

constexpr int kDecodeWavesI8 = 8;

hipError_t launch_append_rope_i8(const AppendLaunch &a, hipStream_t stream) {
    const int64_t tokens = static_cast<int64_t>(a.num_seqs) * a.tokens_per_seq;
    if (tokens == 0) return hipSuccess;
    hipLaunchKernelGGL(k_append_rope_i8, dim3(static_cast<unsigned>(tokens)), dim3(256), 0, stream,
                       static_cast<uint16_t *>(a.q), static_cast<const uint16_t *>(a.k_new),
                       static_cast<const uint16_t *>(a.v_new), static_cast<uint8_t *>(a.k_pool), a.block_tables,
                       a.lens, a.rope, a.tokens_per_seq, a.prefix_mode, a.max_blocks, a.num_pages, a.max_pos,
                       a.flags);
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
    // The non-temporal hint on the codes, by grid size, as measured on MI355X
    // (fused step): from 128 workgroups up (uniform 2048-token batches of 16 to
    // 128 sequences, 256 x 512 tokens, the ragged 256-sequence batch) it is
    // 0-10 % faster, never slower; with 64 workgroups (few long, latency-bound
    // streams) it is 14 % slower.  Hinting the scales as well gains nothing.
    // Priority levelling pays up to 1024 workgroups (0.5 % at 512); above that
    // the form without it ran the ragged 256-sequence batch 4.5 % faster.
    const bool nt = blocks >= kNtMinBlocks;
    const bool level = blocks <= kPrioMaxBlocksI8;
    const dim3 grid(static_cast<unsigned>(blocks)), wg(64 * kDecodeWavesI8);
    auto go = [&](auto order) {
        using Ord = decltype(order);
        constexpr int W = kDecodeWavesI8;
        if (d.fused) {
            if (!nt) hipLaunchKernelGGL((k_decode_paged_i8<W, true, false, true, Ord>), grid, wg, 0, stream, P, order);
            else if (level) hipLaunchKernelGGL((k_decode_paged_i8<W, true, true, true, Ord>), grid, wg, 0, stream, P, order);
            else hipLaunchKernelGGL((k_decode_paged_i8<W, true, true, false, Ord>), grid, wg, 0, stream, P, order);
        } else {
            if (!nt) hipLaunchKernelGGL((k_decode_paged_i8<W, false, false, true, Ord>), grid, wg, 0, stream, P, order);
            else if (level) hipLaunchKernelGGL((k_decode_paged_i8<W, false, true, true, Ord>), grid, wg, 0, stream, P, order);
            else hipLaunchKernelGGL((k_decode_paged_i8<W, false, true, false, Ord>), grid, wg, 0, stream, P, order);
        }
    };
    if (d.order) go(make_dispatch_order(d.order, d.num_seqs, d.num_parts));
    else if (d.order_dev) go(DeviceOrder{d.order_dev, d.num_seqs});
    else go(DispatchOrder<false>{});
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
