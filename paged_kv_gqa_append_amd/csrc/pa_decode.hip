// pa_decode.hip -- split-context paged GQA decode attention for gfx950,
// optionally fused with the KV append + RoPE of the token being decoded.
//
// What is computed: for every sequence s and query head h (KV head j = h/4),
// softmax(scale * q K^T) V over the sequence's L tokens, where K/V rows are
// found through the sequence's block table (samir-vllm article, section
// "Gestion de la KV cache ...": attention reads only the sequence's own
// pages, accumulates weighted V, concatenates nothing and stores no scores).
// The fused variant first appends the new token at position L-1 exactly as
// pa_append_kv_rope does (same fp64 rotation, same bf16 rounding) and rotates
// q in registers, so its results are bitwise those of append-then-decode.
//
// Work decomposition
//   A workgroup of kWaves waves serves one (sequence, KV head, context
//   partition): the 4 query heads of that KV head share every K/V byte, which
//   is read from HBM exactly once.  Waves take the partition's pages
//   round-robin, one 16-token page (a contiguous 2 KiB K tile and 2 KiB V tile
//   of this KV head) per step, with the next page's loads in flight.
//
//   Lanes form 8 groups of 8 (lane = 8g + c).  Every lane holds, for tokens
//   g and g+8 of the page, the 16-byte chunk c*8..c*8+7 of K and of V.
//   q.K: each lane forms the partial dot products of its chunk for the 8
//   (token, head) pairs of its group, then a 3-step reduce-scatter over the 8
//   lanes (DPP lane permutes) leaves every lane with ONE complete score.  For
//   that to need no selects, lane c keeps its K tokens and q heads in an
//   order permuted by its lane bits (tokens by b0^b2, heads by the mask
//   hm(c)): lane c ends up owning pair (token half b0^b2, head hm(c)).
//   Softmax: online, in log2 units (scale*log2 e folded in), with a running
//   max per head that is uniform across the wave and only raised when a score
//   exceeds it by more than 2^8 (lazy rescale; the final division uses sums
//   taken with the same max, so the result is exact in exact arithmetic).
//   Each lane exponentiates only its own score; 9 DPP moves broadcast the 8
//   weights of the group back to all its lanes, whose V chunk slots and
//   accumulator head slots are permuted to match (V tokens by b2, heads by 3*b2).
//   Epilogue: plain sums across the 8 lane groups (one running max per wave),
//   then an LDS merge of the waves (each with its own max).  A sequence whose
//   context fits one partition writes its output directly; longer ones leave
//   (max, sum, acc[64]) per head and partition in the workspace for
//   k_decode_merge.
//
// Page loads come in two forms, chosen by grid size (see launch_decode).
// Whole rows: each lane loads its chunk of token g, then of token g + 8, so one
// load instruction reads 8 whole 128-byte token rows; both tiles carry the
// non-temporal hint, and the lane's slot order above is made with per-lane
// selects where the page is consumed.  Slot order: each lane loads straight
// into its slots, so a load instruction reads half of each of the tile's 16
// rows; no hint, no selects.  The slots hold the same values either way.
//
// The partition size depends on nothing but a constant, so a sequence's
// output is bitwise independent of the batch around it.  The one thing the
// grid size does choose, the load form, changes no arithmetic.
#include <math.h>
#include <stdlib.h>

#include "pa_decode_core.h"

namespace pa {

template <int kWaves, bool kFused, bool kRows, class Ord>
__global__ __launch_bounds__(64 * kWaves, 4) void k_decode_paged(DecodeParams P, Ord order) {
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
    // Issue priority starts high and steps down as the wave's pages run out
    // (see the main loop): two workgroups share each CU, and age-ordered
    // arbitration alone lets the older one finish far ahead of the younger,
    // which then streams alone with half the loads in flight.  Launches given
    // a dispatch order (longest first, for ragged batches) run faster without
    // it (ragged 256-sequence batch, device order: 59.0 -> 58.1 us), launches
    // in slot order with it (the same batch 62.9 -> 61.5 us, batch 64 44.2 ->
    // 44.0 us), so only those level.
    constexpr bool kLevel = std::is_same_v<Ord, DispatchOrder<false>>;
    if (kLevel) __builtin_amdgcn_s_setprio(3);

    __shared__ int s_app_page;  // fused: page of the appended token (last partition)
    __shared__ float s_m[kWaves][kGroup];
    __shared__ float s_l[kWaves][kGroup];
    __shared__ float s_acc[kWaves][kGroup][kD];
    __shared__ __align__(16) uint16_t s_q[kGroup][kD];  // rotated q of the 4 heads (fused)
    __shared__ __align__(16) uint16_t s_newk[kD];       // appended K row, rotated (fused)
    __shared__ __align__(16) uint16_t s_newv[kD];       // appended V row (fused)

    // ---- lane roles --------------------------------------------------------
    const int g = lane >> 3;
    const int c = lane & 7;
    const int b0 = c & 1, b1 = (c >> 1) & 1, b2 = c >> 2;
    const int t0 = b0 ^ b2;                    // token half of K slot A
    const int hm = ((b1 ^ b2) << 1) | b2;      // q slot m holds head m ^ hm
    // Element offsets in a tile of the lane's first K and V load; bit 9 (8
    // tokens x 64) selects the token half, flipped for the second load.  Whole
    // rows: token g (offset 8 * lane) for both.  Slot order: K slot A holds
    // token half t0, V slot u token half u ^ b2.
    const uint32_t offK = (g + (kRows ? 0 : 8 * t0)) * kD + c * 8;
    const uint32_t offV = (g + (kRows ? 0 : 8 * b2)) * kD + c * 8;
    // whole rows: the loads hold the halves in order and the slots swap them
    const bool swapK = kRows && t0, swapV = kRows && b2;

    // ---- prologue loads, in the order they must complete --------------------
    // Vector loads complete in issue order (one counter), so the small loads
    // the prologue waits for go out first and the first page's K/V loads last:
    // waiting for a small load then never waits for page data.
    const int pg0 = part * P.part_pages;
    const int slice = min(P.part_pages, P.max_blocks - pg0);
    const int32_t *bt_row = P.bt + static_cast<int64_t>(s) * P.max_blocks;
    const int L = P.lens[s];
    const int wu = __builtin_amdgcn_readfirstlane(w);
    // Wave w takes pages pg0+w, pg0+w+kWaves, ...; lane i of the wave holds the
    // id of its i-th page (at most 16 per wave), read back with readlane in the
    // loop, so no page id goes through LDS.  The first id is also read by a
    // scalar load, so that page's loads go out as early as possible; any id
    // inside the pool is safe to read, and a page that turns out not to be
    // needed (or an id that fails validation below) is simply never used.
    const int first_id = wu < slice ? bt_row[pg0 + wu] : -1;
    const int my_idx = wu + kWaves * lane;  // partition-relative page of this lane's id
    const int my_id = bt_row[pg0 + min(my_idx, slice - 1)];
    const int64_t qrow0 = (static_cast<int64_t>(s) * kHQ + j * kGroup) * kD;
    const int64_t nrow = (static_cast<int64_t>(s) * kHKV + j) * kD;
    const int pos = L - 1;
    const int pr = tid & 31;
    // fused: raw (i, i+32) pairs of the 4 q heads (threads 0..127), of the
    // appended K row (128..159), and a word of the appended V row (160..191)
    // (every load here is unconditional, from an address that is always valid,
    // so the compiler can count outstanding loads exactly: a load under a branch
    // makes it wait for all of them, page data included)
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
    // fused: the (cos, sin) of pair pr at position L-1, clamped into the table
    // (a bad L is rejected below, before anything computed from it is used)
    double co = 0.0, si = 0.0;
    if (kFused) {
        const int pos_c = min(max(pos, 0), P.max_pos - 1);
        const double *cs = P.rope + static_cast<int64_t>(pos_c) * kD + 2 * pr;
        co = cs[0];
        si = cs[1];
    }
    __builtin_amdgcn_sched_barrier(0);
    const int64_t tile_j = static_cast<int64_t>(j) * kTile;
    auto load_tile = [&](int page_id) {
        // the page id is uniform: keep the tile base in scalar registers
        const int64_t base = static_cast<int64_t>(page_id) * kPageElems + tile_j;
        const uint16_t *kt = P.k_pool + base;
        const uint16_t *vt = P.v_pool + base;
        KVRegs r;
        if (kRows) {
            r.k0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kt + offK));
            r.k1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kt + (offK ^ 512u)));
            r.v0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(vt + offV));
            r.v1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(vt + (offV ^ 512u)));
        } else {
            r.k0 = *reinterpret_cast<const u32x4 *>(kt + offK);
            r.k1 = *reinterpret_cast<const u32x4 *>(kt + (offK ^ 512u));
            r.v0 = *reinterpret_cast<const u32x4 *>(vt + offV);
            r.v1 = *reinterpret_cast<const u32x4 *>(vt + (offV ^ 512u));
        }
        return r;
    };
    // an id outside the pool reads page 0 instead; such a sequence fails validation
    KVRegs cur = load_tile(first_id >= 0 && first_id < P.num_pages ? first_id : 0);
    __builtin_amdgcn_sched_barrier(0);

    // fused: rotation once per workgroup, one pair per thread, into LDS (the
    // rope_pair_bf16 of k_append_rope)
    if (kFused && tid < 192) {
        if (tid < 160) {
            uint16_t *dst = tid < 128 ? &s_q[tid >> 5][0] : &s_newk[0];
            rope_pair_bf16(x0, x1, co, si, dst[pr], dst[pr + 32]);
        } else {
            reinterpret_cast<uint32_t *>(s_newv)[pr] = vword;
        }
    }

    // ---- validation of device-resident lengths and page ids ---------------
    bool len_ok = (L >= 1) && (L <= P.max_blocks * kPage);
    if (kFused) len_ok = len_ok && (L - 1 < P.max_pos);
    const int n_pages = len_ok ? (L + kPage - 1) / kPage : 0;
    const int n_parts_s = (n_pages + P.part_pages - 1) / P.part_pages;
    const int pg1 = min(pg0 + P.part_pages, n_pages);
    const int bad = (my_idx < slice) && (pg0 + my_idx < n_pages) && (my_id < 0 || my_id >= P.num_pages);
    if (kFused) {  // the lane holding the appended token's page publishes it
        const int rel = (pos >> 4) - pg0;
        if (len_ok && rel >= 0 && rel == my_idx && rel < slice) s_app_page = my_id;
    }
    bool ok = len_ok && (__syncthreads_or(bad) == 0);
    if (!order_ok) {  // uniform over the workgroup
        if (tid == 0 && P.flags) atomicOr(P.flags, kDevErrDispatchOrder);
        return;
    }
    if (ok && n_parts_s > 1) {  // long context: the whole row decides, as in every partition
        int bad_row = 0;
        for (int b = tid; b < n_pages; b += kThreads) {
            const int pid = bt_row[b];
            bad_row |= (pid < 0) | (pid >= P.num_pages);
        }
        ok = __syncthreads_or(bad_row) == 0;
    }
    if (!ok) {
        if (part == 0 && tid < kGroup * kD) {  // zero this KV head's 4 output rows, flag once
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
    }
    auto load_page = [&](int p) {
        return load_tile(__builtin_amdgcn_readlane(my_id, (p - pg0 - wu) / kWaves));
    };
    int p = pg0 + wu;

    // ---- per-lane softmax state ----------------------------------------------
    float m_run = kNegBig;  // running max (log2 units) of head hm, uniform over the wave
    float l_run = 0.0f;     // sum of this lane's own weights (pair token t0, head hm)
    float acc[kGroup][8];   // slot e = head e ^ (3*b2), elements c*8 .. c*8+7
#pragma unroll
    for (int e = 0; e < kGroup; ++e)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[e][i] = 0.0f;

    // One page.  process_full: any page but the sequence's last; process_last: the
    // last page, which may be partly empty and, when fused, holds the appended token
    // (its dead slots may hold anything, NaN included, so they are selected out).
    // The slot selects of the whole-row form sit here, where the page is
    // consumed: placed after the loads they would wait for them.
    auto process_full = [&](const KVRegs &r) {
        const float x = page_score(qv, swapK ? r.k1 : r.k0, swapK ? r.k0 : r.k1, P.scale_log2);
        const float pw = softmax_step(x, m_run, l_run, acc);
        float va[8], vb[8];
        unpack8(swapV ? r.v1 : r.v0, va);
        unpack8(swapV ? r.v0 : r.v1, vb);
        accumulate(pw, va, vb, acc);
    };
    auto process_last = [&](KVRegs r, int p) {
        if (kFused && g == (pos & 7)) {  // patch the appended token into the registers
            const u32x4 nk = *reinterpret_cast<const u32x4 *>(&s_newk[c * 8]);
            const u32x4 nv = *reinterpret_cast<const u32x4 *>(&s_newv[c * 8]);
            // register of token half `half`: load order (whole rows) or slot order
            const int half = (pos >> 3) & 1;
            if (kRows ? half : half ^ t0) r.k1 = nk; else r.k0 = nk;
            if (kRows ? half : half ^ b2) r.v1 = nv; else r.v0 = nv;
        }
        const int tb = p * kPage;
        float x = page_score(qv, swapK ? r.k1 : r.k0, swapK ? r.k0 : r.k1, P.scale_log2);
        if (tb + g + 8 * t0 >= L) x = -INFINITY;
        const float pw = softmax_step(x, m_run, l_run, acc);
        float va[8], vb[8];
        unpack8(swapV ? r.v1 : r.v0, va);
        unpack8(swapV ? r.v0 : r.v1, vb);
        const bool ok0 = tb + g + 8 * b2 < L, ok1 = tb + g + 8 * (b2 ^ 1) < L;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            va[i] = ok0 ? va[i] : 0.0f;
            vb[i] = ok1 ? vb[i] : 0.0f;
        }
        accumulate(pw, va, vb, acc);
    };
    // Full pages: two register sets in turn, the next page's loads always in
    // flight.  The sequence's last page is the final page of the wave that owns
    // it; it is prefetched like any other and handled after the loop.
    const int p_stop = (pg1 == n_pages) ? n_pages - 1 : pg1;
    KVRegs alt;
    bool last_in_alt = false;
    // Priority levels by progress through the partition (10/16, 13/16, 15/16):
    // a workgroup that has fallen behind its CU neighbour keeps the higher
    // level and catches up, so both end close together.
    const int span = pg1 - pg0;
    auto level = [&]() {
        if (!kLevel) return;
        const int done16 = 16 * (p - pg0);
        if (done16 >= 15 * span) __builtin_amdgcn_s_setprio(0);
        else if (done16 >= 13 * span) __builtin_amdgcn_s_setprio(1);
        else if (done16 >= 10 * span) __builtin_amdgcn_s_setprio(2);
    };
    // Steady state: both loads of a double step are known to be needed, so they
    // are issued unconditionally.  A load under a branch leaves the compiler's
    // wait counting unsure how many loads are outstanding after the join, and
    // it then waits for all of them (the next page's included) every step.
    while (p + kWaves < p_stop && p + 2 * kWaves < pg1) {
        alt = load_page(p + kWaves);
        process_full(cur);
        p += kWaves;
        level();
        cur = load_page(p + kWaves);
        process_full(alt);
        p += kWaves;
        level();
    }
    // The last page or two of the wave.
    while (p < p_stop) {
        if (p + kWaves < pg1) alt = load_page(p + kWaves);
        process_full(cur);
        p += kWaves;
        level();
        if (p >= p_stop) { last_in_alt = true; break; }
        if (p + kWaves < pg1) cur = load_page(p + kWaves);
        process_full(alt);
        p += kWaves;
        level();
    }
    if (pg1 == n_pages && p == n_pages - 1) {  // this wave owns the sequence's last page
        if (last_in_alt) cur = alt;
        process_last(cur, p);
    }
    // ---- wave epilogue: sums over the 8 lane groups (one max per wave) -----
    // acc[e][i] is reduce-scattered over the groups: the xor-32 step leaves slots
    // e = 0, 1 holding (e, e+2) summed over lane halves, the xor-16 step leaves
    // slot 0 holding slot (g>>1)&1 of that, the xor-8 step completes the sum.
    // Group pair g>>1 then owns accumulator slot e = g>>1, fully summed.
    float l_tot = l_run + dpp_f32<kXor1>(l_run);
    l_tot = sum_groups(l_tot);
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
    }
    __syncthreads();

    // ---- merge the waves: thread (h, d) --------------------------------------
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
        // The appended row and the rotated q are stored last.  Nothing in this
        // kernel reads them back (the loop took the new token from LDS), and a
        // store issued ahead of the page loads would hold up the wave's first
        // wait for page data, since vector memory operations complete in order.
        // Append: last partition only (the sequence is known good here).
        if (tid < 8 && pg1 == n_pages) {
            const int64_t dst = static_cast<int64_t>(s_app_page) * kPageElems + tile_j +
                                (pos & (kPage - 1)) * kD + c * 8;
            *reinterpret_cast<u32x4 *>(P.k_pool + dst) = *reinterpret_cast<const u32x4 *>(&s_newk[c * 8]);
            *reinterpret_cast<u32x4 *>(P.v_pool + dst) = *reinterpret_cast<const u32x4 *>(&s_newv[c * 8]);
        }
        // With one partition no other workgroup reads these q rows (longer
        // contexts leave the rotated q to k_decode_merge).
        if (P.write_q && n_parts_s == 1 && tid >= 64 && tid < 96)
            *reinterpret_cast<u32x4 *>(P.q + qrow0 + (tid - 64) * 8) =
                *reinterpret_cast<const u32x4 *>(&s_q[0][(tid - 64) * 8]);
    }
}


int decode_part_pages() {
    static int cached = [] {
        int v = kMaxPartPages;  // 2048 tokens: one partition for every context up to 2048
        if (const char *e = getenv("PA_DECODE_PART_PAGES")) {
            const int x = atoi(e);
            if (x >= 1 && x <= kMaxPartPages) v = x;
        }
        return v;
    }();
    return cached;
}

constexpr int kDecodeWaves = 8;

hipError_t launch_decode(const DecodeLaunch &d, hipStream_t stream) {
    if (d.num_seqs == 0) return hipSuccess;
    DecodeParams P{};
    P.out = d.out;
    P.q = static_cast<uint16_t *>(d.q);
    P.k_new = static_cast<const uint16_t *>(d.k_new);
    P.v_new = static_cast<const uint16_t *>(d.v_new);
    P.k_pool = static_cast<uint16_t *>(d.k_pool);
    P.v_pool = static_cast<uint16_t *>(d.v_pool);
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
    // The load form by grid size, as measured on MI355X (fused step, 16 layers):
    // from 128 workgroups, whole rows with the non-temporal hint on both tiles
    // (64 x 2048 tokens, 512 workgroups: 44.3 us per launch against 46.3 for
    // the best slot-order form, which hinted K alone; 256 ragged sequences,
    // 2048 workgroups: 61.6 against 69.0 unhinted).  The hint pays only on
    // whole-row loads: a read-only kernel over the same page pattern takes
    // 42.9 us with whole rows and 45.2 us with half rows when K is hinted, and
    // hinting V as well takes the half-row form to 49.4 us.  Below 128
    // workgroups (a few long, latency-bound streams: 8 sequences, 64
    // workgroups) the slot-order form is ahead, 11.9 against 12.9 us.
    const bool rows = blocks >= kNtMinBlocks;
    const dim3 grid(static_cast<unsigned>(blocks)), wg(64 * kDecodeWaves);
    auto go = [&](auto order) {
        using Ord = decltype(order);
        if (d.fused) {
            if (rows) hipLaunchKernelGGL((k_decode_paged<kDecodeWaves, true, true, Ord>), grid, wg, 0, stream, P, order);
            else hipLaunchKernelGGL((k_decode_paged<kDecodeWaves, true, false, Ord>), grid, wg, 0, stream, P, order);
        } else {
            if (rows) hipLaunchKernelGGL((k_decode_paged<kDecodeWaves, false, true, Ord>), grid, wg, 0, stream, P, order);
            else hipLaunchKernelGGL((k_decode_paged<kDecodeWaves, false, false, Ord>), grid, wg, 0, stream, P, order);
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
