// pa_prefill_i8.hip -- chunked prefill attention over INT8 pages.
//
// TinyLoop ("Lifecycle and Memory Model": section "prefill_chunk and scratch
// residency" processes the prompt in row chunks; section "Per-request /
// handle-owned memory" names the INT8 K/V mode).  After the chunk's rows have
// been quantised into their pages and its q rows rotated (k_append_rope_i8 in
// prefix mode), for each chunk row i of sequence s at pos = prefix + i and
// each query head h of KV group j:
//     out[s][i][h] = sum_t softmax_t(scale <q, K_t>) V_t,   t <= pos,
// with K_t, V_t the values code * scale the INT8 format stands for.
//
// A workgroup of 8 waves serves (sequence, KV head j, 32 chunk rows); wave w
// serves rows row0 + 4w .. +3 over every key they see and finishes them
// itself (no merge across waves).  The MFMAs are the INT8 decode's with all
// 16 columns live: column c = 4r + h is row r of the wave's four and query
// head h of the group.
//
// The sequence's pages go through LDS in groups of eight, one per wave: each
// wave loads one page's INT8 tile and writes its codes as the f16 MFMA
// operands (and its scales) into the group's LDS slot, so a page is converted
// once per workgroup; two groups alternate, one barrier per group.  The waves
// take the pages two at a time (32 keys): per page S^T[16 tokens][16 columns]
// = K . Q^T (two v_mfma_f32_16x16x32_f16 on the codes, the accumulator
// starting at minus the code offset's contribution), then for the pair
// O[16 columns][64] += P' . V with four v_mfma_f32_16x16x32_f16 on the f16 hi
// halves of the weights (and four more on the lo halves where the output
// needs them), k = 8 quarter + i taking token 4 quarter + i of the first page
// for i < 4 and of the second for i >= 4 in both operands.  Per (column,
// token) the arithmetic is the INT8 decode's (pa_i8.hip): exact codes, the K
// scale applied to the score, the V scale folded into the weight, online
// softmax in log2 units; here a weight is kept as 2^(x - m - ve) with m the
// column's lazy reference and ve the wave's lazy V exponent, and keys past a
// column's position get weight 0.
#include <math.h>

#include <type_traits>

#include "pa_i8_core.h"

namespace pa {

namespace {

struct PrefillI8Params {
    void *out;
    const uint16_t *q;
    const uint8_t *pool;
    const int32_t *bt;
    const int32_t *prefix_lens;
    uint32_t *flags;
    int chunk_len;
    int max_blocks;
    int num_pages;
    int max_pos;
    int out_fp32;
    int n_tiles;
    float scale_log2;
};

// Eight waves (32 rows) per workgroup, two workgroups per CU.
constexpr int kWavesP8 = 8;
constexpr int kThreadsP8 = 64 * kWavesP8;
constexpr int kRowsP8 = 4 * kWavesP8;  // chunk rows per workgroup
constexpr int kGroupP8 = kWavesP8;     // pages per LDS group: one converted by each wave

// One page's tile as MFMA operands, in LDS (4224 B).  k[h][l]: lane l's K
// operand for dims 8(l/16)+32h .. +7 of token l%16 (f16 values 1152 + code);
// sc[0..15] the K scales times the softmax scale (log2 units, q's power of two
// removed), sc[16..31] the V scales.  vp[n][l] (in the first page of each
// pair): lane l's V operand for dims 16n + l%16 of the pair, tokens 4(l/16) ..
// +3 of the first page (low 8 bytes, written by the wave that converts it) and
// of the second (high 8 bytes), as signed f16 codes.
struct alignas(16) PageOps {
    u32x4 k[2][64];
    float sc[32];
};
struct alignas(16) PairV {
    u32x4 vp[4][64];
};

__global__ __launch_bounds__(kThreadsP8, 2) void k_prefill_attn_i8(PrefillI8Params P) {
    // ids -> (sequence, KV head, tile): the 3 low id bits pick the XCD, which is
    // also the KV head.  An XCD deals its workgroups to its 32 CUs in turn, so
    // its p-th, (p+32)-th, ... share a CU: even turns take the work list (rank
    // r: sequence r / n_tiles, tiles from the highest positions down) forward
    // and odd turns backward, so each CU pairs long tiles with short ones.
    const int bid = blockIdx.x;
    const int j = bid & (kHKV - 1);
    const int pslot = bid >> 3;
    const int base = pslot & ~(kCuPerXcd - 1);
    const int span = min(static_cast<int>(gridDim.x >> 3) - base, kCuPerXcd);  // a last turn may be short
    const int rank = ((pslot / kCuPerXcd) & 1) ? base + span - 1 - (pslot - base) : pslot;
    const int s = rank / P.n_tiles;
    const int tile = P.n_tiles - 1 - rank % P.n_tiles;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar loop control
    const int hh = lane & 15;  // MFMA column: row hh/4 of the wave's four, head hh%4
    const int qd = lane >> 4;  // quarter: K dims 8qd..+7 and 32+8qd..+7; tokens and scales 4qd..+3
    const int C = P.chunk_len;

    __shared__ int s_pages[kMaxBlocksPrefill];
    __shared__ PageOps s_ops[2][kGroupP8];
    __shared__ PairV s_v[2][kGroupP8 / 2];
    __shared__ float s_qmax[kWavesP8];

    // ---- prologue: length, block table (into LDS, checked), this lane's q
    const int prefix = P.prefix_lens[s];
    const int64_t lim = min(static_cast<int64_t>(P.max_blocks) * kPage, static_cast<int64_t>(P.max_pos));
    const bool len_ok = prefix >= 0 && static_cast<int64_t>(prefix) + C <= lim;
    const int total = len_ok ? prefix + C : 0;
    const int n_pages = (total + kPage - 1) / kPage;
    const int32_t *bt_row = P.bt + static_cast<int64_t>(s) * P.max_blocks;
    int bad = 0;
    for (int b = tid; b < n_pages; b += kThreadsP8) {
        const int pid = bt_row[b];
        s_pages[b] = pid;
        bad |= (pid < 0) | (pid >= P.num_pages);
    }
    const int row0 = tile * kRowsP8 + 4 * w;
    // padding rows (past the chunk) compute on its last row and are never stored
    const int row_c = min(row0 + (hh >> 2), C - 1);
    const int pos_c = (len_ok ? prefix : 0) + row_c;
    const uint16_t *qrow = P.q + ((static_cast<int64_t>(s) * C + row_c) * kHQ + j * kGroup + (hh & 3)) * kD;
    const u32x4 qraw0 = *reinterpret_cast<const u32x4 *>(qrow + 8 * qd);
    const u32x4 qraw1 = *reinterpret_cast<const u32x4 *>(qrow + 32 + 8 * qd);
    float qf[16];
    {
        const uint32_t a[8] = {qraw0.x, qraw0.y, qraw0.z, qraw0.w, qraw1.x, qraw1.y, qraw1.z, qraw1.w};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            qf[2 * k] = bf16_lo(a[k]);
            qf[2 * k + 1] = bf16_hi(a[k]);
        }
    }
    {
        float qm = 0.0f;
#pragma unroll
        for (int k = 0; k < 16; ++k) qm = fmaxf(qm, fabsf(qf[k]));
        qm = max_groups(max_lanes8(qm));
        if (lane == 0) s_qmax[w] = qm;
    }

    // ---- validation: the whole sequence's pages (the loop above staged them in LDS)
    const bool ok = len_ok && __syncthreads_or(bad) == 0;
    if (!ok) {
        // zero this wave's rows (4 rows x 4 heads x 64 dims, 16 per lane); flag once
        const int r = row0 + (hh >> 2);
        if (r < C) {
            const int64_t o = ((static_cast<int64_t>(s) * C + r) * kHQ + j * kGroup + (hh & 3)) * kD + 16 * qd;
            const u32x4 z = {0u, 0u, 0u, 0u};
            if (P.out_fp32) {
                u32x4 *dst = reinterpret_cast<u32x4 *>(static_cast<float *>(P.out) + o);
                dst[0] = z, dst[1] = z, dst[2] = z, dst[3] = z;
            } else {
                u32x4 *dst = reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(P.out) + o);
                dst[0] = z, dst[1] = z;
            }
        }
        if (tid == 0 && j == 0 && tile == P.n_tiles - 1 && P.flags)
            atomicOr(P.flags, len_ok ? kDevErrPageId : kDevErrContextLen);
        return;
    }
    // a wave past the chunk's end converts its pages and meets the barriers
    // but attends nothing
    const bool active = row0 < C;
    // the wave's keys: 0 .. the position of its last row
    const int last_pos = prefix + min(row0 + 3, C - 1);
    const int np_w = last_pos / kPage + 1;
    // pages from which some column's causal limit falls inside (or before) the page
    const int first_masked = (prefix + row0) / kPage;
    // the workgroup's pages (those of its last row) and groups of eight
    const int np_g = (prefix + min(tile * kRowsP8 + kRowsP8 - 1, C - 1)) / kPage + 1;
    const int n_groups = (np_g + kGroupP8 - 1) / kGroupP8;

    // ---- q as the f16 B operand, scaled by 2^(15 - e) so that its largest
    // element over the workgroup's 128 columns lies in [2^14, 2^15)
    float qmax = s_qmax[0];
#pragma unroll
    for (int v = 1; v < kWavesP8; ++v) qmax = fmaxf(qmax, s_qmax[v]);
    int qe = 0;
    if (qmax > 0.0f) (void)frexpf(qmax, &qe);
    const int qshift = min(15 - qe, 126);
    const float qscale = ldexpf(1.0f, qshift);
    half8 qb0, qb1;
    {
        uint32_t hq[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) hq[k] = pack_f16x2(qf[2 * k] * qscale, qf[2 * k + 1] * qscale);
        qb0 = __builtin_bit_cast(half8, u32x4{hq[0], hq[1], hq[2], hq[3]});
        qb1 = __builtin_bit_cast(half8, u32x4{hq[4], hq[5], hq[6], hq[7]});
    }
    // -1152 * <q', 1> for column hh: the start of every score accumulator, which
    // removes the offset the code encoding adds
    float ncorr;
    {
        const uint32_t c1152 = 0x64806480u;  // f16 1152.0 twice
        const half8 k1152 = __builtin_bit_cast(half8, u32x4{c1152, c1152, c1152, c1152});
        f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
        z = __builtin_amdgcn_mfma_f32_16x16x32_f16(k1152, qb0, z, 0, 0, 0);
        z = __builtin_amdgcn_mfma_f32_16x16x32_f16(k1152, qb1, z, 0, 0, 0);
        ncorr = -z[0];
    }
    const float sc_log2 = P.scale_log2 * ldexpf(1.0f, -qshift);

    // ---- page conversion: one page's INT8 tile -> its PageOps in LDS
    struct RawPage {
        u32x4 k, v;   // the lane's K unit and V unit
        uint32_t sc;  // scale (l % 32): K scales then V scales
    };
    const int64_t tile_j = static_cast<int64_t>(j) * kI8Tile;
    auto load_raw = [&](int p) {
        const int page = __builtin_amdgcn_readfirstlane(s_pages[p]);
        const uint8_t *t = P.pool + static_cast<int64_t>(page) * kPageBytesI8 + tile_j;
        RawPage r;
        r.k = *reinterpret_cast<const u32x4 *>(t + lane * 16);
        r.v = *reinterpret_cast<const u32x4 *>(t + kI8VOff + lane * 16);
        r.sc = *reinterpret_cast<const uint32_t *>(t + kI8KScOff + 4 * (lane & 31));
        return r;
    };
    // the wave's page in its group: slot w, half w % 2 of pair w / 2's V
    auto store_ops = [&](const RawPage &r, PageOps &d, PairV &pv) {
        d.k[0][lane] = __builtin_bit_cast(u32x4, codes8_to_f16(r.k.x, r.k.y));
        d.k[1][lane] = __builtin_bit_cast(u32x4, codes8_to_f16(r.k.z, r.k.w));
        u32x2 *vh = reinterpret_cast<u32x2 *>(&pv.vp[0][lane]) + (w & 1);
        vh[0] = __builtin_bit_cast(u32x2, codes4_to_f16_signed(r.v.x));
        vh[128] = __builtin_bit_cast(u32x2, codes4_to_f16_signed(r.v.y));
        vh[256] = __builtin_bit_cast(u32x2, codes4_to_f16_signed(r.v.z));
        vh[384] = __builtin_bit_cast(u32x2, codes4_to_f16_signed(r.v.w));
        const float sc = __builtin_bit_cast(float, r.sc);
        if (lane < 32) d.sc[lane] = lane < 16 ? sc * sc_log2 : sc;
    };

    // Softmax state of column hh (the same in its four quarter lanes).  A key's
    // weight is kept as 2^(x - m - ve): m the column's lazy reference, ve the
    // wave's lazy V exponent, so that weight times V scale is the f16 operand
    // directly; l and O carry the same factor 2^-ve, which their ratio drops.
    float m_run = kNegBig;  // reference (log2 units)
    float l_run = 0.0f;     // sum of the lane's weights
    // acc[n]: O[column 4qd + i][dim 16n + hh]
    f32x4 acc[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    int ve = 0;
    float mv = m_run;                                           // m + ve
    float thr = kRescaleLog2;                                   // x - m - ve above this: move m
    uint32_t vlim_bits = __builtin_bit_cast(uint32_t, 128.0f);  // 2^(ve + 7), as bits
    auto scale_rows = [&](float f) {  // accumulator row 4qd + i by column 4qd + i's factor
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float fi = __shfl(f, 4 * qd + i, 64);
#pragma unroll
            for (int n = 0; n < 4; ++n) acc[n][i] *= fi;
        }
    };

    // pages p, p + 1 (slots A, B); masked: some key of the pair lies past some
    // column's position (the wave's last one or two pages, and a page past its
    // last, whose keys are all past)
    auto process_pair = [&](const PageOps &A, const PageOps &B, const PairV &V, int p, bool masked) {
        f32x4 sa = {ncorr, ncorr, ncorr, ncorr}, sb = sa;
        sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, A.k[0][lane]), qb0, sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, B.k[0][lane]), qb0, sb, 0, 0, 0);
        sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, A.k[1][lane]), qb1, sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, B.k[1][lane]), qb1, sb, 0, 0, 0);
        const f32x4 ksa = *reinterpret_cast<const f32x4 *>(&A.sc[4 * qd]);
        const f32x4 ksb = *reinterpret_cast<const f32x4 *>(&B.sc[4 * qd]);
        const f32x4 vsa = *reinterpret_cast<const f32x4 *>(&A.sc[16 + 4 * qd]);
        const f32x4 vsb = *reinterpret_cast<const f32x4 *>(&B.sc[16 + 4 * qd]);
        float sv[8], ks[8], vsl[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sv[i] = sa[i], sv[4 + i] = sb[i];
            ks[i] = ksa[i], ks[4 + i] = ksb[i];
            vsl[i] = vsa[i], vsl[4 + i] = vsb[i];
        }
        // t = x - m - ve, x = the score in log2 units; a key past the column's
        // position gets t = -inf and V scale 0
        float t[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) t[i] = __builtin_fmaf(sv[i], ks[i], -mv);
        auto kill = [&](float *u) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if ((p + (i >> 2)) * kPage + 4 * qd + (i & 3) > pos_c) u[i] = -INFINITY;
        };
        if (masked) {
            kill(t);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if ((p + (i >> 2)) * kPage + 4 * qd + (i & 3) > pos_c) vsl[i] = 0.0f;
        }
        const float tm = fmaxf(fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3])), fmaxf(fmaxf(t[4], t[5]), fmaxf(t[6], t[7])));
        uint32_t vmx = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) vmx = max(vmx, __builtin_bit_cast(uint32_t, vsl[i]));
        const bool need = tm > thr;
        const bool vneed = vmx > vlim_bits;
        if (__builtin_amdgcn_ballot_w64(need || vneed)) {
            if (__builtin_amdgcn_ballot_w64(need)) {
                // the column's largest score of the pair, from the scores themselves
                float x[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) x[i] = sv[i] * ks[i];
                if (masked) kill(x);
                const float xm = max_quarters(fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                                                    fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7]))));
                const float mn = xm > m_run + kRescaleLog2 ? xm : m_run;
                const float f = fast_exp2(m_run - mn);
                m_run = mn;
                l_run *= f;
                scale_rows(f);
            }
            if (__builtin_amdgcn_ballot_w64(vneed)) {
                // the largest live scale over the whole wave (columns mask different tokens)
                const float wmx = __builtin_bit_cast(
                    float, __builtin_amdgcn_readfirstlane(
                               __builtin_bit_cast(int, max_groups(max_lanes8(__builtin_bit_cast(float, vmx))))));
                int e = 0;
                (void)frexpf(wmx, &e);
                const int ve_new = e - 7;
                if (ve_new > ve) {
                    const float f = ldexpf(1.0f, ve - ve_new);
#pragma unroll
                    for (int n = 0; n < 4; ++n)
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[n][i] *= f;
                    l_run *= f;
                    ve = ve_new;
                    thr = kRescaleLog2 - static_cast<float>(ve);
                    vlim_bits = __builtin_bit_cast(uint32_t, ldexpf(1.0f, ve + 7));
                }
            }
            mv = m_run + static_cast<float>(ve);
#pragma unroll
            for (int i = 0; i < 8; ++i) t[i] = __builtin_fmaf(sv[i], ks[i], -mv);
            if (masked) kill(t);
        }
        float pw[8], pv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            pw[i] = fast_exp2(t[i]);
            pv[i] = pw[i] * vsl[i];
        }
        l_run += ((pw[0] + pw[1]) + (pw[2] + pw[3])) + ((pw[4] + pw[5]) + (pw[6] + pw[7]));
        uint32_t hw[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) hw[k] = pack_f16x2(pv[2 * k], pv[2 * k + 1]);
        const half8 ph = __builtin_bit_cast(half8, u32x4{hw[0], hw[1], hw[2], hw[3]});
        half8 vo[4];
#pragma unroll
        for (int n = 0; n < 4; ++n) vo[n] = __builtin_bit_cast(half8, V.vp[n][lane]);
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph, vo[n], acc[n], 0, 0, 0);
        // the lo halves: always for fp32 output; for bf16 output only where some
        // live V scale of the pair exceeds 1/8 (kHiOnlyVScaleBits)
        if (P.out_fp32 || __builtin_amdgcn_ballot_w64(vmx > kHiOnlyVScaleBits)) {
            uint32_t lw[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const half2v e = __builtin_bit_cast(half2v, hw[k]);
                lw[k] = pack_f16x2(pv[2 * k] - static_cast<float>(e[0]), pv[2 * k + 1] - static_cast<float>(e[1]));
            }
            const half8 pl = __builtin_bit_cast(half8, u32x4{lw[0], lw[1], lw[2], lw[3]});
#pragma unroll
            for (int n = 0; n < 4; ++n) acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pl, vo[n], acc[n], 0, 0, 0);
        }
    };

    // ---- the page loop.  Group g holds pages 8g .. 8g+7 (wave w converts page
    // 8g + w; past the last page it converts the last page again, unused).  At
    // the top of step g the group's slots are written and visible, and raw holds
    // group g + 1's page, issued.
    RawPage raw = load_raw(min(w, np_g - 1));
    store_ops(raw, s_ops[0][w], s_v[0][w >> 1]);
    raw = load_raw(min(kGroupP8 + w, np_g - 1));
    __syncthreads();
    for (int g = 0; g < n_groups; ++g) {
        const PageOps *grp = s_ops[g & 1];
        const PairV *gv = s_v[g & 1];
        if (active) {
#pragma unroll
            for (int h = 0; h < kGroupP8 / 2; ++h) {
                const int p = kGroupP8 * g + 2 * h;
                if (p < np_w) process_pair(grp[2 * h], grp[2 * h + 1], gv[h], p, p + 1 >= first_masked);
            }
        }
        if (g + 1 < n_groups) {
            store_ops(raw, s_ops[(g + 1) & 1][w], s_v[(g + 1) & 1][w >> 1]);
            raw = load_raw(min(kGroupP8 * (g + 2) + w, np_g - 1));
        }
        __syncthreads();
    }

    // ---- out[s][row][j*4 + h][16n + hh] = O / l of column 4qd + i (both carry 2^-ve)
    const float l_tot = sum_quarters(l_run);
    const int r = row0 + qd;  // accumulator rows 4qd .. 4qd+3: row qd of the wave's four, heads 0..3
    float inv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) inv[i] = 1.0f / __shfl(l_tot, 4 * qd + i, 64);
    if (r >= C) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t orow = ((static_cast<int64_t>(s) * C + r) * kHQ + j * kGroup + i) * kD + hh;
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const float y = acc[n][i] * inv[i];
            if (P.out_fp32) static_cast<float *>(P.out)[orow + 16 * n] = y;
            else static_cast<uint16_t *>(P.out)[orow + 16 * n] = f32_to_bf16(y);
        }
    }
}

}  // namespace

hipError_t launch_prefill_attention_i8(const PrefillLaunch &p, hipStream_t stream) {
    if (p.num_seqs == 0 || p.chunk_len == 0) return hipSuccess;
    if (p.max_blocks > kMaxBlocksPrefill) return hipErrorInvalidValue;
    PrefillI8Params P{};
    P.out = p.out;
    P.q = static_cast<const uint16_t *>(p.q);
    P.pool = static_cast<const uint8_t *>(p.k_pool);
    P.bt = p.block_tables;
    P.prefix_lens = p.prefix_lens;
    P.flags = p.flags;
    P.chunk_len = p.chunk_len;
    P.max_blocks = p.max_blocks;
    P.num_pages = p.num_pages;
    P.max_pos = p.max_pos;
    P.out_fp32 = p.out_fp32;
    P.n_tiles = (p.chunk_len + kRowsP8 - 1) / kRowsP8;
    P.scale_log2 = p.scale * 1.4426950408889634f;
    const int64_t blocks = static_cast<int64_t>(p.num_seqs) * P.n_tiles * kHKV;
    hipLaunchKernelGGL(k_prefill_attn_i8, dim3(static_cast<unsigned>(blocks)), dim3(kThreadsP8), 0, stream, P);
    return hipGetLastError();
}

}  // namespace pa
