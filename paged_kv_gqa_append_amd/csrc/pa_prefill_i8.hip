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
// A workgroup of 4 waves serves (sequence, KV head j, 16 chunk rows); wave w
// serves rows row0 + 4w .. +3 over every key they see and finishes them
// itself (no merge across waves).  The MFMAs are the INT8 decode's with all
// 16 columns live: column c = 4r + h is row r of the wave's four and query
// head h of the group.  Per page: S^T[16 tokens][16 columns] = K . Q^T (two
// v_mfma_f32_16x16x32_f16 on the codes), then O[16 columns][64] += P' . V
// (four v_mfma_f32_16x16x16_f16 for each half of an f16 hi + lo weight pair).
// The arithmetic per (column, token) is the INT8 decode's (pa_i8.hip): exact
// codes, the 1152 offset subtracted from the score, the K scale applied to
// the score, the V scale folded into the weights with the lazy exponent ve,
// online softmax in log2 units with a lazy running max per column; keys past
// a column's position get weight 0.
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

// Four waves (16 rows) per workgroup, three workgroups per CU: the kernel
// needs about 160 VGPRs (three waves per SIMD); with eight-wave workgroups at
// four waves per SIMD the compiler spilled.
constexpr int kWavesP8 = 4;
constexpr int kThreadsP8 = 64 * kWavesP8;
constexpr int kRowsP8 = 4 * kWavesP8;  // chunk rows per workgroup

__global__ __launch_bounds__(kThreadsP8, 3) void k_prefill_attn_i8(PrefillI8Params P) {
    // ids -> (sequence, KV head, tile): the 3 low id bits pick the XCD, which is
    // also the KV head; each (sequence, head) takes its tiles longest first.
    const int bid = blockIdx.x;
    const int j = bid & (kHKV - 1);
    const int rank = bid >> 3;
    const int s = rank / P.n_tiles;
    const int tile = P.n_tiles - 1 - rank % P.n_tiles;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int hh = lane & 15;  // MFMA column: row hh/4 of the wave's four, head hh%4
    const int qd = lane >> 4;  // quarter: K dims 8qd..+7 and 32+8qd..+7; tokens and scales 4qd..+3
    const int C = P.chunk_len;

    __shared__ int s_pages[kMaxBlocksPrefill];

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
    if (row0 >= C) return;  // a wave past the chunk's end (no barrier follows)

    // the wave's keys: 0 .. the position of its last row
    const int last_pos = prefix + min(row0 + 3, C - 1);
    const int np_w = last_pos / kPage + 1;
    // pages from which some column's causal limit falls inside (or before) the page
    const int first_masked = (prefix + row0) / kPage;

    // ---- q as the f16 B operand, scaled by 2^(15 - e) so that its largest
    // element over the wave's 16 columns lies in [2^14, 2^15)
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

    const int64_t tile_j = static_cast<int64_t>(j) * kI8Tile;
    auto load_page = [&](int p) {
        const int page = __builtin_amdgcn_readfirstlane(s_pages[p]);
        const uint8_t *t = P.pool + static_cast<int64_t>(page) * kPageBytesI8 + tile_j;
        I8Page r;
        r.k = *reinterpret_cast<const u32x4 *>(t + lane * 16);
        r.v = *reinterpret_cast<const u32x4 *>(t + kI8VOff + lane * 16);
        r.ks = *reinterpret_cast<const f32x4 *>(t + kI8KScOff + qd * 16);
        r.vs = *reinterpret_cast<const f32x4 *>(t + kI8VScOff + qd * 16);
        return r;
    };

    float m_run = kNegBig;  // running max (log2 units) of column hh
    float l_run = 0.0f;     // sum of 2^(x - m) over the lane's tokens
    // acc[n]: O[column 4qd + i][dim 16n + hh]
    f32x4 acc[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    int ve = 0;
    float vmul = 1.0f;                                          // 2^-ve
    uint32_t vlim_bits = __builtin_bit_cast(uint32_t, 128.0f);  // 2^(ve + 7), as bits

    // masked: a page in which some column's causal limit falls (the wave's
    // last one or two pages); the others are live for every column
    auto process = [&](const I8Page &r, int p, auto masked_c) {
        constexpr bool masked = decltype(masked_c)::value;
        f32x4 st = {0.0f, 0.0f, 0.0f, 0.0f};
        st = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes8_to_f16(r.k.x, r.k.y), qb0, st, 0, 0, 0);
        st = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes8_to_f16(r.k.z, r.k.w), qb1, st, 0, 0, 0);
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = (st[i] - corr) * (r.ks[i] * sc_log2);
        bool dead[4] = {false, false, false, false};
        if (masked) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                dead[i] = p * kPage + 4 * qd + i > pos_c;
                if (dead[i]) x[i] = -INFINITY;
            }
        }
        const float xm = max_quarters(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
        const bool need = xm > m_run + kRescaleLog2;
        float vsl[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) vsl[i] = (masked && dead[i]) ? 0.0f : r.vs[i];
        const uint32_t vmx = max(max(__builtin_bit_cast(uint32_t, vsl[0]), __builtin_bit_cast(uint32_t, vsl[1])),
                                 max(__builtin_bit_cast(uint32_t, vsl[2]), __builtin_bit_cast(uint32_t, vsl[3])));
        const bool vneed = vmx > vlim_bits;
        if (__builtin_amdgcn_ballot_w64(need || vneed)) {
            if (__builtin_amdgcn_ballot_w64(need)) {
                const float mn = need ? xm : m_run;
                const float f = fast_exp2(m_run - mn);
                m_run = mn;
                l_run *= f;
                // accumulator row 4qd + i is column 4qd + i: its factor is that column's
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float fi = __shfl(f, 4 * qd + i, 64);
#pragma unroll
                    for (int n = 0; n < 4; ++n) acc[n][i] *= fi;
                }
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
            pv[i] = (masked && dead[i]) ? 0.0f : pw[i] * (vsl[i] * vmul);
        }
        l_run += (pw[0] + pw[1]) + (pw[2] + pw[3]);
        const uint32_t h01 = pack_f16x2(pv[0], pv[1]);
        const uint32_t h23 = pack_f16x2(pv[2], pv[3]);
        const half2v e01 = __builtin_bit_cast(half2v, h01), e23 = __builtin_bit_cast(half2v, h23);
        const uint32_t l01 = pack_f16x2(pv[0] - static_cast<float>(e01[0]), pv[1] - static_cast<float>(e01[1]));
        const uint32_t l23 = pack_f16x2(pv[2] - static_cast<float>(e23[0]), pv[3] - static_cast<float>(e23[1]));
        const half4 ph = __builtin_bit_cast(half4, u32x2{h01, h23});
        const half4 pl = __builtin_bit_cast(half4, u32x2{l01, l23});
        const half4 vb[4] = {codes4_to_f16_signed(r.v.x), codes4_to_f16_signed(r.v.y),
                             codes4_to_f16_signed(r.v.z), codes4_to_f16_signed(r.v.w)};
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            acc[n] = __builtin_amdgcn_mfma_f32_16x16x16f16(ph, vb[n], acc[n], 0, 0, 0);
            acc[n] = __builtin_amdgcn_mfma_f32_16x16x16f16(pl, vb[n], acc[n], 0, 0, 0);
        }
    };

    // Pages 0 .. np_w-1, two in flight: at the top of a step cur holds page p
    // and alt page p + 1, both issued.  The steady loop takes unmasked pages
    // two at a time and its two loads are known to be needed, so they are
    // unconditional (see the decode kernels); the rest go one at a time.
    const std::integral_constant<bool, false> kLive;
    const std::integral_constant<bool, true> kMasked;
    int p = 0;
    I8Page cur = load_page(0);
    I8Page alt = load_page(min(1, np_w - 1));
    while (p + 1 < first_masked && p + 3 < np_w) {
        process(cur, p, kLive);
        cur = load_page(p + 2);
        process(alt, p + 1, kLive);
        alt = load_page(p + 3);
        p += 2;
    }
    while (p < np_w) {
        if (p < first_masked) process(cur, p, kLive);
        else process(cur, p, kMasked);
        ++p;
        cur = alt;
        if (p + 1 < np_w) alt = load_page(p + 1);
    }

    // ---- out[s][row][j*4 + h][16n + hh] = O x 2^ve / l of column 4qd + i
    const float l_tot = sum_quarters(l_run);
    const float vback = ldexpf(1.0f, ve);
    const int r = row0 + qd;  // accumulator rows 4qd .. 4qd+3: row qd of the wave's four, heads 0..3
    float inv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) inv[i] = vback / __shfl(l_tot, 4 * qd + i, 64);
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
