// pa_prefill.hip -- causal chunked-prefill attention over the paged pool, on
// bf16 MFMA tiles (gfx950 v_mfma_f32_32x32x16_bf16), fp32 accumulation.
//
// What is computed (TinyLoop, section "prefill_chunk and scratch residency":
// the prompt is processed in row chunks; samir-vllm, "Gestion de la KV cache
// ...": the prompt's pages are filled during prefill): after the chunk's K/V
// rows have been appended and the chunk's q rows rotated in place
// (k_append_rope, prefix mode), every chunk query at absolute position
// p = prefix + i, rotated at p, attends to keys 0..p
// of its sequence, read through the block table:
//     out[s][i][h] = sum_t softmax_t(scale <rope(q[s][i][h], p), K_t>) V_t,  t <= p.
// No score matrix is stored (contrast tiny-vllm's prefill, which keeps a
// 512 x 512 x 32 score buffer, ch.2 buffer table).
//
// Work decomposition
//   One workgroup of 4 waves per (sequence, KV head j, tile of 32 chunk
//   positions).  Each wave holds two of the 4 query heads of that KV head
//   (two independent streams that share every K and V fragment); waves 0-1
//   take the first half of the tile's key blocks, waves 2-3 the second half.
//   The two partial results are merged through LDS at the end, each half
//   finishing 32 of the 64 output dims.  Two workgroups share a CU (2 waves
//   per SIMD, <= 256 VGPRs).  Keys go 32 at a time (two pages).
//   Workgroup ids are mapped so that all tiles of one (sequence, KV head) land
//   on the same XCD (ids are dealt to the 8 XCDs round-robin) and share its
//   L2; the longest tiles start first.
//   Scores are computed transposed, S^T = K Q^T (32 keys x 32 queries): in the
//   MFMA result layout a lane holds 16 keys of ONE query (lane l: query l%32,
//   keys 8i + 4(l/32) + r in register 4i+r), so the online softmax is
//   lane-local plus one exchange with lane l^32.  The output is accumulated
//   transposed too, O^T = V^T P^T (64 d x 32 queries): the same lane-per-query
//   layout, so rescaling is lane-local.  P^T is the MFMA B operand straight
//   from the score registers; the V^T fragments come from natural V rows in
//   LDS through transposing LDS reads.
//   K/V blocks go from the pool straight into LDS (direct-to-LDS loads, no
//   staging registers), four buffers per key half with three blocks in
//   flight; one barrier per block.
//   The loop is software-pipelined by one block: while the weights of block
//   b are formed (exp2, bf16 packing, row sums: VALU work), the score MFMAs
//   of block b+1 run, and the P.V MFMAs of block b overlap the scaling of
//   block b+1's scores; scheduling groups pin that interleave so that the
//   matrix and vector units of one wave work at the same time, and the two
//   streams' products alternate so that none waits for the one before it.
//   Softmax in log2 units against a lazily kept integer reference: per score
//   one fused multiply-add, one exp2, half a packed bf16 conversion and half a
//   dot2 for the row sum (taken over the same bf16 weights the P.V product
//   uses); the block maximum is needed only when the weights outgrow 2^8.
//   With fp32 output the weights are fed as a bf16 hi/lo pair (two MFMAs) so
//   they keep ~16 significant bits.
//   q arrives rotated (the append kernel of the same call rotates it in place
//   before this kernel runs; with out == q the output then overwrites it).
#include <math.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kRows = 32;                   // chunk positions per workgroup (one 32-row tile per wave)
constexpr int kKB = 32;                     // keys per block
constexpr int kBlockBytes = kKB * kD * 2;  // one K or V block in LDS: 32 rows of 128 bytes

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Value of lane l^32 (permlane32 swap; the second operand is hidden from the
// compiler, which would otherwise fold a swap of equal operands).
__device__ __forceinline__ float partner32(float v) {
    const unsigned a = __builtin_bit_cast(unsigned, v);
    unsigned b = a;
    asm volatile("" : "+v"(b));
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    const unsigned r0 = r[0], r1 = r[1];
    // lanes < 32 keep their own value in r0 and get the partner's in r1
    return __lane_id() < 32 ? __builtin_bit_cast(float, r1) : __builtin_bit_cast(float, r0);
}

// max(v, value of lane l^32) in every lane: after the swap one register holds
// the lower lane's value and the other the upper one's, in both halves, so no
// select is needed.
__device__ __forceinline__ float max_partner32(float v) {
    const unsigned a = __builtin_bit_cast(unsigned, v);
    unsigned b = a;
    asm volatile("" : "+v"(b));
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    const unsigned r0 = r[0], r1 = r[1];
    return fmaxf(__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1));
}

// One 16-byte direct-to-LDS load per lane (global_load_lds_dwordx4): lane l's
// 16 bytes at gbase + voff (bytes) land at LDS byte address lds + 16 l.  It is
// issued through inline assembly so that the compiler, which cannot tell which
// LDS buffer it fills, does not hold LDS reads of the other buffers behind it;
// the kernel waits for these loads itself (vmcnt) before the barrier that
// publishes a buffer.  M0 carries the LDS address; its previous value is kept
// and restored, since the compiler may hold one there.  gbase and lds must be
// wave-uniform.
__device__ __forceinline__ void dma16(const void *gbase, uint32_t voff, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %1\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(gbase), "v"(voff), "s"(lds)
        : "memory");
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

typedef float f32x2 __attribute__((ext_vector_type(2)));

// (a, b) -> packed bf16 pair, round to nearest even, one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// K and V blocks in LDS: 32 rows (keys) of 128 bytes, as in the pool, with the
// 16-byte chunk c of row r stored at chunk position c ^ f(r), where
// f(r) = 2 (r mod 4) + (r / 4 mod 2) is a permutation of 0..7 over any 8
// consecutive rows.  Direct-to-LDS loads write each wave's 8 rows as one
// contiguous kilobyte (lane l fetches the chunk that belongs at position l),
// and the swizzle spreads the fragment reads over the 32 banks: a K read (one
// chunk of 8 consecutive rows per 8 lanes) meets 8 positions, and so does a
// transposing V read (chunks 2i, 2i+1 of 4 rows 4j..4j+3 per 16 lanes).
__device__ __forceinline__ int swz_f(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }
__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ swz_f(row)) << 4); }

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Transposing LDS read (gfx950 ds_read_b64_tr_b16): within each group of 16
// lanes, lane i names the 4 consecutive elements of row i/4 of a 4 x 16 block
// (columns 4(i%4)..+3), and lane j receives column j of the block, rows 0..3.
__device__ __forceinline__ bf16x4 read_tr16(const unsigned char *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p));
}

// acc + the sum of the 8 bf16 weights (dot2 against (1, 1): exact products,
// fp32 sums), one chain.
__device__ __forceinline__ float sum8_bf16(bf16x8 v, float acc) {
    const bf16x2 one2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one2, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one2, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one2, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one2, acc, false);
    return acc;
}

}  // namespace

struct PrefillParams {
    void *out;
    const uint16_t *q;
    const uint16_t *k_pool;
    const uint16_t *v_pool;
    const int32_t *bt;
    const int32_t *prefix_lens;
    int chunk_len;
    int max_blocks;
    int num_pages;
    int max_pos;
    int n_tiles;
    int neg;        // scale < 0: q is negated for the products and c = |scale| log2(e)
    float c;        // |scale| * log2(e)
    int out_fp32;
    uint32_t *flags;
};

namespace {

// q fragments of one head over the workgroup's 32 rows (MFMA B operand, as
// stored: the append kernel has rotated the rows already): this lane's query
// row, dims 16kk + 8*half .. +7.
__device__ __forceinline__ void load_q(const PrefillParams &P, int s, int h, int i_c, int half, u32x4 (&raw)[4]) {
    const uint16_t *qrow = P.q + ((static_cast<int64_t>(s) * P.chunk_len + i_c) * kHQ + h) * kD;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) raw[kk] = *reinterpret_cast<const u32x4 *>(qrow + 16 * kk + 8 * half);
}

// The fragments of one 32-key block, read from LDS (sk, sv: the block's K and
// V rows, swizzled, see swz).
//   kf: K as the A operand of S^T = K Q^T: key l%32, dims 16kk + 8(l/32) .. +7.
//   vf: V^T as the A operand of O^T += V^T P^T over keys 16sb..16sb+15: lane l
//       holds dim 32db + l%32 of the keys its P^T operand pairs with.  The score
//       registers give lane half h the keys 16sb + 4h + {0..3} and
//       16sb + 4h + {8..11} (registers 8sb .. 8sb+7), so two transposing reads
//       of 4 rows each fetch exactly those keys for 16 consecutive dims.
__device__ __forceinline__ void read_k(const unsigned char *sk, int lane, bf16x8 (&kf)[4]) {
    const int qc = lane & 31, half = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        kf[kk] = as_bf16x8(*reinterpret_cast<const u32x4 *>(sk + swz(qc, 2 * kk + half)));
}
__device__ __forceinline__ void read_v(const unsigned char *sv, int lane, bf16x8 (&vf)[2][2]) {
    const int half = lane >> 5;
    const int rq = (lane & 15) >> 2;  // row within the 4-row block
    const int col0 = 16 * ((lane & 31) >> 4) + 4 * (lane & 3);
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const int col = 32 * db + col0;
            const int r0 = 16 * sb + 4 * half + rq;
            const bf16x4 lo = read_tr16(sv + swz(r0, col >> 3) + ((col & 7) << 1));
            const bf16x4 hi = read_tr16(sv + swz(r0 + 8, col >> 3) + ((col & 7) << 1));
            vf[db][sb] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
}

// Dead keys of a block get log-weight -inf, hence weight exactly 0: key
// kb*32 + 8(v/4) + 4*half + v%4 of register v is live iff <= lim_pos (the
// row's position, or the sequence's last key).
__device__ __forceinline__ void mask_block(float (&t)[16], int half, int kb, int lim_pos) {
    const int lim = lim_pos - kb * kKB - 4 * half;
#pragma unroll
    for (int v = 0; v < 16; ++v) t[v] = (8 * (v >> 2) + (v & 3)) > lim ? -INFINITY : t[v];
}

// Weights exp2(t - d) of the lane's 16 log-weights t as bf16 (and, for fp32
// output, the bf16 remainders), and their sum over the same bf16 values.
template <bool kHiLo>
__device__ __forceinline__ float block_weights(const float (&t)[16], float d, bf16x8 (&pb)[2], bf16x8 (&pl)[2]) {
    float bs = 0.0f;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = fast_exp2(t[8 * sb + e] - d);
        uint32_t wh[4], wl[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
            wh[e2] = cvt_pk_bf16(p[2 * e2], p[2 * e2 + 1]);
            if (kHiLo) wl[e2] = cvt_pk_bf16(p[2 * e2] - bf16_lo(wh[e2]), p[2 * e2 + 1] - bf16_hi(wh[e2]));
        }
        pb[sb] = as_bf16x8(u32x4{wh[0], wh[1], wh[2], wh[3]});
        bs = sum8_bf16(pb[sb], bs);
        if (kHiLo) {
            pl[sb] = as_bf16x8(u32x4{wl[0], wl[1], wl[2], wl[3]});
            bs = sum8_bf16(pl[sb], bs);
        }
    }
    return bs;
}

// Softmax in log2 units against a lazily kept, integer-valued reference ref
// (-inf while none of the row's keys so far is live; mc = ref, or 0 then): the
// log-weights are t = c x - mc.  The usual block needs no maximum: the weights
// exp2(t) are accepted when the lane's 16 of them sum to at most 2^8 (so each
// is at most 2^8; an overflow or NaN fails the test too).  Otherwise, and on a
// key half's first block, slow_path moves the reference up by d = ceil of the
// row's largest t where that is positive (or sets it when the row had none),
// multiplies O and l by 2^-d and takes the weights again as exp2(t - d) (each
// <= 1 then).  Integer references keep every factor an exact power of two.
template <bool kHiLo>
__device__ __forceinline__ float slow_path(const float (&t)[16], float &ref, float &l, f32x16 (&o)[2],
                                           bf16x8 (&pb)[2], bf16x8 (&pl)[2]) {
    float tmax = t[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) tmax = fmaxf(tmax, t[v]);
    tmax = max_partner32(tmax);
    const bool has = ref > -INFINITY;
    const bool live = tmax > -INFINITY;
    float d = 0.0f, f = 1.0f;
    if (has) {
        if (tmax > 0.0f) {
            const float r_new = ref + ceilf(tmax);
            d = r_new - ref;
            ref = r_new;
            f = fast_exp2(-d);
        }
    } else if (live) {
        // first live key of the row: O and l are still 0
        d = ceilf(tmax);
        ref = d;
        f = 0.0f;
    }
    l *= f;
    o[0] *= f;
    o[1] *= f;
    return block_weights<kHiLo>(t, d, pb, pl);
}

}  // namespace

// LDS layout of one workgroup: two key halves, each with kNBuf K and V block
// buffers; after the block loop the same bytes hold the partial results the
// two halves exchange.
constexpr int kThreads = 256;                           // 4 waves: 2 head pairs x 2 key halves
constexpr int kNBuf = 4;                                // K/V blocks in LDS per key half (3 in flight)
constexpr int kHalfBytes = 2 * kNBuf * kBlockBytes;     // per key half: K and V, kNBuf buffers each
constexpr int kStageBytes = 2 * kHalfBytes;
constexpr int kMergeOBytes = 4 * 2 * 64 * 16 * 4;   // 4 waves x 2 heads x 64 lanes x 16 floats
constexpr int kMergeMLBytes = 4 * 2 * 64 * 2 * 4;   // (reference, l) per wave, head and lane
constexpr int kSmemBytes = kStageBytes > kMergeOBytes + kMergeMLBytes ? kStageBytes : kMergeOBytes + kMergeMLBytes;
static_assert(kMaxBlocksPrefill <= 2 * kThreads, "page validation takes two table entries per thread");

template <bool kHiLo>
// two workgroups per CU, so each SIMD holds 2 waves (<= 256 VGPRs)
__global__ __launch_bounds__(kThreads, 2) void k_prefill_attn(PrefillParams P) {
    // ids -> (sequence, KV head, tile): the 3 low id bits pick the XCD, which
    // is also the KV head, so every tile of (s, j) runs on XCD j.  An XCD's
    // workgroups are dealt to its 32 CUs in turn, so its p-th workgroup shares
    // a CU with the (p+32)-th: the first 32 take the work list longest first
    // and the next 32 in the reverse order, so that each CU pairs a long tile
    // with a short one (rank r: sequence r / n_tiles, tiles from the highest
    // positions down).
    const int bid = blockIdx.x;
    const int p = bid >> 3;
    const int base = p & ~(kCuPerXcd - 1);
    const int span = min(static_cast<int>(gridDim.x >> 3) - base, kCuPerXcd);  // a last turn may be short
    const int rank = ((p / kCuPerXcd) & 1) ? base + span - 1 - (p - base) : p;
    const int sj = (bid & 7) + 8 * (rank / P.n_tiles);
    const int tile = P.n_tiles - 1 - (rank % P.n_tiles);
    const int j = sj & (kHKV - 1);
    const int s = sj >> 3;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int hp = w & 1;             // head pair: query heads 2hp and 2hp+1 of the group, the wave's two streams
    const int kh = w >> 1;            // key half: waves 0-1 take the first half of the blocks, 2-3 the rest
    const int h0 = j * kGroup + 2 * hp;
    const int C = P.chunk_len;
    const int row0 = tile * kRows;
    const int qc = lane & 31;
    const int half = lane >> 5;

    __shared__ int s_pages[kMaxBlocksPrefill];
    __shared__ __align__(16) unsigned char s_raw[kSmemBytes];

    // ---- prologue ----------------------------------------------------------------
    // Every WG starts at once, so each dependent round trip to memory here adds
    // to the whole call.  After the prefix length, the loads that do not depend
    // on validation all go out together: the block table (two entries per
    // thread, for validation and for LDS), this lane's q rows, the page ids of
    // the first blocks and those blocks' K/V (direct to LDS).  All addresses
    // are clamped into their arrays, so a sequence that then fails validation
    // has read only valid memory; its results are never used.
    const int prefix = P.prefix_lens[s];
    const int64_t lim = min(static_cast<int64_t>(P.max_blocks) * kPage, static_cast<int64_t>(P.max_pos));
    const bool len_ok = prefix >= 0 && static_cast<int64_t>(prefix) + C <= lim;
    const int total = len_ok ? prefix + C : 0;
    const int n_pages = (total + kPage - 1) / kPage;  // <= kMaxBlocksPrefill = twice the WG's thread count
    const int32_t *bt_row = P.bt + static_cast<int64_t>(s) * P.max_blocks;
    int pid0 = 0, pid1 = 0;
    if (tid < n_pages) pid0 = bt_row[tid];
    if (tid + kThreads < n_pages) pid1 = bt_row[tid + kThreads];

    // block ranges: keys needed by this tile are 0 .. prefix + last valid row
    const int prefix_c = len_ok ? prefix : 0;
    const int last_key = prefix_c + min(row0 + kRows, C) - 1;
    const int nb = last_key / kKB + 1;
    const int nb0 = (nb + 1) / 2;  // blocks of the first key half (the loop trip count)
    const int kb_begin = kh ? nb0 : 0;
    const int kb_count = kh ? nb - nb0 : nb0;
    // first block that needs the causal / length mask for some row of the tile
    const int first_masked = (prefix_c + row0) / kKB;

    // this lane's q rows of both heads (padding rows compute on the last row,
    // never stored)
    u32x4 qraw[2][4];
    const int i_c = min(row0 + qc, C - 1);
    const int pos0 = prefix_c + i_c;
    load_q(P, s, h0, i_c, half, qraw[0]);
    load_q(P, s, h0 + 1, i_c, half, qraw[1]);

    // LDS of this key half: K buffers 0 .. kNBuf-1, then V buffers (kBlockBytes
    // each), addressed by arithmetic on the shared array (so every access is
    // known to be an LDS access)
    const int half_off = kh * kHalfBytes;
    auto k_buf = [&](int buf) { return s_raw + half_off + buf * kBlockBytes; };
    auto v_buf = [&](int buf) { return s_raw + half_off + (kNBuf + buf) * kBlockBytes; };
    const uint32_t lds_half = static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) unsigned char *)(s_raw + half_off)));

    // Staging: the 2 waves of a key half each bring one page of the block
    // (wave hp: keys 16hp .. 16hp+15, page 2kb + hp) of K and of V straight
    // into LDS, two 16-byte direct-to-LDS loads per lane and tensor: load r,
    // lane l fills chunk position l%8 of block row 16hp + 8r + l/8, which holds
    // the row's chunk (l%8) ^ f(row) (see swz; f depends on the row mod 8
    // only).  Dead keys (>= total) fetch the first row of the same page (a
    // live one), or of the sequence's first page when the whole page lies past
    // the sequence, so no NaN reaches the MFMAs; blocks past the half's range
    // are clamped (re-read, never used).
    const int64_t tile_j = static_cast<int64_t>(j) * kTile;
    const int st_row8 = lane >> 3;
    const uint32_t st_chunk_b = static_cast<uint32_t>(((lane & 7) ^ swz_f(st_row8)) * 16);
    auto stage_with = [&](int kbl, int buf, int page) {
        const int kb = min(kb_begin + kbl, nb - 1);
        const int64_t base = static_cast<int64_t>(page) * kPageElems + tile_j;
        const int key0 = kb * kKB + 16 * hp + st_row8;
        const uint32_t lds_k = __builtin_amdgcn_readfirstlane(lds_half + buf * kBlockBytes + hp * 16 * 128);
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const uint32_t voff =
                key0 + 8 * r < total ? static_cast<uint32_t>((8 * r + st_row8) * kD * 2) + st_chunk_b : st_chunk_b;
            dma16(P.k_pool + base, voff, lds_k + r * 1024);
            dma16(P.v_pool + base, voff, lds_k + r * 1024 + kNBuf * kBlockBytes);
        }
    };
    // the first blocks, from page ids read straight from the table (scalar
    // loads; ids clamped into the pool)
#pragma unroll
    for (int b = 0; b < kNBuf - 1; ++b) {
        if (b < nb0) {
            const int idx = min(2 * min(kb_begin + b, nb - 1) + hp, P.max_blocks - 1);
            const int idx_c = idx < n_pages ? idx : 0;
            int page = bt_row[__builtin_amdgcn_readfirstlane(idx_c)];
            page = min(max(page, 0), P.num_pages - 1);
            stage_with(b, b, __builtin_amdgcn_readfirstlane(page));
        }
    }

    // ---- validation: the whole sequence's pages ------------------------------
    if (tid < n_pages) s_pages[tid] = pid0;
    if (tid + kThreads < n_pages) s_pages[tid + kThreads] = pid1;
    const int bad = ((tid < n_pages) && (pid0 < 0 || pid0 >= P.num_pages)) ||
                    ((tid + kThreads < n_pages) && (pid1 < 0 || pid1 >= P.num_pages));
    const bool ok = len_ok && __syncthreads_or(bad) == 0;

    if (!ok) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's staging loads have landed
        // zero-fill this tile's rows of both heads (the first key half's waves)
        if (kh != 0) return;
        const int i = row0 + qc;
        if (i < C) {
            for (int u = 0; u < 2; ++u) {
                const int64_t o = ((static_cast<int64_t>(s) * C + i) * kHQ + h0 + u) * kD + 32 * half;
                for (int d = 0; d < 32; ++d) {
                    if (P.out_fp32) static_cast<float *>(P.out)[o + d] = 0.0f;
                    else static_cast<uint16_t *>(P.out)[o + d] = 0;
                }
            }
        }
        if (tid == 0 && j == 0 && tile == P.n_tiles - 1 && P.flags)
            atomicOr(P.flags, len_ok ? kDevErrPageId : kDevErrContextLen);
        return;
    }

    // ---- q fragments (negated for scale < 0) -----------------------------------
    bf16x8 qf[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) qf[u][kk] = as_bf16x8(P.neg ? (qraw[u][kk] ^ 0x80008000u) : qraw[u][kk]);

    // The page of this wave's 16 rows of block kb_begin + i, held by lane i
    // (read back with readlane, so staging in the loop waits for no LDS read);
    // blocks from 64 on (contexts past 4096 keys) look theirs up in LDS.
    auto page_of = [&](int kb) {
        const int idx = 2 * kb + hp;
        return s_pages[idx < n_pages ? idx : 0];
    };
    const int my_page = page_of(min(kb_begin + lane, nb - 1));
    auto stage_block = [&](int kbl, int buf) {
        const int kb = min(kb_begin + kbl, nb - 1);
        const int page = __builtin_amdgcn_readfirstlane(kbl < 64 ? __builtin_amdgcn_readlane(my_page, kbl)
                                                                   : page_of(kb));
        stage_with(kbl, buf, page);
    };

    f32x16 o[2][2] = {{f32x16{}, f32x16{}}, {f32x16{}, f32x16{}}};
    float ref[2] = {-INFINITY, -INFINITY}, l[2] = {0.0f, 0.0f};
    const int lim_pos = min(pos0, total - 1);

    // the first blocks have landed (and the q loads); publish them
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // Software pipeline over this half's blocks, two heads (streams) per wave
    // sharing every K and V fragment.  Iteration kbl: (A) the S^T products of
    // block kbl+1 for both heads go out with the weights of block kbl
    // interleaved between them (the two heads' products alternate, so each
    // waits for no other); (B) after the rare rescales, the P.V products of
    // block kbl go out with the log-weights of block kbl+1 interleaved.  Block
    // b is in buffer b % kNBuf; the loads of block kbl+3 go into the buffer of
    // block kbl-1, which every wave finished before the last barrier.  One
    // barrier per block: before it each wave waits until its loads of block
    // kbl+2 (whose K the next iteration reads) have landed, at most the block
    // after it (4 loads) still in flight.  Both key halves run the same trip
    // count (nb0) so that their barriers pair up; the second half may run out
    // of blocks first (its extra iterations compute on stale buffers and keep
    // nothing).
    float t[2][16];  // log-weights of the block being finished, per head
    {
        bf16x8 kf[4];
        read_k(k_buf(0), lane, kf);
        f32x16 st[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int u = 0; u < 2; ++u) st[u] = mfma32(kf[kk], qf[u][kk], st[u]);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
            for (int v = 0; v < 16; ++v) t[u][v] = st[u][v] * P.c;  // reference 0 (ref is -inf)
            if (kb_begin >= first_masked) mask_block(t[u], half, kb_begin, lim_pos);
        }
    }
    for (int kbl = 0;; ++kbl) {
        const bool more = kbl + kNBuf - 1 < nb0;
        if (more) stage_block(kbl + kNBuf - 1, (kbl + kNBuf - 1) & (kNBuf - 1));

        // ---- (A) next block's S^T, this block's weights
        bf16x8 kf[4];
        read_k(k_buf((kbl + 1) & (kNBuf - 1)), lane, kf);
        bf16x8 pb[2][2], pl[2][2];
        float bs[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) bs[u] = block_weights<kHiLo>(t[u], 0.0f, pb[u], pl[u]);
        f32x16 sn[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int u = 0; u < 2; ++u) sn[u] = mfma32(kf[kk], qf[u][kk], sn[u]);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // the K fragment reads
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x002, kHiLo ? 12 : 8, 0);  // weights
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              // one S^T product
        }
        // the weights are used only on the live path below: an empty asm that
        // reads them keeps the compiler from moving their computation there,
        // out of reach of the products they are interleaved with
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            asm volatile("" ::"v"(__builtin_bit_cast(u32x4, pb[u][0])), "v"(__builtin_bit_cast(u32x4, pb[u][1])),
                         "v"(bs[u]));
            if (kHiLo)
                asm volatile("" ::"v"(__builtin_bit_cast(u32x4, pl[u][0])), "v"(__builtin_bit_cast(u32x4, pl[u][1])));
        }

        if (kbl < kb_count) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                if (kbl == 0 || __builtin_amdgcn_ballot_w64(!(bs[u] <= 256.0f)))
                    bs[u] = slow_path<kHiLo>(t[u], ref[u], l[u], o[u], pb[u], pl[u]);
                l[u] += bs[u];
            }

            // ---- (B) this block's P.V, next block's log-weights
            bf16x8 vf[2][2];
            read_v(v_buf(kbl & (kNBuf - 1)), lane, vf);
            // products chained on one accumulator are 4 apart
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int db = 0; db < 2; ++db) {
                        o[u][db] = mfma32(vf[db][sb], pb[u][sb], o[u][db]);
                        if (kHiLo) o[u][db] = mfma32(vf[db][sb], pl[u][sb], o[u][db]);
                    }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const float mc = ref[u] > -INFINITY ? ref[u] : 0.0f;
#pragma unroll
                for (int v = 0; v < 16; ++v) t[u][v] = fmaf(sn[u][v], P.c, -mc);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 8, 1);  // the V fragment reads
#pragma unroll
            for (int g = 0; g < 8; ++g) {
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 1);              // log-weights
                __builtin_amdgcn_sched_group_barrier(0x008, kHiLo ? 2 : 1, 1);  // P.V products
            }
            const int kbn = kb_begin + kbl + 1;
            if (kbn >= first_masked) {
                mask_block(t[0], half, kbn, lim_pos);
                mask_block(t[1], half, kbn, lim_pos);
            }
        }
        if (kbl + 1 >= nb0) break;
        if (more) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }
    __syncthreads();

    // ---- merge the two key halves through LDS -----------------------------------
    // Key half kh finalizes dims 32kh .. 32kh+31 of both heads: each wave
    // leaves the other half's dims of its partial O^T, with its (reference, l),
    // in LDS.  Slot: (key half, head pair, head, lane), 16 floats.
    float *mo = reinterpret_cast<float *>(s_raw);
    float *mml = reinterpret_cast<float *>(s_raw + kMergeOBytes);
    auto slot = [&](int half_k, int u) { return ((half_k * 2 + hp) * 2 + u) * 64 + lane; };
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const f32x16 give = kh ? o[u][0] : o[u][1];
        float *dst = mo + slot(kh, u) * 16;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
            *reinterpret_cast<f32x4 *>(dst + 4 * r4) = f32x4{give[4 * r4], give[4 * r4 + 1], give[4 * r4 + 2],
                                                             give[4 * r4 + 3]};
        mml[slot(kh, u) * 2] = ref[u];
        mml[slot(kh, u) * 2 + 1] = l[u];
    }
    __syncthreads();

    // ---- out[s][i][h][d] = O^T[d][query] / l, d = 32kh + 8r4 + 4*half + r ------
    const int oh = 1 - kh;
    float fA[2], fB[2], inv[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const float rB = mml[slot(oh, u) * 2];
        const float lB = mml[slot(oh, u) * 2 + 1];
        // finite: the first half always holds key 0; a half that had no live
        // key for a row has reference -inf and weight 0
        const float rx = fmaxf(ref[u], rB);
        fA[u] = fast_exp2(ref[u] - rx);
        fB[u] = fast_exp2(rB - rx);
        const float lh = l[u] * fA[u] + lB * fB[u];
        inv[u] = 1.0f / (lh + partner32(lh));  // every lane takes part in the exchange
    }
    const int i = row0 + qc;
    if (i >= C) return;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const float *src = mo + slot(oh, u) * 16;
        const f32x16 mine = kh ? o[u][1] : o[u][0];
        const int64_t orow = ((static_cast<int64_t>(s) * C + i) * kHQ + h0 + u) * kD;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const f32x4 ob = *reinterpret_cast<const f32x4 *>(src + 4 * r4);
            const int d = 32 * kh + 8 * r4 + 4 * half;
            const float y0 = (mine[4 * r4] * fA[u] + ob[0] * fB[u]) * inv[u];
            const float y1 = (mine[4 * r4 + 1] * fA[u] + ob[1] * fB[u]) * inv[u];
            const float y2 = (mine[4 * r4 + 2] * fA[u] + ob[2] * fB[u]) * inv[u];
            const float y3 = (mine[4 * r4 + 3] * fA[u] + ob[3] * fB[u]) * inv[u];
            if (P.out_fp32) {
                *reinterpret_cast<f32x4 *>(static_cast<float *>(P.out) + orow + d) = f32x4{y0, y1, y2, y3};
            } else {
                const uint2 pk = {pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
                *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(P.out) + orow + d) = pk;
            }
        }
    }
}

hipError_t launch_prefill_attention(const PrefillLaunch &p, hipStream_t stream) {
    if (p.num_seqs == 0 || p.chunk_len == 0) return hipSuccess;
    if (p.max_blocks > kMaxBlocksPrefill) return hipErrorInvalidValue;
    PrefillParams P{};
    P.out = p.out;
    P.q = static_cast<const uint16_t *>(p.q);
    P.k_pool = static_cast<const uint16_t *>(p.k_pool);
    P.v_pool = static_cast<const uint16_t *>(p.v_pool);
    P.bt = p.block_tables;
    P.prefix_lens = p.prefix_lens;
    P.chunk_len = p.chunk_len;
    P.max_blocks = p.max_blocks;
    P.num_pages = p.num_pages;
    P.max_pos = p.max_pos;
    P.n_tiles = (p.chunk_len + kRows - 1) / kRows;
    // Scores are taken in units of c = |scale| log2(e) (q is negated when
    // scale < 0).  c is kept >= 1e-30 so that a masked score of -inf always
    // maps to weight 0; for scale == 0 the weights are then exp2(~0) = 1, the
    // uniform average the definition gives.
    const float c = p.scale * 1.4426950408889634f;
    P.neg = c < 0.0f;
    P.c = fmaxf(fabsf(c), 1e-30f);
    P.out_fp32 = p.out_fp32;
    P.flags = p.flags;
    const int64_t blocks = static_cast<int64_t>(p.num_seqs) * kHKV * P.n_tiles;
    if (p.out_fp32)
        hipLaunchKernelGGL(k_prefill_attn<true>, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream, P);
    else
        hipLaunchKernelGGL(k_prefill_attn<false>, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream, P);
    return hipGetLastError();
}

}  // namespace pa
