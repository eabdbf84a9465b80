// pa_decode_core.h -- the lane-level machinery of the paged decode kernels
// (bf16 and INT8 pages), shared so that both compute scores, softmax and the
// split-context merge with the same operations in the same order.
//
// Lane roles (a wave of 64 lanes, lane = 8g + c): every lane holds, for tokens
// g and g+8 of a 16-token page, the 8-element chunk c*8..c*8+7 of K and V, in
// slot orders permuted by its lane bits so that reduce-scatters and weight
// broadcasts over the 8 lanes of a group need no selects (see page_score,
// softmax_step and accumulate).
#pragma once

#include <math.h>

#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

constexpr int kMaxPartPages = 128;
// Grid sizes (workgroups per launch) from which the page loads carry the
// non-temporal hint (bf16: with whole-row loads; INT8: on the code loads).
constexpr int64_t kNtMinBlocks = 128;
// Grid sizes up to which the INT8 kernel levels its wave priorities.
constexpr int64_t kPrioMaxBlocksI8 = 1024;
constexpr float kNegBig = -1.0e30f;   // running-max start (finite, so 2^(x - m) is never NaN)
constexpr float kRescaleLog2 = 8.0f;  // lazy-rescale threshold

// quad_perm broadcasts of quad lane a to the whole quad: [a,a,a,a]
constexpr int kBcast0 = 0x00, kBcast1 = 0x55, kBcast2 = 0xAA, kBcast3 = 0xFF;
constexpr int kXor1 = 0xB1, kXor2 = 0x4E, kHalfMirror = 0x141, kRowRor8 = 0x128;

// Dispatch order, passed by value in the launch arguments.  Workgroups
// 8i .. 8i+7 (the 8 KV heads) serve item[i] = (sequence << 6) | partition;
// the item depends on the workgroup id alone, so its load from the launch
// arguments goes out with the parameters' and adds no step to a workgroup's
// start.  The unordered form is empty: workgroup b serves (sequence, KV head)
// b / num_parts and partition b % num_parts.
constexpr int kOrderPartBits = 6;
static_assert((1 << kOrderPartBits) == kMaxOrderParts, "partition field of a dispatch item");
template <bool kOrd>
struct DispatchOrder {};
template <>
struct DispatchOrder<true> {
    uint16_t item[kMaxDispatchOrder];
};

// A dispatch order in device memory, int32[n] (pa_order_by_length writes
// one): workgroups 8i .. 8i+7 serve partition i % num_parts of sequence
// ord[i / num_parts].  One uniform load, L2-resident after the launch's first
// workgroups, stands before the block-table row; against the order in the
// launch arguments it also keeps the arguments small (2 KiB less to set up per
// launch).  An entry outside [0, n) makes its workgroups flag the error and
// do nothing else.
struct DeviceOrder {
    const int32_t *ord;
    int n;
};

struct WgCoords {
    int s, j, part;
};

template <bool kOrd>
__device__ __forceinline__ WgCoords wg_coords(const DispatchOrder<kOrd> &o, int num_parts) {
    const int b = blockIdx.x;
    if constexpr (kOrd) {
        const int item = o.item[b >> 3];
        return {item >> kOrderPartBits, b & (kHKV - 1), item & (kMaxOrderParts - 1)};
    } else {
        const int sj = b / num_parts;
        return {sj >> 3, sj & (kHKV - 1), b % num_parts};
    }
}

__device__ __forceinline__ WgCoords wg_coords(const DeviceOrder &o, int num_parts) {
    const int b = blockIdx.x;
    const int i = b >> 3;
    const int r = num_parts == 1 ? i : i / num_parts;
    const int s = __builtin_amdgcn_readfirstlane(o.ord[r]);
    return {s, b & (kHKV - 1), i - r * num_parts};
}

// whether the workgroup's sequence index came from a valid order entry
template <class Ord>
__device__ __forceinline__ bool order_entry_ok(const Ord &o, int s) {
    if constexpr (std::is_same_v<Ord, DeviceOrder>) return static_cast<unsigned>(s) < static_cast<unsigned>(o.n);
    else return true;
}

// The ordered form for a host-checked permutation of the n sequences, with
// n * num_parts <= kMaxDispatchOrder and num_parts <= kMaxOrderParts: each
// sequence's partitions follow one another, in the given sequence order.
inline DispatchOrder<true> make_dispatch_order(const int32_t *order, int n, int num_parts) {
    DispatchOrder<true> o{};
    int k = 0;
    for (int i = 0; i < n; ++i)
        for (int p = 0; p < num_parts; ++p) o.item[k++] = static_cast<uint16_t>((order[i] << kOrderPartBits) | p);
    return o;
}

// a page's K and V chunks of one lane, in load order (two loads of each tile)
struct KVRegs {
    u32x4 k0, k1, v0, v1;
};

// Lane pairs (i, i^16) and (i, i^32) through the gfx950 row-swap permutes: with
// the same value in both operands, the two results hold the lower and the upper
// partner's value in every lane.  Two hipcc 7.2 pitfalls are avoided: the
// second operand passes through an empty asm, because a swap of two operands
// known to be equal is folded into two equal results (wrong for these row-wise
// exchanges), and each result is copied to a scalar before it is reinterpreted,
// because __builtin_bit_cast of a vector element is lowered as a load of
// element 0.
__device__ __forceinline__ void xor16_pair(float v, float &lo, float &hi) {
    const unsigned a = __builtin_bit_cast(unsigned, v);
    unsigned b = a;
    asm volatile("" : "+v"(b));
    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    const unsigned r0 = r[0], r1 = r[1];
    lo = __builtin_bit_cast(float, r0);
    hi = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ void xor32_pair(float v, float &lo, float &hi) {
    const unsigned a = __builtin_bit_cast(unsigned, v);
    unsigned b = a;
    asm volatile("" : "+v"(b));
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    const unsigned r0 = r[0], r1 = r[1];
    lo = __builtin_bit_cast(float, r0);
    hi = __builtin_bit_cast(float, r1);
}

// Reduce-scatter step on a pair of values through a row-swap permute: after
// swap(x, y) the lanes of the lower row (or half) hold their own x and their
// partner's x, the upper ones their partner's y and their own y, so x' + y' is
// the pair sum of x in the lower lanes and of y in the upper lanes.
__device__ __forceinline__ float swap16_sum(float x, float y) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, y),
                                                    false, false);
    const unsigned r0 = r[0], r1 = r[1];
    return __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ float swap32_sum(float x, float y) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, y),
                                                    false, false);
    const unsigned r0 = r[0], r1 = r[1];
    return __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
}

// Sum over the 8 lane groups (lanes c, c+8, ..., c+56); every lane gets it.
__device__ __forceinline__ float sum_groups(float v) {
    float lo, hi;
    v += dpp_f32<kRowRor8>(v);
    xor16_pair(v, lo, hi);
    v = lo + hi;
    xor32_pair(v, lo, hi);
    return lo + hi;
}
__device__ __forceinline__ float max_groups(float v) {
    float lo, hi;
    v = fmaxf(v, dpp_f32<kRowRor8>(v));
    xor16_pair(v, lo, hi);
    v = fmaxf(lo, hi);
    xor32_pair(v, lo, hi);
    return fmaxf(lo, hi);
}

// Score of the lane's own (token, head) pair for one page: partial dots of the
// lane's 8-element chunk for the 8 pairs of its group (slot i < 4: token half
// t0, head i^hm; slot i >= 4: token half t0^1), then a reduce-scatter over the
// 8 lanes with partners c^1, c^2 and c^7.  Returns scale*log2(e)*<q, k>.
__device__ __forceinline__ float page_score(const u32x4 (&qv)[kGroup], u32x4 ka, u32x4 kb, float scale_log2) {
    float sa[kGroup], sb[kGroup];
#pragma unroll
    for (int m = 0; m < kGroup; ++m) {
        sa[m] = dot8_bf16(qv[m], ka, 0.0f);
        sb[m] = dot8_bf16(qv[m], kb, 0.0f);
    }
    const float r0 = sa[0] + dpp_f32<kXor1>(sb[0]);
    const float r1 = sa[1] + dpp_f32<kXor1>(sb[1]);
    const float r2 = sa[2] + dpp_f32<kXor1>(sb[2]);
    const float r3 = sa[3] + dpp_f32<kXor1>(sb[3]);
    const float u0 = r0 + dpp_f32<kXor2>(r2);
    const float u1 = r1 + dpp_f32<kXor2>(r3);
    return (u0 + dpp_f32<kHalfMirror>(u1)) * scale_log2;
}

// Online-softmax step for one page: lazily raise the wave's running max of the
// lane's head (rescaling the accumulators of all 4 heads when any lane needs
// it), then return the lane's weight 2^(x - m).  With kSecondSum a second
// per-lane running sum of the lane's head (l2_run) is rescaled with l_run.
template <bool kSecondSum>
__device__ __forceinline__ float softmax_step_t(float x, float &m_run, float &l_run, float &l2_run,
                                                float (&acc)[kGroup][8]) {
    const float xm = fmaxf(x, dpp_f32<kXor1>(x));  // this page's max for the head (both tokens)
    if (__builtin_amdgcn_ballot_w64(xm > m_run + kRescaleLog2)) {
        const float wm = max_groups(xm);
        const float mn = wm > m_run + kRescaleLog2 ? wm : m_run;
        const float f = fast_exp2(m_run - mn);
        m_run = mn;
        l_run *= f;
        if (kSecondSum) l2_run *= f;
        // factors per accumulator slot, routed like the weights in accumulate()
        const float fm = dpp_f32<kHalfMirror>(f);
        const float F0 = dpp_f32<kBcast0>(f), F2 = dpp_f32<kBcast2>(f);
        const float G0 = dpp_f32<kBcast0>(fm), G2 = dpp_f32<kBcast2>(fm);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            acc[0][i] *= F0;
            acc[1][i] *= G0;
            acc[2][i] *= F2;
            acc[3][i] *= G2;
        }
    }
    const float pw = fast_exp2(x - m_run);
    l_run += pw;
    return pw;
}
__device__ __forceinline__ float softmax_step(float x, float &m_run, float &l_run, float (&acc)[kGroup][8]) {
    float unused = 0.0f;
    return softmax_step_t<false>(x, m_run, l_run, unused, acc);
}

__device__ __forceinline__ void unpack8(u32x4 v, float (&f)[8]) {
    const uint32_t a[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        f[2 * k] = bf16_lo(a[k]);
        f[2 * k + 1] = bf16_hi(a[k]);
    }
}

// acc[e] += sum over the group's 8 (token, head) weights of w * V[token]: P_a is
// the weight held by quad lane a, Q_a that of its mirror lane; V slot u (va/vb)
// and accumulator slot e are permuted by the lane bits so that quad lane a's
// pair always lands in slot e = 2*(a>>1) with V slot a&1 (Q_a: e + 1).
__device__ __forceinline__ void accumulate(float pw, const float (&va)[8], const float (&vb)[8],
                                           float (&acc)[kGroup][8]) {
    const float pm = dpp_f32<kHalfMirror>(pw);
    const float P0 = dpp_f32<kBcast0>(pw), P1 = dpp_f32<kBcast1>(pw);
    const float P2 = dpp_f32<kBcast2>(pw), P3 = dpp_f32<kBcast3>(pw);
    const float Q0 = dpp_f32<kBcast0>(pm), Q1 = dpp_f32<kBcast1>(pm);
    const float Q2 = dpp_f32<kBcast2>(pm), Q3 = dpp_f32<kBcast3>(pm);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        acc[0][i] = fmaf(P0, va[i], fmaf(P1, vb[i], acc[0][i]));
        acc[1][i] = fmaf(Q0, va[i], fmaf(Q1, vb[i], acc[1][i]));
        acc[2][i] = fmaf(P2, va[i], fmaf(P3, vb[i], acc[2][i]));
        acc[3][i] = fmaf(Q2, va[i], fmaf(Q3, vb[i], acc[3][i]));
    }
}

struct DecodeParams {
    void *out;
    uint16_t *q;
    const uint16_t *k_new;
    const uint16_t *v_new;
    uint16_t *k_pool;
    uint16_t *v_pool;
    const int32_t *bt;
    const int32_t *lens;
    const double *rope;
    int max_blocks;
    int num_pages;
    int max_pos;
    float scale_log2;
    int out_fp32;
    int part_pages;
    int num_parts;
    int write_q;          // fused only: store the rotated q back (out does not alias q)
    float *ws_ml;
    float *ws_acc;
    uint32_t *flags;
};

// One wave per (sequence, query head): merge that head's partitions.  In the
// fused variant it also stores the rotated q row (all partitions have read q).
template <bool kFused>
__global__ __launch_bounds__(64) void k_decode_merge(DecodeParams P) {
    const int s = blockIdx.x / kHQ;
    const int qh = blockIdx.x % kHQ;
    const int d = threadIdx.x;
    const int L = P.lens[s];
    bool len_ok = (L >= 1) && (L <= P.max_blocks * kPage);
    if (kFused) len_ok = len_ok && (L - 1 < P.max_pos);
    if (!len_ok) return;  // zero-filled by the partial kernel
    const int n_pages = (L + kPage - 1) / kPage;
    const int n_parts_s = (n_pages + P.part_pages - 1) / P.part_pages;
    if (n_parts_s <= 1) return;  // written directly by the partial kernel
    const int32_t *bt_row = P.bt + static_cast<int64_t>(s) * P.max_blocks;
    int bad = 0;
    for (int b = d; b < n_pages; b += 64) bad |= (bt_row[b] < 0) | (bt_row[b] >= P.num_pages);
    if (__syncthreads_or(bad)) return;
    const int64_t row0 = (static_cast<int64_t>(s) * kHQ + qh) * P.num_parts;
    float M = kNegBig;
    for (int k = 0; k < n_parts_s; ++k) M = fmaxf(M, P.ws_ml[(row0 + k) * 2]);
    float Ls = 0.0f, A = 0.0f;
    for (int k = 0; k < n_parts_s; ++k) {
        const float wgt = fast_exp2(P.ws_ml[(row0 + k) * 2] - M);
        Ls = fmaf(wgt, P.ws_ml[(row0 + k) * 2 + 1], Ls);
        A = fmaf(wgt, P.ws_acc[(row0 + k) * kD + d], A);
    }
    const int64_t o = (static_cast<int64_t>(s) * kHQ + qh) * kD + d;
    if (kFused && P.write_q) {
        const int pos = L - 1;
        const int i = d & 31;
        const double co = P.rope[static_cast<int64_t>(pos) * kD + 2 * i];
        const double si = P.rope[static_cast<int64_t>(pos) * kD + 2 * i + 1];
        uint16_t *qr = P.q + o - d;
        // pair (i, i + 32): this thread keeps the half it owns
        uint16_t lo, hi;
        rope_pair_bf16(bf16_to_f32(qr[i]), bf16_to_f32(qr[i + 32]), co, si, lo, hi);
        __syncthreads();  // both halves read before either is written
        qr[d] = d >= 32 ? hi : lo;
    }
    const float r = A / Ls;
    if (P.out_fp32) static_cast<float *>(P.out)[o] = r;
    else static_cast<uint16_t *>(P.out)[o] = f32_to_bf16(r);
}

}  // namespace pa
