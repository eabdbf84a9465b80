// pa_append.hip -- KV append with rotary embedding into the paged pool.
//
// samir-vllm article, section "Gestion de la KV cache et strategies de
// batching": a new token's K and V go into the page that the sequence's block
// table names for its position, at the absolute RoPE position.  One workgroup
// per appended token: it resolves (page, slot) once, rotates the 8 K heads and
// (optionally) the 32 q heads with the fp64 cos/sin table row of that
// position (rope_pair_bf16), and copies V verbatim.  The kernel moves ~10 KiB per token with q, so
// it is bound by latency (length, then block table, then stores), not
// bandwidth; its accesses are fully coalesced (consecutive lanes touch
// consecutive bf16 elements).
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// token = blockIdx.x = s * tokens_per_seq + i.
//   decode (prefix_mode == 0): pos = lens[s] - 1   (tokens_per_seq == 1)
//   prefill (prefix_mode == 1): pos = lens[s] + i  (lens holds prefix lengths)
// Work in units of 4 pairs: K is 8 heads x 8 units (threads 0..63), V 8 heads
// x 8 sixteen-byte chunks copied verbatim (threads 64..127), q 32 heads x 8
// units in place (one per thread).  The rows depend on the token alone, so
// their loads go out first, beside the length's; the table row waits for the
// length and the stores for the page id, and a token that fails either check
// writes nothing.
__global__ __launch_bounds__(256) void k_append_rope(uint16_t *__restrict__ q, const uint16_t *__restrict__ k_new,
                                                     const uint16_t *__restrict__ v_new, uint16_t *__restrict__ k_pool,
                                                     uint16_t *__restrict__ v_pool, const int32_t *__restrict__ bt,
                                                     const int32_t *__restrict__ lens, const double *__restrict__ rope,
                                                     int tokens_per_seq, int prefix_mode, int max_blocks, int num_pages,
                                                     int max_pos, uint32_t *__restrict__ flags) {
    const int tok = blockIdx.x;
    const int s = tok / tokens_per_seq;
    const int i = tok - s * tokens_per_seq;
    const int t = threadIdx.x;
    const int i0 = 4 * (t & 7);
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
        vv = reinterpret_cast<const u32x4 *>(v_new + krow)[t & 7];
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
    const int64_t prow = ((static_cast<int64_t>(page) * kHKV + j) * kPage + slot) * kD;
    if (t < 64) {
        uint2 lo, hi;
        rope4(ka, kb, tb, lo, hi);
        *reinterpret_cast<uint2 *>(k_pool + prow + i0) = lo;
        *reinterpret_cast<uint2 *>(k_pool + prow + i0 + kD / 2) = hi;
    } else if (t < 128) {
        reinterpret_cast<u32x4 *>(v_pool + prow)[t & 7] = vv;
    }
    if (q) {
        uint2 lo, hi;
        rope4(qa, qb, tb, lo, hi);
        *reinterpret_cast<uint2 *>(qrow + i0) = lo;
        *reinterpret_cast<uint2 *>(qrow + i0 + kD / 2) = hi;
    }
}

hipError_t launch_append_rope(const AppendLaunch &a, hipStream_t stream) {
    const int64_t tokens = static_cast<int64_t>(a.num_seqs) * a.tokens_per_seq;
    if (tokens == 0) return hipSuccess;
    hipLaunchKernelGGL(k_append_rope, dim3(static_cast<unsigned>(tokens)), dim3(256), 0, stream,
                       static_cast<uint16_t *>(a.q), static_cast<const uint16_t *>(a.k_new),
                       static_cast<const uint16_t *>(a.v_new), static_cast<uint16_t *>(a.k_pool),
                       static_cast<uint16_t *>(a.v_pool), a.block_tables, a.lens, a.rope, a.tokens_per_seq,
                       a.prefix_mode, a.max_blocks, a.num_pages, a.max_pos, a.flags);
    return hipGetLastError();
}

}  // namespace pa
