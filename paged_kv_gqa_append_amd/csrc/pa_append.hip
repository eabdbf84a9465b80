// pa_append.hip -- KV append with rotary embedding into the paged pool.
//
// samir-vllm article, section "Gestion de la KV cache et strategies de
// batching": a new token's K and V go into the page that the sequence's block
// table names for its position, at the absolute RoPE position.  One workgroup
// per appended token: it resolves (page, slot) once, rotates the 8 K heads and
// (optionally) the 32 q heads with the fp64 cos/sin table row of that
// position (rope_pair_bf16), and copies V verbatim.  The kernel moves ~6 KiB per token, so it is
// bound by launch latency, not bandwidth; it stays simple and fully coalesced
// (consecutive lanes touch consecutive bf16 elements).
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// Rotate-half pair (x_i, x_{i+32}) of a row by (c, s) (rope_pair_bf16).
__device__ __forceinline__ void rope_pair(const uint16_t *src, uint16_t *dst, int i, double c, double s) {
    uint16_t lo, hi;
    rope_pair_bf16(bf16_to_f32(src[i]), bf16_to_f32(src[i + kD / 2]), c, s, lo, hi);
    dst[i] = lo;
    dst[i + kD / 2] = hi;
}

// token = blockIdx.x = s * tokens_per_seq + i.
//   decode (prefix_mode == 0): pos = lens[s] - 1   (tokens_per_seq == 1)
//   prefill (prefix_mode == 1): pos = lens[s] + i  (lens holds prefix lengths)
__global__ __launch_bounds__(256) void k_append_rope(uint16_t *__restrict__ q, const uint16_t *__restrict__ k_new,
                                                     const uint16_t *__restrict__ v_new, uint16_t *__restrict__ k_pool,
                                                     uint16_t *__restrict__ v_pool, const int32_t *__restrict__ bt,
                                                     const int32_t *__restrict__ lens, const double *__restrict__ rope,
                                                     int tokens_per_seq, int prefix_mode, int max_blocks, int num_pages,
                                                     int max_pos, uint32_t *__restrict__ flags) {
    const int tok = blockIdx.x;
    const int s = tok / tokens_per_seq;
    const int i = tok - s * tokens_per_seq;
    const int64_t len = lens[s];
    const int64_t pos = prefix_mode ? len + i : len - 1;
    const bool bad_len = prefix_mode ? (len < 0) : (len < 1);
    if (bad_len || pos >= static_cast<int64_t>(max_blocks) * kPage || pos >= max_pos) {
        if (threadIdx.x == 0 && flags) atomicOr(flags, kDevErrContextLen);
        return;
    }
    const int page = bt[static_cast<int64_t>(s) * max_blocks + (pos >> 4)];
    if (page < 0 || page >= num_pages) {
        if (threadIdx.x == 0 && flags) atomicOr(flags, kDevErrPageId);
        return;
    }
    const int slot = static_cast<int>(pos & (kPage - 1));
    const double *cs = rope + pos * kD;  // [32][2]
    const int t = threadIdx.x;

    // K: 8 heads x 32 pairs, one pair per thread.
    {
        const int j = t >> 5, p = t & 31;
        const uint16_t *src = k_new + (static_cast<int64_t>(tok) * kHKV + j) * kD;
        uint16_t *dst = k_pool + ((static_cast<int64_t>(page) * kHKV + j) * kPage + slot) * kD;
        rope_pair(src, dst, p, cs[2 * p], cs[2 * p + 1]);
    }
    // V: 8 heads x 64 elements, two per thread, verbatim.
    {
        const int j = t >> 5, w = t & 31;
        const uint32_t *src = reinterpret_cast<const uint32_t *>(v_new + (static_cast<int64_t>(tok) * kHKV + j) * kD);
        uint32_t *dst = reinterpret_cast<uint32_t *>(v_pool + ((static_cast<int64_t>(page) * kHKV + j) * kPage + slot) * kD);
        dst[w] = src[w];
    }
    // q: 32 heads x 32 pairs, four per thread, in place.
    if (q) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int idx = t + 256 * r;
            const int h = idx >> 5, p = idx & 31;
            uint16_t *row = q + (static_cast<int64_t>(tok) * kHQ + h) * kD;
            rope_pair(row, row, p, cs[2 * p], cs[2 * p + 1]);
        }
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
