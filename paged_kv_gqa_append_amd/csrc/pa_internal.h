// pa_internal.h -- launch descriptors passed from the C-ABI layer to the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

struct AppendLaunch {
    void *q;              // may be null
    const void *k_new;
    const void *v_new;
    void *k_pool;
    void *v_pool;
    const int32_t *block_tables;
    const int32_t *lens;  // context lengths (decode) or prefix lengths (prefill)
    const double *rope;
    int num_seqs;
    int tokens_per_seq;
    int prefix_mode;      // 0: pos = lens[s]-1, 1: pos = lens[s]+i
    int max_blocks;
    int num_pages;
    int max_pos;
    uint32_t *flags;
};

// Bounds of a dispatch order: at most kMaxDispatchOrder (sequence, partition)
// items (16-bit entries in the launch arguments, 2 KiB), and at most
// kMaxOrderParts partitions per sequence (the item's low 6 bits).
constexpr int kMaxDispatchOrder = 1024;
constexpr int kMaxOrderParts = 64;

struct DecodeLaunch {
    void *out;
    void *q;              // read-only unless fused (then rotated in place when write_q)
    const void *k_new;    // fused only
    const void *v_new;    // fused only
    const double *rope;    // fused only
    int max_pos;          // fused only
    int fused;            // 1: append the token at L-1 and rotate q first
    int write_q;          // fused only: store the rotated q (out does not alias q)
    void *k_pool;
    void *v_pool;
    const int32_t *block_tables;
    const int32_t *context_lens;
    int num_seqs;
    int max_blocks;
    int num_pages;
    float scale;
    int out_fp32;
    int part_pages;       // pages per context partition
    int num_parts;        // ceil(max_blocks / part_pages)
    float *ws_ml;         // [B][32][num_parts][2]  (max in log2 units, sum of weights)
    float *ws_acc;        // [B][32][num_parts][64]
    uint32_t *flags;
    const int32_t *order; // host dispatch order (a checked permutation), or NULL
    const int32_t *order_dev; // device dispatch order int32[num_seqs], or NULL (not with order)
};

struct PrefillLaunch {
    void *out;
    const void *q;        // rotated (by the append kernel of the same call)
    const void *k_pool;
    const void *v_pool;
    const int32_t *block_tables;
    const int32_t *prefix_lens;
    int num_seqs;
    int chunk_len;
    int max_blocks;
    int num_pages;
    int max_pos;
    float scale;
    int out_fp32;
    uint32_t *flags;
};

// Largest block table the prefill kernel stages in LDS (8192 tokens).
constexpr int kMaxBlocksPrefill = 512;

// Decode partition size in pages (fixed per process; the default can be
// overridden with PA_DECODE_PART_PAGES for tuning runs).
int decode_part_pages();

hipError_t launch_append_rope(const AppendLaunch &a, hipStream_t stream);
hipError_t launch_decode(const DecodeLaunch &d, hipStream_t stream);
// A longest-first dispatch order of n <= kMaxDispatchOrder sequences, written
// on the device from their device-resident lengths, dealt in runs of long_run
// long and short_run short sequences (pa_order_by_length).
hipError_t launch_order_by_length(const int32_t *lens, int n, int max_blocks, int long_run, int short_run,
                                  int32_t *order, hipStream_t stream);
hipError_t launch_prefill_attention(const PrefillLaunch &p, hipStream_t stream);
// Chunked prefill attention over an INT8 tile pool (PrefillLaunch::k_pool;
// v_pool unused), after the chunk has been appended into it.
hipError_t launch_prefill_attention_i8(const PrefillLaunch &p, hipStream_t stream);

// INT8 K/V pages (pa_i8.hip).  The tile pool travels in k_pool; v_pool is unused.
hipError_t launch_append_rope_i8(const AppendLaunch &a, hipStream_t stream);
hipError_t launch_decode_i8(const DecodeLaunch &d, hipStream_t stream);
// argmax over logit rows (pa_argmax.hip)
int argmax_chunk_elems(bool bf16);
hipError_t launch_argmax(int32_t *out, const void *logits, int rows, int vocab, bool bf16, bool vec, void *workspace,
                         hipStream_t stream);

// Contiguous-read probe over [buf, buf + bytes), bytes a multiple of 16.
hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream);
hipError_t launch_quantize_pages_i8(void *pool, const void *k_pool, const void *v_pool, const int32_t *page_ids,
                                    int count, int num_pages, uint32_t *flags, hipStream_t stream);

}  // namespace pa
