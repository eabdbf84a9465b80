// pa_api.hip -- the C ABI of libpa.so: argument checks, workspace sizing, launches.
//
// Every entry point validates what the host can see (pointers, sizes,
// alignment, geometry) and returns a status before launching anything; see
// include/pa.h for the contract.  Nothing here allocates or synchronises.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "pa.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t decode_num_parts(int32_t max_blocks) {
    const int pp = pa::decode_part_pages();
    return (static_cast<int64_t>(max_blocks) + pp - 1) / pp;
}


static_assert(PA_MAX_DISPATCH_ORDER == pa::kMaxDispatchOrder, "dispatch order bound");

// A dispatch order: at most PA_MAX_DISPATCH_ORDER entries, each of 0 .. n-1 once.
bool is_permutation(const int32_t *order, int32_t n) {
    if (n > PA_MAX_DISPATCH_ORDER) return false;
    bool seen[PA_MAX_DISPATCH_ORDER] = {};
    for (int32_t i = 0; i < n; ++i) {
        const int32_t s = order[i];
        if (s < 0 || s >= n || seen[s]) return false;
        seen[s] = true;
    }
    return true;
}

// Shared argument checks and launch of the plain and the append-fused decode,
// over bf16 pools (k_pool, v_pool) or an INT8 tile pool (k_pool; v_pool unused).
pa_status decode_common(void *out, void *q, const void *k_new, const void *v_new, void *k_pool, void *v_pool,
                        const int32_t *block_tables, const int32_t *context_lens, const double *rope,
                        int32_t num_seqs, int32_t max_blocks, int32_t num_pages, int32_t page_size, int32_t max_pos,
                        float scale, int32_t out_dtype, void *workspace, size_t workspace_bytes,
                        uint32_t *device_flags, const int32_t *order, const int32_t *order_dev,
                        hipStream_t stream, bool fused, bool i8 = false) {
    if (i8) v_pool = k_pool;
    if (num_seqs < 0 || max_blocks < 1 || num_pages < 1 || !isfinite(scale)) return PA_ERR_INVALID_ARG;
    if (order && order_dev) return PA_ERR_INVALID_ARG;
    if (order && (!is_permutation(order, num_seqs) || decode_num_parts(max_blocks) > pa::kMaxOrderParts ||
                  static_cast<int64_t>(num_seqs) * decode_num_parts(max_blocks) > PA_MAX_DISPATCH_ORDER))
        return PA_ERR_INVALID_ARG;
    if (fused && max_pos < 1) return PA_ERR_INVALID_ARG;
    if (page_size != PA_PAGE_SIZE) return PA_ERR_UNSUPPORTED;
    if (out_dtype != PA_OUT_BF16 && out_dtype != PA_OUT_FP32) return PA_ERR_UNSUPPORTED;
    if (num_seqs == 0) return PA_OK;
    if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens) return PA_ERR_INVALID_ARG;
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(block_tables) ||
        !aligned16(context_lens) || !aligned16(order_dev))
        return PA_ERR_INVALID_ARG;
    if (fused && (!k_new || !v_new || !rope || !aligned16(k_new) || !aligned16(v_new) || !aligned16(rope)))
        return PA_ERR_INVALID_ARG;
    const int64_t np = decode_num_parts(max_blocks);
    const size_t need = pa_decode_workspace_bytes(num_seqs, max_blocks);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace))) return PA_ERR_WORKSPACE;
    float *ws = static_cast<float *>(workspace);
    const int64_t rows = static_cast<int64_t>(num_seqs) * PA_NUM_Q_HEADS * np;
    pa::DecodeLaunch d{};
    d.out = out;
    d.q = q;
    d.k_new = k_new;
    d.v_new = v_new;
    d.rope = rope;
    d.max_pos = max_pos;
    d.fused = fused;
    d.write_q = fused && out != q;
    d.k_pool = k_pool;
    d.v_pool = v_pool;
    d.block_tables = block_tables;
    d.context_lens = context_lens;
    d.num_seqs = num_seqs;
    d.max_blocks = max_blocks;
    d.num_pages = num_pages;
    d.scale = scale;
    d.out_fp32 = out_dtype == PA_OUT_FP32;
    d.part_pages = pa::decode_part_pages();
    d.num_parts = static_cast<int>(np);
    d.ws_ml = need ? ws : nullptr;
    d.ws_acc = need ? ws + rows * 2 : nullptr;
    d.flags = device_flags;
    d.order = order;
    d.order_dev = order_dev;
    return (i8 ? pa::launch_decode_i8(d, stream) : pa::launch_decode(d, stream)) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

// ---- the no-allocation decode entry point's scratch ------------------------
// Decode partials of pa_append_decode_gqa_noalloc live in this file-scope
// device array instead of a caller workspace: PA_NOALLOC_SCRATCH_BYTES per
// GPU, held by each GPU the library runs on until the process ends.  In host
// code the array's name is only a stand-in; the device address is looked up
// once per device with hipGetSymbolAddress (with that device current) and
// kept in g_scratch_ptr, and only that pointer is ever handed to a kernel.
static __device__ __align__(256) float scratch[PA_NOALLOC_SCRATCH_BYTES / sizeof(float)];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxScratchDevices] = {};

// The scratch array's device address on the current device (nullptr on failure).
void *scratch_on_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char *pa_status_string(int status) {
    switch (status) {
        case PA_OK: return "PA_OK";
        case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG";
        case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
        case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE";
        case PA_ERR_HIP: return "PA_ERR_HIP";
        case PA_ERR_REJECTED: return "PA_ERR_REJECTED";
        default: return "PA_ERR_UNKNOWN";
    }
}

int32_t pa_abi_version(void) { return PA_ABI_VERSION; }

// The build id travels in the binary behind a marker, so that the build script
// can also read it from the file without loading the library.
#ifndef PA_BUILD_ID
#define PA_BUILD_ID "0000000000000000000000000000000000000000000000000000000000000000"
#endif
static const char kBuildIdTag[] = "pa-build-id:" PA_BUILD_ID;

const char *pa_build_id(void) { return kBuildIdTag + sizeof("pa-build-id:") - 1; }

int32_t pa_get_device_error(uint32_t *device_flags, int32_t clear, hipStream_t stream) {
    if (!device_flags || (reinterpret_cast<uintptr_t>(device_flags) & 3u)) return -PA_ERR_INVALID_ARG;
    uint32_t word = 0;
    if (hipMemcpyAsync(&word, device_flags, sizeof word, hipMemcpyDeviceToHost, stream) != hipSuccess)
        return -PA_ERR_HIP;
    if (clear && hipMemsetAsync(device_flags, 0, sizeof word, stream) != hipSuccess) return -PA_ERR_HIP;
    if (hipStreamSynchronize(stream) != hipSuccess) return -PA_ERR_HIP;
    return static_cast<int32_t>(word & 0x7FFFFFFFu);
}

pa_status pa_rope_table_fill_host(double *cos_sin_host, int32_t max_pos, double theta) {
    if (!cos_sin_host || max_pos < 1 || !(theta > 1.0)) return PA_ERR_INVALID_ARG;
    for (int32_t pos = 0; pos < max_pos; ++pos) {
        for (int i = 0; i < PA_HEAD_DIM / 2; ++i) {
            const double w = pow(theta, -(2.0 * i) / PA_HEAD_DIM);
            const double a = static_cast<double>(pos) * w;
            cos_sin_host[(static_cast<int64_t>(pos) * (PA_HEAD_DIM / 2) + i) * 2] = cos(a);
            cos_sin_host[(static_cast<int64_t>(pos) * (PA_HEAD_DIM / 2) + i) * 2 + 1] = sin(a);
        }
    }
    return PA_OK;
}

pa_status pa_append_kv_rope(void *q, const void *k_new, const void *v_new, void *k_pool, void *v_pool,
                            const int32_t *block_tables, const int32_t *context_lens, const double *rope_cos_sin,
                            int32_t num_seqs, int32_t max_blocks, int32_t num_pages, int32_t page_size,
                            int32_t max_pos, uint32_t *device_flags, hipStream_t stream) {
    if (num_seqs < 0 || max_blocks < 1 || num_pages < 1 || max_pos < 1) return PA_ERR_INVALID_ARG;
    if (page_size != PA_PAGE_SIZE) return PA_ERR_UNSUPPORTED;
    if (num_seqs == 0) return PA_OK;
    if (!k_new || !v_new || !k_pool || !v_pool || !block_tables || !context_lens || !rope_cos_sin)
        return PA_ERR_INVALID_ARG;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool) ||
        !aligned16(block_tables) || !aligned16(context_lens) || !aligned16(rope_cos_sin) || (q && !aligned16(q)))
        return PA_ERR_INVALID_ARG;
    pa::AppendLaunch a{q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, rope_cos_sin,
                       num_seqs, 1, 0, max_blocks, num_pages, max_pos, device_flags};
    return pa::launch_append_rope(a, stream) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t max_blocks) {
    if (num_seqs <= 0 || max_blocks <= 0) return 0;
    const int64_t np = decode_num_parts(max_blocks);
    if (np <= 1) return 0;
    const int64_t rows = static_cast<int64_t>(num_seqs) * PA_NUM_Q_HEADS * np;
    return static_cast<size_t>(rows * (2 + PA_HEAD_DIM) * sizeof(float));
}

int32_t pa_decode_partition_tokens(void) { return pa::decode_part_pages() * PA_PAGE_SIZE; }

pa_status pa_decode_gqa(void *out, const void *q, const void *k_pool, const void *v_pool,
                        const int32_t *block_tables, const int32_t *context_lens, int32_t num_seqs,
                        int32_t max_blocks, int32_t num_pages, int32_t page_size, float scale, int32_t out_dtype,
                        void *workspace, size_t workspace_bytes, uint32_t *device_flags,
                        const int32_t *dispatch_order, const int32_t *device_order, hipStream_t stream) {
    return decode_common(out, const_cast<void *>(q), nullptr, nullptr, const_cast<void *>(k_pool),
                         const_cast<void *>(v_pool), block_tables, context_lens, nullptr, num_seqs, max_blocks,
                         num_pages, page_size, 0, scale, out_dtype, workspace, workspace_bytes, device_flags,
                         dispatch_order, device_order, stream, false);
}

pa_status pa_append_decode_gqa(void *out, void *q, const void *k_new, const void *v_new, void *k_pool, void *v_pool,
                               const int32_t *block_tables, const int32_t *context_lens, const double *rope_cos_sin,
                               int32_t num_seqs, int32_t max_blocks, int32_t num_pages, int32_t page_size,
                               int32_t max_pos, float scale, int32_t out_dtype, void *workspace,
                               size_t workspace_bytes, uint32_t *device_flags, const int32_t *dispatch_order,
                               const int32_t *device_order, hipStream_t stream) {
    return decode_common(out, q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, rope_cos_sin, num_seqs,
                         max_blocks, num_pages, page_size, max_pos, scale, out_dtype, workspace, workspace_bytes,
                         device_flags, dispatch_order, device_order, stream, true);
}

pa_status pa_append_decode_gqa_noalloc(void *out, void *q, const void *k_new, const void *v_new, void *k_pool,
                                       void *v_pool, const int32_t *block_tables, const int32_t *context_lens,
                                       const double *rope_cos_sin, int32_t num_seqs, int32_t max_blocks,
                                       int32_t num_pages, int32_t page_size, int32_t max_pos, float scale,
                                       int32_t out_dtype, uint32_t *device_flags, const int32_t *dispatch_order,
                                       const int32_t *device_order, hipStream_t stream) {
    // Sizes first, so that an oversized call fails before anything else.
    const size_t need = pa_decode_workspace_bytes(num_seqs, max_blocks);
    if (need > PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_WORKSPACE;
    void *ws = nullptr;
    if (need > 0) {
        ws = scratch_on_current_device();
        if (!ws) return PA_ERR_HIP;
    }
    return decode_common(out, q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, rope_cos_sin, num_seqs,
                         max_blocks, num_pages, page_size, max_pos, scale, out_dtype, ws,
                         need > 0 ? static_cast<size_t>(PA_NOALLOC_SCRATCH_BYTES) : 0, device_flags, dispatch_order,
                         device_order, stream, true);
}

pa_status pa_prefill_chunk(void *out, void *q, const void *k_chunk, const void *v_chunk, void *k_pool, void *v_pool,
                           const int32_t *block_tables, const int32_t *prefix_lens, const double *rope_cos_sin,
                           int32_t num_seqs, int32_t chunk_len, int32_t max_blocks, int32_t num_pages,
                           int32_t page_size, int32_t max_pos, float scale, int32_t out_dtype,
                           uint32_t *device_flags, hipStream_t stream) {
    if (num_seqs < 0 || chunk_len < 0 || max_blocks < 1 || num_pages < 1 || max_pos < 1 || !isfinite(scale))
        return PA_ERR_INVALID_ARG;
    if (page_size != PA_PAGE_SIZE) return PA_ERR_UNSUPPORTED;
    if (max_blocks > pa::kMaxBlocksPrefill) return PA_ERR_UNSUPPORTED;
    if (out_dtype != PA_OUT_BF16 && out_dtype != PA_OUT_FP32) return PA_ERR_UNSUPPORTED;
    if (num_seqs == 0 || chunk_len == 0) return PA_OK;
    if (!out || !q || !k_chunk || !v_chunk || !k_pool || !v_pool || !block_tables || !prefix_lens || !rope_cos_sin)
        return PA_ERR_INVALID_ARG;
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_chunk) || !aligned16(v_chunk) || !aligned16(k_pool) ||
        !aligned16(v_pool) || !aligned16(block_tables) || !aligned16(prefix_lens) || !aligned16(rope_cos_sin))
        return PA_ERR_INVALID_ARG;
    // K/V rows of the chunk go into their pages and the chunk's q rows are
    // rotated in place first; the attention kernel reads q rotated.
    pa::AppendLaunch a{q, k_chunk, v_chunk, k_pool, v_pool, block_tables, prefix_lens, rope_cos_sin,
                       num_seqs, chunk_len, 1, max_blocks, num_pages, max_pos, device_flags};
    if (pa::launch_append_rope(a, stream) != hipSuccess) return PA_ERR_HIP;
    pa::PrefillLaunch p{out, q, k_pool, v_pool, block_tables, prefix_lens, num_seqs, chunk_len,
                        max_blocks, num_pages, max_pos, scale, out_dtype == PA_OUT_FP32, device_flags};
    return pa::launch_prefill_attention(p, stream) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

size_t pa_i8_pool_bytes(int32_t num_pages) {
    return num_pages < 1 ? 0 : static_cast<size_t>(num_pages) * PA_NUM_KV_HEADS * PA_I8_TILE_BYTES;
}

pa_status pa_quantize_pages_i8(void *kv_pool_i8, const void *k_pool, const void *v_pool, const int32_t *page_ids,
                               int32_t count, int32_t num_pages, uint32_t *device_flags, hipStream_t stream) {
    if (count < 0 || num_pages < 1) return PA_ERR_INVALID_ARG;
    if (!page_ids && count > num_pages) return PA_ERR_INVALID_ARG;
    if (count == 0) return PA_OK;
    if (!kv_pool_i8 || !k_pool || !v_pool) return PA_ERR_INVALID_ARG;
    if (!aligned16(kv_pool_i8) || !aligned16(k_pool) || !aligned16(v_pool) || (page_ids && !aligned16(page_ids)))
        return PA_ERR_INVALID_ARG;
    return pa::launch_quantize_pages_i8(kv_pool_i8, k_pool, v_pool, page_ids, count, num_pages, device_flags,
                                        stream) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_prefill_chunk_i8(void *out, void *q, const void *k_chunk, const void *v_chunk, void *kv_pool_i8,
                              const int32_t *block_tables, const int32_t *prefix_lens, const double *rope_cos_sin,
                              int32_t num_seqs, int32_t chunk_len, int32_t max_blocks, int32_t num_pages,
                              int32_t page_size, int32_t max_pos, float scale, int32_t out_dtype,
                              uint32_t *device_flags, hipStream_t stream) {
    if (num_seqs < 0 || chunk_len < 0 || max_blocks < 1 || num_pages < 1 || max_pos < 1 || !isfinite(scale))
        return PA_ERR_INVALID_ARG;
    if (page_size != PA_PAGE_SIZE) return PA_ERR_UNSUPPORTED;
    if (max_blocks > pa::kMaxBlocksPrefill) return PA_ERR_UNSUPPORTED;
    if (out_dtype != PA_OUT_BF16 && out_dtype != PA_OUT_FP32) return PA_ERR_UNSUPPORTED;
    if (num_seqs == 0 || chunk_len == 0) return PA_OK;
    if (!out || !q || !k_chunk || !v_chunk || !kv_pool_i8 || !block_tables || !prefix_lens || !rope_cos_sin)
        return PA_ERR_INVALID_ARG;
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_chunk) || !aligned16(v_chunk) || !aligned16(kv_pool_i8) ||
        !aligned16(block_tables) || !aligned16(prefix_lens) || !aligned16(rope_cos_sin))
        return PA_ERR_INVALID_ARG;
    // The chunk's rows are quantised into their pages and its q rows rotated
    // first; the attention kernel reads q rotated and every key from the pool.
    pa::AppendLaunch a{q, k_chunk, v_chunk, kv_pool_i8, nullptr, block_tables, prefix_lens, rope_cos_sin,
                       num_seqs, chunk_len, 1, max_blocks, num_pages, max_pos, device_flags};
    if (pa::launch_append_rope_i8(a, stream) != hipSuccess) return PA_ERR_HIP;
    pa::PrefillLaunch p{out, q, kv_pool_i8, nullptr, block_tables, prefix_lens, num_seqs, chunk_len,
                        max_blocks, num_pages, max_pos, scale, out_dtype == PA_OUT_FP32, device_flags};
    return pa::launch_prefill_attention_i8(p, stream) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_append_kv_rope_i8(void *q, const void *k_new, const void *v_new, void *kv_pool_i8,
                               const int32_t *block_tables, const int32_t *context_lens,
                               const double *rope_cos_sin, int32_t num_seqs, int32_t max_blocks,
                               int32_t num_pages, int32_t page_size, int32_t max_pos,
                               uint32_t *device_flags, hipStream_t stream) {
    if (num_seqs < 0 || max_blocks < 1 || num_pages < 1 || max_pos < 1) return PA_ERR_INVALID_ARG;
    if (page_size != PA_PAGE_SIZE) return PA_ERR_UNSUPPORTED;
    if (num_seqs == 0) return PA_OK;
    if (!k_new || !v_new || !kv_pool_i8 || !block_tables || !context_lens || !rope_cos_sin) return PA_ERR_INVALID_ARG;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(kv_pool_i8) || !aligned16(block_tables) ||
        !aligned16(context_lens) || !aligned16(rope_cos_sin) || (q && !aligned16(q)))
        return PA_ERR_INVALID_ARG;
    pa::AppendLaunch a{q, k_new, v_new, kv_pool_i8, nullptr, block_tables, context_lens, rope_cos_sin,
                       num_seqs, 1, 0, max_blocks, num_pages, max_pos, device_flags};
    return pa::launch_append_rope_i8(a, stream) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_decode_gqa_i8(void *out, const void *q, const void *kv_pool_i8, const int32_t *block_tables,
                           const int32_t *context_lens, int32_t num_seqs, int32_t max_blocks, int32_t num_pages,
                           int32_t page_size, float scale, int32_t out_dtype, void *workspace,
                           size_t workspace_bytes, uint32_t *device_flags, const int32_t *dispatch_order,
                           const int32_t *device_order, hipStream_t stream) {
    return decode_common(out, const_cast<void *>(q), nullptr, nullptr, const_cast<void *>(kv_pool_i8), nullptr,
                         block_tables, context_lens, nullptr, num_seqs, max_blocks, num_pages, page_size, 0, scale,
                         out_dtype, workspace, workspace_bytes, device_flags, dispatch_order, device_order, stream,
                         false, true);
}

pa_status pa_append_decode_gqa_i8(void *out, void *q, const void *k_new, const void *v_new, void *kv_pool_i8,
                                  const int32_t *block_tables, const int32_t *context_lens,
                                  const double *rope_cos_sin, int32_t num_seqs, int32_t max_blocks,
                                  int32_t num_pages, int32_t page_size, int32_t max_pos, float scale,
                                  int32_t out_dtype, void *workspace, size_t workspace_bytes,
                                  uint32_t *device_flags, const int32_t *dispatch_order,
                                  const int32_t *device_order, hipStream_t stream) {
    return decode_common(out, q, k_new, v_new, kv_pool_i8, nullptr, block_tables, context_lens, rope_cos_sin,
                         num_seqs, max_blocks, num_pages, page_size, max_pos, scale, out_dtype, workspace,
                         workspace_bytes, device_flags, dispatch_order, device_order, stream, true, true);
}

size_t pa_argmax_workspace_bytes(int32_t num_rows, int32_t vocab, int32_t logits_dtype) {
    if (num_rows < 1 || vocab < 1 || (logits_dtype != PA_LOGITS_BF16 && logits_dtype != PA_LOGITS_FP32)) return 0;
    const int64_t chunk = pa::argmax_chunk_elems(logits_dtype == PA_LOGITS_BF16);
    const int64_t splits = (static_cast<int64_t>(vocab) + chunk - 1) / chunk;
    // Per row: the running key and the arrival count, one 64-bit word each.
    return splits <= 1 ? 0 : static_cast<size_t>(num_rows) * 2 * sizeof(uint64_t);
}

pa_status pa_argmax(int32_t *out_index, const void *logits, int32_t num_rows, int32_t vocab, int32_t logits_dtype,
                    void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (num_rows < 0 || vocab < 1) return PA_ERR_INVALID_ARG;
    if (logits_dtype != PA_LOGITS_BF16 && logits_dtype != PA_LOGITS_FP32) return PA_ERR_UNSUPPORTED;
    if (num_rows > 65535) return PA_ERR_UNSUPPORTED;  // rows are the grid's second dimension
    if (num_rows == 0) return PA_OK;
    const bool bf16 = logits_dtype == PA_LOGITS_BF16;
    const size_t esz = bf16 ? 2 : 4;
    if (!out_index || !logits) return PA_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(out_index) & 3u) || (reinterpret_cast<uintptr_t>(logits) & (esz - 1)))
        return PA_ERR_INVALID_ARG;
    const size_t need = pa_argmax_workspace_bytes(num_rows, vocab, logits_dtype);
    if (need > 0 && (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 7u)))
        return PA_ERR_WORKSPACE;
    const bool vec = aligned16(logits) && (static_cast<size_t>(vocab) * esz) % 16 == 0;
    return pa::launch_argmax(out_index, logits, num_rows, vocab, bf16, vec, workspace, stream) == hipSuccess
               ? PA_OK : PA_ERR_HIP;
}

pa_status pa_dispatch_order_longest_first(const int32_t *lengths, int32_t n, int32_t *order) {
    if (n < 0 || (n > 0 && (!lengths || !order))) return PA_ERR_INVALID_ARG;
    for (int32_t i = 0; i < n; ++i) order[i] = i;
    std::stable_sort(order, order + n, [lengths](int32_t a, int32_t b) { return lengths[a] > lengths[b]; });
    return PA_OK;
}

pa_status pa_order_by_length(const int32_t *context_lens, int32_t num_seqs, int32_t max_blocks, int32_t long_run,
                             int32_t short_run, int32_t *order, hipStream_t stream) {
    if (num_seqs < 0 || num_seqs > PA_MAX_DISPATCH_ORDER || max_blocks < 1) return PA_ERR_INVALID_ARG;
    if (long_run < 1 || long_run > PA_MAX_ORDER_RUN || short_run < 0 || short_run > PA_MAX_ORDER_RUN)
        return PA_ERR_INVALID_ARG;
    if (num_seqs == 0) return PA_OK;
    if (!context_lens || !order || !aligned16(context_lens) || !aligned16(order)) return PA_ERR_INVALID_ARG;
    const uintptr_t a = reinterpret_cast<uintptr_t>(context_lens), b = reinterpret_cast<uintptr_t>(order);
    const uintptr_t bytes = static_cast<uintptr_t>(num_seqs) * sizeof(int32_t);
    if (a < b + bytes && b < a + bytes) return PA_ERR_INVALID_ARG;
    return pa::launch_order_by_length(context_lens, num_seqs, max_blocks, long_run, short_run, order, stream) ==
                   hipSuccess
               ? PA_OK
               : PA_ERR_HIP;
}

pa_status pa_probe_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream) {
    if (bytes == 0) return PA_OK;
    if (!buf || !sink || !aligned16(buf) || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(sink) & 3u))
        return PA_ERR_INVALID_ARG;
    return pa::launch_stream_read(buf, bytes, sink, stream) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // extern "C"
