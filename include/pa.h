/*
 * pa.h -- C ABI of libpa.so: paged grouped-query attention for MI355X (gfx950).
 *
 * The problem these calls solve is the paged KV cache of a small decoder LLM
 * engine as the samir-vllm article describes it (section "Gestion de la KV
 * cache et strategies de batching"): K and V of every layer live in one shared
 * pool of physical pages of 16 tokens; each (sequence, layer) owns a block table
 * naming its pages; at decode time each new token is appended at its absolute
 * RoPE position; paged attention reads only the sequence's own pages, never
 * concatenates a contiguous prefix and never stores the attention scores.
 * Geometry is Llama-3.2-1B's (tiny-vllm chapter "Weight Loading and GPU Buffer
 * Design", section "Preallocating the 16 compute buffers"): 32 query heads,
 * KV width 512 = 8 KV heads x head dim 64, bf16 storage.  Like that engine the
 * geometry is fixed at compile time (samir-vllm, section "Limitations").
 *
 * ---------------------------------------------------------------- layouts --
 *   bf16 = IEEE binary32 truncated to its upper 16 bits (1-8-7).
 *   k_pool, v_pool : [num_pages][8 kv heads][16 slots][64] bf16.  Page p of the
 *                    K pool and page p of the V pool hold the same 16 tokens.
 *                    One (page, kv head) is a contiguous 2 KiB tile.
 *   block_tables   : [num_seqs][max_blocks] int32.  Entry b is the physical page
 *                    of tokens 16b..16b+15; entries at or past ceil(L/16) are
 *                    never read and may be -1 (unassigned, as in tiny-vllm's
 *                    init, section "What else is set up ...").  One layer is
 *                    selected by passing that layer's table; all layers share
 *                    the pool.
 *   context_lens   : [num_seqs] int32, the sequence length INCLUDING the token
 *                    being appended; that token's position is L-1 (0-based).
 *   q              : [num_seqs][32][64] bf16; q head h reads KV head h/4.
 *   k_new, v_new   : [num_seqs][8][64] bf16 (the decode-time K/V batch buffers
 *                    of tiny-vllm, BATCH_SIZE x KV_DIM).
 *   rope_cos_sin   : [max_pos][32][2] fp64: (cos, sin) of pos * w_i,
 *                    w_i = theta^(-2i/64); pair i rotates elements (i, i+32)
 *                    ("rotate-half").  Build it with pa_rope_table_fill_host.
 *
 * ------------------------------------------------------------- conventions --
 *   Ownership: every array is caller-owned device memory (hipMalloc or any
 *     allocator); scalars are host values.  The library allocates nothing and
 *     keeps no mutable global state.
 *   Streams: each call enqueues its kernels on `stream` and returns without
 *     synchronising.  Calls that touch the same pool, q or out must be ordered
 *     by the caller (one stream, or events); concurrent calls on disjoint
 *     buffers are safe.
 *   Alignment: every array pointer must be 16-byte aligned.
 *   Errors: a call returns PA_OK, or an error code *before launching anything*
 *     when a host-checkable argument is wrong (NULL pointer, non-positive size,
 *     misalignment, page_size != 16, workspace too small).  Launch failures map
 *     to PA_ERR_HIP.  Table contents live on the device and cannot be checked
 *     on the host: a bad length or page id found by a kernel is never
 *     dereferenced; the kernel skips (append) or zero-fills (decode/prefill)
 *     the affected sequence and ORs a PA_DEVERR_* bit into *device_flags when
 *     that pointer is not NULL (pa_get_device_error reads it back).
 *   Values: inputs are finite bf16; every score scale * <q, K_t> must be
 *     finite in fp32 (|score| < 2^127), and max |V| times the context length
 *     must stay below 2^119 (the weighted V sums are accumulated in fp32 with
 *     weights up to 2^8: e.g. |V| < 2^108, about 3e32, at 2048 tokens).  The
 *     outputs are then finite.
 */
#ifndef PAGED_KV_GQA_APPEND_PA_H
#define PAGED_KV_GQA_APPEND_PA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_NUM_Q_HEADS 32
#define PA_NUM_KV_HEADS 8
#define PA_HEAD_DIM 64
#define PA_PAGE_SIZE 16

typedef enum {
    PA_OK = 0,
    PA_ERR_INVALID_ARG = 1, /* NULL, non-positive size, misaligned pointer    */
    PA_ERR_UNSUPPORTED = 2, /* page_size other than 16, dtype not supported   */
    PA_ERR_WORKSPACE = 3,   /* decode workspace missing or too small          */
    PA_ERR_HIP = 4,         /* the HIP runtime refused a launch               */
    PA_ERR_REJECTED = 5     /* request budget exceeds the whole pool (pa_kvm) */
} pa_status;

typedef enum { PA_OUT_BF16 = 0, PA_OUT_FP32 = 1 } pa_out_dtype;

/* Bits a kernel ORs into *device_flags (caller-owned uint32, may be NULL). */
#define PA_DEVERR_CONTEXT_LEN 0x1u /* L < 1, or L beyond max_blocks*16 / max_pos */
#define PA_DEVERR_PAGE_ID 0x2u     /* a used block-table entry outside [0, num_pages) */
#define PA_DEVERR_DISPATCH_ORDER 0x4u /* a device_order entry outside [0, num_seqs)      */

/* Human-readable name of a status code (static string, never NULL).  Every
 * call reports failure through its return value and the caller must not go on
 * with what the failed call was to produce (TinyLoop, "Lifecycle and Memory
 * Model", section "Internal allocation phases": a failed load hands back
 * nothing and the caller must stop there; tiny-vllm ch.2 "Weight Loading and
 * GPU Buffer Design", opening section: the device check reports a missing GPU
 * as an error return rather than aborting).                                  */
const char *pa_status_string(int status);

/* Device-side errors, read back (debug helper; SYNCHRONISES).  The kernels
 * never abort: a bad length or page id found in device-resident tables is
 * flagged by OR-ing a PA_DEVERR_* bit into the caller's *device_flags word
 * (see "Errors" above), so that, as in TinyLoop's "Internal allocation
 * phases", the failure reaches the caller, who must not use the affected
 * outputs.  This call waits for `stream` to drain, copies the word to the host
 * and returns it (a combination of PA_DEVERR_* bits, 0 when nothing was
 * flagged); with clear != 0 it also resets the word to 0, in stream order,
 * before returning.  Returns -PA_ERR_INVALID_ARG for a NULL or misaligned
 * pointer and -PA_ERR_HIP when the runtime fails (including an asynchronous
 * error of earlier work on the stream).  Not for hot loops or graph capture. */
int32_t pa_get_device_error(uint32_t *device_flags, int32_t clear, hipStream_t stream);

/* ABI version of this header, bumped on any signature or layout change;
 * pa_abi_version() returns the value of the header the library was built
 * from, so a caller can refuse a library built from another header.  Like the
 * fixed geometry (samir-vllm, section "Limitations et perspectives": changing
 * the architecture means recompiling), a mismatch is refused, not adapted to. */
#define PA_ABI_VERSION 14
int32_t pa_abi_version(void);

/* Identity of the sources the library was built from: the sha256 (64 hex
 * characters, static string) of its kernel and ABI sources and compile
 * flags, so a binding can refuse a library older than the sources beside it. */
const char *pa_build_id(void);

/* The RoPE frequency table the initialization block builds (tiny-vllm ch.2,
 * section "What else is set up in the initialization block").  Fill a HOST
 * table [max_pos][32][2] fp64 with (cos, sin)(a), a = pos * pow(theta,
 * -2i/64), each a double operation of the C library.  The caller copies it to
 * the device.  Frequencies are unscaled; theta = 500000 for Llama 3.
 * Returns PA_ERR_INVALID_ARG for a NULL table, max_pos < 1 or theta <= 1.     */
pa_status pa_rope_table_fill_host(double *cos_sin_host, int32_t max_pos, double theta);

/* Decode-time KV append (samir-vllm, section "Gestion de la KV cache ...": each
 * new token is written at its absolute RoPE position).  For every sequence s,
 * pos = context_lens[s]-1, page = block_tables[s][pos/16], slot = pos%16:
 *   k_pool[page][j][slot][:] = bf16_rne(rope(k_new[s][j][:], pos))   j < 8
 *   v_pool[page][j][slot][:] = v_new[s][j][:]                           (copy)
 *   q[s][h][:] = bf16_rne(rope(q[s][h][:], pos)) in place, h < 32 (skipped when
 *   q is NULL).
 * Rotation in fp64 from the table values, every product and the sum rounded
 * on its own (no fused multiply-add), then rounded once to bf16 (RNE): the
 * operations of the plain double-precision definition, so the stored rows are
 * bitwise those of such an evaluation.
 * Device errors: L < 1 or pos >= min(max_blocks*16, max_pos) -> CONTEXT_LEN,
 * page id out of range -> PAGE_ID; that sequence is left untouched.           */
pa_status pa_append_kv_rope(void *q, const void *k_new, const void *v_new, void *k_pool, void *v_pool,
                            const int32_t *block_tables, const int32_t *context_lens,
                            const double *rope_cos_sin, int32_t num_seqs, int32_t max_blocks,
                            int32_t num_pages, int32_t page_size, int32_t max_pos,
                            uint32_t *device_flags, hipStream_t stream);

/* Bytes of device workspace pa_decode_gqa needs for num_seqs sequences whose
 * block tables have max_blocks entries (0 when one context partition always
 * suffices).  The workspace holds per-partition softmax partials; it needs no
 * initialisation and its contents are dead between calls.  As with the
 * engines' compute buffers, the caller allocates it once, up front, and hands
 * it to every call (tiny-vllm ch.2, section "Preallocating the 16 compute
 * buffers"; TinyLoop, "Lifecycle and Memory Model", section "Why this memory
 * design exists": no allocation churn in hot paths).                         */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t max_blocks);

/* Tokens per context partition pa_decode_gqa uses (a multiple of 16; 2048 by
 * default, the engines' whole context window, samir-vllm "Limitations et
 * perspectives").  It does not depend on the batch, so a sequence's result
 * does not either (the article notes its engine's batched results may differ
 * from single runs; this library's do not).
 * Test switch: the environment variable PA_DECODE_PART_PAGES (1 .. 128 pages),
 * read once per process at the first decode call, overrides the default.  It
 * changes the summation order, hence the output bits, of every decode in the
 * process; results stay within the same tolerance of the exact attention and
 * remain batch-invariant within the process.  It exists to exercise the
 * partition merge; production callers leave it unset.                        */
int32_t pa_decode_partition_tokens(void);

/* dispatch_order (every decode entry point; HOST int32[num_seqs], may be NULL):
 * the order in which the sequences' workgroups are dispatched, a permutation
 * of 0 .. num_seqs-1 (entry 0 first).  The array must hold exactly num_seqs
 * entries: the library reads num_seqs of them and cannot see a shorter or
 * longer array (the Python binding refuses one whose length differs).  NULL dispatches in slot order.  It
 * changes no result: each sequence is computed the same way wherever it is
 * dispatched.  A caller that knows its lengths on the host can pass them
 * longest first, so that long sequences do not start last and form the
 * launch's tail (ragged batches).  The order is copied into the launch's
 * arguments, so the array may be reused when the call returns.  With
 * P = ceil(max_blocks * 16 / pa_decode_partition_tokens()) partitions per
 * sequence, PA_ERR_INVALID_ARG when it is not a permutation, when
 * num_seqs * P exceeds PA_MAX_DISPATCH_ORDER, or when P exceeds 64.          */
#define PA_MAX_DISPATCH_ORDER 1024

/* Host helper: order[0 .. n-1] = the indices 0 .. n-1 sorted by lengths[i],
 * longest first, equal lengths in index order (a stable sort): the dispatch
 * order that starts long sequences first.  lengths and order are HOST arrays
 * of n int32 (they may not overlap).  PA_ERR_INVALID_ARG for n < 0 or a NULL
 * array with n > 0.                                                           */
pa_status pa_dispatch_order_longest_first(const int32_t *lengths, int32_t n, int32_t *order);

/* device_order (every decode entry point; DEVICE int32[num_seqs], may be NULL;
 * not together with dispatch_order, PA_ERR_INVALID_ARG): the same as
 * dispatch_order, read by the kernels from device memory, so that an order
 * computed on the device (pa_order_by_length) needs no copy to the host and
 * one order serves every layer of a step.  Workgroups of the i-th dispatched
 * item serve sequence device_order[i / P], partition i % P.  It must be a
 * permutation of 0 .. num_seqs-1: the host cannot check device memory, so a
 * repeated entry leaves some sequence unserved, unflagged (pa_order_by_length
 * always writes a permutation).  An entry outside [0, num_seqs) is never
 * dereferenced: its workgroups do nothing and OR PA_DEVERR_DISPATCH_ORDER into
 * *device_flags; the whole call's outputs are then unusable.  Any num_seqs
 * and any P; 16-byte aligned.                                                */

/* The longest-first order of a ragged batch, computed on the device (a
 * continuous-batching decode batch mixes contexts of very different lengths:
 * samir-vllm, "Gestion de la KV cache et strategies de batching", admission as
 * soon as a request's page budget is free).  Writes order[0 .. num_seqs-1]
 * (DEVICE int32) from context_lens (DEVICE int32[num_seqs]).  The sequences
 * are ranked by length class, longest class first, index order within a
 * class, where class c of a valid length L (1 <= L <= 16 * max_blocks) is
 * (ceil(L/16) - 1) / ceil(max_blocks/64), 64 classes across the table width;
 * an invalid length has class 0, the last (the decode rejects it as usual).
 * The ranks are then dealt in runs: long_run sequences from the long end,
 * short_run from the short end, and again, until the two ends meet (1, 0 is
 * plain longest first; with 3, 2 a batch of 10 is ranks 0 1 2 9 8 3 4 5 7 6).
 * Mixing a few short sequences in among the long ones keeps the CUs streaming
 * while the short ones pay their fixed costs, and the launch still ends on
 * short sequences.  Pass the result as device_order to every decode of the
 * step; no result changes.  One workgroup on `stream`, nothing allocated; the
 * lengths must not change between this call and the decodes that use its
 * order (stream order).  PA_ERR_INVALID_ARG for num_seqs outside [0,
 * PA_MAX_DISPATCH_ORDER], max_blocks < 1, long_run outside [1,
 * PA_MAX_ORDER_RUN], short_run outside [0, PA_MAX_ORDER_RUN], a NULL or
 * misaligned array, or arrays that overlap.                                  */
#define PA_MAX_ORDER_RUN 64
pa_status pa_order_by_length(const int32_t *context_lens, int32_t num_seqs, int32_t max_blocks, int32_t long_run,
                             int32_t short_run, int32_t *order, hipStream_t stream);

/* Paged GQA decode (samir-vllm, batched-decode paragraph of "Gestion de la KV
 * cache ..."; tiny-vllm ch.2, "One buffer, two roles": the attention output is
 * written over the q buffer).  For each s, h < 32, j = h/4, L = context_lens[s]:
 *   x_t = scale * <q[s][h], K_t>,  K_t, V_t = pool rows of token t < L, head j
 *   out[s][h][:] = sum_t exp(x_t - max x) V_t / sum_t exp(x_t - max x)
 * accumulated in fp32 (online softmax over context partitions, exact merge),
 * stored as bf16 (RNE) or fp32 per out_dtype.  out MAY ALIAS q exactly
 * (same pointer); no other overlap is allowed.  q must already be rotated.
 * Device errors: L < 1 or L > max_blocks*16 -> CONTEXT_LEN and the sequence's
 * output rows are zero-filled; a used page id out of range -> PAGE_ID and the
 * same.                                                                       */
pa_status pa_decode_gqa(void *out, const void *q, const void *k_pool, const void *v_pool,
                        const int32_t *block_tables, const int32_t *context_lens, int32_t num_seqs,
                        int32_t max_blocks, int32_t num_pages, int32_t page_size, float scale,
                        int32_t out_dtype, void *workspace, size_t workspace_bytes,
                        uint32_t *device_flags, const int32_t *dispatch_order, const int32_t *device_order,
                        hipStream_t stream);

/* One decode step of a layer in a single launch: pa_append_kv_rope followed by
 * pa_decode_gqa, fused (samir-vllm, "Gestion de la KV cache ...": the new
 * token is appended at its absolute RoPE position, then paged attention reads
 * the sequence's pages).  Arguments are the union of the two calls; q holds the
 * UN-rotated query and receives the rotated one in place (unless out == q, in
 * which case it receives the attention output).  Results are bitwise those of
 * the two separate calls: the same fp64 rotation and bf16 rounding, and the
 * appended K/V row is written to its slot exactly as pa_append_kv_rope does.
 * Device errors: the union of both calls' (L-1 >= max_pos also counts as
 * CONTEXT_LEN); a failing sequence is neither appended nor attended, its out
 * rows are zero-filled.                                                        */
pa_status pa_append_decode_gqa(void *out, void *q, const void *k_new, const void *v_new, void *k_pool, void *v_pool,
                               const int32_t *block_tables, const int32_t *context_lens,
                               const double *rope_cos_sin, int32_t num_seqs, int32_t max_blocks,
                               int32_t num_pages, int32_t page_size, int32_t max_pos, float scale,
                               int32_t out_dtype, void *workspace, size_t workspace_bytes,
                               uint32_t *device_flags, const int32_t *dispatch_order, const int32_t *device_order,
                               hipStream_t stream);

/* pa_append_decode_gqa without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  It allocates nothing: the decode partials
 * go to a scratch array of PA_NOALLOC_SCRATCH_BYTES that the library holds in
 * every GPU it runs on (static device memory, kept until the process ends).
 * Everything else, results included, is exactly pa_append_decode_gqa's.
 * Limit: pa_decode_workspace_bytes(num_seqs, max_blocks) must not exceed
 * PA_NOALLOC_SCRATCH_BYTES (8 MiB: for example 64 sequences of up to 30720
 * tokens, or 256 of up to 6144), else PA_ERR_WORKSPACE before anything runs.
 * The scratch needs no initialisation and holds nothing between calls, but it
 * is one array per GPU: calls on one GPU whose executions overlap (on
 * different streams, or concurrently from several host threads on streams
 * that are not ordered) race on it and must be serialised by the caller.
 * `stream` must belong to the current device.  PA_ERR_HIP if the scratch
 * cannot be located on the current device.                                  */
#define PA_NOALLOC_SCRATCH_BYTES (8u << 20)
pa_status pa_append_decode_gqa_noalloc(void *out, void *q, const void *k_new, const void *v_new, void *k_pool,
                                       void *v_pool, const int32_t *block_tables, const int32_t *context_lens,
                                       const double *rope_cos_sin, int32_t num_seqs, int32_t max_blocks,
                                       int32_t num_pages, int32_t page_size, int32_t max_pos, float scale,
                                       int32_t out_dtype, uint32_t *device_flags, const int32_t *dispatch_order,
                                       const int32_t *device_order, hipStream_t stream);

/* Chunked prefill (TinyLoop, section "prefill_chunk and scratch residency":
 * the prompt is processed in row chunks; samir-vllm: the prompt's pages are
 * filled during prefill).  For each s and chunk token i < chunk_len at
 * pos = prefix_lens[s] + i: append k_chunk[s][i] / v_chunk[s][i] as
 * pa_append_kv_rope does and rotate q[s][i] in place; then every chunk query
 * attends causally (keys 0..pos inclusive) to its sequence's pages:
 *   out[s][i][h][:] = softmax_t(scale * <q[s][i][h], K_t>) . V_t,  t <= pos
 * with bf16 MFMA tiles and fp32 accumulation; no score matrix is stored.
 * q, out: [num_seqs][chunk_len][32][64]; k_chunk, v_chunk: [num_seqs][chunk_len][8][64].
 * out may alias q exactly.  max_blocks may be at most 512 (contexts up to
 * 8192 tokens; larger tables return PA_ERR_UNSUPPORTED).  Device errors: a
 * chunk token whose position (prefix < 0, or beyond max_blocks*16 or max_pos)
 * or page id is invalid is not appended (nor is its q row rotated), exactly as
 * pa_append_kv_rope treats one token; a sequence whose length or any used page
 * id is invalid has all its out rows zero-filled; the matching PA_DEVERR_* bit
 * is set.                                                                       */
pa_status pa_prefill_chunk(void *out, void *q, const void *k_chunk, const void *v_chunk, void *k_pool,
                           void *v_pool, const int32_t *block_tables, const int32_t *prefix_lens,
                           const double *rope_cos_sin, int32_t num_seqs, int32_t chunk_len,
                           int32_t max_blocks, int32_t num_pages, int32_t page_size, int32_t max_pos,
                           float scale, int32_t out_dtype, uint32_t *device_flags, hipStream_t stream);

/* ------------------------------------------------------ INT8 K/V pages --
 * An INT8 KV cache (TinyLoop, "Lifecycle and Memory Model", section
 * "Per-request / handle-owned memory": the runtime KV cache holds K/V as FP16
 * or INT8).  The pages give no quantisation rule; this library's format is one
 * symmetric fp32 scale per (token, KV head) row of 64 values:
 *   scale = max|x| / 127,  code = round-half-even(x / scale) in [-127, 127],
 * both in IEEE binary32, scale 0 and codes 0 for an all-zero row (rows must be
 * finite; the decode accepts V over the same range as the bf16 pools, see
 * "Values" above).  Accuracy: the products run on f16 MFMAs; the weights
 * times the V scales reach them through one running power-of-two exponent
 * per wave, so they never overflow, and a (sequence, KV head)'s outputs are
 * within the usual rounding of the exact attention plus 2^-16 of the largest
 * |V| it attends (rows about 2^30 below that largest one lose precision
 * first; with V rows of ordinary spread the extra term is negligible).  The value a code stands for is
 * code * scale.  K rows are quantised
 * after RoPE from the bf16-rounded rotated row (the row pa_append_kv_rope would
 * store), V rows from their bf16 input.
 *
 *   kv_pool_i8 : [num_pages][8 kv heads] tiles of PA_I8_TILE_BYTES = 2176 bytes,
 *                K and V together (there is no separate V pool); for slot t
 *                (0..15) and element d (0..63) of the row:
 *                  K code at byte ((d%32)/8*16 + t)*16 + (d/32)*8 + d%8
 *                    (sixteen-byte units ordered by dim quarter, then token),
 *                  V code at byte 1024 + ((t/4)*16 + d%16)*16 + (d/16)*4 + t%4
 *                    (units ordered by token quad, then dim mod 16),
 *                  K scale (fp32) at byte 2048 + 4t, V scale at 2112 + 4t.
 *                A token costs 8 x 136 = 1088 bytes per layer, against 2048 in
 *                bf16.
 * Block tables, lengths, q, k_new, v_new, the RoPE table, out, workspace and
 * device_flags mean exactly what they mean for the bf16 calls above; the decode
 * workspace is sized by pa_decode_workspace_bytes.                           */
#define PA_I8_TILE_BYTES 2176

/* Bytes of an INT8 pool of num_pages pages (0 for num_pages < 1). */
size_t pa_i8_pool_bytes(int32_t num_pages);

/* Quantise whole pages of a bf16 pool pair into the INT8 pool: for each listed
 * page id p (page_ids: device int32[count]; NULL means pages 0..count-1), all
 * 16 slots of all 8 heads of k_pool/v_pool page p go to INT8 page p.  Slots
 * that hold no token are quantised too (their codes are never read by decode).
 * Device errors: an id outside [0, num_pages) -> PAGE_ID, that page skipped.  */
pa_status pa_quantize_pages_i8(void *kv_pool_i8, const void *k_pool, const void *v_pool, const int32_t *page_ids,
                               int32_t count, int32_t num_pages, uint32_t *device_flags, hipStream_t stream);

/* pa_append_kv_rope into an INT8 pool: the rotated K row (bf16-rounded) and the
 * V row of every KV head are quantised into slot pos%16 of page
 * block_tables[s][pos/16], pos = context_lens[s]-1; q rotated in place as by
 * pa_append_kv_rope (skipped when q is NULL).  Device errors as there.        */
pa_status pa_append_kv_rope_i8(void *q, const void *k_new, const void *v_new, void *kv_pool_i8,
                               const int32_t *block_tables, const int32_t *context_lens,
                               const double *rope_cos_sin, int32_t num_seqs, int32_t max_blocks,
                               int32_t num_pages, int32_t page_size, int32_t max_pos,
                               uint32_t *device_flags, hipStream_t stream);

/* pa_decode_gqa over an INT8 pool: K_t, V_t are the values the codes stand for
 * (code * scale); everything else as pa_decode_gqa, out may alias q.  The
 * weights (softmax weight x V scale) enter the products as f16 hi + lo halves;
 * with PA_OUT_BF16 a page whose live V scales are all <= 1/8 takes the hi
 * halves alone (within 2^-11 * 16 < 8e-3 of exact).                          */
pa_status pa_decode_gqa_i8(void *out, const void *q, const void *kv_pool_i8, const int32_t *block_tables,
                           const int32_t *context_lens, int32_t num_seqs, int32_t max_blocks, int32_t num_pages,
                           int32_t page_size, float scale, int32_t out_dtype, void *workspace,
                           size_t workspace_bytes, uint32_t *device_flags, const int32_t *dispatch_order,
                           const int32_t *device_order, hipStream_t stream);

/* Chunked prefill into INT8 pages (TinyLoop, "Lifecycle and Memory Model":
 * section "prefill_chunk and scratch residency" processes the prompt in row
 * chunks, section "Per-request / handle-owned memory" names the INT8 K/V
 * mode).  pa_prefill_chunk over an INT8 pool: for each s and chunk token i at
 * pos = prefix_lens[s] + i, k_chunk[s][i] and v_chunk[s][i] are appended as
 * pa_append_kv_rope_i8 appends one token (K rotated, rounded to bf16 and
 * quantised; V quantised; q[s][i] rotated in place); then every chunk query
 * attends causally (keys 0..pos inclusive) to its sequence's keys, with K_t,
 * V_t the values code * scale:
 *   out[s][i][h][:] = softmax_t(scale * <q[s][i][h], K_t>) . V_t,  t <= pos
 * on f16 MFMAs with the INT8 decode's arithmetic (exact codes, scales in
 * fp32), accumulated in fp32.  The weights (softmax weight x V scale) go in as
 * f16 hi + lo halves for PA_OUT_FP32; for PA_OUT_BF16 the lo half is dropped
 * for keys taken together (two pages) whose V scales are all <= 1/8, where f16
 * weights alone keep the output within 2^-11 * 16 < 8e-3 of exact.  Shapes, aliasing (out may
 * alias q exactly), max_blocks <= 512 and device errors as pa_prefill_chunk;
 * the pool is the PA_I8_TILE_BYTES tile pool of pa_decode_gqa_i8.            */
pa_status pa_prefill_chunk_i8(void *out, void *q, const void *k_chunk, const void *v_chunk, void *kv_pool_i8,
                              const int32_t *block_tables, const int32_t *prefix_lens, const double *rope_cos_sin,
                              int32_t num_seqs, int32_t chunk_len, int32_t max_blocks, int32_t num_pages,
                              int32_t page_size, int32_t max_pos, float scale, int32_t out_dtype,
                              uint32_t *device_flags, hipStream_t stream);

/* pa_append_kv_rope_i8 followed by pa_decode_gqa_i8 in one launch, bitwise equal
 * to the two calls (same rotation, rounding and quantisation); q as in
 * pa_append_decode_gqa.                                                       */
pa_status pa_append_decode_gqa_i8(void *out, void *q, const void *k_new, const void *v_new, void *kv_pool_i8,
                                  const int32_t *block_tables, const int32_t *context_lens,
                                  const double *rope_cos_sin, int32_t num_seqs, int32_t max_blocks,
                                  int32_t num_pages, int32_t page_size, int32_t max_pos, float scale,
                                  int32_t out_dtype, void *workspace, size_t workspace_bytes,
                                  uint32_t *device_flags, const int32_t *dispatch_order,
                                  const int32_t *device_order, hipStream_t stream);

/* --------------------------------------------------------------- argmax --
 * Greedy next-token choice on the GPU (samir-vllm, section "Architecture et
 * flux d'inference": the argmax runs on the GPU; tiny-vllm ch.2, section
 * "Preallocating the 16 compute buffers": the CPU argmax it replaces scans the
 * logits row with a strict greater-than, so the first maximum wins).
 *   out_index[r] = lowest i with logits[r][i] = max over the row's non-NaN
 *                  entries (-0.0 == +0.0); 0 for a row holding only NaN.
 *   logits : [num_rows][vocab] bf16 or fp32 (logits_dtype), caller-owned device
 *            memory, 2-byte (bf16) or 4-byte (fp32) aligned; rows that start on
 *            16-byte boundaries with a 16-byte multiple of bytes take the
 *            vector path, any other layout a scalar one (same results).
 *   out_index : [num_rows] int32, device.
 *   workspace : pa_argmax_workspace_bytes(num_rows, vocab, logits_dtype) bytes
 *            (16 per row when a row spans more than one chunk, else 0),
 *            8-byte aligned, may be NULL when that is 0.  It must be all zero
 *            before its first use; every call that returns PA_OK leaves it all
 *            zero again once its kernel has finished (the last chunk of each
 *            row resets the row's words), so a workspace is zeroed once, at
 *            allocation.  Calls sharing one workspace must not overlap in time
 *            (same stream, or ordered by the caller).  Stream-ordered, one
 *            launch, no synchronisation, nothing allocated.
 *   Errors: PA_ERR_UNSUPPORTED for another dtype or more than 65535 rows.     */
typedef enum { PA_LOGITS_BF16 = 0, PA_LOGITS_FP32 = 1 } pa_logits_dtype;

size_t pa_argmax_workspace_bytes(int32_t num_rows, int32_t vocab, int32_t logits_dtype);

pa_status pa_argmax(int32_t *out_index, const void *logits, int32_t num_rows, int32_t vocab, int32_t logits_dtype,
                    void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------ host KV page manager --
 * Host-side bookkeeping that produces the block tables and lengths the calls
 * above consume (samir-vllm, section "Gestion de la KV cache et strategies de
 * batching": one shared pool of 16-token pages, a block table per sequence and
 * per layer, admission once a request's page budget is available, the budget
 * being prompt_tokens + allowed_new_tokens - 1 tokens rounded up to 16-token
 * pages for every layer, continuous or static batching, explicit refusal of a
 * request larger than the pool).  Initial state as tiny-vllm ch.2 "What else is
 * set up ...": all pages free, all block-table entries -1, all slots free.
 *
 * Ownership: the manager is a host object created by pa_kvm_create and owned by
 * the caller until pa_kvm_destroy; it allocates host memory only, never device
 * memory, and the caller uploads the tables it exposes.  Not thread-safe: one
 * thread (or external locking) per manager.
 * Policies: budgets are reserved at admission and pages are taken from the free
 * list as a slot grows (so growth within the budget cannot fail); the free list
 * is a stack (page 0 first on a fresh pool, the page freed last is reused
 * first); admission is first-come first-served with no overtaking.          */
typedef struct pa_kv_manager pa_kv_manager;
typedef enum { PA_BATCH_CONTINUOUS = 0, PA_BATCH_STATIC = 1 } pa_batching;

/* Pages a request reserves: ceil((prompt + max_new - 1) / 16) * num_layers; the
 * last generated token is never appended, hence the -1.  -1 for a non-positive
 * argument.                                                                  */
int64_t pa_admission_credit_pages(int32_t prompt_tokens, int32_t max_new_tokens, int32_t num_layers);

/* Create a manager for a pool of num_pages pages shared by num_layers layers,
 * max_slots batch slots and block tables of max_blocks entries.  batching is a
 * pa_batching value.  *out receives the handle (NULL on error).              */
pa_status pa_kvm_create(int32_t num_pages, int32_t num_layers, int32_t max_slots, int32_t max_blocks,
                        int32_t batching, pa_kv_manager **out);
void pa_kvm_destroy(pa_kv_manager *m);

/* Queue a request.  PA_ERR_REJECTED when its budget exceeds the pool or its
 * token budget exceeds max_blocks*16 (it could never run); PA_ERR_INVALID_ARG
 * for prompt_tokens < 1 or max_new_tokens < 1.  *request_id gets a
 * non-negative id, or -1 on error.                                           */
pa_status pa_kvm_submit(pa_kv_manager *m, int32_t prompt_tokens, int32_t max_new_tokens, int32_t *request_id);

/* Admit queued requests in arrival order while the head's budget fits in the
 * unreserved pages and a slot is free (static batching: only when no slot is
 * active).  Writes the admitted slots to admitted_slots[0..n) and returns n
 * (at most max_out), or -1 for bad arguments.  An admitted slot starts at
 * length 0 with its budget reserved.                                         */
int32_t pa_kvm_schedule(pa_kv_manager *m, int32_t *admitted_slots, int32_t max_out);

/* Grow an active slot to len tokens (its context_lens value): blocks
 * ceil(old/16) .. ceil(len/16)-1 get pages from the free list in every layer.
 * PA_ERR_INVALID_ARG for a free slot, a shrinking len or len beyond the slot's
 * budget of prompt + max_new - 1 tokens.                                     */
pa_status pa_kvm_set_length(pa_kv_manager *m, int32_t slot, int32_t len);

/* Finish a slot: its pages return to the free list (all layers), its budget is
 * released, its table rows become -1 and its length 0.                       */
pa_status pa_kvm_release(pa_kv_manager *m, int32_t slot);

/* Read-only views, valid until the next call that modifies the manager:
 * block tables [num_layers][max_slots][max_blocks] int32 (-1 unassigned; the
 * table of layer l is the slice at l*max_slots*max_blocks) and lengths
 * [max_slots] int32 (0 for a free slot).                                     */
const int32_t *pa_kvm_block_tables(const pa_kv_manager *m);
const int32_t *pa_kvm_lengths(const pa_kv_manager *m);
int32_t pa_kvm_slot_request(const pa_kv_manager *m, int32_t slot);  /* request id, -1 if free */
int32_t pa_kvm_slot_budget(const pa_kv_manager *m, int32_t slot);   /* token budget, -1 if bad */
int32_t pa_kvm_free_pages(const pa_kv_manager *m);                  /* pages on the free list   */
int64_t pa_kvm_reserved_pages(const pa_kv_manager *m);              /* budgets of active slots   */
int32_t pa_kvm_queued(const pa_kv_manager *m);                      /* requests not yet admitted */

/* ------------------------------------------------------------ diagnostics --
 * Contiguous-read probe, for measurement: reads bytes from buf (device,
 * 16-byte aligned, bytes a multiple of 16) once, with 16-byte loads and no
 * other memory traffic, so its time gives the read bandwidth a plain stream
 * reaches on this GPU, the ceiling the decode kernels' figures are set
 * against.  sink (device uint32, 4-byte aligned) receives a fixed constant
 * (0x9E3779B9) only if the 32-bit XOR of the words one lane read equals that
 * constant, never for all-zero data; it exists so the loads are kept.
 * PA_ERR_INVALID_ARG for a NULL or misaligned pointer or a bad size; 0 bytes
 * is a no-op.  Stream-ordered, nothing allocated.                            */
pa_status pa_probe_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* PAGED_KV_GQA_APPEND_PA_H */
