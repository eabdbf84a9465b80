/*
 * oracle.c -- plain, slow, fp64 CPU reference for paged GQA decode, KV append
 * with rotary embedding, and causal chunked prefill.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library (paged_kv_gqa_append_amd)
 * links, includes or calls this file; only the tests, the smoke check and the
 * benchmark's CPU-baseline leg do.  It shares no code, header or table with the
 * HIP path.
 *
 * What it computes, and where the pages state it:
 *  - samir-vllm article, section "Gestion de la KV cache et strategies de
 *    batching": K and V live in a shared pool of physical pages of 16 tokens,
 *    each (sequence, layer) has a block table naming its pages, and during
 *    decode every new token is appended at its absolute RoPE position.  The
 *    same section's batched-decode paragraph: paged attention reads only the
 *    sequence's own pages, accumulates weighted V, never concatenates a
 *    contiguous prefix and never stores the scores.  (This oracle does keep one
 *    score row per (sequence, head) in a scratch array: it is a checker, and
 *    a plain two-pass softmax is the obviously-correct definition.)
 *  - tiny-vllm chapter "Weight Loading and GPU Buffer Design", section
 *    "Preallocating the 16 compute buffers": 32 query heads, KV width 512
 *    (8 KV heads of 64), and section "What else is set up ...": block table
 *    entries start at -1 (unassigned), a RoPE frequency table exists.
 *
 * Readings where the pages are silent (all listed in the design notes):
 *  - rotary: rotate-half pairs (i, i+32), frequency w_i = theta^(-2i/64),
 *    no frequency scaling, theta passed in (500000 for the Llama-3 family);
 *    angle = pos * w_i evaluated in fp64 with libm cos/sin.
 *  - q head h reads KV head floor(h/4).
 *  - pool layout [page][kv head][slot 0..15][d 0..63], bf16.
 *  - context_lens counts the appended token; its position is L-1.
 *  - stored results (rotated K, rotated q) are rounded once, fp64 -> bf16,
 *    to nearest even.  Attention outputs stay fp64.
 *
 * Everything is double precision; every bf16 input is exact in double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define O_HQ 32
#define O_HKV 8
#define O_D 64
#define O_PS 16

/* Return codes (match nothing in the library on purpose; tests read them). */
#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1
#define ORACLE_BAD_LEN 2
#define ORACLE_BAD_PAGE 3

/* ---------------------------------------------------------------- bf16 -- */

double oracle_bf16_to_f64(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f; /* exact: bf16 is the top half of a binary32 */
}

/* Round a double to the nearest bf16 (ties to even) in ONE rounding step.
 * bf16 keeps 8 significant bits; the spacing of representable values at
 * magnitude 2^e (normal range) is 2^(e-7), and 2^-133 below 2^-126.
 * Rounding x/spacing to an integer with rint() (round-half-even in the
 * default mode) and scaling back is exact in double arithmetic because both
 * steps only touch the exponent.  The result is a bf16 value, hence exactly
 * representable as a binary32 whose low 16 bits are zero.                  */
uint16_t oracle_f64_to_bf16(double x)
{
    if (isnan(x)) return 0x7FC0;
    if (isinf(x)) return x > 0 ? 0x7F80 : 0xFF80;
    if (x == 0.0) return signbit(x) ? 0x8000 : 0x0000;
    int e;
    frexp(fabs(x), &e);           /* |x| = m * 2^e, m in [0.5, 1) -> 2^(e-1) <= |x| */
    int qexp = (e - 1) - 7;        /* exponent of the spacing in the normal range    */
    if (qexp < -133) qexp = -133;  /* subnormal bf16 spacing                           */
    double r = rint(ldexp(x, -qexp));
    double y = ldexp(r, qexp);
    if (fabs(y) >= 0x1p128) return x > 0 ? 0x7F80 : 0xFF80; /* overflow to inf */
    float f = (float)y;            /* exact */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

/* ---------------------------------------------------------------- rope -- */

/* Rotate one 64-wide head (bf16 in) to fp64 out at absolute position pos.   */
void oracle_rope_head(const uint16_t *x, int64_t pos, double theta, double *y)
{
    for (int i = 0; i < O_D / 2; ++i) {
        double w = pow(theta, -(2.0 * i) / (double)O_D);
        double a = (double)pos * w;
        double c = cos(a), s = sin(a);
        double x0 = oracle_bf16_to_f64(x[i]);
        double x1 = oracle_bf16_to_f64(x[i + O_D / 2]);
        y[i] = x0 * c - x1 * s;
        y[i + O_D / 2] = x1 * c + x0 * s;
    }
}

static size_t pool_index(int64_t page, int head, int slot)
{
    return (((size_t)page * O_HKV + (size_t)head) * O_PS + (size_t)slot) * O_D;
}

/* Write one token's rotated K and raw V into its page, rotate its q heads.
 * q_tok may be NULL.  Returns ORACLE_BAD_PAGE if the page id is unusable.   */
static int append_token(uint16_t *q_tok, const uint16_t *k_tok, const uint16_t *v_tok,
                        uint16_t *k_pool, uint16_t *v_pool, const int32_t *bt_row,
                        int32_t max_blocks, int32_t num_pages, int64_t pos, double theta)
{
    int64_t blk = pos / O_PS;
    int slot = (int)(pos % O_PS);
    if (blk >= max_blocks) return ORACLE_BAD_LEN;
    int64_t page = bt_row[blk];
    if (page < 0 || page >= num_pages) return ORACLE_BAD_PAGE;
    double y[O_D];
    for (int j = 0; j < O_HKV; ++j) {
        oracle_rope_head(k_tok + (size_t)j * O_D, pos, theta, y);
        uint16_t *kd = k_pool + pool_index(page, j, slot);
        uint16_t *vd = v_pool + pool_index(page, j, slot);
        for (int d = 0; d < O_D; ++d) {
            kd[d] = oracle_f64_to_bf16(y[d]);
            vd[d] = v_tok[(size_t)j * O_D + d];
        }
    }
    if (q_tok) {
        for (int h = 0; h < O_HQ; ++h) {
            oracle_rope_head(q_tok + (size_t)h * O_D, pos, theta, y);
            for (int d = 0; d < O_D; ++d) q_tok[(size_t)h * O_D + d] = oracle_f64_to_bf16(y[d]);
        }
    }
    return ORACLE_OK;
}

/* Decode-time append: one new token per sequence at pos = context_lens[s]-1.
 * q: [B][32][64] (may be NULL), k_new/v_new: [B][8][64], pools as above,
 * block_tables: [B][max_blocks].  All bf16 as uint16.                       */
int oracle_append_kv_rope(uint16_t *q, const uint16_t *k_new, const uint16_t *v_new,
                          uint16_t *k_pool, uint16_t *v_pool, const int32_t *block_tables,
                          const int32_t *context_lens, int32_t num_seqs, int32_t max_blocks,
                          int32_t num_pages, double theta)
{
    if (num_seqs < 0 || max_blocks <= 0 || num_pages <= 0) return ORACLE_BAD_ARG;
    int rc = ORACLE_OK;
    for (int32_t s = 0; s < num_seqs; ++s) {
        int64_t L = context_lens[s];
        if (L < 1) { rc = ORACLE_BAD_LEN; continue; }
        int r = append_token(q ? q + (size_t)s * O_HQ * O_D : NULL,
                             k_new + (size_t)s * O_HKV * O_D, v_new + (size_t)s * O_HKV * O_D,
                             k_pool, v_pool, block_tables + (size_t)s * max_blocks,
                             max_blocks, num_pages, L - 1, theta);
        if (r != ORACLE_OK) rc = r;
    }
    return rc;
}

/* ----------------------------------------------------------- attention -- */

/* Softmax attention of one 64-wide query over tokens 0..n-1 of one KV head of
 * one sequence, read through its block table.  score_buf holds n doubles.   */
static int attend(double *out, const uint16_t *q_head, const uint16_t *k_pool,
                  const uint16_t *v_pool, const int32_t *bt_row, int32_t max_blocks,
                  int32_t num_pages, int kv_head, int64_t n, double scale, double *score_buf)
{
    double qd[O_D];
    for (int d = 0; d < O_D; ++d) qd[d] = oracle_bf16_to_f64(q_head[d]);
    if ((n + O_PS - 1) / O_PS > max_blocks) return ORACLE_BAD_LEN;
    /* scores x_t = scale * <q, K_t> */
    double m = -INFINITY;
    for (int64_t t = 0; t < n; ++t) {
        int64_t page = bt_row[t / O_PS];
        if (page < 0 || page >= num_pages) return ORACLE_BAD_PAGE;
        const uint16_t *kr = k_pool + pool_index(page, kv_head, (int)(t % O_PS));
        double acc = 0.0;
        for (int d = 0; d < O_D; ++d) acc += qd[d] * oracle_bf16_to_f64(kr[d]);
        score_buf[t] = scale * acc;
        if (score_buf[t] > m) m = score_buf[t];
    }
    /* w_t = exp(x_t - m); out = sum_t w_t V_t / sum_t w_t */
    double z = 0.0;
    double o[O_D];
    for (int d = 0; d < O_D; ++d) o[d] = 0.0;
    for (int64_t t = 0; t < n; ++t) {
        int64_t page = bt_row[t / O_PS];
        const uint16_t *vr = v_pool + pool_index(page, kv_head, (int)(t % O_PS));
        double w = exp(score_buf[t] - m);
        z += w;
        for (int d = 0; d < O_D; ++d) o[d] += w * oracle_bf16_to_f64(vr[d]);
    }
    for (int d = 0; d < O_D; ++d) out[d] = o[d] / z;
    return ORACLE_OK;
}

/* Decode: out[s][h][:] = softmax over t < L_s of scale*<q[s][h], K_t> times V_t,
 * K/V of KV head floor(h/4), read through block_tables[s].  out: [B][32][64] fp64. */
int oracle_decode_gqa(double *out, const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                      const int32_t *block_tables, const int32_t *context_lens, int32_t num_seqs,
                      int32_t max_blocks, int32_t num_pages, double scale)
{
    if (num_seqs < 0 || max_blocks <= 0 || num_pages <= 0) return ORACLE_BAD_ARG;
    int rc = ORACLE_OK;
    int64_t maxn = 0;
    for (int32_t s = 0; s < num_seqs; ++s)
        if (context_lens[s] > maxn) maxn = context_lens[s];
    #pragma omp parallel for schedule(dynamic) collapse(2) reduction(max : rc)
    for (int32_t s = 0; s < num_seqs; ++s) {
        for (int h = 0; h < O_HQ; ++h) {
            double *o = out + ((size_t)s * O_HQ + h) * O_D;
            int64_t L = context_lens[s];
            int r;
            if (L < 1) {
                r = ORACLE_BAD_LEN;
            } else {
                double *buf = (double *)malloc(sizeof(double) * (size_t)(maxn > 0 ? maxn : 1));
                r = attend(o, q + ((size_t)s * O_HQ + h) * O_D, k_pool, v_pool,
                           block_tables + (size_t)s * max_blocks, max_blocks, num_pages, h / (O_HQ / O_HKV),
                           L, scale, buf);
                free(buf);
            }
            if (r != ORACLE_OK) {
                for (int d = 0; d < O_D; ++d) o[d] = NAN;
                if (r > rc) rc = r;
            }
        }
    }
    return rc;
}

/* Chunked prefill.  For each sequence s and chunk token i (position
 * p = prefix_lens[s] + i): append it as in decode (rotated K, raw V, rotated q
 * in place), then every chunk query attends causally, inclusively, to tokens
 * 0..p of its sequence through the pages.
 * q: [B][C][32][64] (rotated in place), k_chunk/v_chunk: [B][C][8][64],
 * out: [B][C][32][64] fp64.                                                    */
int oracle_prefill_chunk(double *out, uint16_t *q, const uint16_t *k_chunk, const uint16_t *v_chunk,
                         uint16_t *k_pool, uint16_t *v_pool, const int32_t *block_tables,
                         const int32_t *prefix_lens, int32_t num_seqs, int32_t chunk_len,
                         int32_t max_blocks, int32_t num_pages, double theta, double scale)
{
    if (num_seqs < 0 || chunk_len < 0 || max_blocks <= 0 || num_pages <= 0) return ORACLE_BAD_ARG;
    int rc = ORACLE_OK;
    for (int32_t s = 0; s < num_seqs; ++s) {
        if (prefix_lens[s] < 0) { rc = ORACLE_BAD_LEN; continue; }
        for (int32_t i = 0; i < chunk_len; ++i) {
            size_t tok = (size_t)s * chunk_len + i;
            int r = append_token(q + tok * O_HQ * O_D, k_chunk + tok * O_HKV * O_D,
                                 v_chunk + tok * O_HKV * O_D, k_pool, v_pool,
                                 block_tables + (size_t)s * max_blocks, max_blocks, num_pages,
                                 (int64_t)prefix_lens[s] + i, theta);
            if (r != ORACLE_OK) rc = r;
        }
    }
    if (rc != ORACLE_OK) return rc;
    int64_t maxn = 0;
    for (int32_t s = 0; s < num_seqs; ++s)
        if ((int64_t)prefix_lens[s] + chunk_len > maxn) maxn = (int64_t)prefix_lens[s] + chunk_len;
    #pragma omp parallel for schedule(dynamic) collapse(2) reduction(max : rc)
    for (int32_t s = 0; s < num_seqs; ++s) {
        for (int32_t i = 0; i < chunk_len; ++i) {
            double *buf = (double *)malloc(sizeof(double) * (size_t)(maxn > 0 ? maxn : 1));
            for (int h = 0; h < O_HQ; ++h) {
                size_t row = ((size_t)s * chunk_len + i) * O_HQ + h;
                int r = attend(out + row * O_D, q + row * O_D, k_pool, v_pool,
                               block_tables + (size_t)s * max_blocks, max_blocks, num_pages,
                               h / (O_HQ / O_HKV), (int64_t)prefix_lens[s] + i + 1, scale, buf);
                if (r > rc) rc = r;
            }
            free(buf);
        }
    }
    return rc;
}

/* ----------------------------------------------------------- INT8 pages --
 * A KV cache stored as INT8 K/V (TinyLoop, "Lifecycle and Memory Model",
 * RuntimeKVCache INT8 K/V mode).  The pages give no quantisation rule; the
 * reading taken (and the library's documented format) is one symmetric scale
 * per (token, KV head) row of 64 values:
 *     scale = max|x| / 127,   code = round-half-even(x / scale) in [-127, 127],
 * taken in IEEE binary32 (the precision the decision is made in on the device;
 * x86-64 SSE float arithmetic is exactly that), a zero row giving scale 0 and
 * codes 0.  The value a code stands for is code * scale, exact in double.
 * K rows are quantised after RoPE from their bf16-rounded values, V rows from
 * their bf16 input.
 * Tile of (page, head): 2176 bytes = K codes [0,1024) + V codes [1024,2048) +
 * the 16 K scales (float) at 2048+4t + the 16 V scales at 2112+4t.  Code of
 * element d of token t:
 *   K: 16-byte unit ((d mod 32) div 8)*16 + t, byte (d div 32)*8 + d mod 8 in it;
 *   V: 16-byte unit (t div 4)*16 + d mod 16, byte (d div 16)*4 + t mod 4 in it.
 * (A storage layout of this library's own choosing; the pages give none.)  */
#define O_I8_TILE 2176

static size_t i8_tile(int64_t page, int head) { return ((size_t)page * O_HKV + (size_t)head) * O_I8_TILE; }
static size_t i8_kpos(int t, int d) { return (size_t)((((d % 32) / 8) * 16 + t) * 16 + (d / 32) * 8 + d % 8); }
static size_t i8_vpos(int t, int d) { return (size_t)(1024 + ((t / 4) * 16 + d % 16) * 16 + (d / 16) * 4 + t % 4); }
static size_t i8_kscale(int t) { return (size_t)(2048 + 4 * t); }
static size_t i8_vscale(int t) { return (size_t)(2112 + 4 * t); }

/* One row: x given as 64 bf16 patterns. */
void oracle_quantize_row_i8(const uint16_t *x, int8_t *codes, float *scale_out)
{
    float v[O_D];
    float amax = 0.0f;
    for (int d = 0; d < O_D; ++d) {
        v[d] = (float)oracle_bf16_to_f64(x[d]); /* exact */
        if (fabsf(v[d]) > amax) amax = fabsf(v[d]);
    }
    float scale = amax / 127.0f;
    for (int d = 0; d < O_D; ++d) {
        float c = 0.0f;
        if (scale > 0.0f) {
            c = rintf(v[d] / scale);
            if (c > 127.0f) c = 127.0f;
            if (c < -127.0f) c = -127.0f;
        }
        codes[d] = (int8_t)c;
    }
    *scale_out = scale;
}

/* Quantise one row into slot `slot` of a tile: is_v selects the V block. */
static void store_row_i8(uint8_t *tile, int is_v, int slot, const uint16_t *row)
{
    int8_t codes[O_D];
    float sc;
    oracle_quantize_row_i8(row, codes, &sc);
    for (int d = 0; d < O_D; ++d) tile[is_v ? i8_vpos(slot, d) : i8_kpos(slot, d)] = (uint8_t)codes[d];
    memcpy(tile + (is_v ? i8_vscale(slot) : i8_kscale(slot)), &sc, 4);
}

static int append_token_i8(uint16_t *q_tok, const uint16_t *k_tok, const uint16_t *v_tok, uint8_t *pool,
                           const int32_t *bt_row, int32_t max_blocks, int32_t num_pages, int64_t pos, double theta)
{
    int64_t blk = pos / O_PS;
    int slot = (int)(pos % O_PS);
    if (blk >= max_blocks) return ORACLE_BAD_LEN;
    int64_t page = bt_row[blk];
    if (page < 0 || page >= num_pages) return ORACLE_BAD_PAGE;
    double y[O_D];
    uint16_t kb[O_D];
    for (int j = 0; j < O_HKV; ++j) {
        uint8_t *tile = pool + i8_tile(page, j);
        oracle_rope_head(k_tok + (size_t)j * O_D, pos, theta, y);
        for (int d = 0; d < O_D; ++d) kb[d] = oracle_f64_to_bf16(y[d]);
        store_row_i8(tile, 0, slot, kb);
        store_row_i8(tile, 1, slot, v_tok + (size_t)j * O_D);
    }
    if (q_tok) {
        for (int h = 0; h < O_HQ; ++h) {
            oracle_rope_head(q_tok + (size_t)h * O_D, pos, theta, y);
            for (int d = 0; d < O_D; ++d) q_tok[(size_t)h * O_D + d] = oracle_f64_to_bf16(y[d]);
        }
    }
    return ORACLE_OK;
}

/* Decode-time append into an INT8 pool (pool: num_pages * 8 * 2176 bytes). */
int oracle_append_kv_rope_i8(uint16_t *q, const uint16_t *k_new, const uint16_t *v_new, uint8_t *pool,
                             const int32_t *block_tables, const int32_t *context_lens, int32_t num_seqs,
                             int32_t max_blocks, int32_t num_pages, double theta)
{
    if (num_seqs < 0 || max_blocks <= 0 || num_pages <= 0) return ORACLE_BAD_ARG;
    int rc = ORACLE_OK;
    for (int32_t s = 0; s < num_seqs; ++s) {
        int64_t L = context_lens[s];
        if (L < 1) { rc = ORACLE_BAD_LEN; continue; }
        int r = append_token_i8(q ? q + (size_t)s * O_HQ * O_D : NULL, k_new + (size_t)s * O_HKV * O_D,
                                v_new + (size_t)s * O_HKV * O_D, pool, block_tables + (size_t)s * max_blocks,
                                max_blocks, num_pages, L - 1, theta);
        if (r != ORACLE_OK) rc = r;
    }
    return rc;
}

/* Quantise whole pages of a bf16 pool pair (K, V: [P][8][16][64]) into an
 * INT8 pool of the same page count, every (page, head, slot) row through
 * oracle_quantize_row_i8.  A row holding a non-finite value is not a value
 * the format can represent: its bytes are left as they are.                */
static int row_finite(const uint16_t *row)
{
    for (int d = 0; d < O_D; ++d)
        if (!isfinite(oracle_bf16_to_f64(row[d]))) return 0;
    return 1;
}

void oracle_quantize_pages_i8(uint8_t *pool, const uint16_t *k_pool, const uint16_t *v_pool, int32_t num_pages)
{
    for (int64_t p = 0; p < num_pages; ++p)
        for (int j = 0; j < O_HKV; ++j)
            for (int t = 0; t < O_PS; ++t) {
                size_t src = pool_index(p, j, t);
                uint8_t *tile = pool + i8_tile(p, j);
                if (row_finite(k_pool + src)) store_row_i8(tile, 0, t, k_pool + src);
                if (row_finite(v_pool + src)) store_row_i8(tile, 1, t, v_pool + src);
            }
}

/* Value of element d of token t of a tile's K (is_v 0) or V (is_v 1) row.  */
static double i8_value(const uint8_t *tile, int is_v, int t, int d)
{
    float sc;
    memcpy(&sc, tile + (is_v ? i8_vscale(t) : i8_kscale(t)), 4);
    return (double)(int8_t)tile[is_v ? i8_vpos(t, d) : i8_kpos(t, d)] * (double)sc;
}

static int attend_i8(double *out, const uint16_t *q_head, const uint8_t *pool, const int32_t *bt_row,
                     int32_t max_blocks, int32_t num_pages, int kv_head, int64_t n, double scale, double *score_buf)
{
    double qd[O_D];
    for (int d = 0; d < O_D; ++d) qd[d] = oracle_bf16_to_f64(q_head[d]);
    if ((n + O_PS - 1) / O_PS > max_blocks) return ORACLE_BAD_LEN;
    double m = -INFINITY;
    for (int64_t t = 0; t < n; ++t) {
        int64_t page = bt_row[t / O_PS];
        if (page < 0 || page >= num_pages) return ORACLE_BAD_PAGE;
        const uint8_t *tile = pool + i8_tile(page, kv_head);
        double acc = 0.0;
        for (int d = 0; d < O_D; ++d) acc += qd[d] * i8_value(tile, 0, (int)(t % O_PS), d);
        score_buf[t] = scale * acc;
        if (score_buf[t] > m) m = score_buf[t];
    }
    double z = 0.0, o[O_D];
    for (int d = 0; d < O_D; ++d) o[d] = 0.0;
    for (int64_t t = 0; t < n; ++t) {
        const uint8_t *tile = pool + i8_tile(bt_row[t / O_PS], kv_head);
        double w = exp(score_buf[t] - m);
        z += w;
        for (int d = 0; d < O_D; ++d) o[d] += w * i8_value(tile, 1, (int)(t % O_PS), d);
    }
    for (int d = 0; d < O_D; ++d) out[d] = o[d] / z;
    return ORACLE_OK;
}

/* Decode over an INT8 pool: the decode definition with K_t, V_t the values
 * the codes stand for.  out: [B][32][64] fp64.                             */
int oracle_decode_gqa_i8(double *out, const uint16_t *q, const uint8_t *pool, const int32_t *block_tables,
                         const int32_t *context_lens, int32_t num_seqs, int32_t max_blocks, int32_t num_pages,
                         double scale)
{
    if (num_seqs < 0 || max_blocks <= 0 || num_pages <= 0) return ORACLE_BAD_ARG;
    int rc = ORACLE_OK;
    int64_t maxn = 0;
    for (int32_t s = 0; s < num_seqs; ++s)
        if (context_lens[s] > maxn) maxn = context_lens[s];
    #pragma omp parallel for schedule(dynamic) collapse(2) reduction(max : rc)
    for (int32_t s = 0; s < num_seqs; ++s) {
        for (int h = 0; h < O_HQ; ++h) {
            double *o = out + ((size_t)s * O_HQ + h) * O_D;
            int64_t L = context_lens[s];
            int r;
            if (L < 1) {
                r = ORACLE_BAD_LEN;
            } else {
                double *buf = (double *)malloc(sizeof(double) * (size_t)(maxn > 0 ? maxn : 1));
                r = attend_i8(o, q + ((size_t)s * O_HQ + h) * O_D, pool, block_tables + (size_t)s * max_blocks,
                              max_blocks, num_pages, h / (O_HQ / O_HKV), L, scale, buf);
                free(buf);
            }
            if (r != ORACLE_OK) {
                for (int d = 0; d < O_D; ++d) o[d] = NAN;
                if (r > rc) rc = r;
            }
        }
    }
    return rc;
}

/* ------------------------------------------------------------- argmax --
 * Greedy next-token choice over a row of logits (samir-vllm article, section
 * "Architecture et flux d'inference": the argmax runs on the GPU; tiny-vllm
 * ch.2, section "Preallocating the 16 compute buffers": a CPU argmax over the
 * logits row, scanning with a strict greater-than, so the first maximum wins).
 * Reading where the pages are silent: NaN entries are never chosen; the
 * result is the lowest index holding the maximum of the non-NaN entries
 * (-0.0 and +0.0 are equal), and 0 for a row that holds only NaN.
 * logits: [rows][vocab], bf16 patterns (is_bf16) or fp32; out: [rows] int32. */
int oracle_argmax(int32_t *out, const void *logits, int32_t rows, int32_t vocab, int is_bf16)
{
    if (rows < 0 || vocab < 1) return ORACLE_BAD_ARG;
    for (int32_t r = 0; r < rows; ++r) {
        int64_t best = -1;
        double bv = 0.0;
        for (int64_t i = 0; i < vocab; ++i) {
            size_t k = (size_t)r * (size_t)vocab + (size_t)i;
            double v;
            if (is_bf16) {
                v = oracle_bf16_to_f64(((const uint16_t *)logits)[k]);
            } else {
                v = (double)((const float *)logits)[k];
            }
            if (isnan(v)) continue;
            if (best < 0 || v > bv) {
                best = i;
                bv = v;
            }
        }
        out[r] = best < 0 ? 0 : (int32_t)best;
    }
    return ORACLE_OK;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
