/*
 * pa_oracle.c -- plain, slow CPU reference for paged KV-cache attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this file.  It exists so that tests, the smoke check and the
 * CPU-baseline leg of the benchmark can compare the HIP kernels against an
 * independent, obviously correct computation.  It shares no source, header,
 * table or helper with the HIP library.
 *
 * Sources (web pages; cited by title and section):
 *   [L33]  "Lecture 33: KV Cache memory management -- PagedAttention,
 *          Continuous Batching and Chunked Prefill" (lilinji.mintlify.site)
 *   [VM]   "PagedAttention: managing the KV cache like virtual memory"
 *          (inference-learning-path.pages.dev, Part 5)
 *
 * What is computed, and why it is the plain definition:
 *   [L33] §8.1 (misconception table, item 1) states that paging changes only
 *   how addresses are formed; the arithmetic is that of standard attention.
 *   [VM] §6 states that the result equals attention over contiguous KV.
 *   The online softmax of [L33] §2.3 and any split into partitions only
 *   reassociate the same sums.  The oracle is therefore dense softmax
 *   attention over the logically ordered KV, gathered one token at a time
 *   through the block table, evaluated in double precision.  There is no
 *   online softmax, no partitioning and no tiling here.
 *
 * Readings where the pages are silent (each one is also listed with the
 * design notes of the repository):
 *   - GQA: query head h reads KV head floor(h / G), G = Hq / Hkv
 *     (contiguous groups).  [VM] §9 names GQA but gives no mapping.
 *   - Softmax: max-subtracted, no bias, window, soft-cap or sink terms.
 *   - fp8 KV: OCP E4M3FN (bias 7, no infinities, S.1111.111 is NaN, max
 *     magnitude 448).  Stored code e = nearest code to x * (1/s) after
 *     saturation to +-448, ties to the code with even mantissa LSB; the
 *     reciprocal 1/s and the product are both taken in fp32.  Dequantised
 *     value = value(e) * s.  [VM] §3.1 and §9 name an fp8 KV cache only.
 *   - context_lens includes every token the query attends to, its own
 *     token included (written before the read).
 *   - Chunked prefill: a chunk of n rows that ends a request of total
 *     length C starts at P = C - n; row j attends keys [0, P + j]
 *     ([L33] §4.2: a chunk attends to the cached earlier chunks as history,
 *     causal inside the chunk).
 *   - Parity pins for every function are in tests/test_oracle_pins.py; no
 *     function here is "parity unpinned".
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Element types of stored data (values fixed by the oracle's own API). */
enum { OR_F32 = 0, OR_BF16 = 1, OR_FP8 = 2 };

/* ------------------------------------------------------------------ */
/* Scalar codecs                                                      */
/* ------------------------------------------------------------------ */

/* bf16 is the upper half of an IEEE binary32: widen by a 16-bit shift. */
static double bf16_value(uint16_t bits)
{
    uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* OCP 8-bit floating point, E4M3 variant: 1 sign bit, 4 exponent bits
 * (bias 7), 3 mantissa bits; exponent field 0 holds subnormals m * 2^-9;
 * the all-ones exponent with all-ones mantissa is NaN; no infinities. */
double oracle_fp8_value(uint8_t code)
{
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double mag;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* Encode one fp32 value to E4M3 by exhaustive search over the codes of the
 * value's own sign: nearest magnitude wins, ties go to the even code.
 * NaN maps to the NaN code of the same sign; magnitudes beyond 448
 * (infinities included) saturate to 448 first. */
uint8_t oracle_fp8_encode(float y)
{
    int neg = signbit(y) ? 1 : 0;
    double a = fabs((double)y);
    int best = -1;
    double best_err = 0.0;
    if (isnan(y))
        return (uint8_t)((neg << 7) | 0x7F);
    if (a > 448.0)
        a = 448.0;
    for (int c = 0; c < 0x7F; ++c) { /* 0x7F is NaN: skipped */
        double err = fabs(oracle_fp8_value((uint8_t)c) - a);
        if (best < 0 || err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            best_err = err;
        }
    }
    return (uint8_t)((neg << 7) | best);
}

/* Quantise as the cache write does: y = x * (1/s), both steps in fp32. */
uint8_t oracle_fp8_quantize(float x, float kv_scale)
{
    volatile float inv = 1.0f / kv_scale;
    volatile float y = x * inv;
    return oracle_fp8_encode(y);
}

/* Value of element `idx` of an array of the given storage type; fp8 values
 * are dequantised with kv_scale. */
static double stored_value(const void *base, int dtype, int64_t idx, double kv_scale)
{
    switch (dtype) {
    case OR_F32:
        return (double)((const float *)base)[idx];
    case OR_BF16:
        return bf16_value(((const uint16_t *)base)[idx]);
    default:
        return oracle_fp8_value(((const uint8_t *)base)[idx]) * kv_scale;
    }
}

static size_t elt_bytes(int dtype)
{
    return dtype == OR_F32 ? 4 : dtype == OR_BF16 ? 2 : 1;
}

/* ------------------------------------------------------------------ */
/* Cache write: [L33] §2.1 (a new token fills the last block) and     */
/* [VM] §3.3 (decode-step growth); slot = physical block * 16 + offset */
/* ([L33] §2.2 addressing walk-through).                              */
/* ------------------------------------------------------------------ */

/* For every token n with slot_mapping[n] >= 0, copy k[n] and v[n]
 * ([Hkv, d] each, type src_dtype) into pool row `slot` (type cache_dtype).
 * Identity for equal types; fp8 caches store oracle_fp8_quantize(x, s).
 * A pool is [num_slots, Hkv, d]; no other byte is touched. */
void oracle_reshape_and_cache(const void *k, const void *v, void *k_cache, void *v_cache,
                              const int64_t *slot_mapping, int64_t num_tokens,
                              int src_dtype, int cache_dtype, int num_kv_heads,
                              int head_dim, float kv_scale)
{
    int64_t row = (int64_t)num_kv_heads * head_dim;
    for (int64_t n = 0; n < num_tokens; ++n) {
        int64_t slot = slot_mapping[n];
        if (slot < 0)
            continue;
        for (int side = 0; side < 2; ++side) {
            const void *src = side ? v : k;
            void *dst = side ? v_cache : k_cache;
            for (int64_t e = 0; e < row; ++e) {
                int64_t si = n * row + e;
                int64_t di = slot * row + e;
                if (cache_dtype == OR_FP8) {
                    float x = (float)stored_value(src, src_dtype, si, 1.0);
                    ((uint8_t *)dst)[di] = oracle_fp8_quantize(x, kv_scale);
                } else {
                    size_t b = elt_bytes(cache_dtype);
                    memcpy((char *)dst + di * b, (const char *)src + si * b, b);
                }
            }
        }
    }
}

/* Copy-on-write ([L33] §2.4): for every (src, dst) pair, in order, the
 * token rows of block src in both pools are copied over the rows of block
 * dst (pools [num_slots, Hkv, d]; a block is block_bytes of consecutive
 * rows).  A pair naming a block outside [0, num_blocks) is skipped. */
void oracle_copy_blocks(void *k_cache, void *v_cache, const int64_t *pairs, int64_t num_pairs,
                        int64_t num_blocks, int64_t block_bytes)
{
    for (int64_t p = 0; p < num_pairs; ++p) {
        int64_t src = pairs[2 * p], dst = pairs[2 * p + 1];
        if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks)
            continue;
        memmove((char *)k_cache + dst * block_bytes, (const char *)k_cache + src * block_bytes,
                (size_t)block_bytes);
        memmove((char *)v_cache + dst * block_bytes, (const char *)v_cache + src * block_bytes,
                (size_t)block_bytes);
    }
}

/* Swapping ([L33] §5.2): for every (src, dst) pair, in order, block src of
 * the source pools is copied over block dst of the destination pools (two
 * separate pools of the same row layout).  Pairs naming a block outside
 * its pool are skipped. */
void oracle_swap_blocks(const void *src_k, const void *src_v, int64_t src_blocks, void *dst_k,
                        void *dst_v, int64_t dst_blocks, const int64_t *pairs, int64_t num_pairs,
                        int64_t block_bytes)
{
    for (int64_t p = 0; p < num_pairs; ++p) {
        int64_t src = pairs[2 * p], dst = pairs[2 * p + 1];
        if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks)
            continue;
        memcpy((char *)dst_k + dst * block_bytes, (const char *)src_k + src * block_bytes,
               (size_t)block_bytes);
        memcpy((char *)dst_v + dst * block_bytes, (const char *)src_v + src * block_bytes,
               (size_t)block_bytes);
    }
}

/* ------------------------------------------------------------------ */
/* Attention over a paged history                                     */
/* ------------------------------------------------------------------ */

typedef struct {
    /* problem */
    const void *q;
    int q_dtype;
    const void *k_cache, *v_cache;
    int cache_dtype;
    double kv_scale;
    const int32_t *block_tables;
    int32_t max_blocks_per_seq;
    int32_t block_size;        /* tokens per block */
    int num_q_heads, num_kv_heads, head_dim;
    double scale;
    /* decode: query row of seq i is row i; prefill: row index given */
    const int32_t *item_row;   /* query row of each work item            */
    const int32_t *item_seq;   /* table row (sequence) of each work item */
    const int32_t *item_head;  /* query head of each work item           */
    const int32_t *item_nkeys; /* keys 0 .. nkeys-1 are attended         */
    int64_t num_items;
    double *out;               /* [num_items, head_dim]                  */
    /* work distribution */
    int64_t next;
    pthread_mutex_t lock;
} attn_job;

/* Physical slot of logical token t of sequence `seq`: logical block
 * t / B, offset t % B, physical block from the table, slot = block * B +
 * offset, for B tokens per block ([L33] §2.2 walk-through with B = 16; the
 * same formula in its appendix Q1). */
static int64_t token_slot(const attn_job *J, int seq, int64_t t)
{
    int64_t B = J->block_size;
    int64_t logical_block = t / B;
    int64_t offset = t % B;
    int64_t physical_block = J->block_tables[(int64_t)seq * J->max_blocks_per_seq + logical_block];
    return physical_block * B + offset;
}

/* One output row: softmax(scale * q K^T) V over keys [0, nkeys). */
static void attend_one(const attn_job *J, int64_t it, double *scores)
{
    int row = J->item_row[it], seq = J->item_seq[it], h = J->item_head[it];
    int64_t nkeys = J->item_nkeys[it];
    int d = J->head_dim;
    int group = J->num_q_heads / J->num_kv_heads;
    int g = h / group;
    int64_t q_off = ((int64_t)row * J->num_q_heads + h) * d;
    double *o = J->out + it * d;
    double m = -INFINITY, z = 0.0;

    for (int c = 0; c < d; ++c)
        o[c] = 0.0;
    if (nkeys <= 0)
        return;
    for (int64_t t = 0; t < nkeys; ++t) {
        int64_t base = (token_slot(J, seq, t) * J->num_kv_heads + g) * d;
        double s = 0.0;
        for (int c = 0; c < d; ++c)
            s += stored_value(J->q, J->q_dtype, q_off + c, 1.0) *
                 stored_value(J->k_cache, J->cache_dtype, base + c, J->kv_scale);
        scores[t] = J->scale * s;
        if (scores[t] > m)
            m = scores[t];
    }
    for (int64_t t = 0; t < nkeys; ++t) {
        double w = exp(scores[t] - m);
        int64_t base = (token_slot(J, seq, t) * J->num_kv_heads + g) * d;
        z += w;
        for (int c = 0; c < d; ++c)
            o[c] += w * stored_value(J->v_cache, J->cache_dtype, base + c, J->kv_scale);
    }
    for (int c = 0; c < d; ++c)
        o[c] /= z;
}

static void *attn_worker(void *arg)
{
    attn_job *J = (attn_job *)arg;
    int64_t cap = 0;
    double *scores = NULL;
    for (;;) {
        int64_t it;
        pthread_mutex_lock(&J->lock);
        it = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (it >= J->num_items)
            break;
        if (J->item_nkeys[it] > cap) {
            cap = J->item_nkeys[it];
            free(scores);
            scores = (double *)malloc((size_t)cap * sizeof(double));
            if (!scores)
                abort();
        }
        attend_one(J, it, scores);
    }
    free(scores);
    return NULL;
}

static void run_items(attn_job *J, int num_threads)
{
    pthread_t tid[256];
    if (num_threads < 1)
        num_threads = 1;
    if (num_threads > 256)
        num_threads = 256;
    J->next = 0;
    pthread_mutex_init(&J->lock, NULL);
    for (int i = 0; i < num_threads; ++i)
        pthread_create(&tid[i], NULL, attn_worker, J);
    for (int i = 0; i < num_threads; ++i)
        pthread_join(tid[i], NULL);
    pthread_mutex_destroy(&J->lock);
}

/* Decode attention ([L33] §2.3: one query per sequence reads its own
 * scattered blocks through the table).  Work items are (seq, q head)
 * pairs given by sel_seq / sel_head (num_sel of them), so that a caller
 * can ask for a sample of outputs; out is [num_sel, head_dim].
 * q is [S, Hq, d]; pools are [N*16 slots, Hkv, d]; a sequence attends
 * context_lens[seq] tokens. */
int oracle_decode(double *out, const void *q, int q_dtype, const void *k_cache,
                  const void *v_cache, int cache_dtype, double kv_scale,
                  const int32_t *block_tables, int32_t max_blocks_per_seq,
                  const int32_t *context_lens, int num_q_heads, int num_kv_heads,
                  int head_dim, double scale, const int32_t *sel_seq,
                  const int32_t *sel_head, int64_t num_sel, int num_threads, int block_size)
{
    attn_job J;
    int32_t *nkeys;
    if (num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 || block_size <= 0)
        return -1;
    nkeys = (int32_t *)malloc((size_t)(num_sel > 0 ? num_sel : 1) * sizeof(int32_t));
    if (!nkeys)
        return -2;
    for (int64_t i = 0; i < num_sel; ++i)
        nkeys[i] = context_lens[sel_seq[i]];
    memset(&J, 0, sizeof J);
    J.q = q; J.q_dtype = q_dtype;
    J.k_cache = k_cache; J.v_cache = v_cache; J.cache_dtype = cache_dtype;
    J.kv_scale = kv_scale;
    J.block_tables = block_tables; J.max_blocks_per_seq = max_blocks_per_seq;
    J.block_size = block_size;
    J.num_q_heads = num_q_heads; J.num_kv_heads = num_kv_heads; J.head_dim = head_dim;
    J.scale = scale;
    J.item_row = sel_seq; J.item_seq = sel_seq; J.item_head = sel_head;
    J.item_nkeys = nkeys; J.num_items = num_sel; J.out = out;
    run_items(&J, num_threads);
    free(nkeys);
    return 0;
}

/* Chunked prefill ([L33] §4.2): request r owns query rows
 * [query_start[r], query_start[r+1]) of q ([Tq, Hq, d]); its chunk is the
 * last n_r tokens of its context_lens[r] cached tokens, so row j of the
 * chunk attends keys [0, context_lens[r] - n_r + j].  Work items are
 * (query row, q head) pairs from sel_row / sel_head; out is
 * [num_sel, head_dim]. */
int oracle_prefill(double *out, const void *q, int q_dtype, const void *k_cache,
                   const void *v_cache, int cache_dtype, double kv_scale,
                   const int32_t *block_tables, int32_t max_blocks_per_seq,
                   const int32_t *query_start, const int32_t *context_lens,
                   int num_requests, int num_q_heads, int num_kv_heads, int head_dim,
                   double scale, const int32_t *sel_row, const int32_t *sel_head,
                   int64_t num_sel, int num_threads, int block_size)
{
    attn_job J;
    int32_t *nkeys, *seq;
    if (num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 || block_size <= 0)
        return -1;
    nkeys = (int32_t *)malloc((size_t)(num_sel > 0 ? num_sel : 1) * sizeof(int32_t));
    seq = (int32_t *)malloc((size_t)(num_sel > 0 ? num_sel : 1) * sizeof(int32_t));
    if (!nkeys || !seq) {
        free(nkeys);
        free(seq);
        return -2;
    }
    for (int64_t i = 0; i < num_sel; ++i) {
        int r = -1;
        for (int k = 0; k < num_requests; ++k)
            if (sel_row[i] >= query_start[k] && sel_row[i] < query_start[k + 1])
                r = k;
        if (r < 0) {
            free(nkeys);
            free(seq);
            return -3;
        }
        {
            int n = query_start[r + 1] - query_start[r];
            int j = sel_row[i] - query_start[r];
            seq[i] = r;
            nkeys[i] = context_lens[r] - n + j + 1;
        }
    }
    memset(&J, 0, sizeof J);
    J.q = q; J.q_dtype = q_dtype;
    J.k_cache = k_cache; J.v_cache = v_cache; J.cache_dtype = cache_dtype;
    J.kv_scale = kv_scale;
    J.block_tables = block_tables; J.max_blocks_per_seq = max_blocks_per_seq;
    J.block_size = block_size;
    J.num_q_heads = num_q_heads; J.num_kv_heads = num_kv_heads; J.head_dim = head_dim;
    J.scale = scale;
    J.item_row = sel_row; J.item_seq = seq; J.item_head = sel_head;
    J.item_nkeys = nkeys; J.num_items = num_sel; J.out = out;
    run_items(&J, num_threads);
    free(nkeys);
    free(seq);
    return 0;
}
