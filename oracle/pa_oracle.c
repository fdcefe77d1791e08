/*
 * Oracle for the paged-KV-cache hot path: a plain, slow, fp64 CPU
 * implementation used ONLY as test infrastructure.  It may be loaded by the
 * test suite, by the smoke check and by the benchmark's cpu_baseline leg;
 * the product library never links, loads or calls it, and it shares no code,
 * header, table or helper with the GPU path.
 *
 * Sources (pages are named by address; sections as they number them):
 *   [5688vip]  5688vip.com, "4、PagedAttention：显存管理、分页机制、块大小选择"
 *   [lpnh-2758356]  lpnh.cn/news/2758356 (block mapping, on-demand
 *              allocation, copy-on-write), sections 1-5
 *   [lpnh-1824136]  lpnh.cn/news/1824136 (the SOSP 2023 paper and vLLM),
 *              sections 1-4
 *
 * What it computes:
 *
 *  - Cache layout: one tensor per layer of fixed-size physical blocks, each
 *    block a contiguous [num_kv_heads, block_size, head_dim] slab.  The pages
 *    give the per-block shape as block_size x kv heads x head_dim and keep
 *    each block's data contiguous while blocks are scattered
 *    ([lpnh-2758356] 2.1 and the note after 2.2).
 *
 *  - Address translation: logical token position p is found in physical
 *    block table[p / block_size] at offset p % block_size ([5688vip]
 *    section 分页机制, block-table figure; [lpnh-2758356] 2.2).
 *
 *  - Scatter (reshape-and-cache): each new token's K and V vectors go to the
 *    slot its block table assigns ([lpnh-1824136] 3.1: the kernels write
 *    results back into the proper blocks).
 *
 *  - Block copy: copy-on-write gives the writer a fresh block holding a copy
 *    of the whole shared block ([lpnh-2758356] 4.2, third step).
 *
 *  - Decode attention: the new token attends to every cached K/V of its
 *    sequence, which is ordinary attention over the logically contiguous
 *    K/V since paging is invisible to the model ([lpnh-2758356] 2.2;
 *    [lpnh-1824136] 2.2).  The pages never write the formula; the reading
 *    taken is textbook scaled dot-product softmax attention
 *        z_t = scale * <q, k_t>,  w = softmax(z),  out = sum_t w_t v_t,
 *    and a sequence of length 0 gives an all-zero output.
 *
 * All values are IEEE binary16 bit patterns (uint16_t) on input; arithmetic
 * is binary64.  Outputs of the attention routines are binary64.
 */
#include <errno.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL -1
#define ORACLE_ENOMEM -2
#define ORACLE_ERANGE -3

/* IEEE 754 binary16 -> binary64 straight from the format: 1 sign bit,
 * 5 exponent bits with bias 15, 10 fraction bits. */
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);               /* subnormal: f * 2^-24   */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);   /* (1 + f/2^10) * 2^(e-15) */
    return sign ? -v : v;
}

/* ---------------------------------------------------------------------- */
/* Softmax attention of one query over n contiguous keys/values (fp64).   */
/* ---------------------------------------------------------------------- */
static int attend(double *out, const double *q, const double *K,
                  const double *V, int64_t n, int D, double scale)
{
    if (n == 0) {
        for (int d = 0; d < D; ++d) out[d] = 0.0;
        return ORACLE_OK;
    }
    double *w = (double *)malloc((size_t)n * sizeof(double));
    if (!w) return ORACLE_ENOMEM;
    double m = -INFINITY;
    for (int64_t t = 0; t < n; ++t) {
        double z = 0.0;
        for (int d = 0; d < D; ++d) z += q[d] * K[t * D + d];
        z *= scale;
        w[t] = z;
        if (z > m) m = z;
    }
    double sum = 0.0;
    for (int64_t t = 0; t < n; ++t) {
        w[t] = exp(w[t] - m);
        sum += w[t];
    }
    for (int d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int64_t t = 0; t < n; ++t) acc += w[t] * V[t * D + d];
        out[d] = acc / sum;
    }
    free(w);
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------- */
/* Work splitting over (sequence, head) pairs with plain pthreads.        */
/* ---------------------------------------------------------------------- */
typedef int (*item_fn)(void *ctx, int64_t item);

struct pool_arg {
    void *ctx;
    item_fn fn;
    int64_t n_items;
    int tid, nthreads;
    int status;
};

static void *pool_main(void *p)
{
    struct pool_arg *a = (struct pool_arg *)p;
    a->status = ORACLE_OK;
    for (int64_t i = a->tid; i < a->n_items; i += a->nthreads) {
        int rc = a->fn(a->ctx, i);
        if (rc != ORACLE_OK) { a->status = rc; break; }
    }
    return NULL;
}

static int run_items(void *ctx, item_fn fn, int64_t n_items, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > n_items) nthreads = n_items > 0 ? (int)n_items : 1;
    struct pool_arg args[256];
    pthread_t th[256];
    for (int i = 0; i < nthreads; ++i) {
        args[i].ctx = ctx; args[i].fn = fn; args[i].n_items = n_items;
        args[i].tid = i; args[i].nthreads = nthreads; args[i].status = ORACLE_OK;
    }
    if (nthreads == 1) {
        pool_main(&args[0]);
        return args[0].status;
    }
    int started = 0, rc = ORACLE_OK;
    for (; started < nthreads; ++started)
        if (pthread_create(&th[started], NULL, pool_main, &args[started]) != 0) break;
    if (started < nthreads) {           /* finish the unstarted shares inline */
        for (int i = started; i < nthreads; ++i) pool_main(&args[i]);
    }
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    for (int i = 0; i < nthreads; ++i)
        if (args[i].status != ORACLE_OK) rc = args[i].status;
    return rc;
}

/* ---------------------------------------------------------------------- */
/* Paged decode: gather through the block table, then attend.             */
/* ---------------------------------------------------------------------- */
struct decode_ctx {
    double *out;
    const uint16_t *q, *k_cache, *v_cache;
    const int32_t *block_tables, *context_lens;
    int32_t max_blocks, H, Hkv, D, B;
    int64_t num_blocks;
    double scale;
};

static int decode_item(void *vctx, int64_t item)
{
    const struct decode_ctx *c = (const struct decode_ctx *)vctx;
    int64_t s = item / c->H;
    int h = (int)(item % c->H);
    int kvh = h / (c->H / c->Hkv);            /* query head -> its KV head */
    int D = c->D, B = c->B;
    int64_t n = c->context_lens[s];
    if (n < 0 || n > (int64_t)c->max_blocks * B) return ORACLE_ERANGE;

    double *q = (double *)malloc((size_t)D * sizeof(double));
    double *K = (double *)malloc((size_t)(n ? n : 1) * D * sizeof(double));
    double *V = (double *)malloc((size_t)(n ? n : 1) * D * sizeof(double));
    if (!q || !K || !V) { free(q); free(K); free(V); return ORACLE_ENOMEM; }

    for (int d = 0; d < D; ++d)
        q[d] = oracle_half_to_double(c->q[(s * c->H + h) * D + d]);

    /* gather: logical position p -> (physical block, offset) */
    for (int64_t p = 0; p < n; ++p) {
        int64_t phys = c->block_tables[s * c->max_blocks + p / B];
        if (phys < 0 || phys >= c->num_blocks) {
            free(q); free(K); free(V);
            return ORACLE_ERANGE;
        }
        int64_t base = ((phys * c->Hkv + kvh) * B + p % B) * (int64_t)D;
        for (int d = 0; d < D; ++d) {
            K[p * D + d] = oracle_half_to_double(c->k_cache[base + d]);
            V[p * D + d] = oracle_half_to_double(c->v_cache[base + d]);
        }
    }
    int rc = attend(c->out + (s * c->H + h) * (int64_t)D, q, K, V, n, D, c->scale);
    free(q); free(K); free(V);
    return rc;
}

/*
 * out[S, H, D] (fp64) = attention of q[S, H, D] over each sequence's first
 * context_lens[s] cached tokens, found through block_tables[S, max_blocks].
 * Caches are [num_blocks, Hkv, B, D].  Query head h reads KV head
 * h / (H / Hkv).  Returns 0, or a negative code on bad arguments / a table
 * entry outside [0, num_blocks).
 */
int oracle_decode(double *out, const uint16_t *q, const uint16_t *k_cache,
                  const uint16_t *v_cache, const int32_t *block_tables,
                  int32_t max_blocks, const int32_t *context_lens,
                  int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                  int32_t head_dim, int32_t block_size, int64_t num_blocks,
                  double scale, int32_t nthreads)
{
    if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
        return ORACLE_EINVAL;
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 ||
        num_heads % num_kv_heads || head_dim <= 0 || block_size <= 0 ||
        max_blocks < 0 || num_blocks < 0)
        return ORACLE_EINVAL;
    struct decode_ctx c = {out, q, k_cache, v_cache, block_tables, context_lens,
                           max_blocks, num_heads, num_kv_heads, head_dim,
                           block_size, num_blocks, scale};
    return run_items(&c, decode_item, (int64_t)num_seqs * num_heads, nthreads);
}

/* ---------------------------------------------------------------------- */
/* Paged prefill / chunked prefill: several new tokens of a sequence,     */
/* each attending causally to the cached positions up to its own.         */
/*                                                                        */
/* Sequence s has n = context_lens[s] cached tokens, the last m of which  */
/* are its new ones (m = query_start[s+1] - query_start[s]); query row    */
/* query_start[s] + i is the token at position n - m + i and attends to   */
/* positions 0 .. n - m + i.  This is the prompt path of a request (the   */
/* pages: [lpnh-1824136] 3.2 second step; the attention kernels must read */
/* the paged cache since a contiguous-memory kernel cannot, [n1n] on the  */
/* limits of FlashAttention), with the same textbook softmax attention as */
/* decode; m = 1 is decode.                                               */
/* ---------------------------------------------------------------------- */
struct prefill_ctx {
    double *out;
    const uint16_t *q, *k_cache, *v_cache;
    const int32_t *block_tables, *context_lens, *query_start;
    int32_t max_blocks, H, Hkv, D, B;
    int64_t num_blocks;
    double scale;
};

static int prefill_item(void *vctx, int64_t item)
{
    const struct prefill_ctx *c = (const struct prefill_ctx *)vctx;
    int64_t s = item / c->H;
    int h = (int)(item % c->H);
    int kvh = h / (c->H / c->Hkv);
    int D = c->D, B = c->B;
    int64_t n = c->context_lens[s];
    int64_t q0 = c->query_start[s], m = c->query_start[s + 1] - q0;
    if (n < 0 || m < 0 || m > n || n > (int64_t)c->max_blocks * B) return ORACLE_ERANGE;
    if (m == 0) return ORACLE_OK;

    double *q = (double *)malloc((size_t)D * sizeof(double));
    double *K = (double *)malloc((size_t)n * D * sizeof(double));
    double *V = (double *)malloc((size_t)n * D * sizeof(double));
    if (!q || !K || !V) { free(q); free(K); free(V); return ORACLE_ENOMEM; }
    for (int64_t p = 0; p < n; ++p) {
        int64_t phys = c->block_tables[s * c->max_blocks + p / B];
        if (phys < 0 || phys >= c->num_blocks) { free(q); free(K); free(V); return ORACLE_ERANGE; }
        int64_t base = ((phys * c->Hkv + kvh) * B + p % B) * (int64_t)D;
        for (int d = 0; d < D; ++d) {
            K[p * D + d] = oracle_half_to_double(c->k_cache[base + d]);
            V[p * D + d] = oracle_half_to_double(c->v_cache[base + d]);
        }
    }
    int rc = ORACLE_OK;
    for (int64_t i = 0; i < m && rc == ORACLE_OK; ++i) {
        int64_t row = (q0 + i) * c->H + h;
        for (int d = 0; d < D; ++d) q[d] = oracle_half_to_double(c->q[row * D + d]);
        /* causal: the token at position n - m + i sees positions 0 .. n - m + i */
        rc = attend(c->out + row * D, q, K, V, n - m + i + 1, D, c->scale);
    }
    free(q); free(K); free(V);
    return rc;
}

int oracle_prefill(double *out, const uint16_t *q, const uint16_t *k_cache,
                   const uint16_t *v_cache, const int32_t *block_tables,
                   int32_t max_blocks, const int32_t *context_lens,
                   const int32_t *query_start, int32_t num_seqs, int32_t num_heads,
                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                   int64_t num_blocks, double scale, int32_t nthreads)
{
    if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start)
        return ORACLE_EINVAL;
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 ||
        num_heads % num_kv_heads || head_dim <= 0 || block_size <= 0 ||
        max_blocks < 0 || num_blocks < 0)
        return ORACLE_EINVAL;
    struct prefill_ctx c = {out, q, k_cache, v_cache, block_tables, context_lens, query_start,
                            max_blocks, num_heads, num_kv_heads, head_dim, block_size,
                            num_blocks, scale};
    return run_items(&c, prefill_item, (int64_t)num_seqs * num_heads, nthreads);
}

/* ---------------------------------------------------------------------- */
/* Attention over logically contiguous K/V (no paging).                   */
/* ---------------------------------------------------------------------- */
struct contig_ctx {
    double *out;
    const uint16_t *q, *k, *v;
    const int64_t *seq_start;
    const int32_t *lens;
    int32_t H, Hkv, D;
    double scale;
};

static int contig_item(void *vctx, int64_t item)
{
    const struct contig_ctx *c = (const struct contig_ctx *)vctx;
    int64_t s = item / c->H;
    int h = (int)(item % c->H);
    int kvh = h / (c->H / c->Hkv);
    int D = c->D;
    int64_t n = c->lens[s];
    if (n < 0) return ORACLE_ERANGE;
    double *q = (double *)malloc((size_t)D * sizeof(double));
    double *K = (double *)malloc((size_t)(n ? n : 1) * D * sizeof(double));
    double *V = (double *)malloc((size_t)(n ? n : 1) * D * sizeof(double));
    if (!q || !K || !V) { free(q); free(K); free(V); return ORACLE_ENOMEM; }
    for (int d = 0; d < D; ++d)
        q[d] = oracle_half_to_double(c->q[(s * c->H + h) * D + d]);
    for (int64_t p = 0; p < n; ++p) {
        int64_t base = ((c->seq_start[s] + p) * c->Hkv + kvh) * (int64_t)D;
        for (int d = 0; d < D; ++d) {
            K[p * D + d] = oracle_half_to_double(c->k[base + d]);
            V[p * D + d] = oracle_half_to_double(c->v[base + d]);
        }
    }
    int rc = attend(c->out + (s * c->H + h) * (int64_t)D, q, K, V, n, D, c->scale);
    free(q); free(K); free(V);
    return rc;
}

/*
 * Same attention with K/V given contiguously: sequence s owns tokens
 * [seq_start[s], seq_start[s] + lens[s]) of k/v, laid out [tokens, Hkv, D].
 */
int oracle_attention_contig(double *out, const uint16_t *q, const uint16_t *k,
                            const uint16_t *v, const int64_t *seq_start,
                            const int32_t *lens, int32_t num_seqs,
                            int32_t num_heads, int32_t num_kv_heads,
                            int32_t head_dim, double scale, int32_t nthreads)
{
    if (!out || !q || !k || !v || !seq_start || !lens) return ORACLE_EINVAL;
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 ||
        num_heads % num_kv_heads || head_dim <= 0)
        return ORACLE_EINVAL;
    struct contig_ctx c = {out, q, k, v, seq_start, lens, num_heads,
                           num_kv_heads, head_dim, scale};
    return run_items(&c, contig_item, (int64_t)num_seqs * num_heads, nthreads);
}

/* ---------------------------------------------------------------------- */
/* Scatter of new tokens into their slots, bit for bit.                   */
/* ---------------------------------------------------------------------- */
/*
 * For every token t with slot_mapping[t] >= 0, copy key[t, h, :] and
 * value[t, h, :] (token stride kv_token_stride elements, head stride D) into
 * cache[slot / B, h, slot % B, :] for all h < Hkv.  A negative slot is
 * skipped.  Slots must lie below num_blocks * B.
 */
int oracle_reshape_and_cache(const uint16_t *key, const uint16_t *value,
                             int64_t kv_token_stride,
                             const int64_t *slot_mapping, int32_t num_tokens,
                             uint16_t *k_cache, uint16_t *v_cache,
                             int64_t num_blocks, int32_t num_kv_heads,
                             int32_t block_size, int32_t head_dim)
{
    if (num_tokens < 0 || num_kv_heads <= 0 || block_size <= 0 || head_dim <= 0)
        return ORACLE_EINVAL;
    if (num_tokens > 0 && (!key || !value || !slot_mapping || !k_cache || !v_cache))
        return ORACLE_EINVAL;
    for (int32_t t = 0; t < num_tokens; ++t) {
        int64_t slot = slot_mapping[t];
        if (slot < 0) continue;
        if (slot >= num_blocks * block_size) return ORACLE_ERANGE;
        int64_t blk = slot / block_size, off = slot % block_size;
        for (int32_t h = 0; h < num_kv_heads; ++h) {
            const uint16_t *ks = key + t * kv_token_stride + (int64_t)h * head_dim;
            const uint16_t *vs = value + t * kv_token_stride + (int64_t)h * head_dim;
            int64_t dst = ((blk * num_kv_heads + h) * block_size + off) * head_dim;
            memcpy(k_cache + dst, ks, (size_t)head_dim * sizeof(uint16_t));
            memcpy(v_cache + dst, vs, (size_t)head_dim * sizeof(uint16_t));
        }
    }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------- */
/* Whole-block copies for copy-on-write, applied as if simultaneous.      */
/* ---------------------------------------------------------------------- */
/*
 * For every layer l < num_layers and pair i: block pairs[2i+1] of
 * k_caches[l] / v_caches[l] becomes a copy of block pairs[2i].  All sources
 * are read before any destination is written.
 */
int oracle_copy_blocks(uint16_t *const *k_caches, uint16_t *const *v_caches,
                       int32_t num_layers, const int64_t *pairs,
                       int32_t num_pairs, int64_t block_elems,
                       int64_t num_blocks)
{
    if (num_layers < 0 || num_pairs < 0 || block_elems <= 0) return ORACLE_EINVAL;
    if (num_pairs == 0 || num_layers == 0) return ORACLE_OK;
    if (!k_caches || !v_caches || !pairs) return ORACLE_EINVAL;
    for (int32_t i = 0; i < 2 * num_pairs; ++i)
        if (pairs[i] < 0 || pairs[i] >= num_blocks) return ORACLE_ERANGE;
    size_t bytes = (size_t)block_elems * sizeof(uint16_t);
    uint16_t *snap = (uint16_t *)malloc(bytes * (size_t)num_pairs * 2);
    if (!snap) return ORACLE_ENOMEM;
    for (int32_t l = 0; l < num_layers; ++l) {
        for (int32_t i = 0; i < num_pairs; ++i) {
            memcpy(snap + (2 * (size_t)i) * block_elems,
                   k_caches[l] + pairs[2 * i] * block_elems, bytes);
            memcpy(snap + (2 * (size_t)i + 1) * block_elems,
                   v_caches[l] + pairs[2 * i] * block_elems, bytes);
        }
        for (int32_t i = 0; i < num_pairs; ++i) {
            memcpy(k_caches[l] + pairs[2 * i + 1] * block_elems,
                   snap + (2 * (size_t)i) * block_elems, bytes);
            memcpy(v_caches[l] + pairs[2 * i + 1] * block_elems,
                   snap + (2 * (size_t)i + 1) * block_elems, bytes);
        }
    }
    free(snap);
    return ORACLE_OK;
}
