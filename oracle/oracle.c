/*
 * Plain CPU oracle for paged decode attention and its two block operations.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this file: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or helper with the
 * HIP library; the two meet only through the seeded input generators.
 *
 * Everything is single-threaded, unblocked and unfused, and every floating
 * point step runs in IEEE binary64.  Stored f32 / f16 / bf16 values are decoded
 * to binary64 exactly (every such value is representable).
 *
 * Sources (four web pages on vLLM's PagedAttention):
 *  - "PagedAttention" concept report (compassingai.com), §5: the cache is cut
 *    into fixed-size physical blocks of B tokens; a per-request block table
 *    (an integer array) maps logical block j to a physical block id; the kernel
 *    walks the table and reads a token at (physical block base + offset).
 *  - same page, §8: decode attention is the query's dot product with every key,
 *    a softmax over those scores, and the softmax-weighted sum of the values;
 *    the kernel's outer loop walks blocks in table order, the inner loop tokens.
 *  - same page, §6: before a write into a block whose reference count exceeds
 *    one, a new block is allocated and the old block's content copied into it.
 *  - KV-cache / paging tutorial (wmrh.cn), "KV cache" part: at a decode step only
 *    the newest token's K and V are computed; the prediction attends over the
 *    cached K/V of all earlier tokens plus the newest one.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *  - K and V live in two pools of identical layout [num_blocks][H_kv][B][d].
 *  - context_lens[s] counts the newest token, which is written first.
 *  - query head h reads KV head h / (H_q / H_kv).
 *  - a context of length 0 yields an all-zero output.
 *  - slot = physical_block * B + offset; a negative slot is skipped.
 *
 * ORACLE_MUTANT (compile-time, tests only) plants one known mistake so the test
 * suite can show that its pins catch it; the shipped build defines it as 0.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

enum { ORACLE_F32 = 0, ORACLE_F16 = 1, ORACLE_BF16 = 2 };
enum { ORACLE_OK = 0, ORACLE_BAD_ARG = 1, ORACLE_BAD_INDEX = 2, ORACLE_NO_MEM = 3 };

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double f16_bits_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);                 /* zero or subnormal */
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), expo - 25);  /* (1.frac) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32 word. */
static double bf16_bits_to_f64(uint16_t b)
{
    uint32_t w = (uint32_t)b << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

double oracle_load(const void *base, int64_t idx, int dtype)
{
    if (dtype == ORACLE_F32) {
        float f;
        memcpy(&f, (const char *)base + idx * 4, 4);
        return (double)f;
    }
    uint16_t u;
    memcpy(&u, (const char *)base + idx * 2, 2);
    return dtype == ORACLE_F16 ? f16_bits_to_f64(u) : bf16_bits_to_f64(u);
}

static int elem_bytes(int dtype)
{
    return dtype == ORACLE_F32 ? 4 : (dtype == ORACLE_F16 || dtype == ORACLE_BF16) ? 2 : 0;
}

/* Element offset of K or V for (physical block b, kv head k, in-block slot o, dim j). */
static int64_t pool_index(int64_t b, int k, int o, int j, int Hkv, int B, int d)
{
#if ORACLE_MUTANT == 7
    /* planted: head and slot axes swapped */
    return ((b * B + o) * Hkv + k) * d + j;
#else
    return ((b * Hkv + k) * B + o) * d + j;
#endif
}

/*
 * out[s][h][:]  (binary64, [S][H_q][d]) for every sequence s and query head h:
 *   n   = context_lens[s]
 *   x_t = scale * sum_j q[s][h][j] * K(t)[j]            for t < n
 *   p_t = exp(x_t - max_t x_t),   Z = sum_t p_t
 *   out = sum_t p_t * V(t) / Z
 * where K(t), V(t) are read at physical block block_tables[s][t / B], slot t % B,
 * KV head h / (H_q / H_kv).  Returns ORACLE_BAD_INDEX if a table entry needed
 * for t < n is outside [0, num_blocks) or t / B reaches max_blocks_per_seq.
 */
int oracle_decode(double *out, const void *query, const void *key_cache, const void *value_cache,
                  const int32_t *block_tables, int max_blocks_per_seq, const int32_t *context_lens,
                  int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                  int num_blocks, double scale, int dtype)
{
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        num_q_heads % num_kv_heads != 0 || elem_bytes(dtype) == 0)
        return ORACLE_BAD_ARG;
    const int g = num_q_heads / num_kv_heads;
    const int d = head_dim, B = block_size, Hkv = num_kv_heads;

    for (int s = 0; s < num_seqs; ++s) {
        const int n = context_lens[s];
        if (n < 0) return ORACLE_BAD_ARG;
        double *x = (double *)malloc(sizeof(double) * (n > 0 ? n : 1));
        if (!x) return ORACLE_NO_MEM;
        for (int h = 0; h < num_q_heads; ++h) {
#if ORACLE_MUTANT == 2
            const int k = h % Hkv;           /* planted: wrong group mapping */
#else
            const int k = h / g;
#endif
            double *o_row = out + ((int64_t)s * num_q_heads + h) * d;
            const int64_t q_row = ((int64_t)s * num_q_heads + h) * d;
            if (n == 0) {
                for (int j = 0; j < d; ++j) o_row[j] = 0.0;
                continue;
            }
            /* scores, walking the block table */
            for (int t = 0; t < n; ++t) {
                const int lb = t / B;
#if ORACLE_MUTANT == 3
                const int off = (t + 1) % B;  /* planted: off-by-one slot */
#else
                const int off = t % B;
#endif
                if (lb >= max_blocks_per_seq) { free(x); return ORACLE_BAD_INDEX; }
                const int64_t pb = block_tables[(int64_t)s * max_blocks_per_seq + lb];
                if (pb < 0 || pb >= num_blocks) { free(x); return ORACLE_BAD_INDEX; }
                double dot = 0.0;
                for (int j = 0; j < d; ++j)
                    dot += oracle_load(query, q_row + j, dtype) *
                           oracle_load(key_cache, pool_index(pb, k, off, j, Hkv, B, d), dtype);
#if ORACLE_MUTANT == 1
                x[t] = dot;                   /* planted: scale dropped */
#else
                x[t] = scale * dot;
#endif
            }
            /* softmax */
            double m = x[0];
            for (int t = 1; t < n; ++t)
                if (x[t] > m) m = x[t];
#if ORACLE_MUTANT == 4
            m = 0.0;                          /* planted: no max subtraction */
#endif
            double Z = 0.0;
#if ORACLE_MUTANT == 5
            for (int t = 0; t + 1 < n; ++t)   /* planted: last token left out of Z */
#else
            for (int t = 0; t < n; ++t)
#endif
            {
#if ORACLE_MUTANT == 10
                x[t] = exp(m - x[t]);         /* planted: sign flipped */
#else
                x[t] = exp(x[t] - m);
#endif
                Z += x[t];
            }
#if ORACLE_MUTANT == 5
            x[n - 1] = exp(x[n - 1] - m);
#endif
            /* weighted sum of values */
            for (int j = 0; j < d; ++j) {
                double acc = 0.0;
                for (int t = 0; t < n; ++t) {
                    const int64_t pb = block_tables[(int64_t)s * max_blocks_per_seq + t / B];
#if ORACLE_MUTANT == 6
                    const void *vsrc = key_cache;   /* planted: K used in place of V */
#else
                    const void *vsrc = value_cache;
#endif
                    acc += x[t] * oracle_load(vsrc, pool_index(pb, k, t % B, j, Hkv, B, d), dtype);
                }
                o_row[j] = acc / Z;
            }
        }
        free(x);
    }
    return ORACLE_OK;
}

/*
 * For every token i with slot = slot_mapping[i] >= 0: physical block slot / B,
 * in-block position slot % B; for every KV head k, copy key[i][k][:] into the key
 * pool and value[i][k][:] into the value pool at that place, bit for bit.
 * ORACLE_BAD_INDEX if slot / B >= num_blocks.
 */
int oracle_reshape_and_cache(const void *key, const void *value, void *key_cache, void *value_cache,
                             const int32_t *slot_mapping, int num_tokens, int num_kv_heads,
                             int head_dim, int block_size, int num_blocks, int dtype)
{
    const int eb = elem_bytes(dtype);
    if (eb == 0 || num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0)
        return ORACLE_BAD_ARG;
    for (int i = 0; i < num_tokens; ++i) {
        const int64_t slot = slot_mapping[i];
        if (slot < 0) continue;
#if ORACLE_MUTANT == 8
        const int64_t b = slot % block_size, off = slot / block_size; /* planted: swapped */
#else
        const int64_t b = slot / block_size, off = slot % block_size;
#endif
        if (b >= num_blocks || off >= block_size) return ORACLE_BAD_INDEX;
        for (int k = 0; k < num_kv_heads; ++k)
            for (int j = 0; j < head_dim; ++j) {
                const int64_t src = ((int64_t)i * num_kv_heads + k) * head_dim + j;
                const int64_t dst = pool_index(b, k, (int)off, j, num_kv_heads, block_size, head_dim);
                memcpy((char *)key_cache + dst * eb, (const char *)key + src * eb, eb);
                memcpy((char *)value_cache + dst * eb, (const char *)value + src * eb, eb);
            }
    }
    return ORACLE_OK;
}

/*
 * For each pair p in order: the whole physical block src[p] (every KV head,
 * every slot, every dim) of both pools is copied onto block dst[p], bit for bit.
 * ORACLE_BAD_INDEX if an id is outside [0, num_blocks).
 */
int oracle_copy_blocks(void *key_cache, void *value_cache, const int32_t *src, const int32_t *dst,
                       int num_pairs, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                       int dtype)
{
    const int eb = elem_bytes(dtype);
    if (eb == 0 || num_pairs < 0) return ORACLE_BAD_ARG;
    const int64_t block_elems = (int64_t)num_kv_heads * block_size * head_dim;
    for (int p = 0; p < num_pairs; ++p) {
        if (src[p] < 0 || src[p] >= num_blocks || dst[p] < 0 || dst[p] >= num_blocks)
            return ORACLE_BAD_INDEX;
        for (int64_t e = 0; e < block_elems; ++e) {
            const int64_t so = (int64_t)src[p] * block_elems + e;
            const int64_t dO = (int64_t)dst[p] * block_elems + e;
            memcpy((char *)key_cache + dO * eb, (const char *)key_cache + so * eb, eb);
#if ORACLE_MUTANT != 9
            memcpy((char *)value_cache + dO * eb, (const char *)value_cache + so * eb, eb);
#endif
        }
    }
    return ORACLE_OK;
}

/*
 * Whole-block moves between two different pools of the same block shape ("PagedAttention"
 * concept report §6 and §11: a request's blocks move to CPU memory under pressure and
 * back later): for each pair p, block src[p] of (src_k, src_v) is copied onto block
 * dst[p] of (dst_k, dst_v), bit for bit.  ORACLE_BAD_INDEX if an id is out of range.
 */
int oracle_swap_blocks(const void *src_k, const void *src_v, void *dst_k, void *dst_v,
                       const int32_t *src, const int32_t *dst, int num_pairs, int num_kv_heads,
                       int head_dim, int block_size, int src_blocks, int dst_blocks, int dtype)
{
    const int eb = elem_bytes(dtype);
    if (eb == 0 || num_pairs < 0) return ORACLE_BAD_ARG;
    const int64_t block_bytes = (int64_t)num_kv_heads * block_size * head_dim * eb;
    for (int p = 0; p < num_pairs; ++p) {
        if (src[p] < 0 || src[p] >= src_blocks || dst[p] < 0 || dst[p] >= dst_blocks)
            return ORACLE_BAD_INDEX;
        memcpy((char *)dst_k + dst[p] * block_bytes, (const char *)src_k + src[p] * block_bytes,
               (size_t)block_bytes);
        memcpy((char *)dst_v + dst[p] * block_bytes, (const char *)src_v + src[p] * block_bytes,
               (size_t)block_bytes);
    }
    return ORACLE_OK;
}
