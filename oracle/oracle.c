/*
 * Plain CPU oracle for paged decode attention and its two block operations.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this file: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or helper with the
 * HIP library; the two meet only through the seeded input generators.
 *
 * Everything is single-threaded, unblocked and unfused, and every floating
 * point step runs in IEEE binary64.  Stored f32 / f16 / bf16 / E4M3 values are
 * decoded to binary64 exactly (every such value is representable).  The one
 * binary32 step is the division that picks an E4M3 code (reshape into E4M3
 * pools), done in the precision the device decides it in.
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
 *  - compressed pools (kwkr.cn §1.5 quantising older blocks; compassingai.com §15
 *    lossy block compression): OCP E4M3 codes with one fp32 scale per (physical
 *    block, KV head) for K and one for V; encoding rounds to nearest, ties to the
 *    even code, and saturates at +-448.
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

enum { ORACLE_F32 = 0, ORACLE_F16 = 1, ORACLE_BF16 = 2, ORACLE_FP8 = 3 };
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

/*
 * OCP 8-bit floating point, E4M3 variant without infinities: 1 sign bit, 4 exponent
 * bits (bias 7), 3 fraction bits.  Exponent field 0 holds zero and the subnormals
 * frac * 2^-9; the fraction pattern 111 with exponent field 1111 is NaN (0x7F, 0xFF);
 * every other code is (1 + frac/8) * 2^(e-7), up to 448.
 */
double oracle_fp8_value(uint8_t c)
{
    const int sign = c >> 7;
    const int expo = (c >> 3) & 15;
    const int frac = c & 7;
    double v;
    if (expo == 15 && frac == 7)
        return NAN;
#if ORACLE_MUTANT == 11
    if (expo == 0)
        v = ldexp((double)frac, -10);                /* planted: bias 8 */
    else
        v = ldexp((double)(8 + frac), expo - 11);
#else
    if (expo == 0)
        v = ldexp((double)frac, -9);                 /* (frac / 8) * 2^(1-7) */
    else
        v = ldexp((double)(8 + frac), expo - 10);    /* (1 + frac/8) * 2^(e-7) */
#endif
    return sign ? -v : v;
}

/*
 * The E4M3 code nearest to y, found by trying every finite code; of two equally near
 * codes the one with an even code (fraction bit 0) wins.  Magnitudes of 448 and above
 * (infinity too) give the largest finite code of y's sign; NaN gives 0x7F; the sign of
 * a zero result is y's sign.
 */
uint8_t oracle_fp8_encode(float y)
{
    if (y != y)
        return 0x7F;
    const uint8_t sign = signbit(y) ? 0x80 : 0;
    const double a = fabs((double)y);
#if ORACLE_MUTANT == 14
    if (a >= 464.0)
        return 0x7F;                                  /* planted: no saturation */
#endif
    if (a >= 448.0)
        return sign | 0x7E;
    static double value[0x7F];  /* oracle_fp8_value of the finite non-negative codes */
    static int have_values = 0;
    if (!have_values) {
        for (int c = 0; c <= 0x7E; ++c)
            value[c] = oracle_fp8_value((uint8_t)c);
        have_values = 1;
    }
    int best = 0;
    double best_dist = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
        const double dist = fabs(value[c] - a);
#if ORACLE_MUTANT == 13
        if (dist <= best_dist) {                      /* planted: ties away from zero */
#else
        if (dist < best_dist || (dist == best_dist && (c & 1) == 0)) {
#endif
            best = c;
            best_dist = dist;
        }
    }
    return (uint8_t)(sign | best);
}

double oracle_load(const void *base, int64_t idx, int dtype)
{
    if (dtype == ORACLE_FP8)
        return oracle_fp8_value(((const uint8_t *)base)[idx]);
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
    return dtype == ORACLE_F32 ? 4 : (dtype == ORACLE_F16 || dtype == ORACLE_BF16) ? 2
                                     : dtype == ORACLE_FP8 ? 1 : 0;
}

/* Query and output types: the 16- and 32-bit floating point formats. */
static int is_wide(int dtype)
{
    return dtype == ORACLE_F32 || dtype == ORACLE_F16 || dtype == ORACLE_BF16;
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
 * Scale of the stored values of physical block pb, KV head k: 1 for pools in the
 * query's type; for E4M3 pools the per-(block, head) factor from `scales`
 * ([num_blocks][H_kv]).
 */
static double block_scale(const float *scales, int64_t pb, int k, int Hkv)
{
    return scales ? (double)scales[pb * Hkv + k] : 1.0;
}

/*
 * out[s][h][:]  (binary64, [S][H_q][d]) for every sequence s and query head h:
 *   n   = context_lens[s]
 *   x_t = scale * sum_j q[s][h][j] * K(t)[j]            for t < n
 *   p_t = exp(x_t - max_t x_t),   Z = sum_t p_t
 *   out = sum_t p_t * V(t) / Z
 * where K(t), V(t) are read at physical block block_tables[s][t / B], slot t % B,
 * KV head h / (H_q / H_kv), and multiplied by that block's scale (E4M3 pools).
 * Returns ORACLE_BAD_INDEX if a table entry needed for t < n is outside
 * [0, num_blocks) or t / B reaches max_blocks_per_seq.
 */
static int decode_impl(double *out, const void *query, const void *key_cache, const void *value_cache,
                       const float *k_scales, const float *v_scales, const int32_t *block_tables,
                       int max_blocks_per_seq, const int32_t *context_lens, int num_seqs,
                       int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                       int num_blocks, double scale, int qdtype, int kvdtype)
{
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        num_q_heads % num_kv_heads != 0 || !is_wide(qdtype) || elem_bytes(kvdtype) == 0)
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
#if ORACLE_MUTANT == 15
                const double ks = block_scale(k_scales, lb, k, Hkv);  /* planted: logical block */
#else
                const double ks = block_scale(k_scales, pb, k, Hkv);
#endif
                double dot = 0.0;
                for (int j = 0; j < d; ++j)
                    dot += oracle_load(query, q_row + j, qdtype) *
                           (oracle_load(key_cache, pool_index(pb, k, off, j, Hkv, B, d), kvdtype) * ks);
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
#if ORACLE_MUTANT == 12
                    const double vs = block_scale(k_scales, pb, k, Hkv);  /* planted: K's scale */
#else
                    const double vs = block_scale(v_scales, pb, k, Hkv);
#endif
                    acc += x[t] * (oracle_load(vsrc, pool_index(pb, k, t % B, j, Hkv, B, d), kvdtype) * vs);
                }
                o_row[j] = acc / Z;
            }
        }
        free(x);
    }
    return ORACLE_OK;
}

/* Decode over pools stored in the query's type (f32, f16 or bf16). */
int oracle_decode(double *out, const void *query, const void *key_cache, const void *value_cache,
                  const int32_t *block_tables, int max_blocks_per_seq, const int32_t *context_lens,
                  int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                  int num_blocks, double scale, int dtype)
{
    if (!is_wide(dtype))
        return ORACLE_BAD_ARG;
    return decode_impl(out, query, key_cache, value_cache, NULL, NULL, block_tables,
                       max_blocks_per_seq, context_lens, num_seqs, num_q_heads, num_kv_heads,
                       head_dim, block_size, num_blocks, scale, dtype, dtype);
}

/*
 * Decode over E4M3 pools: a stored code c of block pb, head k stands for
 * value(c) * k_scales[pb][k] (keys) or value(c) * v_scales[pb][k] (values); the query
 * is f16 or bf16 (qdtype).  Compressing cached blocks to fewer bits is the direction
 * of "vLLM PagedAttention 技术深度解析" (kwkr.cn) §1.5 and of the "PagedAttention"
 * concept report §15; the format and the per-block scale are this oracle's reading.
 */
int oracle_decode_fp8(double *out, const void *query, const void *key_cache, const void *value_cache,
                      const float *k_scales, const float *v_scales, const int32_t *block_tables,
                      int max_blocks_per_seq, const int32_t *context_lens, int num_seqs,
                      int num_q_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                      double scale, int qdtype)
{
    if (!k_scales || !v_scales)
        return ORACLE_BAD_ARG;
    return decode_impl(out, query, key_cache, value_cache, k_scales, v_scales, block_tables,
                       max_blocks_per_seq, context_lens, num_seqs, num_q_heads, num_kv_heads,
                       head_dim, block_size, num_blocks, scale, qdtype, ORACLE_FP8);
}

/*
 * Several query tokens per sequence over the paged cache (chunked prefill, a prefix-
 * cache hit: "PagedAttention 深度解析" (5ulink.com) §六 item 5; the same gather through
 * the block table as decode, "PagedAttention" concept report §5 and §8).  Sequence s
 * owns query rows query_start[s] .. query_start[s+1]-1 (n_s of them, n_s <= ctx); row
 * i of s is the token at position p = ctx - n_s + i, whose K/V are already cached, and
 * it attends causally to the tokens t <= p:
 *   out[row][h] = sum_{t <= p} softmax_t(scale * <q[row][h], K(t)>) * V(t).
 * query, out: [T][H_q][d], T = query_start[num_seqs].
 */
int oracle_multi_query(double *out, const void *query, const void *key_cache, const void *value_cache,
                       const int32_t *block_tables, int max_blocks_per_seq, const int32_t *context_lens,
                       const int32_t *query_start, int num_seqs, int num_q_heads, int num_kv_heads,
                       int head_dim, int block_size, int num_blocks, double scale, int dtype)
{
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        num_q_heads % num_kv_heads != 0 || !is_wide(dtype) || query_start[0] != 0)
        return ORACLE_BAD_ARG;
    const int g = num_q_heads / num_kv_heads;
    const int d = head_dim, B = block_size, Hkv = num_kv_heads;
    for (int s = 0; s < num_seqs; ++s) {
        const int n = context_lens[s];
        const int nq = query_start[s + 1] - query_start[s];
        if (n < 0 || nq < 0 || nq > n) return ORACLE_BAD_ARG;
        for (int lb = 0; lb * B < n; ++lb) {
            if (lb >= max_blocks_per_seq) return ORACLE_BAD_INDEX;
            const int64_t pb = block_tables[(int64_t)s * max_blocks_per_seq + lb];
            if (pb < 0 || pb >= num_blocks) return ORACLE_BAD_INDEX;
        }
        double *x = (double *)malloc(sizeof(double) * (n > 0 ? n : 1));
        if (!x) return ORACLE_NO_MEM;
        for (int i = 0; i < nq; ++i) {
            const int64_t row = query_start[s] + i;
#if ORACLE_MUTANT == 17
            const int p = n - nq + i + 1;        /* planted: positions shifted by one */
#else
            const int p = n - nq + i;
#endif
#if ORACLE_MUTANT == 16
            const int last = p - 1;              /* planted: a token does not see itself */
#else
            const int last = p;
#endif
            for (int h = 0; h < num_q_heads; ++h) {
                const int k = h / g;
                const int64_t q_row = (row * num_q_heads + h) * d;
                double *o_row = out + (row * num_q_heads + h) * d;
                double m = -INFINITY;
                for (int t = 0; t <= last && t < n; ++t) {
                    const int64_t pb = block_tables[(int64_t)s * max_blocks_per_seq + t / B];
                    double dot = 0.0;
                    for (int j = 0; j < d; ++j)
                        dot += oracle_load(query, q_row + j, dtype) *
                               oracle_load(key_cache, pool_index(pb, k, t % B, j, Hkv, B, d), dtype);
                    x[t] = scale * dot;
                    if (x[t] > m) m = x[t];
                }
                double Z = 0.0;
                for (int t = 0; t <= last && t < n; ++t) {
                    x[t] = exp(x[t] - m);
                    Z += x[t];
                }
                for (int j = 0; j < d; ++j) {
                    double acc = 0.0;
                    for (int t = 0; t <= last && t < n; ++t) {
                        const int64_t pb = block_tables[(int64_t)s * max_blocks_per_seq + t / B];
                        acc += x[t] * oracle_load(value_cache, pool_index(pb, k, t % B, j, Hkv, B, d), dtype);
                    }
                    o_row[j] = Z > 0.0 ? acc / Z : 0.0;
                }
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
 * The slot scatter into E4M3 pools: element x (key/value in src_dtype) of token i, KV
 * head k goes to block b = slot / B as oracle_fp8_encode(x / scale), scale taken from
 * k_scales[b][k] (keys) or v_scales[b][k] (values); the division is one binary32
 * division, so that the code is decided in the precision the device uses.
 */
int oracle_reshape_and_cache_fp8(const void *key, const void *value, uint8_t *key_cache,
                                 uint8_t *value_cache, const float *k_scales, const float *v_scales,
                                 const int32_t *slot_mapping, int num_tokens, int num_kv_heads,
                                 int head_dim, int block_size, int num_blocks, int src_dtype)
{
    if (!is_wide(src_dtype) || num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0 || !k_scales || !v_scales)
        return ORACLE_BAD_ARG;
    for (int i = 0; i < num_tokens; ++i) {
        const int64_t slot = slot_mapping[i];
        if (slot < 0) continue;
        const int64_t b = slot / block_size, off = slot % block_size;
        if (b >= num_blocks) return ORACLE_BAD_INDEX;
        for (int k = 0; k < num_kv_heads; ++k) {
            const float ks = k_scales[b * num_kv_heads + k];
            const float vs = v_scales[b * num_kv_heads + k];
            for (int j = 0; j < head_dim; ++j) {
                const int64_t src = ((int64_t)i * num_kv_heads + k) * head_dim + j;
                const int64_t dst = pool_index(b, k, (int)off, j, num_kv_heads, block_size, head_dim);
                const float xk = (float)oracle_load(key, src, src_dtype);
                const float xv = (float)oracle_load(value, src, src_dtype);
                const float yk = xk / ks;
                const float yv = xv / vs;
                key_cache[dst] = oracle_fp8_encode(yk);
                value_cache[dst] = oracle_fp8_encode(yv);
            }
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
