/*
 * pa.h — C ABI of libpa: paged decode attention on AMD Instinct MI355X (gfx950).
 *
 * The operations follow four web pages on vLLM's PagedAttention:
 *   [kwkr]   "vLLM PagedAttention 技术深度解析" (kwkr.cn/news/58438)
 *   [wmrh]   KV cache / memory paging / paged attention tutorial (wmrh.cn/news/286280)
 *   [5ulink] "PagedAttention 深度解析：vLLM 连续批处理与显存分页的工程奇迹" (5ulink.com)
 *   [cpai]   "PagedAttention" concept report (compassingai.com/zh-hant/concept/pagedattention)
 *
 * Data layout (one attention layer):
 *   key_cache, value_cache  [num_blocks][num_kv_heads][block_size][head_dim] of `dtype`:
 *                           the physical block pool; one (block, head) tile is
 *                           block_size * head_dim contiguous elements ([cpai] §5).
 *   block_tables            int32 [num_seqs][max_blocks_per_seq]: entry j of row s is the
 *                           physical block that holds tokens [j*B, (j+1)*B) of sequence s
 *                           ([cpai] §5, [5ulink] §二); entries past ceil(ctx/B) are never
 *                           read (pad them with -1).
 *   context_lens            int32 [num_seqs]: tokens of sequence s, including the one being
 *                           decoded, whose K/V must already be in the cache ([wmrh] "KV cache").
 *   slot_mapping            int32 [num_tokens]: slot = physical_block * block_size + offset;
 *                           a negative slot marks a padding token and is skipped.
 *   query, out              [num_seqs][num_q_heads][head_dim] of `dtype`; query head h reads
 *                           KV head h / (num_q_heads / num_kv_heads).
 *
 * Supported: dtype f32 / f16 / bf16; head_dim 64 or 128; block_size 16, 32, 64 or 128;
 * num_q_heads / num_kv_heads in {1, 2, 4, 8, 16}.  Compressed pools (pa_decode_fp8,
 * pa_reshape_and_cache_fp8) hold one-byte E4M3 codes with an fp32 scale per
 * (physical block, KV head); their query and output are f16 or bf16.
 *
 * Ownership and ordering: every device pointer is borrowed from the caller and must
 * stay valid until the work queued on `stream` (a hipStream_t; NULL = the null stream)
 * has finished.  Device calls only validate host-visible arguments, enqueue kernels and
 * return; they never allocate, free or synchronise.  Work on one stream runs in order,
 * which is what makes it safe to reuse a freed block at once ([kwkr] §1.3.2).
 *
 * Errors: every call returns a pa_status.  Argument errors are reported before anything
 * is enqueued.  Faults in device data cannot be reported synchronously; instead the
 * kernels never touch memory outside the pools, and a sequence whose table holds an
 * entry outside [0, num_blocks) for a token < ctx, or whose ctx is negative (or, with
 * partitions, larger than max_context_len), gets NaN in every element of its output
 * ([cpai] §13: bounds are checked in the kernel as well as by the scheduler).
 * pa_check_tables validates host copies of the tables beforehand.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
    PA_OK = 0,
    PA_ERR_INVALID = 1,     /* bad argument, unknown sequence, double free */
    PA_ERR_BOUNDS = 2,      /* index outside the pool or the table */
    PA_ERR_OOM = 3,         /* no free block left ([cpai] §13); state unchanged */
    PA_ERR_UNSUPPORTED = 4, /* dtype / head_dim / block_size / group not built */
    PA_ERR_HIP = 5          /* the HIP runtime reported an error (see pa_last_error) */
} pa_status;

/* PA_FP8_E4M3: one-byte OCP E4M3 codes (no infinities; 0x7F / 0xFF are NaN; largest
 * finite 448).  Pool storage only: accepted by pa_copy_blocks and pa_swap_blocks, and
 * the pool type of pa_decode_fp8 / pa_reshape_and_cache_fp8. */
typedef enum pa_dtype { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2, PA_FP8_E4M3 = 3 } pa_dtype;

/* Decode-attention variants (pa_decode's `variant` argument): a kernel choice in the
 * low 4 bits, optionally OR-ed with PA_DECODE_SHARED_KV. */
typedef enum pa_variant {
    PA_VARIANT_AUTO = 0, /* MFMA when the group size is >= 2 and dtype is 16-bit, else VALU */
    PA_VARIANT_VALU = 1, /* vector-ALU kernel: one wavefront row per token */
    PA_VARIANT_MFMA = 2, /* matrix-core kernel for grouped-query heads (16-bit only) */
    /* Hint: the batch's tables share physical blocks (forked sequences, shared prefixes,
     * [cpai] §6).  K/V are then read with cacheable loads so sequences that read the same
     * block can hit in L2; without it they are read non-temporally, which is faster when
     * every block is read once per step.  Results are identical either way. */
    PA_DECODE_SHARED_KV = 16
} pa_variant;

/* Static text for a status code. */
const char *pa_status_str(int status);
/* Detail of the last failed call on this thread ("" if none). */
const char *pa_last_error(void);
/* ABI version (incremented on any incompatible change). */
int pa_abi_version(void);

/* ------------------------------------------------------------------ device ops */

/* pa_decode's partition_size for the balanced split (see pa_decode). */
#define PA_PARTITION_BALANCED (-1)

/*
 * Bytes of scratch pa_decode needs for a given partition size (0 when
 * partition_size == 0).  Partials are kept in fp32: a running max, a sum of weights
 * and head_dim weighted sums per query head, for every (sequence, partition) or, with
 * PA_PARTITION_BALANCED, for every wave the current device can hold plus every
 * (sequence, KV head); the balanced size therefore depends on the current device.
 */
size_t pa_decode_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                 int max_context_len, int partition_size);

/*
 * Decode attention over the paged cache ([cpai] §8: scores of the query against every
 * cached key, softmax, weighted sum of the values; the kernel walks the block table):
 *   out[s][h] = sum_t softmax_t(scale * <query[s][h], K_t>) * V_t,  t < context_lens[s]
 * with K_t, V_t read at block block_tables[s][t / B], slot t % B, KV head h / g.
 * Softmax and accumulation run in fp32; out is rounded to `dtype` (round to nearest
 * even).  context_lens[s] == 0 gives zeros.
 *
 * partition_size == 0: one pass per (sequence, KV head).  A multiple of block_size
 * (and of 16): each partition of that many tokens is reduced on its own and a second
 * kernel merges the partials with log-sum-exp weights; max_context_len must bound
 * every context_lens[s].  PA_PARTITION_BALANCED (at most 4096 sequences; either
 * kernel): the batch's work, as one list of fixed-size chunks over KV heads and
 * sequences, is cut into equal ranges for all the waves the device holds at once,
 * whatever the length mix; each wave writes a partial per (sequence, KV head) it
 * touches and a second kernel merges them.  With partitions `workspace` must hold
 * pa_decode_workspace_bytes(...) bytes of device memory (contents need not be set).
 * `variant` selects the kernel (pa_variant).
 */
int pa_decode(void *out, const void *query, const void *key_cache, const void *value_cache,
              const int32_t *block_tables, int max_blocks_per_seq, const int32_t *context_lens,
              int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
              int num_blocks, int max_context_len, float scale, int dtype, int partition_size,
              int variant, void *workspace, size_t workspace_bytes, void *stream);

/*
 * The decode step in one call: each sequence's newest token, new_key[s] / new_value[s]
 * ([num_seqs][num_kv_heads][head_dim] of `dtype`, device), is stored at position
 * context_lens[s] - 1 of its table (block table[(ctx-1) / B], slot (ctx-1) % B) and
 * the attention of pa_decode is computed over all ctx tokens.  The result and the
 * pools afterwards equal pa_reshape_and_cache with those slots followed by pa_decode
 * (up to the order of the fp32 sums).  One launch (plus the merge when partitioned or
 * balanced) on either kernel; the vector kernel's balanced split (PA_PARTITION_BALANCED
 * with the vector kernel chosen) returns PA_ERR_UNSUPPORTED.  Sequences with ctx <= 0
 * store nothing.  The block holding
 * position ctx - 1 must not appear in another sequence's table (it is exclusive once the
 * step's copy-on-write copies have run, [cpai] §6).  Other arguments and errors as
 * pa_decode.
 */
int pa_decode_append(void *out, const void *query, const void *new_key, const void *new_value,
                     void *key_cache, void *value_cache, const int32_t *block_tables,
                     int max_blocks_per_seq, const int32_t *context_lens, int num_seqs, int num_q_heads,
                     int num_kv_heads, int head_dim, int block_size, int num_blocks, int max_context_len,
                     float scale, int dtype, int partition_size, int variant, void *workspace,
                     size_t workspace_bytes, void *stream);

/*
 * Write the newest tokens' K/V into their slots ([wmrh] "KV cache": at a decode step
 * only the newest token's K and V are computed and cached; [cpai] §5 base + offset):
 *   key_cache[slot / B][k][slot % B][:] = key[i][k][:]   (same for value)
 * for every token i with 0 <= slot_mapping[i] < num_blocks * B; a bitwise copy.
 * key, value: device [num_tokens][num_kv_heads][head_dim]; slot_mapping device.
 */
int pa_reshape_and_cache(const void *key, const void *value, void *key_cache, void *value_cache,
                         const int32_t *slot_mapping, int num_tokens, int num_kv_heads,
                         int head_dim, int block_size, int num_blocks, int dtype, void *stream);

/*
 * Copy-on-write block copies ([cpai] §6: before a write into a shared block, a new
 * block gets a copy of its content): for every pair p, the whole block src[p] (all KV
 * heads, all slots) of both pools is copied onto block dst[p], bit for bit.
 * src, dst: device int32 [num_pairs].  A pair with an id outside [0, num_blocks) is
 * skipped.  The dst ids must be distinct and must not appear among the src ids (the
 * allocator's pairs always are); pa_check_copy_pairs checks host copies.  A block's
 * bytes (num_kv_heads * block_size * head_dim * element size) must be a multiple of 4:
 * the per-(block, KV head) scales of E4M3 pools are moved with the same call, as pools
 * of PA_F32 with head_dim = block_size = 1.
 */
int pa_copy_blocks(void *key_cache, void *value_cache, const int32_t *src, const int32_t *dst,
                   int num_pairs, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                   int dtype, void *stream);

/*
 * Move whole blocks between two different pools of the same shape (per block: all KV
 * heads, all slots, bit for bit): dst_*[dst[p]] = src_*[src[p]] for both K and V.
 * Either pool may be device memory or pinned host memory mapped into the device's
 * address space (hipHostMalloc / a pinned tensor): this is the swap-out and swap-in
 * data mover for preemption ([cpai] §6 and §11: a request's blocks move to CPU memory
 * under memory pressure and come back when it is rescheduled).  src, dst: int32
 * [num_pairs] readable by the device.  A pair with an id outside its pool is skipped.
 */
int pa_swap_blocks(const void *src_key_cache, const void *src_value_cache, void *dst_key_cache,
                   void *dst_value_cache, const int32_t *src, const int32_t *dst, int num_pairs,
                   int num_kv_heads, int head_dim, int block_size, int src_num_blocks,
                   int dst_num_blocks, int dtype, void *stream);

/*
 * Several query tokens per sequence (chunked prefill, a prefix-cache hit: [5ulink] §六
 * item 5), over the same paged cache and tables as pa_decode ([cpai] §5, §8).  Sequence
 * s owns rows query_start[s] .. query_start[s+1]-1 of query and out ([T][num_q_heads]
 * [head_dim] of `dtype`, T = num_query_tokens); with n_s such rows, row i is the token
 * at position ctx_s - n_s + i, whose K/V must already be in the cache (written with
 * pa_reshape_and_cache), and it attends causally:
 *   out[row][h] = sum_{t <= ctx_s - n_s + i} softmax_t(scale * <query[row][h], K_t>) * V_t.
 * query_start: device int32 [num_seqs + 1], nondecreasing from 0.  max_query_len must
 * bound every n_s.  dtype f16 or bf16 (matrix cores); head_dim 64 or 128; group sizes
 * 1 to 16.  A sequence with n_s > ctx_s, n_s > max_query_len, ctx_s < 0 or a needed
 * table entry outside [0, num_blocks) gets NaN in its rows (rows past max_query_len are
 * not written); rows outside [0, T) are never read or written.
 */
int pa_multi_query(void *out, const void *query, const void *key_cache, const void *value_cache,
                   const int32_t *block_tables, int max_blocks_per_seq, const int32_t *context_lens,
                   const int32_t *query_start, int num_seqs, int num_query_tokens, int max_query_len,
                   int num_q_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                   float scale, int dtype, void *stream);

/* ------------------------------------------------------- compressed (E4M3) pools */

/*
 * Compressed KV blocks ([kwkr] §1.5: quantising older blocks, dynamic precision;
 * [cpai] §15: lossy compression of physical blocks to raise the effective capacity).
 * The pools hold PA_FP8_E4M3 codes in the usual [num_blocks][num_kv_heads][B][d]
 * layout, and k_scales / v_scales (device fp32 [num_blocks][num_kv_heads]) give each
 * (physical block, KV head) tile its own scale: a key code c of block b, head k stands
 * for value(c) * k_scales[b][k] (values likewise with v_scales).  The caller owns the
 * scales: it sets a block's scales before the block's first write and moves them with
 * the block (pa_copy_blocks / pa_swap_blocks on the scale arrays, see there).
 */

/*
 * E4M3 counterpart of pa_reshape_and_cache: element x of key[i][k][:] (dtype f32, f16
 * or bf16) is stored in block b = slot / B as the E4M3 code nearest to
 * y = x / k_scales[b][k] (one correctly rounded fp32 division): round to nearest, ties
 * to the even code, |y| >= 448 (infinities too) saturating to +-448, NaN to 0x7F.
 * Values likewise with v_scales.  Slots outside [0, num_blocks * B) are skipped.
 */
int pa_reshape_and_cache_fp8(const void *key, const void *value, void *key_cache, void *value_cache,
                             const float *k_scales, const float *v_scales,
                             const int32_t *slot_mapping, int num_tokens, int num_kv_heads,
                             int head_dim, int block_size, int num_blocks, int dtype, void *stream);

/*
 * pa_decode over E4M3 pools: the same attention with K_t = value(code) * k_scale and
 * V_t = value(code) * v_scale of the block and KV head holding token t.  query and out
 * are `dtype` (PA_F16 or PA_BF16); codes are widened exactly, products and softmax run
 * in fp32.  Every other argument, partitioning, the workspace and the error behaviour
 * are those of pa_decode; the vector kernel serves every variant (PA_VARIANT_MFMA
 * returns PA_ERR_UNSUPPORTED), and group sizes go up to 8.
 */
int pa_decode_fp8(void *out, const void *query, const void *key_cache, const void *value_cache,
                  const float *k_scales, const float *v_scales, const int32_t *block_tables,
                  int max_blocks_per_seq, const int32_t *context_lens, int num_seqs,
                  int num_q_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                  int max_context_len, float scale, int dtype, int partition_size, int variant,
                  void *workspace, size_t workspace_bytes, void *stream);

/* pa_decode_append over E4M3 pools: new_key / new_value are `dtype` (f16 or bf16) and are
 * stored as the codes pa_reshape_and_cache_fp8 would write (same rounding, bit for bit). */
int pa_decode_fp8_append(void *out, const void *query, const void *new_key, const void *new_value,
                         void *key_cache, void *value_cache, const float *k_scales, const float *v_scales,
                         const int32_t *block_tables, int max_blocks_per_seq, const int32_t *context_lens,
                         int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                         int num_blocks, int max_context_len, float scale, int dtype, int partition_size,
                         int variant, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Decode attention for batches whose sequences share leading blocks ([cpai] §6 and
 * [wmrh] "paged attention": forked samples of one prompt hold the prompt's physical
 * blocks with a reference count, so their tables start with the same block ids).  The
 * result is that of pa_decode_append (new_key, new_value given: each sequence's newest
 * K/V stored at position ctx - 1, then attended) or of pa_decode (both NULL), up to
 * rounding order; the shared blocks are read once per group instead of once per
 * sequence.
 *
 * Groups are runs of consecutive sequences: group j holds sequences group_start[j] ..
 * group_start[j + 1] - 1 (device int32 [num_groups + 1], ascending, group_start[0] = 0,
 * group_start[num_groups] = num_seqs), at most max_group_size (1..16) of them, whose first
 * group_parts[j] spans of partition_size tokens (device int32 [num_groups]) are reached
 * through the same table entries.  Those spans run once per (group, KV head) on the
 * matrix cores, every member's query a row of the product, leaving a partial (max, sum,
 * weighted value sums) per member and head in the workspace; the rest of each context
 * runs in one pass on the vector kernel, which also stores the newest token and folds
 * the partial in.
 *
 * A sequence is served by its group only when the group is well formed (at most
 * max_group_size members, 1 <= group_parts[j] <= max_group_parts), its shared
 * spans end before its newest token (group_parts[j] * partition_size <= ctx - 1)
 * and its table entries for them equal the group's first sequence's and lie in the pool
 * (a device-side plan kernel checks this); any other sequence is attended in full by the
 * vector kernel, so a wrong group description costs speed, not results.
 *
 * Supported: one query head per KV head (num_q_heads == num_kv_heads), f16 or bf16,
 * head_dim 64 or 128, block_size 16..128 dividing partition_size (> 0), max_group_parts
 * * partition_size <= max_context_len (0: no shared-prefix pass).  variant: PA_VARIANT_AUTO
 * or PA_VARIANT_VALU, optionally | PA_DECODE_SHARED_KV.  workspace: at least
 * pa_decode_grouped_workspace_bytes(...) bytes.  Other errors as pa_decode.
 */
size_t pa_decode_grouped_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                         int max_context_len, int partition_size);
int pa_decode_grouped(void *out, const void *query, const void *new_key, const void *new_value,
                      void *key_cache, void *value_cache, const int32_t *block_tables, int max_blocks_per_seq,
                      const int32_t *context_lens, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                      int block_size, int num_blocks, int max_context_len, float scale, int dtype,
                      int partition_size, const int32_t *group_start, const int32_t *group_parts,
                      int num_groups, int max_group_size, int max_group_parts, int variant, void *workspace,
                      size_t workspace_bytes, void *stream);

/*
 * For callers that cannot allocate device memory (code under graph capture, serving
 * loops that must not allocate, harnesses that forbid allocation): pa_decode with its
 * partials (partitions or the balanced split) kept in a fixed device array of the
 * library instead of a caller workspace.  The call allocates and frees nothing.
 *
 * Every GPU the library runs on holds its own copy of that array, PA_NOALLOC_SCRATCH_BYTES
 * bytes, from the first use of the library on it until the process ends.  A call whose
 * partials need more (pa_decode_workspace_bytes(...) > PA_NOALLOC_SCRATCH_BYTES) returns
 * PA_ERR_INVALID before anything is enqueued.  All calls on one GPU share its array and
 * its contents are whatever the last call left (the kernels write every partial before
 * reading it, so nothing needs clearing): calls that can overlap on one GPU (several
 * streams, several host threads) race on it and must be serialised by the caller.
 * partition_size == 0 uses no scratch.  Arguments, results and errors otherwise as
 * pa_decode.
 */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int pa_decode_noalloc(void *out, const void *query, const void *key_cache, const void *value_cache,
                      const int32_t *block_tables, int max_blocks_per_seq, const int32_t *context_lens,
                      int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                      int num_blocks, int max_context_len, float scale, int dtype, int partition_size,
                      int variant, void *stream);

/*
 * Measurement helper, not part of the attention path: reads `bytes` bytes of device
 * memory at buf once (16-byte non-temporal loads spread over the whole device) and
 * folds them into a value that is stored to *sink (device, 4 bytes) only when it
 * equals a fixed constant, so the reads cannot be elided.  The achievable read
 * bandwidth that the decode kernels' HBM roofline is compared against.  buf 16-byte
 * aligned, bytes a positive multiple of 16; PA_ERR_INVALID otherwise.
 */
int pa_stream_read(const void *buf, size_t bytes, void *sink, void *stream);

/*
 * Measurement helper, not part of the attention path: the achievable read rate for
 * the decode kernels' own access pattern.  Reads num_tiles tiles of tile_bytes bytes
 * once, tile i at device address tile_addrs[i] (a device array of num_tiles addresses,
 * each 16-byte aligned), with 16-byte non-temporal loads, one wave per tile and two
 * tiles in flight per wave, spread over the whole device; the folded value is stored to
 * *sink (device, 4 bytes) only when it equals a fixed constant.  A decode step's tiles
 * are the (physical block, KV head) tiles of both pools its tables reach
 * ("PagedAttention" concept report (compassingai.com) §5: a block's tokens sit at
 * consecutive offsets).  tile_bytes is 1024, 2048, 4096 or 8192 (a larger tile is
 * passed as consecutive pieces); num_tiles >= 0 (0: nothing is launched).  The
 * addresses are the caller's: each must point at tile_bytes readable device bytes,
 * which the library cannot check.  PA_ERR_INVALID for the checkable errors.
 */
int pa_gather_read(const uint64_t *tile_addrs, int num_tiles, int tile_bytes, void *sink, void *stream);

/* Host-side checks ([cpai] §13).  PA_ERR_BOUNDS names the first offending entry in
 * pa_last_error. */
int pa_check_tables(const int32_t *block_tables, const int32_t *context_lens, int num_seqs,
                    int max_blocks_per_seq, int block_size, int num_blocks);
int pa_check_copy_pairs(const int32_t *src, const int32_t *dst, int num_pairs, int num_blocks);

/* ------------------------------------------------------------ host allocator */

/*
 * Block allocator ([kwkr] §1.2.2 allocation flow, §1.3.2 sharing; [cpai] §6 reference
 * counts and copy-on-write, §11 free list, §13 out-of-memory).  An opaque handle owned
 * by the library; all calls on one handle are serialised by an internal mutex.
 * Free blocks form a LIFO stack whose pops return 0, 1, 2, ... unless set otherwise;
 * blocks released by pa_alloc_free_seq are pushed in table order.
 */
typedef struct pa_allocator pa_allocator;

/* Pool figures for monitoring.  The rates are those "vLLM PagedAttention 技术深度解析"
 * (kwkr.cn) §1.4.1 names, with the paged pool's quantities: blocks in use over all
 * blocks; shared blocks over all blocks; memory that is free but unusable over all
 * memory, where in a paged pool any free block serves any request, so the unusable part
 * is the allocated slots no token fills (the tails of last blocks); and the effective
 * memory utilisation of the "PagedAttention" concept report (compassingai.com) §7:
 * KV that requests need over KV allocated to them, here stored tokens over the slots of
 * the blocks in use (a shared block counted once; 0 with no block in use). */
typedef struct pa_alloc_stats {
    int64_t total_blocks;
    int64_t used_blocks;    /* reference count > 0 */
    int64_t free_blocks;
    int64_t shared_blocks;  /* reference count > 1 */
    int64_t num_seqs;
    int64_t logical_tokens; /* sum of context lengths */
    int64_t stored_tokens;  /* filled slots, counting a shared block once */
    int64_t wasted_slots;   /* used_blocks * B - stored_tokens */
    double block_utilisation;  /* used_blocks / total_blocks */
    double sharing_rate;       /* shared_blocks / total_blocks */
    double fragmentation_rate; /* wasted_slots / (total_blocks * B) */
    double emu;                /* stored_tokens / (used_blocks * B) */
} pa_alloc_stats;

int pa_alloc_create(int num_blocks, int block_size, pa_allocator **out);
void pa_alloc_destroy(pa_allocator *a);
/* Pops return ids[0], ids[1], ...: ids must be a permutation of [0, num_blocks) and
 * no block may be in use. */
int pa_alloc_set_free_order(pa_allocator *a, const int32_t *ids, int n);
int pa_alloc_new_seq(pa_allocator *a, int64_t *seq);
/*
 * Reserve the slot of seq's next token.  A full (or missing) last block takes a free
 * block.  A partly filled last block that is shared (count > 1) is replaced by a
 * fresh block and (*cow_src, *cow_dst) name the copy to run with pa_copy_blocks
 * before the write; otherwise both are -1.  With no free block: PA_ERR_OOM and no
 * change.
 */
int pa_alloc_append_slot(pa_allocator *a, int64_t seq, int32_t *slot, int32_t *cow_src,
                         int32_t *cow_dst);
/*
 * n appends in order (seqs[i] may repeat).  slots[i] receives each slot; the copies
 * raised are written to cow_src/cow_dst (capacity n) and counted in *num_cow.  All or
 * nothing ([cpai] §13: running work stays untouched by an out-of-memory error): when an
 * append fails (PA_ERR_OOM, or PA_ERR_INVALID for an unknown sequence) the appends
 * before it are taken back, the allocator is left exactly as before the call (free
 * stack order included), *num_cow and *num_done are 0 and pa_last_error names the
 * failing append.  On success *num_done (may be NULL) = n.
 */
int pa_alloc_append_slots(pa_allocator *a, const int64_t *seqs, int n, int32_t *slots,
                          int32_t *cow_src, int32_t *cow_dst, int *num_cow, int *num_done);
/* New sequence of num_tokens tokens on ceil(num_tokens / B) fresh blocks (count 1),
 * whose ids are written to block_ids in table order (capacity cap): the receiving end
 * of a swap.  With too few free blocks: PA_ERR_OOM and no change. */
int pa_alloc_adopt(pa_allocator *a, int num_tokens, int64_t *seq, int32_t *block_ids, int cap);
/* New sequence sharing all of parent's blocks (each count + 1), same length. */
int pa_alloc_fork(pa_allocator *a, int64_t parent, int64_t *child);
/* Release the sequence; blocks whose count drops to 0 return to the free stack. */
int pa_alloc_free_seq(pa_allocator *a, int64_t seq);
/* One table: up to cap entries to out; *num_blocks and *context_len may be NULL. */
int pa_alloc_block_table(pa_allocator *a, int64_t seq, int32_t *out, int cap, int *num_blocks,
                         int *context_len);
/* Padded tables of n sequences: out [n][max_blocks_per_seq] (-1 padding) and
 * context_lens [n]; PA_ERR_BOUNDS if a table is longer than max_blocks_per_seq. */
int pa_alloc_block_tables(pa_allocator *a, const int64_t *seqs, int n, int32_t *out,
                          int max_blocks_per_seq, int32_t *context_lens);
int pa_alloc_refcount(pa_allocator *a, int32_t block, int *refcount);
int pa_alloc_get_stats(pa_allocator *a, pa_alloc_stats *out);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
