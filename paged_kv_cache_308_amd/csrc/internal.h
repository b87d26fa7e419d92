// Internal declarations shared by the libpa sources (not part of the ABI).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

// Record a message for pa_last_error() and return `status`.
int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear the thread's last error.
void clear_error();

// Everything a decode launch needs (validated by the dispatcher).
struct DecodeArgs {
    void *out;
    const void *query;
    const void *key_cache;
    const void *value_cache;
    const float *k_scales;  // E4M3 pools: [num_blocks][H_kv] scales (else null)
    const float *v_scales;
    const int32_t *block_tables;
    const int32_t *context_lens;
    float *ws_max;   // [S][H_q][P] running max (log2 domain), partitioned runs only
    float *ws_sum;   // [S][H_q][P] sum of weights
    float *ws_acc;   // [S][H_q][P][d] weighted value sums
    int32_t *ws_hdr; // balanced split: list header and per-sequence chunk prefix
    int max_workers; // balanced split: partial slots reserved for this many waves
    int max_blocks_per_seq;
    int num_seqs;
    int num_q_heads;
    int num_kv_heads;
    int head_dim;
    int block_size;
    int num_blocks;
    int partition_size;  // 0 = one pass
    int max_partitions;  // grid extent along partitions (1 for one pass)
    float scale_log2;    // scale * log2(e)
    bool cached_kv;      // K/V through cacheable loads (blocks shared between sequences)
    int dtype;           // query / output type
    bool kv_fp8;         // pools hold E4M3 codes (k_scales / v_scales set)
    // newest tokens to store and attend to in the same launch (pa_decode_append): [S][H_kv][d]
    // of the query's type; key_out / value_out are the pools, written at position ctx - 1
    const void *new_key;
    const void *new_value;
    void *key_out;
    void *value_out;
    // several query tokens per sequence (pa_multi_query)
    const int32_t *query_start;  // [S + 1]: the sequence's rows of query / out
    int num_query_tokens;        // rows of query / out
    int max_query_len;           // bound on query_start[s + 1] - query_start[s]
    // shared-prefix groups (pa_decode_grouped)
    const int32_t *group_start;  // [num_groups + 1]: group j is sequences group_start[j] ..
    const int32_t *group_parts;  // [num_groups]: leading spans its members share
    int32_t *seq_group;          // workspace [S]: group serving sequence s (-1: none)
    int32_t *seq_parts;          // workspace [S]: leading spans served by its group
    const int32_t *skip_parts;   // for the one-pass vector kernel: spans already attended
    int num_groups;
    int max_group_parts;         // bound on group_parts[j] (grid extent)
    int group_rows;              // rows of the grouped score product: 2, 4, 8 or 16
    int group_span;              // tokens per shared span (0 outside pa_decode_grouped)
    void *stream;
};

// Workspace partition for `a` (pointers into `ws`); returns bytes needed.
size_t workspace_layout(int num_seqs, int num_q_heads, int head_dim, int max_partitions,
                        void *ws, float **m, float **l, float **acc);
// Balanced split: header ints then (waves + H_kv * S) partial slots of G heads.
size_t workspace_layout_balanced(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                 int max_workers, void *ws, int32_t **hdr, float **m, float **l,
                                 float **acc);
// pa_decode_grouped: one shared-prefix partial per (sequence, query head), then the plan's
// seq_group and seq_parts (pointers set in *a when ws is given); returns bytes needed.
struct DecodeArgs;
size_t grouped_workspace_layout(int num_seqs, int num_q_heads, int head_dim, void *ws, DecodeArgs *a);
// Most waves the current device can hold at once (0 if unknown).
int device_max_waves();
constexpr int kBalancedMaxSeqs = 4096;

// Kernel launchers (return PA_OK, PA_ERR_UNSUPPORTED or PA_ERR_HIP).
int launch_decode_valu(const DecodeArgs &a);
int launch_decode_mfma(const DecodeArgs &a);
// Log-sum-exp merge of partition partials into `out` (after a partitioned decode).
int launch_lse_merge(const DecodeArgs &a);
bool mfma_supported(int dtype, int head_dim, int block_size, int group);
int launch_reshape_and_cache(const void *key, const void *value, void *key_cache,
                             void *value_cache, const int32_t *slot_mapping, int num_tokens,
                             int num_kv_heads, int head_dim, int block_size, int num_blocks,
                             int elem_bytes, void *stream);
// E4M3 scatter; src_dtype is the pa_dtype of key / value (f32, f16 or bf16).
int launch_reshape_and_cache_fp8(const void *key, const void *value, void *key_cache,
                                 void *value_cache, const float *k_scales, const float *v_scales,
                                 const int32_t *slot_mapping, int num_tokens, int num_kv_heads,
                                 int head_dim, int block_size, int num_blocks, int src_dtype,
                                 void *stream);
int launch_stream_read(const void *buf, size_t bytes, void *sink, void *stream);
int launch_gather_read(const uint64_t *tile_addrs, int num_tiles, int tile_bytes, void *sink, void *stream);
int launch_decode_mfma_grouped(const DecodeArgs &a);
int launch_move_blocks(const void *src_key, const void *src_value, void *dst_key, void *dst_value,
                       const int32_t *src, const int32_t *dst, int num_pairs, int num_kv_heads,
                       int head_dim, int block_size, int src_blocks, int dst_blocks, int elem_bytes,
                       void *stream);

// Per-dtype launchers (one translation unit each).
int launch_decode_valu_f32(const DecodeArgs &a);
int launch_decode_valu_f16(const DecodeArgs &a);
int launch_decode_valu_bf16(const DecodeArgs &a);
int launch_lse_merge_f32(const DecodeArgs &a);
int launch_lse_merge_f16(const DecodeArgs &a);
int launch_lse_merge_bf16(const DecodeArgs &a);
int launch_decode_valu_fp8_f16(const DecodeArgs &a);
int launch_decode_valu_fp8_bf16(const DecodeArgs &a);
int launch_decode_mfma_f16(const DecodeArgs &a);
int launch_multi_query_f16(const DecodeArgs &a);
int launch_multi_query_bf16(const DecodeArgs &a);
int launch_decode_mfma_bf16(const DecodeArgs &a);
int launch_decode_mfma_grouped_f16(const DecodeArgs &a);
int launch_decode_mfma_grouped_bf16(const DecodeArgs &a);

// Map a HIP error after a launch to PA_ERR_HIP with its text.
int check_launch(const char *what);

}  // namespace pa
