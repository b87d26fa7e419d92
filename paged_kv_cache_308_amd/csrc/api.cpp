// C ABI entry points of libpa: argument validation, variant choice, launches.
// Nothing here allocates device memory or synchronises; see pa.h for the contract.
#include <hip/hip_runtime.h>

#include <cstring>

#include "internal.h"

namespace pa {

int check_launch(const char *what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return PA_OK;
}

// Element bytes of the query / output types (0 for anything else).
static int elem_bytes(int dtype) {
    return dtype == PA_F32 ? 4 : (dtype == PA_F16 || dtype == PA_BF16) ? 2 : 0;
}

// Element bytes of every pool type (block moves are bitwise).
static int pool_elem_bytes(int dtype) { return dtype == PA_FP8_E4M3 ? 1 : elem_bytes(dtype); }

static bool pow2_in(int x, int lo, int hi) { return x >= lo && x <= hi && (x & (x - 1)) == 0; }

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int launch_decode_valu(const DecodeArgs &a) {
    if (a.kv_fp8) {
        if (a.dtype == PA_F16) return launch_decode_valu_fp8_f16(a);
        if (a.dtype == PA_BF16) return launch_decode_valu_fp8_bf16(a);
        return fail(PA_ERR_UNSUPPORTED, "E4M3 pools with query dtype %d", a.dtype);
    }
    switch (a.dtype) {
        case PA_F32: return launch_decode_valu_f32(a);
        case PA_F16: return launch_decode_valu_f16(a);
        case PA_BF16: return launch_decode_valu_bf16(a);
    }
    return fail(PA_ERR_UNSUPPORTED, "dtype %d", a.dtype);
}

int launch_lse_merge(const DecodeArgs &a) {
    switch (a.dtype) {
        case PA_F32: return launch_lse_merge_f32(a);
        case PA_F16: return launch_lse_merge_f16(a);
        case PA_BF16: return launch_lse_merge_bf16(a);
    }
    return fail(PA_ERR_UNSUPPORTED, "dtype %d", a.dtype);
}

bool mfma_supported(int dtype, int head_dim, int block_size, int group) {
    return (dtype == PA_F16 || dtype == PA_BF16) && (head_dim == 64 || head_dim == 128) &&
           block_size >= 16 && (group == 2 || group == 4 || group == 8 || group == 16);
}

int launch_decode_mfma(const DecodeArgs &a) {
    if (a.dtype == PA_F16) return launch_decode_mfma_f16(a);
    if (a.dtype == PA_BF16) return launch_decode_mfma_bf16(a);
    return fail(PA_ERR_UNSUPPORTED, "MFMA dtype %d", a.dtype);
}

int launch_decode_mfma_grouped(const DecodeArgs &a) {
    if (a.dtype == PA_F16) return launch_decode_mfma_grouped_f16(a);
    if (a.dtype == PA_BF16) return launch_decode_mfma_grouped_bf16(a);
    return fail(PA_ERR_UNSUPPORTED, "MFMA dtype %d", a.dtype);
}

size_t workspace_layout(int S, int Hq, int d, int P, void *ws, float **m, float **l, float **acc) {
    const size_t n = (size_t)S * Hq * P;
    const size_t bm = align256(n * sizeof(float));
    const size_t bacc = align256(n * (size_t)d * sizeof(float));
    if (ws) {
        char *p = (char *)ws;
        *m = (float *)p;
        *l = (float *)(p + bm);
        *acc = (float *)(p + 2 * bm);
    }
    return 2 * bm + bacc;
}

size_t workspace_layout_balanced(int S, int Hq, int Hkv, int d, int W, void *ws, int32_t **hdr,
                                 float **m, float **l, float **acc) {
    const size_t bh = align256((size_t)(4 + S + 1) * sizeof(int32_t));
    const size_t n = ((size_t)W + (size_t)Hkv * S) * (size_t)(Hq / Hkv);
    const size_t bm = align256(n * sizeof(float));
    const size_t bacc = align256(n * (size_t)d * sizeof(float));
    if (ws) {
        char *p = (char *)ws;
        *hdr = (int32_t *)p;
        *m = (float *)(p + bh);
        *l = (float *)(p + bh + bm);
        *acc = (float *)(p + bh + 2 * bm);
    }
    return bh + 2 * bm + bacc;
}

// pa_decode_grouped: the shared-prefix partials (one partition) then seq_group, seq_parts.
size_t grouped_workspace_layout(int S, int Hq, int d, void *ws, DecodeArgs *a) {
    const size_t base = workspace_layout(S, Hq, d, 1, nullptr, nullptr, nullptr, nullptr);
    const size_t plan = align256((size_t)S * sizeof(int32_t));
    if (ws) {
        workspace_layout(S, Hq, d, 1, ws, &a->ws_max, &a->ws_sum, &a->ws_acc);
        a->seq_group = (int32_t *)((char *)ws + base);
        a->seq_parts = (int32_t *)((char *)ws + base + plan);
    }
    return base + 2 * plan;
}

int device_max_waves() {
    int dev = 0, cus = 0, threads = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&threads, hipDeviceAttributeMaxThreadsPerMultiProcessor, dev) != hipSuccess)
        return 0;
    return cus * (threads / 64);
}

}  // namespace pa

using namespace pa;

extern "C" {

static int max_partitions_for(int max_context_len, int partition_size) {
    if (partition_size == 0) return 1;
    return max_context_len <= 0 ? 1 : (max_context_len + partition_size - 1) / partition_size;
}

size_t pa_decode_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                 int max_context_len, int partition_size) {
    if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        num_q_heads % num_kv_heads)
        return 0;
    if (partition_size == PA_PARTITION_BALANCED) {
        const int w = device_max_waves();
        if (w <= 0) return 0;
        return workspace_layout_balanced(num_seqs, num_q_heads, num_kv_heads, head_dim, w, nullptr,
                                         nullptr, nullptr, nullptr, nullptr);
    }
    if (partition_size <= 0) return 0;
    return workspace_layout(num_seqs, num_q_heads, head_dim,
                            max_partitions_for(max_context_len, partition_size), nullptr, nullptr,
                            nullptr, nullptr);
}

// Validation, workspace carving and kernel choice shared by pa_decode and pa_decode_fp8.
static int decode_common(DecodeArgs &a, int max_context_len, float scale, int variant, void *workspace,
                         size_t workspace_bytes) {
    const int num_seqs = a.num_seqs, num_q_heads = a.num_q_heads, num_kv_heads = a.num_kv_heads;
    const int head_dim = a.head_dim, block_size = a.block_size, num_blocks = a.num_blocks;
    const int partition_size = a.partition_size, dtype = a.dtype;
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 ||
        a.max_blocks_per_seq <= 0)
        return fail(PA_ERR_INVALID, "bad sizes: S=%d Hq=%d Hkv=%d blocks=%d max_blocks=%d",
                    num_seqs, num_q_heads, num_kv_heads, num_blocks, a.max_blocks_per_seq);
    if (num_seqs == 0) return PA_OK;
    if (!a.out || !a.query || !a.key_cache || !a.value_cache || !a.block_tables || !a.context_lens)
        return fail(PA_ERR_INVALID, "NULL device pointer");
    if (a.kv_fp8 && (!a.k_scales || !a.v_scales)) return fail(PA_ERR_INVALID, "NULL scale array");
    if (elem_bytes(dtype) == 0 || (a.kv_fp8 && dtype == PA_F32))
        return fail(PA_ERR_UNSUPPORTED, "dtype %d", dtype);
    if (head_dim != 64 && head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "head_dim %d", head_dim);
    if (!pow2_in(block_size, 16, 128)) return fail(PA_ERR_UNSUPPORTED, "block_size %d", block_size);
    if (num_q_heads % num_kv_heads)
        return fail(PA_ERR_INVALID, "num_q_heads %d not a multiple of num_kv_heads %d", num_q_heads,
                    num_kv_heads);
    const int group = num_q_heads / num_kv_heads;
    if (!pow2_in(group, 1, a.kv_fp8 ? 8 : 16)) return fail(PA_ERR_UNSUPPORTED, "group size %d", group);
    if ((int64_t)num_blocks * num_kv_heads * block_size * head_dim > ((int64_t)1 << 40))
        return fail(PA_ERR_UNSUPPORTED, "pool too large");
    if (!(scale == scale)) return fail(PA_ERR_INVALID, "scale is NaN");
    const bool balanced = partition_size == PA_PARTITION_BALANCED;
    if ((partition_size < 0 && !balanced) ||
        (partition_size > 0 && (partition_size % block_size || partition_size % 16)))
        return fail(PA_ERR_INVALID,
                    "partition_size %d must be 0, PA_PARTITION_BALANCED or a multiple of block_size %d and 16",
                    partition_size, block_size);
    if (balanced && num_seqs > kBalancedMaxSeqs)
        return fail(PA_ERR_UNSUPPORTED, "balanced split takes at most %d sequences", kBalancedMaxSeqs);
    if (partition_size > 0 && max_context_len <= 0)
        return fail(PA_ERR_INVALID, "max_context_len %d with partitions", max_context_len);
    const int kernel_choice = variant & 15;
    if (kernel_choice > PA_VARIANT_MFMA || (variant & ~(15 | PA_DECODE_SHARED_KV)))
        return fail(PA_ERR_INVALID, "variant %d", variant);
    const bool grouped = a.group_start != nullptr;
    if (grouped) {
        if (partition_size <= 0)
            return fail(PA_ERR_INVALID, "shared-prefix groups need partitions (partition_size %d)", partition_size);
        if (group != 1 || a.kv_fp8 || (dtype != PA_F16 && dtype != PA_BF16))
            return fail(PA_ERR_UNSUPPORTED, "shared-prefix groups take f16/bf16 pools with one query head per "
                                            "KV head (group %d, dtype %d)", group, dtype);
        if (kernel_choice == PA_VARIANT_MFMA)
            return fail(PA_ERR_UNSUPPORTED, "shared-prefix groups run their private tokens on the vector kernel");
        if (!a.group_parts) return fail(PA_ERR_INVALID, "NULL group_parts");
        if (a.num_groups < 1) return fail(PA_ERR_INVALID, "num_groups %d", a.num_groups);
        if (a.group_rows < 1 || a.group_rows > 16)
            return fail(PA_ERR_INVALID, "max_group_size %d (1..16)", a.group_rows);
        if (a.max_group_parts < 0 || (int64_t)a.max_group_parts * partition_size > max_context_len)
            return fail(PA_ERR_INVALID, "max_group_parts %d with partitions of %d and max_context_len %d",
                        a.max_group_parts, partition_size, max_context_len);
        if ((int64_t)a.num_groups * num_kv_heads > INT32_MAX)  // one workgroup per (group, KV head)
            return fail(PA_ERR_UNSUPPORTED, "too many groups");
        a.group_rows = a.group_rows <= 2 ? 2 : a.group_rows <= 4 ? 4 : a.group_rows <= 8 ? 8 : 16;
    }
    const bool mfma_ok = !a.kv_fp8 && mfma_supported(dtype, head_dim, block_size, group);
    const bool on_mfma = mfma_ok && (kernel_choice == PA_VARIANT_MFMA ||
                                     (kernel_choice == PA_VARIANT_AUTO && group >= 2));
    if (a.new_key) {
        // the fused newest-token store lives in every form but the vector kernel's
        // balanced split
        if (!a.new_value || !a.key_out || !a.value_out) return fail(PA_ERR_INVALID, "NULL new token pointer");
        if (balanced && !on_mfma)
            return fail(PA_ERR_UNSUPPORTED, "the fused newest-token store does not run on the vector "
                                            "kernel's balanced split");
    }

    a.max_partitions = max_partitions_for(max_context_len, partition_size);
    a.scale_log2 = scale * 1.4426950408889634f;
    a.cached_kv = (variant & PA_DECODE_SHARED_KV) != 0;
    if (balanced) {
        // partial slots for every wave the device can hold at once
        const int w = device_max_waves();
        if (w <= 0) return fail(PA_ERR_HIP, "device properties unavailable");
        const size_t need = workspace_layout_balanced(num_seqs, num_q_heads, num_kv_heads, head_dim, w,
                                                      nullptr, nullptr, nullptr, nullptr, nullptr);
        if (!workspace || workspace_bytes < need)
            return fail(PA_ERR_INVALID, "workspace of %zu bytes, need %zu", workspace_bytes, need);
        a.max_workers = w;
        workspace_layout_balanced(num_seqs, num_q_heads, num_kv_heads, head_dim, w, workspace, &a.ws_hdr,
                                  &a.ws_max, &a.ws_sum, &a.ws_acc);
    } else if (grouped) {
        // one partial per (sequence, query head) from the shared-prefix pass, then the plan
        const size_t need = grouped_workspace_layout(num_seqs, num_q_heads, head_dim, nullptr, &a);
        if (!workspace || workspace_bytes < need)
            return fail(PA_ERR_INVALID, "workspace of %zu bytes, need %zu", workspace_bytes, need);
        grouped_workspace_layout(num_seqs, num_q_heads, head_dim, workspace, &a);
    } else if (partition_size > 0) {
        const size_t need = workspace_layout(num_seqs, num_q_heads, head_dim, a.max_partitions,
                                             nullptr, nullptr, nullptr, nullptr);
        if (!workspace || workspace_bytes < need)
            return fail(PA_ERR_INVALID, "workspace of %zu bytes, need %zu", workspace_bytes, need);
        workspace_layout(num_seqs, num_q_heads, head_dim, a.max_partitions, workspace, &a.ws_max,
                         &a.ws_sum, &a.ws_acc);
    }
    if (grouped) {
        // spans of partition_size tokens; the private tokens run in one pass
        a.group_span = partition_size;
        a.partition_size = 0;
        a.max_partitions = 1;
        if (a.max_group_parts > 0) {
            // the plan (which sequences each group serves) and the shared spans, one launch
            const int rc = launch_decode_mfma_grouped(a);
            if (rc != PA_OK) return rc;
            a.skip_parts = a.seq_parts;
        }
        return launch_decode_valu(a);
    }
    if (kernel_choice == PA_VARIANT_MFMA) {
        if (a.kv_fp8) return fail(PA_ERR_UNSUPPORTED, "E4M3 pools run on the vector kernel");
        if (!mfma_ok)
            return fail(PA_ERR_UNSUPPORTED, "MFMA kernel needs 16-bit dtype and group >= 2 (group %d)",
                        group);
        return launch_decode_mfma(a);
    }
    if (kernel_choice == PA_VARIANT_AUTO && mfma_ok && group >= 2) return launch_decode_mfma(a);
    return launch_decode_valu(a);
}

static DecodeArgs decode_args(void *out, const void *query, const void *key_cache, const void *value_cache,
                              const int32_t *block_tables, int max_blocks_per_seq,
                              const int32_t *context_lens, int num_seqs, int num_q_heads,
                              int num_kv_heads, int head_dim, int block_size, int num_blocks, int dtype,
                              int partition_size, void *stream) {
    DecodeArgs a{};
    a.out = out;
    a.query = query;
    a.key_cache = key_cache;
    a.value_cache = value_cache;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.head_dim = head_dim;
    a.block_size = block_size;
    a.num_blocks = num_blocks;
    a.partition_size = partition_size;
    a.dtype = dtype;
    a.stream = stream;
    return a;
}

int pa_decode(void *out, const void *query, const void *key_cache, const void *value_cache,
              const int32_t *block_tables, int max_blocks_per_seq, const int32_t *context_lens,
              int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
              int num_blocks, int max_context_len, float scale, int dtype, int partition_size,
              int variant, void *workspace, size_t workspace_bytes, void *stream) {
    clear_error();
    DecodeArgs a = decode_args(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq,
                               context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                               num_blocks, dtype, partition_size, stream);
    return decode_common(a, max_context_len, scale, variant, workspace, workspace_bytes);
}

int pa_decode_append(void *out, const void *query, const void *new_key, const void *new_value,
                     void *key_cache, void *value_cache, const int32_t *block_tables,
                     int max_blocks_per_seq, const int32_t *context_lens, int num_seqs, int num_q_heads,
                     int num_kv_heads, int head_dim, int block_size, int num_blocks, int max_context_len,
                     float scale, int dtype, int partition_size, int variant, void *workspace,
                     size_t workspace_bytes, void *stream) {
    clear_error();
    if (num_seqs > 0 && (!new_key || !new_value)) return fail(PA_ERR_INVALID, "NULL new token pointer");
    DecodeArgs a = decode_args(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq,
                               context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                               num_blocks, dtype, partition_size, stream);
    a.new_key = new_key;
    a.new_value = new_value;
    a.key_out = key_cache;
    a.value_out = value_cache;
    return decode_common(a, max_context_len, scale, variant, workspace, workspace_bytes);
}

size_t pa_decode_grouped_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                         int max_context_len, int partition_size) {
    (void)max_context_len;
    if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || num_q_heads % num_kv_heads ||
        partition_size <= 0)
        return 0;
    return grouped_workspace_layout(num_seqs, num_q_heads, head_dim, nullptr, nullptr);
}

int pa_decode_grouped(void *out, const void *query, const void *new_key, const void *new_value,
                      void *key_cache, void *value_cache, const int32_t *block_tables, int max_blocks_per_seq,
                      const int32_t *context_lens, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                      int block_size, int num_blocks, int max_context_len, float scale, int dtype,
                      int partition_size, const int32_t *group_start, const int32_t *group_parts,
                      int num_groups, int max_group_size, int max_group_parts, int variant, void *workspace,
                      size_t workspace_bytes, void *stream) {
    clear_error();
    if (num_seqs > 0 && !group_start) return fail(PA_ERR_INVALID, "NULL group_start");
    if (num_seqs > 0 && (!new_key) != (!new_value)) return fail(PA_ERR_INVALID, "new_key and new_value: both or neither");
    DecodeArgs a = decode_args(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq,
                               context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                               num_blocks, dtype, partition_size, stream);
    if (new_key) {
        a.new_key = new_key;
        a.new_value = new_value;
        a.key_out = key_cache;
        a.value_out = value_cache;
    }
    a.group_start = group_start;
    a.group_parts = group_parts;
    a.num_groups = num_groups;
    a.group_rows = max_group_size;
    a.max_group_parts = max_group_parts;
    return decode_common(a, max_context_len, scale, variant, workspace, workspace_bytes);
}

int pa_decode_fp8_append(void *out, const void *query, const void *new_key, const void *new_value,
                         void *key_cache, void *value_cache, const float *k_scales, const float *v_scales,
                         const int32_t *block_tables, int max_blocks_per_seq, const int32_t *context_lens,
                         int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                         int num_blocks, int max_context_len, float scale, int dtype, int partition_size,
                         int variant, void *workspace, size_t workspace_bytes, void *stream) {
    clear_error();
    if (num_seqs > 0 && (!new_key || !new_value)) return fail(PA_ERR_INVALID, "NULL new token pointer");
    DecodeArgs a = decode_args(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq,
                               context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                               num_blocks, dtype, partition_size, stream);
    a.kv_fp8 = true;
    a.k_scales = k_scales;
    a.v_scales = v_scales;
    a.new_key = new_key;
    a.new_value = new_value;
    a.key_out = key_cache;
    a.value_out = value_cache;
    return decode_common(a, max_context_len, scale, variant, workspace, workspace_bytes);
}

int pa_decode_fp8(void *out, const void *query, const void *key_cache, const void *value_cache,
                  const float *k_scales, const float *v_scales, const int32_t *block_tables,
                  int max_blocks_per_seq, const int32_t *context_lens, int num_seqs,
                  int num_q_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                  int max_context_len, float scale, int dtype, int partition_size, int variant,
                  void *workspace, size_t workspace_bytes, void *stream) {
    clear_error();
    DecodeArgs a = decode_args(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq,
                               context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                               num_blocks, dtype, partition_size, stream);
    a.kv_fp8 = true;
    a.k_scales = k_scales;
    a.v_scales = v_scales;
    return decode_common(a, max_context_len, scale, variant, workspace, workspace_bytes);
}

int pa_reshape_and_cache(const void *key, const void *value, void *key_cache, void *value_cache,
                         const int32_t *slot_mapping, int num_tokens, int num_kv_heads,
                         int head_dim, int block_size, int num_blocks, int dtype, void *stream) {
    clear_error();
    const int eb = elem_bytes(dtype);
    if (eb == 0) return fail(PA_ERR_UNSUPPORTED, "dtype %d", dtype);
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
        return fail(PA_ERR_INVALID, "bad sizes");
    if ((head_dim * eb) % 16) return fail(PA_ERR_UNSUPPORTED, "head_dim * elem_bytes must be a multiple of 16");
    if ((int64_t)num_blocks * block_size > INT32_MAX) return fail(PA_ERR_INVALID, "slot ids overflow int32");
    if (num_tokens == 0) return PA_OK;
    if (!key || !value || !key_cache || !value_cache || !slot_mapping)
        return fail(PA_ERR_INVALID, "NULL device pointer");
    return launch_reshape_and_cache(key, value, key_cache, value_cache, slot_mapping, num_tokens,
                                    num_kv_heads, head_dim, block_size, num_blocks, eb, stream);
}

int pa_multi_query(void *out, const void *query, const void *key_cache, const void *value_cache,
                   const int32_t *block_tables, int max_blocks_per_seq, const int32_t *context_lens,
                   const int32_t *query_start, int num_seqs, int num_query_tokens, int max_query_len,
                   int num_q_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                   float scale, int dtype, void *stream) {
    clear_error();
    if (num_seqs < 0 || num_query_tokens < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
        num_blocks <= 0 || max_blocks_per_seq <= 0)
        return fail(PA_ERR_INVALID, "bad sizes");
    if (num_seqs == 0 || num_query_tokens == 0) return PA_OK;
    if (max_query_len <= 0) return fail(PA_ERR_INVALID, "max_query_len %d", max_query_len);
    if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens || !query_start)
        return fail(PA_ERR_INVALID, "NULL device pointer");
    if (dtype != PA_F16 && dtype != PA_BF16)
        return fail(PA_ERR_UNSUPPORTED, "multi-query attention runs on the matrix cores: f16 or bf16, not %d",
                    dtype);
    if (head_dim != 64 && head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "head_dim %d", head_dim);
    if (!pow2_in(block_size, 16, 128)) return fail(PA_ERR_UNSUPPORTED, "block_size %d", block_size);
    if (num_q_heads % num_kv_heads)
        return fail(PA_ERR_INVALID, "num_q_heads %d not a multiple of num_kv_heads %d", num_q_heads,
                    num_kv_heads);
    const int group = num_q_heads / num_kv_heads;
    if (!pow2_in(group, 1, 16)) return fail(PA_ERR_UNSUPPORTED, "group size %d", group);
    if ((int64_t)num_blocks * num_kv_heads * block_size * head_dim > ((int64_t)1 << 40))
        return fail(PA_ERR_UNSUPPORTED, "pool too large");
    if (!(scale == scale)) return fail(PA_ERR_INVALID, "scale is NaN");
    DecodeArgs a = decode_args(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq,
                               context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                               num_blocks, dtype, 0, stream);
    a.query_start = query_start;
    a.num_query_tokens = num_query_tokens;
    a.max_query_len = max_query_len;
    a.scale_log2 = scale * 1.4426950408889634f;
    return dtype == PA_F16 ? launch_multi_query_f16(a) : launch_multi_query_bf16(a);
}

int pa_reshape_and_cache_fp8(const void *key, const void *value, void *key_cache, void *value_cache,
                             const float *k_scales, const float *v_scales,
                             const int32_t *slot_mapping, int num_tokens, int num_kv_heads,
                             int head_dim, int block_size, int num_blocks, int dtype, void *stream) {
    clear_error();
    if (elem_bytes(dtype) == 0) return fail(PA_ERR_UNSUPPORTED, "source dtype %d", dtype);
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
        return fail(PA_ERR_INVALID, "bad sizes");
    if (head_dim % 4) return fail(PA_ERR_UNSUPPORTED, "head_dim must be a multiple of 4");
    if ((int64_t)num_blocks * block_size > INT32_MAX) return fail(PA_ERR_INVALID, "slot ids overflow int32");
    if (num_tokens == 0) return PA_OK;
    if (!key || !value || !key_cache || !value_cache || !k_scales || !v_scales || !slot_mapping)
        return fail(PA_ERR_INVALID, "NULL device pointer");
    return launch_reshape_and_cache_fp8(key, value, key_cache, value_cache, k_scales, v_scales,
                                        slot_mapping, num_tokens, num_kv_heads, head_dim, block_size,
                                        num_blocks, dtype, stream);
}

int pa_copy_blocks(void *key_cache, void *value_cache, const int32_t *src, const int32_t *dst,
                   int num_pairs, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                   int dtype, void *stream) {
    clear_error();
    const int eb = pool_elem_bytes(dtype);
    if (eb == 0) return fail(PA_ERR_UNSUPPORTED, "dtype %d", dtype);
    if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
        return fail(PA_ERR_INVALID, "bad sizes");
    if (((int64_t)num_kv_heads * block_size * head_dim * eb) % 4)
        return fail(PA_ERR_UNSUPPORTED, "block bytes must be a multiple of 4");
    if (num_pairs == 0) return PA_OK;
    if (!key_cache || !value_cache || !src || !dst) return fail(PA_ERR_INVALID, "NULL device pointer");
    return launch_move_blocks(key_cache, value_cache, key_cache, value_cache, src, dst, num_pairs,
                              num_kv_heads, head_dim, block_size, num_blocks, num_blocks, eb, stream);
}

int pa_stream_read(const void *buf, size_t bytes, void *sink, void *stream) {
    clear_error();
    if (!buf || !sink) return fail(PA_ERR_INVALID, "NULL device pointer");
    if (bytes == 0 || bytes % 16 || ((uintptr_t)buf & 15)) return fail(PA_ERR_INVALID, "buffer of %zu bytes", bytes);
    return launch_stream_read(buf, bytes, sink, stream);
}

int pa_gather_read(const uint64_t *tile_addrs, int num_tiles, int tile_bytes, void *sink, void *stream) {
    clear_error();
    if (num_tiles < 0) return fail(PA_ERR_INVALID, "num_tiles %d", num_tiles);
    if (tile_bytes != 1024 && tile_bytes != 2048 && tile_bytes != 4096 && tile_bytes != 8192)
        return fail(PA_ERR_INVALID, "tile of %d bytes (1024, 2048, 4096 or 8192)", tile_bytes);
    if (num_tiles == 0) return PA_OK;
    if (!tile_addrs || !sink) return fail(PA_ERR_INVALID, "NULL device pointer");
    return launch_gather_read(tile_addrs, num_tiles, tile_bytes, sink, stream);
}

int pa_swap_blocks(const void *src_key_cache, const void *src_value_cache, void *dst_key_cache,
                   void *dst_value_cache, const int32_t *src, const int32_t *dst, int num_pairs,
                   int num_kv_heads, int head_dim, int block_size, int src_num_blocks,
                   int dst_num_blocks, int dtype, void *stream) {
    clear_error();
    const int eb = pool_elem_bytes(dtype);
    if (eb == 0) return fail(PA_ERR_UNSUPPORTED, "dtype %d", dtype);
    if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || src_num_blocks <= 0 ||
        dst_num_blocks <= 0)
        return fail(PA_ERR_INVALID, "bad sizes");
    if (((int64_t)num_kv_heads * block_size * head_dim * eb) % 4)
        return fail(PA_ERR_UNSUPPORTED, "block bytes must be a multiple of 4");
    if (num_pairs == 0) return PA_OK;
    if (!src_key_cache || !src_value_cache || !dst_key_cache || !dst_value_cache || !src || !dst)
        return fail(PA_ERR_INVALID, "NULL pointer");
    if (src_key_cache == dst_key_cache || src_value_cache == dst_value_cache)
        return fail(PA_ERR_INVALID, "source and destination pools must differ (use pa_copy_blocks)");
    return launch_move_blocks(src_key_cache, src_value_cache, dst_key_cache, dst_value_cache, src, dst,
                              num_pairs, num_kv_heads, head_dim, block_size, src_num_blocks,
                              dst_num_blocks, eb, stream);
}

}  // extern "C"
