// Block-pool write kernels: the newest-token scatter and the copy-on-write block copy.
//
// Both are bitwise moves of 16-byte words (one dwordx4 per lane), so they work for
// any element type.  Pool layout [num_blocks][H_kv][B][d]: the row of token `o` of
// head `h` in block `b` starts at ((b * H_kv + h) * B + o) * d elements.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// "KV cache / 内存分页 / paged attention" tutorial (wmrh.cn), "KV cache" part: a decode
// step computes and caches only the newest token's K and V.  "PagedAttention" concept
// report (compassingai.com) §5: a token lives at its physical block's base plus the
// in-block offset.  One workgroup per token; lanes stride over the token's
// H_kv * d elements in 16-byte words.  Out-of-range or negative slots are skipped.
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const u32x4 *__restrict__ key, const u32x4 *__restrict__ value, u32x4 *__restrict__ key_cache,
    u32x4 *__restrict__ value_cache, const int32_t *__restrict__ slot_mapping, int num_kv_heads,
    int words_per_row, int block_size, int64_t num_slots) {
    const int i = blockIdx.x;
    const int64_t slot = slot_mapping[i];
    if (slot < 0 || slot >= num_slots) return;
    const int64_t b = slot / block_size;
    const int64_t o = slot - b * block_size;
    const int per_token = num_kv_heads * words_per_row;
    const u32x4 *k_src = key + (int64_t)i * per_token;
    const u32x4 *v_src = value + (int64_t)i * per_token;
    for (int c = threadIdx.x; c < per_token; c += blockDim.x) {
        const int h = c / words_per_row;
        const int r = c - h * words_per_row;
        const int64_t dst = ((b * num_kv_heads + h) * block_size + o) * words_per_row + r;
        key_cache[dst] = k_src[c];
        value_cache[dst] = v_src[c];
    }
}

// Whole-block moves between two pools (which may be the same pool).
// "PagedAttention" concept report (compassingai.com) §6: before a write into a shared
// block, a fresh block receives a copy of its content; §6 and §11: under memory
// pressure a request's blocks are moved out to CPU memory and moved back later.
// grid = (word groups, pairs, pool); each workgroup moves 4 words per lane (16 KiB)
// of one block of one pool.  A pair with an id outside its pool is skipped.
constexpr int COPY_THREADS = 256;
constexpr int COPY_UNROLL = 4;

__global__ __launch_bounds__(COPY_THREADS) void move_blocks_kernel(
    const u32x4 *src_key, const u32x4 *src_value, u32x4 *dst_key, u32x4 *dst_value,
    const int32_t *__restrict__ src, const int32_t *__restrict__ dst, int64_t words_per_block,
    int src_blocks, int dst_blocks) {
    const int pair = blockIdx.y;
    const int32_t s = src[pair];
    const int32_t d = dst[pair];
    if (s < 0 || s >= src_blocks || d < 0 || d >= dst_blocks) return;
    const u32x4 *from = (blockIdx.z == 0 ? src_key : src_value) + (int64_t)s * words_per_block;
    u32x4 *to = (blockIdx.z == 0 ? dst_key : dst_value) + (int64_t)d * words_per_block;
    const int64_t base = (int64_t)blockIdx.x * COPY_THREADS * COPY_UNROLL + threadIdx.x;
    u32x4 w[COPY_UNROLL];
#pragma unroll
    for (int u = 0; u < COPY_UNROLL; ++u) {
        const int64_t e = base + u * COPY_THREADS;
        if (e < words_per_block) w[u] = from[e];
    }
#pragma unroll
    for (int u = 0; u < COPY_UNROLL; ++u) {
        const int64_t e = base + u * COPY_THREADS;
        if (e < words_per_block) to[e] = w[u];
    }
}

}  // namespace

int launch_reshape_and_cache(const void *key, const void *value, void *key_cache, void *value_cache,
                             const int32_t *slot_mapping, int num_tokens, int num_kv_heads,
                             int head_dim, int block_size, int num_blocks, int elem_bytes,
                             void *stream) {
    const int words_per_row = head_dim * elem_bytes / 16;
    const int per_token = num_kv_heads * words_per_row;
    const int threads = per_token >= 256 ? 256 : (per_token >= 128 ? 128 : 64);
    hipLaunchKernelGGL(reshape_and_cache_kernel, dim3(num_tokens), dim3(threads), 0,
                       (hipStream_t)stream, (const u32x4 *)key, (const u32x4 *)value,
                       (u32x4 *)key_cache, (u32x4 *)value_cache, slot_mapping, num_kv_heads,
                       words_per_row, block_size, (int64_t)num_blocks * block_size);
    return check_launch("reshape_and_cache");
}

int launch_move_blocks(const void *src_key, const void *src_value, void *dst_key, void *dst_value,
                       const int32_t *src, const int32_t *dst, int num_pairs, int num_kv_heads,
                       int head_dim, int block_size, int src_blocks, int dst_blocks, int elem_bytes,
                       void *stream) {
    const int64_t words = (int64_t)num_kv_heads * block_size * head_dim * elem_bytes / 16;
    const int64_t per_wg = COPY_THREADS * COPY_UNROLL;
    const unsigned gx = (unsigned)((words + per_wg - 1) / per_wg);
    for (int off = 0; off < num_pairs; off += 65535) {  // grid.y is limited
        const int n = num_pairs - off < 65535 ? num_pairs - off : 65535;
        hipLaunchKernelGGL(move_blocks_kernel, dim3(gx, n, 2), dim3(COPY_THREADS), 0, (hipStream_t)stream,
                           (const u32x4 *)src_key, (const u32x4 *)src_value, (u32x4 *)dst_key,
                           (u32x4 *)dst_value, src + off, dst + off, words, src_blocks, dst_blocks);
        const int rc = check_launch("move_blocks");
        if (rc != PA_OK) return rc;
    }
    return PA_OK;
}

}  // namespace pa
