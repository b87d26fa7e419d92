// Block-pool write kernels: the newest-token scatter (bitwise, or rounded to E4M3
// codes), and the whole-block moves of copy-on-write and swapping.
//
// The bitwise kernels move 16-byte words (4-byte words for blocks of other sizes), so
// they work for any element type.  Pool layout [num_blocks][H_kv][B][d]: the row of
// token `o` of head `h` in block `b` starts at ((b * H_kv + h) * B + o) * d elements.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "kernel_common.h"

namespace pa {
namespace {

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

// E4M3 counterpart of the scatter ("vLLM PagedAttention 技术深度解析" (kwkr.cn) §1.5
// and the "PagedAttention" concept report §15: cached blocks compressed to fewer bits).
// Element x of head h goes to block b as the E4M3 code nearest to x / scale[b][h] (an
// IEEE fp32 division: the library is built with correctly rounded division).  One
// workgroup per token; each lane turns 4 elements into one 4-byte word of codes.
template <typename T>
__device__ inline void load4(const uint8_t *p, float (&x)[4]);
template <>
__device__ inline void load4<F32>(const uint8_t *p, float (&x)[4]) {
    const u32x4 w = *(const u32x4 *)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(w[i]);
}
template <>
__device__ inline void load4<F16>(const uint8_t *p, float (&x)[4]) {
    const uint2 w = *(const uint2 *)p;
    const f16x2 a = __builtin_bit_cast(f16x2, w.x), b = __builtin_bit_cast(f16x2, w.y);
    x[0] = (float)a[0];
    x[1] = (float)a[1];
    x[2] = (float)b[0];
    x[3] = (float)b[1];
}
template <>
__device__ inline void load4<BF16>(const uint8_t *p, float (&x)[4]) {
    const uint2 w = *(const uint2 *)p;
    x[0] = __uint_as_float(w.x << 16);
    x[1] = __uint_as_float(w.x & 0xffff0000u);
    x[2] = __uint_as_float(w.y << 16);
    x[3] = __uint_as_float(w.y & 0xffff0000u);
}

template <typename T>
__global__ __launch_bounds__(256) void reshape_and_cache_fp8_kernel(
    const uint8_t *__restrict__ key, const uint8_t *__restrict__ value, uint32_t *__restrict__ key_cache,
    uint32_t *__restrict__ value_cache, const float *__restrict__ k_scales,
    const float *__restrict__ v_scales, const int32_t *__restrict__ slot_mapping, int num_kv_heads,
    int quads_per_row, int block_size, int64_t num_slots) {
    const int i = blockIdx.x;
    const int64_t slot = slot_mapping[i];
    if (slot < 0 || slot >= num_slots) return;
    const int64_t b = slot / block_size;
    const int64_t o = slot - b * block_size;
    const int per_token = num_kv_heads * quads_per_row;
    for (int c = threadIdx.x; c < per_token; c += blockDim.x) {
        const int h = c / quads_per_row;
        const int r = c - h * quads_per_row;
        const int64_t src = ((int64_t)i * per_token + c) * 4 * T::bytes;
        const int64_t dst = ((b * num_kv_heads + h) * block_size + o) * quads_per_row + r;
        const float ks = k_scales[b * num_kv_heads + h];
        const float vs = v_scales[b * num_kv_heads + h];
        float xk[4], xv[4];
        load4<T>(key + src, xk);
        load4<T>(value + src, xv);
        uint32_t wk = 0, wv = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            wk |= e4m3_encode(xk[e] / ks) << (8 * e);
            wv |= e4m3_encode(xv[e] / vs) << (8 * e);
        }
        key_cache[dst] = wk;
        value_cache[dst] = wv;
    }
}

// Whole-block moves between two pools (which may be the same pool).
// "PagedAttention" concept report (compassingai.com) §6: before a write into a shared
// block, a fresh block receives a copy of its content; §6 and §11: under memory
// pressure a request's blocks are moved out to CPU memory and moved back later.
// grid = (word groups, pairs, pool); each workgroup moves 4 words per lane of one
// block of one pool (W = 16-byte words, or 4-byte words for blocks whose size is not
// a multiple of 16 bytes, such as per-block scale arrays).  A pair with an id outside
// its pool is skipped.
constexpr int COPY_THREADS = 256;
constexpr int COPY_UNROLL = 4;

template <typename W>
__global__ __launch_bounds__(COPY_THREADS) void move_blocks_kernel(
    const W *src_key, const W *src_value, W *dst_key, W *dst_value, const int32_t *__restrict__ src,
    const int32_t *__restrict__ dst, int64_t words_per_block, int src_blocks, int dst_blocks) {
    const int pair = blockIdx.y;
    const int32_t s = src[pair];
    const int32_t d = dst[pair];
    if (s < 0 || s >= src_blocks || d < 0 || d >= dst_blocks) return;
    const W *from = (blockIdx.z == 0 ? src_key : src_value) + (int64_t)s * words_per_block;
    W *to = (blockIdx.z == 0 ? dst_key : dst_value) + (int64_t)d * words_per_block;
    const int64_t base = (int64_t)blockIdx.x * COPY_THREADS * COPY_UNROLL + threadIdx.x;
    W w[COPY_UNROLL];
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

template <typename W>
int move_blocks(const void *src_key, const void *src_value, void *dst_key, void *dst_value,
                const int32_t *src, const int32_t *dst, int num_pairs, int64_t block_bytes,
                int src_blocks, int dst_blocks, void *stream) {
    const int64_t words = block_bytes / (int64_t)sizeof(W);
    const int64_t per_wg = COPY_THREADS * COPY_UNROLL;
    const unsigned gx = (unsigned)((words + per_wg - 1) / per_wg);
    for (int off = 0; off < num_pairs; off += 65535) {  // grid.y is limited
        const int n = num_pairs - off < 65535 ? num_pairs - off : 65535;
        hipLaunchKernelGGL(move_blocks_kernel<W>, dim3(gx, n, 2), dim3(COPY_THREADS), 0, (hipStream_t)stream,
                           (const W *)src_key, (const W *)src_value, (W *)dst_key, (W *)dst_value, src + off,
                           dst + off, words, src_blocks, dst_blocks);
        const int rc = check_launch("move_blocks");
        if (rc != PA_OK) return rc;
    }
    return PA_OK;
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

int launch_reshape_and_cache_fp8(const void *key, const void *value, void *key_cache,
                                 void *value_cache, const float *k_scales, const float *v_scales,
                                 const int32_t *slot_mapping, int num_tokens, int num_kv_heads,
                                 int head_dim, int block_size, int num_blocks, int src_dtype,
                                 void *stream) {
    const int quads = head_dim / 4;
    const int per_token = num_kv_heads * quads;
    const int threads = per_token >= 256 ? 256 : (per_token >= 128 ? 128 : 64);
    const int64_t slots = (int64_t)num_blocks * block_size;
    auto launch = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3(num_tokens), dim3(threads), 0, (hipStream_t)stream,
                           (const uint8_t *)key, (const uint8_t *)value, (uint32_t *)key_cache,
                           (uint32_t *)value_cache, k_scales, v_scales, slot_mapping, num_kv_heads, quads,
                           block_size, slots);
        return check_launch("reshape_and_cache_fp8");
    };
    switch (src_dtype) {
        case PA_F32: return launch(reshape_and_cache_fp8_kernel<F32>);
        case PA_F16: return launch(reshape_and_cache_fp8_kernel<F16>);
        case PA_BF16: return launch(reshape_and_cache_fp8_kernel<BF16>);
    }
    return fail(PA_ERR_UNSUPPORTED, "dtype %d", src_dtype);
}

int launch_move_blocks(const void *src_key, const void *src_value, void *dst_key, void *dst_value,
                       const int32_t *src, const int32_t *dst, int num_pairs, int num_kv_heads,
                       int head_dim, int block_size, int src_blocks, int dst_blocks, int elem_bytes,
                       void *stream) {
    const int64_t bytes = (int64_t)num_kv_heads * block_size * head_dim * elem_bytes;
    if (bytes % 16 == 0)
        return move_blocks<u32x4>(src_key, src_value, dst_key, dst_value, src, dst, num_pairs, bytes,
                                  src_blocks, dst_blocks, stream);
    return move_blocks<uint32_t>(src_key, src_value, dst_key, dst_value, src, dst, num_pairs, bytes,
                                 src_blocks, dst_blocks, stream);
}

// Read-bandwidth probe: per step a workgroup reads SR_U consecutive 4 KiB pieces (each
// wave 1 KiB of each), then jumps by the whole grid's span; the last, partial span is
// read word by word.
constexpr int SR_U = 8;
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *__restrict__ p, int64_t n,
                                                           uint32_t *__restrict__ sink) {
    uint32_t x = 0;
    const int64_t stride = (int64_t)gridDim.x * 256 * SR_U;
    int64_t i = (int64_t)blockIdx.x * 256 * SR_U + threadIdx.x;
    for (; i + (SR_U - 1) * 256 < n; i += stride) {
        u32x4 v[SR_U];
#pragma unroll
        for (int u = 0; u < SR_U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * 256);
#pragma unroll
        for (int u = 0; u < SR_U; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (int u = 0; u < SR_U; ++u)
        if (i + u * 256 < n) {
            const u32x4 a = __builtin_nontemporal_load(p + i + u * 256);
            x ^= a[0] ^ a[1] ^ a[2] ^ a[3];
        }
    if (x == 0x9e3779b9u) *sink = x;
}

int launch_stream_read(const void *buf, size_t bytes, void *sink, void *stream) {
    const int64_t n = (int64_t)(bytes / 16);
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return fail(PA_ERR_HIP, "device properties unavailable");
    int64_t grid = (int64_t)cus * 8;
    const int64_t need = (n + 256 * SR_U - 1) / (256 * SR_U);
    if (grid > need) grid = need;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream,
                       (const u32x4 *)buf, n, (uint32_t *)sink);
    return check_launch("stream_read");
}

// Tile-gather read probe: wave w of the grid reads tiles w, w + W, w + 2W, ... (W waves
// in all), two tiles in flight (tile t and t + W loaded before either is folded); each
// tile is TB / 1024 wave loads of 1 KiB, 16 bytes per lane.
template <int TB>
__global__ __launch_bounds__(256) void gather_read_kernel(const uint64_t *__restrict__ tile_addrs, int num_tiles,
                                                          uint32_t *__restrict__ sink) {
    constexpr int LOADS = TB / 1024;
    const int lane = threadIdx.x & 63;
    const int nw = gridDim.x * 4;
    uint32_t x = 0;
    for (int t = blockIdx.x * 4 + (int)(threadIdx.x >> 6); t < num_tiles; t += 2 * nw) {
        const uint8_t *a = (const uint8_t *)tile_addrs[t];
        const int t1 = t + nw;
        const uint8_t *b = t1 < num_tiles ? (const uint8_t *)tile_addrs[t1] : a;
        u32x4 v[2 * LOADS];
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            v[i] = __builtin_nontemporal_load((const u32x4 *)(a + i * 1024 + lane * 16));
            v[LOADS + i] = __builtin_nontemporal_load((const u32x4 *)(b + i * 1024 + lane * 16));
        }
#pragma unroll
        for (int i = 0; i < 2 * LOADS; ++i) x ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
    }
    if (x == 0x9e3779b9u) *sink = x;
}

int launch_gather_read(const uint64_t *tile_addrs, int num_tiles, int tile_bytes, void *sink, void *stream) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return fail(PA_ERR_HIP, "device properties unavailable");
    int64_t grid = (int64_t)cus * 8;
    const int64_t need = ((int64_t)num_tiles + 3) / 4;
    if (grid > need) grid = need;
    hipStream_t st = (hipStream_t)stream;
    uint32_t *sk = (uint32_t *)sink;
    switch (tile_bytes) {
        case 1024: hipLaunchKernelGGL(gather_read_kernel<1024>, dim3((unsigned)grid), dim3(256), 0, st, tile_addrs, num_tiles, sk); break;
        case 2048: hipLaunchKernelGGL(gather_read_kernel<2048>, dim3((unsigned)grid), dim3(256), 0, st, tile_addrs, num_tiles, sk); break;
        case 4096: hipLaunchKernelGGL(gather_read_kernel<4096>, dim3((unsigned)grid), dim3(256), 0, st, tile_addrs, num_tiles, sk); break;
        case 8192: hipLaunchKernelGGL(gather_read_kernel<8192>, dim3((unsigned)grid), dim3(256), 0, st, tile_addrs, num_tiles, sk); break;
        default: return fail(PA_ERR_INVALID, "tile of %d bytes", tile_bytes);
    }
    return check_launch("gather_read");
}


}  // namespace pa
