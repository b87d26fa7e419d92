#pragma once
// Grouped-query paged decode attention on the matrix cores (gfx950 MFMA).
//
// What is computed is the same as the vector kernel ("PagedAttention" concept report
// (compassingai.com) §8: scores of the query against every cached key, softmax, the
// weighted sum of the values, walking the block table; §5 base + offset addressing).
// With g = H_q / H_kv query heads per KV head, a tile of cached keys against the
// group's queries is a small dense product, so it runs on v_mfma_f32_16x16x32_{bf16,f16}
// (heads padded to 16):
//
//   S^T[t][h]  = sum_d K[t][d] Q[h][d]          A = K rows (16 tokens x 32 d), B = Q^T
//   O^T[d][h] += sum_t V[t][d] P[h][t]          A = V^T (16 d x 32 tokens),   B = P^T
//
// Operand layouts (checked on gfx950): lane l supplies A[l%16][8(l/16)..+8] and
// B[8(l/16)..+8][l%16] and receives D[4(l/16)..+4][l%16].  Consequences:
//  * a K operand is a plain 16-byte load of one token row per lane, straight from HBM;
//  * the score fragment S^T already holds, per lane, one head's scores for 4+4 tokens,
//    which is exactly a P^T operand once the k order is chosen to match (no shuffle);
//  * the O^T fragment holds one head per lane column, so the online-softmax rescale
//    and the final division use per-lane values;
//  * V must be read transposed (8 tokens of one d per lane): each wave copies its V
//    rows HBM -> LDS with direct 16-byte LDS loads (global_load_lds_dwordx4, no
//    register staging) into its own double-buffered region, 1 KiB per wave load with
//    32 bytes of padding after each KiB so the four rows read together fall in
//    different banks, and reads them back 16 bits at a time.
// Softmax runs in fp32 (online, exp2 domain).  P enters the second product rounded to
// the storage type; the normaliser sums the rounded weights, so numerator and
// denominator use the same weights.  Accumulation is fp32.
//
// Work decomposition, XCD-aware numbering and the partition partials are those of the
// vector kernel, so the same log-sum-exp merge kernel finishes a partitioned run.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "kernel_common.h"

namespace pa {
namespace mfma {

#ifndef PA_MFMA_WAVES
#define PA_MFMA_WAVES 4
#endif
constexpr int MW = PA_MFMA_WAVES;  // waves per workgroup
constexpr int CT = 32;             // tokens per chunk: two 16-token tiles

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Mma;
template <>
struct Mma<F16> {
    static __device__ inline f32x4 run(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    // round to the storage type; returns the 16 bits and the rounded value
    static __device__ inline uint32_t round(float x, float &back) {
        const _Float16 h = (_Float16)x;
        back = (float)h;
        return (uint32_t)__builtin_bit_cast(uint16_t, h);
    }
};
template <>
struct Mma<BF16> {
    static __device__ inline f32x4 run(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    static __device__ inline uint32_t round(float x, float &back) {
        // x is a finite weight in [0, 1]: round to nearest even
        const uint32_t u = __float_as_uint(x);
        const uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u;
        back = __uint_as_float(r);
        return r >> 16;
    }
};

template <typename T, int D, int G, bool SPLIT, bool NT>
__global__ __launch_bounds__(MW * 64) void decode_mfma_kernel(
    void *__restrict__ out, const uint8_t *__restrict__ query, const uint8_t *__restrict__ key_cache,
    const uint8_t *__restrict__ value_cache, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ context_lens, float *__restrict__ ws_max, float *__restrict__ ws_sum,
    float *__restrict__ ws_acc, int max_blocks_per_seq, int num_seqs, int num_kv_heads,
    int log2_block, int num_blocks, int partition_size, int max_partitions, float scale_log2) {
    constexpr int ROW = D * 2;            // bytes per token row
    constexpr int NKK = D / 32;           // 32-wide d steps of the score product
    constexpr int NN = D / 16;            // 16-row d fragments of the output
    constexpr int VL = 16 * ROW / 1024;   // 1 KiB wave loads per 16-token V tile
    constexpr int RPK = 1024 / ROW;       // token rows per KiB
    constexpr int KSTR = 1024 + 32;       // LDS stride of one KiB group (padded)
    constexpr int STAGE = 2 * VL * KSTR;  // LDS bytes of one chunk's V
    constexpr int WAVE_LDS = 2 * STAGE;   // double-buffered

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15;  // head column / token row within a tile
    const int q = lane >> 4;  // k group

    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int part = L % max_partitions;
    const int rest = L / max_partitions;
    const int s = rest % num_seqs;
    const int kvh = rest / num_seqs;
    const int num_q_heads = num_kv_heads * G;

    const int ctx = context_lens[s];
    int start = 0, end = ctx;
    if (SPLIT) {
        start = part * partition_size;
        if (ctx < 0 || start >= ctx) return;
        end = min(ctx, start + partition_size);
    }

    __shared__ __attribute__((aligned(16))) uint8_t lds[MW * WAVE_LDS];
    static_assert((2 * MW * G + MW * G * D) * 4 <= MW * WAVE_LDS, "merge area must fit the staging area");
    uint8_t *wave_lds = lds + wave * WAVE_LDS;

    const int block_size = 1 << log2_block;
    const int32_t *table = block_tables + (int64_t)s * max_blocks_per_seq;
    const int64_t head_off = (int64_t)kvh * block_size * ROW;
    const int64_t block_bytes = (int64_t)num_kv_heads * block_size * ROW;

    // Q^T operand: lane holds Q[head n][32 kk + 8 q .. +8]; heads past the group are zero
    u32x4 qb[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        qb[kk] = u32x4{0, 0, 0, 0};
        if (n < G)
            qb[kk] = *(const u32x4 *)(query + ((int64_t)(s * num_q_heads + kvh * G + n) * D + 32 * kk + 8 * q) * 2);
    }

    float m = -INFINITY;  // running max of head n (same in the 4 lanes of a column)
    float lsum = 0.f;     // this lane's share of the normaliser
    f32x4 o[NN];
#pragma unroll
    for (int i = 0; i < NN; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    bool bad = ctx < 0;

    const int ntok = ctx < 0 ? 0 : end - start;
    const int nchunks = (ntok + CT - 1) / CT;

    // Byte offset of the first row of 16-token tile `tt` of chunk c, or -1.  A tile with
    // no data (past `end`, or a bad entry) reads block 0's first rows instead (inside
    // the pool; masked like any row past `end`): no branch around a load, because one
    // makes the compiler wait for every outstanding load.
    auto tile_base = [&](int c, int tt) -> int64_t {
        const int tok = start + c * CT + 16 * tt;
        if (tok >= end) return -1;
        const int lb = tok >> log2_block;
        if (lb >= max_blocks_per_seq) {
            bad = true;
            return -1;
        }
        const int32_t pb = table[lb];
        if (pb < 0 || pb >= num_blocks) {
            bad = true;
            return -1;
        }
        return (int64_t)pb * block_bytes + head_off + (int64_t)(tok & (block_size - 1)) * ROW;
    };

    // a chunk's K operands live in registers; its V rows go to LDS stage `st`
    struct Chunk {
        u32x4 k[2][NKK];
    };
    auto issue = [&](Chunk &b, int c, int st) {
        uint8_t *stage = wave_lds + st * STAGE;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            int64_t base = tile_base(c, tt);
            base = base < 0 ? 0 : base;
#pragma unroll
            for (int i = 0; i < VL; ++i)
                __builtin_amdgcn_global_load_lds(
                    (const void *)(value_cache + base + i * 1024 + lane * 16),
                    (__attribute__((address_space(3))) void *)(stage + (tt * VL + i) * KSTR), 16, 0, 0);
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
                b.k[tt][kk] = kv_load<NT>(
                    (const u32x4 *)(key_cache + base + n * ROW + (32 * kk + 8 * q) * 2));
        }
    };
    // LDS address of V[row r of the chunk][byte col]
    auto v_at = [&](const uint8_t *stage, int r, int col) -> const uint8_t * {
        return stage + (r / RPK) * KSTR + (r % RPK) * ROW + col;
    };
    auto consume = [&](const Chunk &b, int c, int st) {
        const uint8_t *stage = wave_lds + st * STAGE;
        const int tok0 = start + c * CT;
        const bool tail = tok0 + CT > end;
        // scores S^T: lane holds tokens 16 tt + 4 q + i of head n
        float sc[2][4];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) acc = Mma<T>::run(b.k[tt][kk], qb[kk], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = !tail || (tok0 + 16 * tt + 4 * q + i < end);
                sc[tt][i] = ok ? acc[i] * scale_log2 : -INFINITY;
            }
        }
        float cm = sc[0][0];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) cm = fmaxf(cm, sc[tt][i]);
        cm = fmaxf(cm, __shfl_xor(cm, 16));
        cm = fmaxf(cm, __shfl_xor(cm, 32));
        const float mn = fmaxf(m, cm);
        const float ms = mn == -INFINITY ? 0.f : mn;
        const float alpha = fast_exp2(m - ms);
        m = mn;
        // P^T operand: k slot j < 4 -> token 4q + j (tile 0), j >= 4 -> token 16 + 4q + j - 4
        uint32_t pk[4];
        float psum = 0.f;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
                float b0, b1;
                const uint32_t h0 = Mma<T>::round(fast_exp2(sc[tt][i] - ms), b0);
                const uint32_t h1 = Mma<T>::round(fast_exp2(sc[tt][i + 1] - ms), b1);
                psum += b0 + b1;
                pk[2 * tt + i / 2] = h0 | (h1 << 16);
            }
        lsum = lsum * alpha + psum;
        const u32x4 pb = u32x4{pk[0], pk[1], pk[2], pk[3]};
#pragma unroll
        for (int nn = 0; nn < NN; ++nn) o[nn] *= alpha;
        // this chunk's V rows have landed in LDS: its V loads were issued before its K
        // loads, which the score product above already waited for
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (tail) {
            // rows past `end` as zeros: 0 * NaN would poison the product
            for (int r = max(0, end - tok0); r < CT; ++r)
                for (int col = lane * 4; col < ROW; col += 256)
                    *(uint32_t *)v_at(stage, r, col) = 0u;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        // V^T operand per 16-row d fragment: lane reads V[t(q, j)][16 nn + n]
#pragma unroll
        for (int nn = 0; nn < NN; ++nn) {
            uint32_t vk[4];
#pragma unroll
            for (int j = 0; j < 8; j += 2) {
                const int t0 = j < 4 ? 4 * q + j : 16 + 4 * q + (j - 4);
                const uint16_t a = *(const uint16_t *)v_at(stage, t0, (16 * nn + n) * 2);
                const uint16_t c2 = *(const uint16_t *)v_at(stage, t0 + 1, (16 * nn + n) * 2);
                vk[j / 2] = (uint32_t)a | ((uint32_t)c2 << 16);
            }
            o[nn] = Mma<T>::run(u32x4{vk[0], vk[1], vk[2], vk[3]}, pb, o[nn]);
        }
        // the stage is rewritten by a later chunk's loads: finish reading it first
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    {
        // this wave's chunks are wave, wave + MW, ...; the steady-state loop always has
        // a next chunk to prefetch (see tile_base), the last one or two run after it
        const int mine = nchunks > wave ? (nchunks - wave + MW - 1) / MW : 0;
        Chunk A, Bf;
        if (mine > 0) {
            issue(A, wave, 0);
            int j = 0;
            for (; j + 2 < mine; j += 2) {
                issue(Bf, wave + (j + 1) * MW, 1);
                consume(A, wave + j * MW, 0);
                issue(A, wave + (j + 2) * MW, 0);
                consume(Bf, wave + (j + 1) * MW, 1);
            }
            if (j + 1 < mine) {
                issue(Bf, wave + (j + 1) * MW, 1);
                consume(A, wave + j * MW, 0);
                consume(Bf, wave + (j + 1) * MW, 1);
            } else {
                consume(A, wave + j * MW, 0);
            }
        }
    }

    // normaliser of head n over the 4 lanes of its column
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);

    // merge the waves through LDS (the staging area is free now)
    __syncthreads();
    float *sm_m = (float *)lds;          // [MW][G]
    float *sm_l = sm_m + MW * G;         // [MW][G]
    float *sm_acc = sm_l + MW * G;       // [MW][G][D]
    __shared__ int sm_bad;
    if (threadIdx.x == 0) sm_bad = 0;
    __syncthreads();
    if (bad) sm_bad = 1;
    if (n < G) {
        if (q == 0) {
            sm_m[wave * G + n] = m;
            sm_l[wave * G + n] = lsum;
        }
#pragma unroll
        for (int nn = 0; nn < NN; ++nn)
#pragma unroll
            for (int i = 0; i < 4; ++i) sm_acc[(wave * G + n) * D + 16 * nn + 4 * q + i] = o[nn][i];
    }
    __syncthreads();
    const bool any_bad = sm_bad != 0;
    for (int t = threadIdx.x; t < G * D; t += MW * 64) {
        const int g = t / D;
        const int j = t - g * D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < MW; ++w) M = fmaxf(M, sm_m[w * G + g]);
        const float Ms = M == -INFINITY ? 0.f : M;
        float Lsum = 0.f, A = 0.f;
#pragma unroll
        for (int w = 0; w < MW; ++w) {
            const float f = fast_exp2(sm_m[w * G + g] - Ms);
            Lsum += sm_l[w * G + g] * f;
            A += sm_acc[(w * G + g) * D + j] * f;
        }
        const int h = kvh * G + g;
        if (SPLIT) {
            const int64_t pi = ((int64_t)s * num_q_heads + h) * max_partitions + part;
            if (j == 0) {
                ws_max[pi] = any_bad ? NAN : M;
                ws_sum[pi] = Lsum;
            }
            ws_acc[pi * D + j] = A;
        } else {
            float ov = Lsum > 0.f ? A / Lsum : 0.f;
            if (any_bad) ov = NAN;
            store_out<T>(out, ((int64_t)s * num_q_heads + h) * D + j, ov);
        }
    }
}

template <typename T, int D, int G, bool NT>
int launch_t(const DecodeArgs &a) {
    const int log2b = __builtin_ctz(a.block_size);
    const bool split = a.partition_size > 0;
    const unsigned grid = (unsigned)a.num_seqs * a.num_kv_heads * (split ? a.max_partitions : 1);
    hipStream_t st = (hipStream_t)a.stream;
    if (split) {
        hipLaunchKernelGGL((decode_mfma_kernel<T, D, G, true, NT>), dim3(grid), dim3(MW * 64), 0, st,
                           a.out, (const uint8_t *)a.query, (const uint8_t *)a.key_cache,
                           (const uint8_t *)a.value_cache, a.block_tables, a.context_lens, a.ws_max,
                           a.ws_sum, a.ws_acc, a.max_blocks_per_seq, a.num_seqs, a.num_kv_heads,
                           log2b, a.num_blocks, a.partition_size, a.max_partitions, a.scale_log2);
        const int rc = check_launch("decode_mfma (partitions)");
        if (rc != PA_OK) return rc;
        return launch_lse_merge(a);
    }
    hipLaunchKernelGGL((decode_mfma_kernel<T, D, G, false, NT>), dim3(grid), dim3(MW * 64), 0, st,
                       a.out, (const uint8_t *)a.query, (const uint8_t *)a.key_cache,
                       (const uint8_t *)a.value_cache, a.block_tables, a.context_lens, nullptr,
                       nullptr, nullptr, a.max_blocks_per_seq, a.num_seqs, a.num_kv_heads, log2b,
                       a.num_blocks, 0, 1, a.scale_log2);
    return check_launch("decode_mfma");
}

template <typename T, int D, int G>
int by_cache(const DecodeArgs &a) {
    return a.cached_kv ? launch_t<T, D, G, false>(a) : launch_t<T, D, G, true>(a);
}

template <typename T, int D>
int by_group(const DecodeArgs &a) {
    switch (a.num_q_heads / a.num_kv_heads) {
        case 2: return by_cache<T, D, 2>(a);
        case 4: return by_cache<T, D, 4>(a);
        case 8: return by_cache<T, D, 8>(a);
        case 16: return by_cache<T, D, 16>(a);
    }
    return fail(PA_ERR_UNSUPPORTED, "MFMA group %d", a.num_q_heads / a.num_kv_heads);
}

template <typename T>
int by_dim(const DecodeArgs &a) {
    if (a.head_dim == 64) return by_group<T, 64>(a);
    if (a.head_dim == 128) return by_group<T, 128>(a);
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d", a.head_dim);
}

}  // namespace mfma

}  // namespace pa
