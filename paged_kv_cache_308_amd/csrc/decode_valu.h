#pragma once
// Paged decode attention on the vector ALUs (gfx950), one pass or split by context
// partition, and the log-sum-exp merge of partition partials.
//
// What is computed ("PagedAttention" concept report (compassingai.com) §8): for each
// sequence and query head, the query's dot product with every cached key, a softmax
// over those scores, and the softmax-weighted sum of the cached values; the kernel
// walks the block table (outer loop over blocks, inner loop over the block's
// tokens) and reads each token at physical block base + in-block offset (§5).
//
// Mapping to CDNA4:
//  * one workgroup of NW wave64s per (sequence, KV head, context partition);
//  * a "chunk" is C consecutive tokens of one KV head inside one physical block.
//    Each lane loads 16 contiguous bytes per token row, so a wave load covers
//    TPW = 64 / LPT whole token rows (LPT = lanes per row = d*esz/16) and every
//    load instruction reads 1 KiB of consecutive memory;
//  * the LPT lanes of a row hold one token: its q.k partial sums are combined
//    with DPP row operations inside the row; each lane keeps the fp32 running
//    max / sum / weighted value sum of the tokens of its row (online softmax) for
//    its own LPT-th of the head dimension, so no value ever crosses lanes in the
//    token loop and nothing is staged in LDS;
//  * chunks of a wave are double-buffered in registers (the next chunk's K and V
//    loads are in flight while the current one is reduced);
//  * at the end the rows of a wave, then the waves of the workgroup (through LDS),
//    are merged with log-sum-exp weights;
//  * workgroup ids are remapped so that each XCD runs a contiguous range of work
//    items (partition fastest, then sequence, then KV head): the XCDs get equal
//    shares, and consecutive sequences of one KV head share an XCD's L2 when their
//    tables point at the same blocks (shared prefixes).
#include <hip/hip_runtime.h>

#include "internal.h"
#include "kernel_common.h"

namespace pa {
namespace valu {

#ifndef PA_VALU_WAVES
#define PA_VALU_WAVES 8
#endif
#ifndef PA_VALU_LOADS
#define PA_VALU_LOADS 4
#endif
constexpr int NW = PA_VALU_WAVES;  // waves per workgroup
constexpr int NL = PA_VALU_LOADS;  // wave loads (of K and of V) per chunk

template <typename T, int D, int G, bool SPLIT, bool NT>
__global__ __launch_bounds__(NW * 64) void decode_valu_kernel(
    void *__restrict__ out, const uint8_t *__restrict__ query, const uint8_t *__restrict__ key_cache,
    const uint8_t *__restrict__ value_cache, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ context_lens, float *__restrict__ ws_max, float *__restrict__ ws_sum,
    float *__restrict__ ws_acc, int max_blocks_per_seq, int num_seqs, int num_kv_heads,
    int log2_block, int num_blocks, int partition_size, int max_partitions, float scale_log2) {
    constexpr int EB = T::bytes;
    constexpr int EPL = 16 / EB;            // elements per lane per row
    constexpr int LPT = D * EB / 16;        // lanes per token row
    constexpr int TPW = 64 / LPT;           // token rows per wave load
    constexpr int C = NL * TPW;             // tokens per chunk
    constexpr int ROW_BYTES = D * EB;

    const int lane = threadIdx.x & 63;
    // wave-uniform: keeps table lookups on the scalar unit and branches scalar
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row = lane / LPT;
    const int col = lane % LPT;

    // work item order: partition fastest, then sequence, then KV head, so every XCD's
    // contiguous range holds whole sequences (balanced) and a head's sequences are
    // neighbours (shared-prefix siblings land on one XCD)
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
        if (ctx < 0 || start >= ctx) return;  // nothing here (the merge handles bad lengths)
        end = min(ctx, start + partition_size);
    }

    const int block_size = 1 << log2_block;
    const int32_t *table = block_tables + (int64_t)s * max_blocks_per_seq;
    const int64_t head_off = (int64_t)kvh * block_size * ROW_BYTES;
    const int64_t block_bytes = (int64_t)num_kv_heads * block_size * ROW_BYTES;

    // this lane's slice of every query head of the group
    u32x4 qv[G];
#pragma unroll
    for (int g = 0; g < G; ++g)
        qv[g] = *(const u32x4 *)(query + ((int64_t)(s * num_q_heads + kvh * G + g) * D + col * EPL) * EB);

    float m[G], l[G], acc[G][EPL];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
    }
    bool bad = ctx < 0;

    const int ntok = ctx < 0 ? 0 : end - start;
    const int nfull = ntok / C;
    const bool has_tail = (ntok % C) != 0;

    // Byte offset of the first row of wave load i of chunk c (uniform), or -1 when the
    // load lies past `end` or its table entry is outside the pool.  The last block
    // looked up is remembered: the loads of a chunk usually share one block.
    // A load with no data (past `end` in the tail chunk, or through a bad entry) reads
    // block 0's first rows instead (always inside the pool; masked or discarded
    // later): no branch around a load, because one makes the compiler wait for every
    // outstanding load.
    int cached_lb = -1;
    int64_t cached_base = -1;
    auto load_offset = [&](int c, int i) -> int64_t {
        const int tok = start + c * C + i * TPW;
        if (tok >= end) return -1;
        const int lb = tok >> log2_block;
        if (lb != cached_lb) {
            cached_lb = lb;
            cached_base = -1;
            if (lb >= max_blocks_per_seq) {  // context longer than the table row
                bad = true;
            } else {
                const int32_t pb = table[lb];
                if (pb < 0 || pb >= num_blocks)
                    bad = true;
                else
                    cached_base = (int64_t)pb * block_bytes + head_off;
            }
        }
        if (cached_base < 0) return -1;
        return cached_base + (int64_t)(tok & (block_size - 1)) * ROW_BYTES;
    };

    struct Chunk {
        u32x4 k[NL], v[NL];
    };
    auto issue = [&](Chunk &b, int c) {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            int64_t off = load_offset(c, i);
            off = off < 0 ? 0 : off;
            b.k[i] = kv_load<NT>((const u32x4 *)(key_cache + off + lane * 16));
            b.v[i] = kv_load<NT>((const u32x4 *)(value_cache + off + lane * 16));
        }
    };
    auto consume = [&](const Chunk &b, int c, bool tail) {
        const int tok0 = start + c * C + row;
        float sc[G][NL];
        bool valid[NL];
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            valid[i] = !tail || (tok0 + i * TPW < end);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float dot = row_sum<LPT>(dot16<T>(qv[g], b.k[i]));
                sc[g][i] = valid[i] ? dot * scale_log2 : -INFINITY;
            }
        }
        float vf[NL][EPL];
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            u32x4 w = b.v[i];
            if (tail && !valid[i]) w = u32x4{0, 0, 0, 0};  // never multiply a slot past ctx
            to_f32<T>(w, vf[i]);
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float cm = sc[g][0];
#pragma unroll
            for (int i = 1; i < NL; ++i) cm = fmaxf(cm, sc[g][i]);
            const float mn = fmaxf(m[g], cm);
            const float ms = mn == -INFINITY ? 0.f : mn;
            const float alpha = fast_exp2(m[g] - ms);
            float p[NL], psum = 0.f;
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                p[i] = fast_exp2(sc[g][i] - ms);
                psum += p[i];
            }
            l[g] = l[g] * alpha + psum;
            m[g] = mn;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                float a = acc[g][e] * alpha;
#pragma unroll
                for (int i = 0; i < NL; ++i) a = fmaf(p[i], vf[i][e], a);
                acc[g][e] = a;
            }
        }
    };

    // double-buffered walk over this wave's full chunks: wave, wave + NW, ...
    // This wave's full chunks are wave, wave + NW, ...  The steady-state loop always
    // has a next chunk to prefetch, so its loads are unconditional and the compiler
    // waits only for the chunk being reduced; the last one or two run after it.
    {
        const int mine = nfull > wave ? (nfull - wave + NW - 1) / NW : 0;
        Chunk A, Bf;
        if (mine > 0) {
            issue(A, wave);
            int j = 0;
            for (; j + 2 < mine; j += 2) {
                issue(Bf, wave + (j + 1) * NW);
                consume(A, wave + j * NW, false);
                issue(A, wave + (j + 2) * NW);
                consume(Bf, wave + (j + 1) * NW, false);
            }
            if (j + 1 < mine) {
                issue(Bf, wave + (j + 1) * NW);
                consume(A, wave + j * NW, false);
                consume(Bf, wave + (j + 1) * NW, false);
            } else {
                consume(A, wave + j * NW, false);
            }
        }
        if (has_tail && (nfull % NW) == wave) {
            issue(A, nfull);
            consume(A, nfull, true);
        }
    }

    // merge the rows of this wave (lanes col, col + LPT, ... hold the same dims)
#pragma unroll
    for (int step = LPT; step < 64; step <<= 1) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float mo = __shfl_xor(m[g], step);
            const float lo = __shfl_xor(l[g], step);
            const float mn = fmaxf(m[g], mo);
            const float ms = mn == -INFINITY ? 0.f : mn;
            const float a = fast_exp2(m[g] - ms);
            const float bsc = fast_exp2(mo - ms);
            l[g] = l[g] * a + lo * bsc;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const float ao = __shfl_xor(acc[g][e], step);
                acc[g][e] = acc[g][e] * a + ao * bsc;
            }
            m[g] = mn;
        }
    }

    // merge the waves through LDS
    __shared__ float sm_m[NW][G], sm_l[NW][G], sm_acc[NW][G][D];
    __shared__ int sm_bad;
    if (threadIdx.x == 0) sm_bad = 0;
    __syncthreads();
    if (bad) sm_bad = 1;
    if (row == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) sm_acc[wave][g][col * EPL + e] = acc[g][e];
            if (col == 0) {
                sm_m[wave][g] = m[g];
                sm_l[wave][g] = l[g];
            }
        }
    }
    __syncthreads();
    const bool any_bad = sm_bad != 0;
    for (int t = threadIdx.x; t < G * D; t += NW * 64) {
        const int g = t / D;
        const int j = t - g * D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][g]);
        const float Ms = M == -INFINITY ? 0.f : M;
        float Lsum = 0.f, A = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float f = fast_exp2(sm_m[w][g] - Ms);
            Lsum += sm_l[w][g] * f;
            A += sm_acc[w][g][j] * f;
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
            float o = Lsum > 0.f ? A / Lsum : 0.f;
            if (any_bad) o = NAN;
            store_out<T>(out, ((int64_t)s * num_q_heads + h) * D + j, o);
        }
    }
}

// Log-sum-exp merge of the partition partials of one (sequence, query head):
//   M = max_p m_p,  L = sum_p l_p 2^(m_p - M),  out = sum_p 2^(m_p - M) acc_p / L.
template <typename T, int D>
__global__ __launch_bounds__(64) void lse_merge_kernel(
    void *__restrict__ out, const float *__restrict__ ws_max, const float *__restrict__ ws_sum,
    const float *__restrict__ ws_acc, const int32_t *__restrict__ context_lens, int num_q_heads,
    int partition_size, int max_partitions) {
    const int sh = blockIdx.x;  // s * H_q + h
    const int s = sh / num_q_heads;
    const int ctx = context_lens[s];
    const int64_t obase = (int64_t)sh * D;
    const int n = ctx <= 0 ? 0 : (ctx + partition_size - 1) / partition_size;
    if (ctx < 0 || n > max_partitions) {
        for (int j = threadIdx.x; j < D; j += 64) store_out<T>(out, obase + j, NAN);
        return;
    }
    const float *mp = ws_max + (int64_t)sh * max_partitions;
    const float *lp = ws_sum + (int64_t)sh * max_partitions;
    float M = -INFINITY;
    bool bad = false;
    for (int p = 0; p < n; ++p) {
        const float x = mp[p];
        bad |= x != x;
        M = fmaxf(M, x);
    }
    const float Ms = M == -INFINITY ? 0.f : M;
    float Lsum = 0.f;
    for (int p = 0; p < n; ++p) Lsum += lp[p] * fast_exp2(mp[p] - Ms);
    for (int j = threadIdx.x; j < D; j += 64) {
        float A = 0.f;
        for (int p = 0; p < n; ++p)
            A += fast_exp2(mp[p] - Ms) * ws_acc[((int64_t)sh * max_partitions + p) * D + j];
        float o = Lsum > 0.f ? A / Lsum : 0.f;
        if (bad) o = NAN;
        store_out<T>(out, obase + j, o);
    }
}

template <typename T, int D, int G, bool NT>
int launch_t(const DecodeArgs &a) {
    const int log2b = __builtin_ctz(a.block_size);
    const bool split = a.partition_size > 0;
    const unsigned grid = (unsigned)a.num_seqs * a.num_kv_heads * (split ? a.max_partitions : 1);
    hipStream_t st = (hipStream_t)a.stream;
    if (split) {
        hipLaunchKernelGGL((decode_valu_kernel<T, D, G, true, NT>), dim3(grid), dim3(NW * 64), 0, st,
                           a.out, (const uint8_t *)a.query, (const uint8_t *)a.key_cache,
                           (const uint8_t *)a.value_cache, a.block_tables, a.context_lens, a.ws_max,
                           a.ws_sum, a.ws_acc, a.max_blocks_per_seq, a.num_seqs, a.num_kv_heads,
                           log2b, a.num_blocks, a.partition_size, a.max_partitions, a.scale_log2);
        const int rc = check_launch("decode_valu (partitions)");
        if (rc != PA_OK) return rc;
        return launch_lse_merge(a);
    }
    hipLaunchKernelGGL((decode_valu_kernel<T, D, G, false, NT>), dim3(grid), dim3(NW * 64), 0, st,
                       a.out, (const uint8_t *)a.query, (const uint8_t *)a.key_cache,
                       (const uint8_t *)a.value_cache, a.block_tables, a.context_lens, nullptr,
                       nullptr, nullptr, a.max_blocks_per_seq, a.num_seqs, a.num_kv_heads, log2b,
                       a.num_blocks, 0, 1, a.scale_log2);
    return check_launch("decode_valu");
}

template <typename T, int D, int G>
int by_cache(const DecodeArgs &a) {
    return a.cached_kv ? launch_t<T, D, G, false>(a) : launch_t<T, D, G, true>(a);
}

template <typename T, int D>
int by_group(const DecodeArgs &a) {
    switch (a.num_q_heads / a.num_kv_heads) {
        case 1: return by_cache<T, D, 1>(a);
        case 2: return by_cache<T, D, 2>(a);
        case 4: return by_cache<T, D, 4>(a);
        case 8: return by_cache<T, D, 8>(a);
        case 16: return by_cache<T, D, 16>(a);
    }
    return fail(PA_ERR_UNSUPPORTED, "group %d", a.num_q_heads / a.num_kv_heads);
}

template <typename T>
int by_dim(const DecodeArgs &a) {
    if (a.head_dim == 64) return by_group<T, 64>(a);
    if (a.head_dim == 128) return by_group<T, 128>(a);
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d", a.head_dim);
}

template <typename T, int D>
int merge_t(const DecodeArgs &a) {
    hipLaunchKernelGGL((lse_merge_kernel<T, D>), dim3(a.num_seqs * a.num_q_heads), dim3(64), 0,
                       (hipStream_t)a.stream, a.out, a.ws_max, a.ws_sum, a.ws_acc, a.context_lens,
                       a.num_q_heads, a.partition_size, a.max_partitions);
    return check_launch("lse_merge");
}

template <typename T>
int merge_dim(const DecodeArgs &a) {
    return a.head_dim == 64 ? merge_t<T, 64>(a) : merge_t<T, 128>(a);
}

}  // namespace valu

}  // namespace pa
