#pragma once
// Several causal query tokens per sequence over the paged cache, on the matrix cores
// (gfx950 MFMA): the chunked-prefill / prefix-cache-hit case ("PagedAttention 深度解析"
// (5ulink.com) §六 item 5) of the same attention through the block table ("PagedAttention"
// concept report (compassingai.com) §5 and §8).  Sequence s has n_s query tokens, the
// last n_s positions of its context (their K/V already cached); the token at position
// p attends to the cached tokens t <= p.
//
// A workgroup takes one (KV head, sequence, tile of 16 query rows), a row being one
// (query token, query head of the group) pair: 16 / g tokens times the g heads that
// share the KV head.  Its four waves split the keys the tile can see ([0, last row's
// position]) in 32-key chunks and merge through LDS at the end.  Per chunk and wave:
//
//   S^T[t][r]  = sum_d K[t][d] Q[r][d]          A = K rows (16 keys x 32 d), B = Q^T
//   O^T[d][r] += sum_t V[t][d] P[r][t]          A = V^T (16 d x 32 keys),   B = P^T
//
// on v_mfma_f32_16x16x32_{f16,bf16}, with the operand layouts and the staging of the
// grouped-query decode kernel (K straight from HBM into registers, V through per-wave
// double-buffered LDS by direct 16-byte LDS loads, the score fragment reused as the P^T
// operand by matching the k order); the causal mask compares each key's position with
// its row's.  Softmax is fp32 online in the exp2 domain; P enters the second product
// rounded to the storage type and the normaliser sums the rounded weights.
//
// Tiles are numbered row tile fastest, then sequence, then KV head, and spread over the
// XCDs in contiguous ranges, so the tiles that read the same sequence's blocks share an
// XCD's L2 (K and V are read with cacheable loads: every row tile of a sequence reads
// them).
#include <hip/hip_runtime.h>

#include "decode_mfma.h"
#include "internal.h"
#include "kernel_common.h"

namespace pa {
namespace mq {

using mfma::Mma;
using mfma::f32x4;
constexpr int MW = 4;   // waves per workgroup
constexpr int CT = 32;  // keys per chunk: two 16-key tiles

template <typename T, int D, int G>
__global__ __launch_bounds__(MW * 64) void multi_query_kernel(
    void *__restrict__ out, const uint8_t *__restrict__ query, const uint8_t *__restrict__ key_cache,
    const uint8_t *__restrict__ value_cache, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ context_lens, const int32_t *__restrict__ query_start,
    int max_blocks_per_seq, int num_seqs, int num_kv_heads, int num_query_tokens, int tiles_per_seq,
    int max_query_len, int log2_block, int num_blocks, float scale_log2) {
    constexpr int ROW = D * 2;            // bytes per token row
    constexpr int NKK = D / 32;           // 32-wide d steps of the score product
    constexpr int NN = D / 16;            // 16-row d fragments of the output
    constexpr int VL = 16 * ROW / 1024;   // 1 KiB wave loads per 16-key V tile
    constexpr int RPK = 1024 / ROW;       // token rows per KiB
    constexpr int KSTR = 1024 + 32;       // LDS stride of one KiB group (padded)
    constexpr int STAGE = 2 * VL * KSTR;  // LDS bytes of one chunk's V
    constexpr int WAVE_LDS = 2 * STAGE;   // double-buffered

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15;  // query row of the tile / key row within a 16-key tile
    const int q = lane >> 4;  // k group

    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int tile = L % tiles_per_seq;
    const int rest = L / tiles_per_seq;
    const int s = rest % num_seqs;
    const int kvh = rest / num_seqs;
    const int num_q_heads = num_kv_heads * G;

    const int ctx = context_lens[s];
    const int q0 = query_start[s];
    const int nq = query_start[s + 1] - q0;
    const int rows = nq * G;  // flattened (token, head) rows of the sequence
    if (nq <= 0 || 16 * tile >= rows) return;
    // invalid lengths: this tile's rows become NaN (no key is read)
    const bool bad_len = ctx < 0 || nq > ctx || nq > max_query_len;

    // this lane's row: token i, head g; its position, and the tile's last position
    const int r = 16 * tile + n;
    const bool row_ok = r < rows;
    const int ti = (row_ok ? r : rows - 1) / G;
    const int g = (row_ok ? r : rows - 1) % G;
    const int pos = ctx - nq + ti;  // sees keys t <= pos
    const int last_row = min(rows, 16 * tile + 16) - 1;
    const int end = bad_len ? 0 : ctx - nq + last_row / G + 1;  // keys the tile reads
    const int64_t out_row = (int64_t)q0 + ti;  // row of query / out
    const bool io_ok = row_ok && out_row >= 0 && out_row < num_query_tokens;

    __shared__ __attribute__((aligned(16))) uint8_t lds[MW * WAVE_LDS];
    static_assert((2 * MW * 16 + MW * 16 * D) * 4 <= MW * WAVE_LDS, "merge area must fit the staging area");
    uint8_t *wave_lds = lds + wave * WAVE_LDS;

    const int block_size = 1 << log2_block;
    const int32_t *table = block_tables + (int64_t)s * max_blocks_per_seq;
    const int64_t head_off = (int64_t)kvh * block_size * ROW;
    const int64_t block_bytes = (int64_t)num_kv_heads * block_size * ROW;

    // Q^T operand: lane holds Q[row n][32 kk + 8 q .. +8]; rows past the sequence are zero
    u32x4 qb[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        qb[kk] = u32x4{0, 0, 0, 0};
        if (io_ok)
            qb[kk] = *(const u32x4 *)(query + ((out_row * num_q_heads + kvh * G + g) * D + 32 * kk + 8 * q) * 2);
    }

    float m = -INFINITY;  // running max of row n (same in the 4 lanes of a column)
    float lsum = 0.f;     // this lane's share of the normaliser
    f32x4 o[NN];
#pragma unroll
    for (int i = 0; i < NN; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    bool bad = bad_len;

    const int nchunks = (end + CT - 1) / CT;

    // Byte offset of the first row of 16-key tile `tt` of chunk c, or -1 (past `end` or
    // a bad entry: the loads then read block 0's first rows, masked like any key past
    // `end`, so no branch surrounds a load).
    auto tile_base = [&](int c, int tt) -> int64_t {
        const int tok = c * CT + 16 * tt;
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
                b.k[tt][kk] = *(const u32x4 *)(key_cache + base + n * ROW + (32 * kk + 8 * q) * 2);
        }
    };
    auto v_at = [&](const uint8_t *stage, int rr, int col) -> const uint8_t * {
        return stage + (rr / RPK) * KSTR + (rr % RPK) * ROW + col;
    };
    auto consume = [&](const Chunk &b, int c, int st) {
        const uint8_t *stage = wave_lds + st * STAGE;
        const int tok0 = c * CT;
        // scores S^T: lane holds keys tok0 + 16 tt + 4 q + i of row n, masked causally
        float sc[2][4];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) acc = Mma<T>::run(b.k[tt][kk], qb[kk], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = tok0 + 16 * tt + 4 * q + i;
                sc[tt][i] = (key <= pos && key < end) ? acc[i] * scale_log2 : -INFINITY;
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
        // P^T operand: k slot j < 4 -> key 4q + j (tile 0), j >= 4 -> key 16 + 4q + j - 4
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
        // the chunk's V rows have landed in LDS (issued before its K loads, which the
        // score product has waited for)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (tok0 + CT > end) {
            // keys past `end` as zeros: 0 * NaN would poison the product
            for (int rr = max(0, end - tok0); rr < CT; ++rr)
                for (int col = lane * 4; col < ROW; col += 256)
                    *(uint32_t *)v_at(stage, rr, col) = 0u;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
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
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    {
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

    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);

    // merge the waves through LDS (the staging area is free now)
    __syncthreads();
    float *sm_m = (float *)lds;     // [MW][16]
    float *sm_l = sm_m + MW * 16;   // [MW][16]
    float *sm_acc = sm_l + MW * 16; // [MW][16][D]
    __shared__ int sm_bad;
    if (threadIdx.x == 0) sm_bad = 0;
    __syncthreads();
    if (bad) sm_bad = 1;
    if (q == 0) {
        sm_m[wave * 16 + n] = m;
        sm_l[wave * 16 + n] = lsum;
    }
#pragma unroll
    for (int nn = 0; nn < NN; ++nn)
#pragma unroll
        for (int i = 0; i < 4; ++i) sm_acc[(wave * 16 + n) * D + 16 * nn + 4 * q + i] = o[nn][i];
    __syncthreads();
    const bool any_bad = sm_bad != 0;
    for (int t = threadIdx.x; t < 16 * D; t += MW * 64) {
        const int rn = t / D;
        const int j = t - rn * D;
        const int rr = 16 * tile + rn;
        if (rr >= rows) continue;
        const int64_t orow = (int64_t)q0 + rr / G;
        if (orow < 0 || orow >= num_query_tokens) continue;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < MW; ++w) M = fmaxf(M, sm_m[w * 16 + rn]);
        const float Ms = M == -INFINITY ? 0.f : M;
        float Lsum = 0.f, A = 0.f;
#pragma unroll
        for (int w = 0; w < MW; ++w) {
            const float f = fast_exp2(sm_m[w * 16 + rn] - Ms);
            Lsum += sm_l[w * 16 + rn] * f;
            A += sm_acc[(w * 16 + rn) * D + j] * f;
        }
        float ov = Lsum > 0.f ? A / Lsum : 0.f;
        if (any_bad) ov = NAN;
        store_out<T>(out, (orow * num_q_heads + kvh * G + rr % G) * D + j, ov);
    }
}

template <typename T, int D, int G>
int launch_t(const DecodeArgs &a) {
    const int tiles = (a.max_query_len * G + 15) / 16;
    const int64_t grid = (int64_t)a.num_kv_heads * a.num_seqs * tiles;
    if (grid > 0x7fffffff) return fail(PA_ERR_UNSUPPORTED, "grid of %lld workgroups", (long long)grid);
    hipLaunchKernelGGL((multi_query_kernel<T, D, G>), dim3((unsigned)grid), dim3(MW * 64), 0,
                       (hipStream_t)a.stream, a.out, (const uint8_t *)a.query, (const uint8_t *)a.key_cache,
                       (const uint8_t *)a.value_cache, a.block_tables, a.context_lens, a.query_start,
                       a.max_blocks_per_seq, a.num_seqs, a.num_kv_heads, a.num_query_tokens, tiles,
                       a.max_query_len, __builtin_ctz(a.block_size), a.num_blocks, a.scale_log2);
    return check_launch("multi_query");
}

template <typename T, int D>
int by_group(const DecodeArgs &a) {
    switch (a.num_q_heads / a.num_kv_heads) {
        case 1: return launch_t<T, D, 1>(a);
        case 2: return launch_t<T, D, 2>(a);
        case 4: return launch_t<T, D, 4>(a);
        case 8: return launch_t<T, D, 8>(a);
        case 16: return launch_t<T, D, 16>(a);
    }
    return fail(PA_ERR_UNSUPPORTED, "group %d", a.num_q_heads / a.num_kv_heads);
}

template <typename T>
int by_dim(const DecodeArgs &a) {
    if (a.head_dim == 64) return by_group<T, 64>(a);
    if (a.head_dim == 128) return by_group<T, 128>(a);
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d", a.head_dim);
}

}  // namespace mq
}  // namespace pa
