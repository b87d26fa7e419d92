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
//  * V must be read transposed (8 tokens of one d per lane): each wave loads its V rows
//    into registers two chunks ahead (16-byte loads, 1 KiB per wave load), stores them
//    into its own double-buffered LDS region with 32 bytes of padding after each KiB,
//    and reads the V^T operand with gfx950's LDS transpose read ds_read_b64_tr_b16 (two
//    per operand).  (Direct HBM -> LDS loads would save the stores, but while one is in
//    flight the compiler turns every wait for a register load into a wait for all
//    loads, which limits the pipeline to one chunk ahead.)  The tokens of a 16-token
//    tile are taken in the order tile_row gives (the K operand's rows are loaded in that
//    order, which permutes rows within one load instruction), so the four rows one
//    16-lane group reads together lie in different padded KiB groups: different banks.
// Softmax runs in fp32 (online, exp2 domain).  P enters the second product rounded to
// the storage type; the normaliser sums the rounded weights, so numerator and
// denominator use the same weights.  Accumulation is fp32.
//
// Work decomposition, XCD-aware numbering and the partition partials are those of the
// vector kernel, so the same log-sum-exp merge kernel finishes a partitioned run.
#include <hip/hip_runtime.h>

#include "balanced.h"
#include "group_plan.h"
#include "internal.h"
#include "kernel_common.h"

namespace pa {
namespace mfma {

// Cost of starting an item in the matrix-core balanced split, in chunks: the list gives
// every item this many units before its chunks, so a worker whose range starts an item
// takes that many chunks fewer (an item start drains the workgroup's load pipeline, merges
// its waves and refills; about three chunks' time at 2 workgroups per CU).
#ifndef PA_BAL_ITEM_UNITS
#define PA_BAL_ITEM_UNITS 3
#endif
#ifndef PA_MFMA_WAVES
#define PA_MFMA_WAVES 4
#endif
#ifndef PA_MFMA_BAL_PER_CU
#define PA_MFMA_BAL_PER_CU 0  // balanced split: workgroups per CU (0: as many as fit)
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

// Tile geometry of head dimension D (16-bit elements).
template <int D>
struct Geom {
    static constexpr int ROW = D * 2;            // bytes per token row
    static constexpr int NKK = D / 32;           // 32-wide d steps of the score product
    static constexpr int NN = D / 16;            // 16-row d fragments of the output
    static constexpr int VL = 16 * ROW / 1024;   // 1 KiB wave loads per 16-token V tile
    static constexpr int RPK = 1024 / ROW;       // token rows per KiB
    static constexpr int KSTR = 1024 + 32;       // LDS stride of one KiB group (padded)
    static constexpr int STAGE = 2 * VL * KSTR;  // LDS bytes of one chunk's V
    static constexpr int WAVE_LDS = 2 * STAGE;   // double-buffered
};

// LDS address of V[row r of the chunk][byte col] in a stage
template <int D>
__device__ inline uint8_t *v_at(uint8_t *stage, int r, int col) {
    using Gm = Geom<D>;
    return stage + (r / Gm::RPK) * Gm::KSTR + (r % Gm::RPK) * Gm::ROW + col;
}

// Token (row of a 16-token tile) in k slot m of lane group a (a, m in 0..3) of the score
// and value products.  S^T row 4a + m holds this token, and the transpose read of lane
// group a returns V rows tile_row(a, 0..3).  Chosen so that the four rows a group reads
// lie at different bank offsets of the LDS stage (KiB groups padded by 32 bytes):
// d = 128 (4 rows per KiB): rows a, a + 4, a + 8, a + 12, one per KiB group;
// d = 64 (8 rows per KiB): rows 2a, 2a + 1, 2a + 8, 2a + 9 (two groups, odd and even rows
// half a KiB-period apart).
template <int D>
__device__ inline int tile_row(int a, int m) {
    static_assert(D == 64 || D == 128, "head dim");
    if constexpr (D == 128)
        return 4 * m + a;
    else
        return 8 * (m >> 1) + (m & 1) + 2 * a;
}

// One chunk of CT tokens starting at position tok0 (rows at or past `end` masked) folded
// into a wave's online-softmax state: m (running max of head n), lsum (this lane's share
// of the normaliser) and o (O^T fragments).  k: the chunk's K operands; its V rows are
// in the LDS stage, read as V^T operands fragment by fragment.
// ds_read_b64_tr_b16 (lane mapping checked on gfx950): within each 16-lane group, lane j
// receives element j % 4 of the 8-byte reads of lanes 4k + j / 4, k = 0..3.  Lane (n, q)
// reads 8 bytes of row tile_row(q, n / 4) at d = 16 nn + 4 (n % 4), so it receives
// V[tile_row(q, k)][16 nn + n] for k = 0..3: tile 0's k slots; the same read 16 rows
// further gives tile 1's.  P^T operand: k slot j < 4 -> token tile_row(q, j) (tile 0),
// j >= 4 -> token 16 + tile_row(q, j - 4) (tile 1).
template <typename T, int D>
__device__ __forceinline__ void consume_chunk(const u32x4 (&k)[2][Geom<D>::NKK], const u32x4 (&qb)[Geom<D>::NKK],
                                                  uint8_t *stage, int tok0, int end, float scale_log2, int n, int q,
                                                  float &m, float &lsum, f32x4 (&o)[Geom<D>::NN]) {
    using Gm = Geom<D>;
    const bool tail = tok0 + CT > end;
    float sc[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < Gm::NKK; ++kk) acc = Mma<T>::run(k[tt][kk], qb[kk], acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool ok = !tail || (tok0 + 16 * tt + tile_row<D>(q, i) < end);
            sc[tt][i] = ok ? acc[i] * scale_log2 : -INFINITY;
        }
    }
    float cm = sc[0][0];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) cm = fmaxf(cm, sc[tt][i]);
    cm = max_over_column(cm);
    const float mn = fmaxf(m, cm);
    const float ms = mn == -INFINITY ? 0.f : mn;
    const float alpha = fast_exp2(m - ms);
    m = mn;
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
    for (int nn = 0; nn < Gm::NN; ++nn) o[nn] *= alpha;
    // rows past `end` as zeros (0 * NaN would poison the product); word w of an operand
    // holds k slots 2w (low half) and 2w + 1
    u32x4 keep = u32x4{~0u, ~0u, ~0u, ~0u};
    if (tail) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int t0 = (w < 2 ? 0 : 16) + tile_row<D>(q, (2 * w) & 3);
            const int t1 = (w < 2 ? 0 : 16) + tile_row<D>(q, (2 * w + 1) & 3);
            keep[w] = (tok0 + t0 < end ? 0x0000ffffu : 0u) | (tok0 + t1 < end ? 0xffff0000u : 0u);
        }
    }
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    const int vrow = tile_row<D>(q, n >> 2);
#pragma unroll
    for (int nn = 0; nn < Gm::NN; ++nn) {
        const int col = (16 * nn + 4 * (n & 3)) * 2;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4 *)v_at<D>(stage, vrow, col));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4 *)v_at<D>(stage, 16 + vrow, col));
        const uint2 lw = __builtin_bit_cast(uint2, lo), hw = __builtin_bit_cast(uint2, hi);
        const u32x4 va = u32x4{lw.x, lw.y, hw.x, hw.y} & keep;
        o[nn] = Mma<T>::run(va, pb, o[nn]);
    }
}

// Q^T operand of (sequence s, KV head kvh): lane holds Q[head n][32 kk + 8 q .. +8];
// heads past the group are zero
template <int D, int G>
__device__ __forceinline__ void load_q(u32x4 (&qb)[Geom<D>::NKK], const uint8_t *query, int s, int kvh,
                                       int num_q_heads, int n, int q) {
#pragma unroll
    for (int kk = 0; kk < Geom<D>::NKK; ++kk) {
        qb[kk] = u32x4{0, 0, 0, 0};
        if (n < G)
            qb[kk] = *(const u32x4 *)(query + ((int64_t)(s * num_q_heads + kvh * G + n) * D + 32 * kk + 8 * q) * 2);
    }
}

// Q^T operand with one query row per member of a group of consecutive sequences (one
// query head per KV head): row n, when bit n of `rows` is set, is the query of head kvh
// of sequence s + n; other rows are zero
template <int D>
__device__ __forceinline__ void load_q_rows(u32x4 (&qb)[Geom<D>::NKK], const uint8_t *query, int s, int kvh,
                                            int num_q_heads, uint32_t rows, int n, int q) {
#pragma unroll
    for (int kk = 0; kk < Geom<D>::NKK; ++kk) {
        qb[kk] = u32x4{0, 0, 0, 0};
        if ((rows >> n) & 1u)
            qb[kk] = *(const u32x4 *)(query + ((int64_t)((s + n) * num_q_heads + kvh) * D + 32 * kk + 8 * q) * 2);
    }
}

// Per-wave online-softmax state of one range: m (running max of head n, same in the 4
// lanes of a column), lsum (this lane's share of the normaliser), o (O^T fragments).
template <int D>
struct WaveState {
    float m, lsum;
    f32x4 o[Geom<D>::NN];
    bool bad;
};

// The workgroup's MW waves over tokens [start, end) of (sequence s, KV head kvh):
// wave w takes the CT-token chunks w, w + MW, ... of the range through a pipeline: K
// operands loaded one chunk ahead into registers, V rows two chunks ahead into registers
// and then into the wave's two LDS stages.
//
// Newest token given (new_k non-null; the range ends at the context's end): the chunks
// stop before position end - 1, and the wave that would take the next chunk then stores
// the given K/V row (new_k, new_v: D elements each) into the pools at that position's
// slot and folds it into its state from registers: the score by vector dot products
// over the 4 lanes of each head's column, the weight rounded to T as the matrix-core
// path rounds it.  A wave whose 16-row tile holds that slot treats the row as past the
// end (score -inf, V operand zeroed), whichever value it read.
template <typename T, int D, int G, bool NT>
__device__ __forceinline__ void attend_range(WaveState<D> &st, uint8_t *wave_lds, const uint8_t *query,
                                             const uint8_t *key_cache, const uint8_t *value_cache,
                                             const int32_t *table, int max_blocks_per_seq, int s, int kvh,
                                             int num_kv_heads, int log2_block, int num_blocks, int start,
                                             int end, float scale_log2, int wave, int lane,
                                             const uint8_t *new_k = nullptr, const uint8_t *new_v = nullptr,
                                             uint8_t *key_out = nullptr, uint8_t *value_out = nullptr,
                                             uint32_t group_rows = 0) {
    using Gm = Geom<D>;
    constexpr int ROW = Gm::ROW;
    constexpr int NKK = Gm::NKK;
    const int n = lane & 15;  // head column / token row within a tile
    const int q = lane >> 4;  // k group
    const int num_q_heads = num_kv_heads * G;
    const int block_size = 1 << log2_block;
    const int64_t head_off = (int64_t)kvh * block_size * ROW;
    const int64_t block_bytes = (int64_t)num_kv_heads * block_size * ROW;

    u32x4 qb[NKK];
    if (group_rows)  // one query row per sequence of a group (shared-prefix pass)
        load_q_rows<D>(qb, query, s, kvh, num_kv_heads, group_rows, n, q);
    else
        load_q<D, G>(qb, query, s, kvh, num_q_heads, n, q);

    st.m = -INFINITY;
    st.lsum = 0.f;
#pragma unroll
    for (int i = 0; i < Gm::NN; ++i) st.o[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    const bool append = new_k != nullptr && end > start;
    const int tnew = end - 1;  // position of the newest token when appending
    if (append) end = tnew;
    const int ntok = end > start ? end - start : 0;
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
            st.bad = true;
            return -1;
        }
        const int32_t pb = table[lb];
        if (pb < 0 || pb >= num_blocks) {
            st.bad = true;
            return -1;
        }
        return (int64_t)pb * block_bytes + head_off + (int64_t)(tok & (block_size - 1)) * ROW;
    };
    struct Chunk {
        u32x4 k[2][NKK];
    };
    auto bases = [&](int c, int64_t (&base)[2]) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            base[tt] = tile_base(c, tt);
            base[tt] = base[tt] < 0 ? 0 : base[tt];
        }
    };
    // V rows through registers (ordinary loads, like K): with every load of one kind the
    // compiler's waits count exactly, so V can run two chunks ahead.
    struct VSet {
        u32x4 v[2 * Gm::VL];
    };
    auto issue_vr = [&](VSet &b, int c) {
        int64_t base[2];
        bases(c, base);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int i = 0; i < Gm::VL; ++i)
                b.v[tt * Gm::VL + i] = kv_load<NT>((const u32x4 *)(value_cache + base[tt] + i * 1024 + lane * 16));
    };
    // into the wave's stage, 1 KiB groups padded by 32 B (the layout tile_row's bank spread
    // assumes); the stage's previous chunk was read two chunks ago (a wave's LDS operations
    // run in order)
    auto stage_vr = [&](const VSet &b, int stage) {
        uint8_t *sp = wave_lds + stage * Gm::STAGE;
#pragma unroll
        for (int j = 0; j < 2 * Gm::VL; ++j) *(u32x4 *)(sp + j * Gm::KSTR + lane * 16) = b.v[j];
    };
    auto issue_kr = [&](Chunk &b, int c) {
        int64_t base[2];
        bases(c, base);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
                b.k[tt][kk] = kv_load<NT>((const u32x4 *)(key_cache + base[tt] + tile_row<D>(n >> 2, n & 3) * ROW +
                                                          (32 * kk + 8 * q) * 2));
    };
    auto stage_at = [&](int stage) { return wave_lds + stage * Gm::STAGE; };
    auto consume_lds = [&](const Chunk &b, int c, int stage) {
        consume_chunk<T, D>(b.k, qb, stage_at(stage), start + c * CT, end, scale_log2, n, q, st.m, st.lsum, st.o);
    };

    const int mine = nchunks > wave ? (nchunks - wave + MW - 1) / MW : 0;
    auto cidx = [&](int i) { return wave + i * MW; };
    // This wave's chunks are c_i = wave + i MW, i < mine.  Chunk i's V rows are loaded two
    // chunks ahead into register set i % 2 and stored into stage i % 2 once the stage's
    // previous chunk has been read out; its K operands are loaded one chunk ahead into K
    // set i % 2; then the chunk is used (K from registers, V^T read from the stage).  The
    // loop starts with loads and ends with the next chunk's store, so the compiler's waits
    // for register loads fall inside an iteration, where it counts them exactly.  Loads in
    // the steady-state loop are unconditional (no branch around a load); the last one to
    // three chunks run after it; loads past the range read block 0's rows, never used.
    Chunk K0, K1;
    VSet V0, V1;
    if (mine > 0) {
        issue_vr(V0, cidx(0));
        issue_vr(V1, cidx(1));
        issue_kr(K0, cidx(0));
        stage_vr(V0, 0);
        int i = 0;
        for (; i + 3 < mine; i += 2) {
            issue_vr(V0, cidx(i + 2));
            issue_kr(K1, cidx(i + 1));
            consume_lds(K0, cidx(i), 0);
            stage_vr(V1, 1);
            issue_vr(V1, cidx(i + 3));
            issue_kr(K0, cidx(i + 2));
            consume_lds(K1, cidx(i + 1), 1);
            stage_vr(V0, 0);
        }
        const int left = mine - i;  // 1 to 3; chunk i's V is in stage 0, chunk i + 1's in V1
        if (left == 3) issue_vr(V0, cidx(i + 2));
        if (left >= 2) issue_kr(K1, cidx(i + 1));
        consume_lds(K0, cidx(i), 0);
        if (left >= 2) {
            stage_vr(V1, 1);
            if (left == 3) issue_kr(K0, cidx(i + 2));
            consume_lds(K1, cidx(i + 1), 1);
        }
        if (left == 3) {
            stage_vr(V0, 0);
            consume_lds(K0, cidx(i + 2), 0);
        }
    }
    if (append && wave == nchunks % MW) {
        const int lb = tnew >> log2_block;
        int64_t base = -1;
        if (lb < max_blocks_per_seq) {
            const int32_t pb = table[lb];
            if (pb >= 0 && pb < num_blocks)
                base = (int64_t)pb * block_bytes + head_off + (int64_t)(tnew & (block_size - 1)) * ROW;
        }
        if (base < 0) st.bad = true;
        // the store: lanes 0.. carry K, lanes 32.. carry V, 16 bytes each
        const int w16 = lane & 31;
        if (w16 < ROW / 16 && base >= 0) {
            const uint8_t *src = lane < 32 ? new_k : new_v;
            uint8_t *dst = lane < 32 ? key_out : value_out;
            *(u32x4 *)(dst + base + w16 * 16) = *(const u32x4 *)(src + w16 * 16);
        }
        // score of head n: lane (n, q) holds the products over d = 32 kk + 8 q .. +8
        float part = 0.f;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) part += dot16<T>(qb[kk], *(const u32x4 *)(new_k + (32 * kk + 8 * q) * 2));
        const float sc = sum_over_column(part) * scale_log2;
        const float mn = fmaxf(st.m, sc);
        const float ms = mn == -INFINITY ? 0.f : mn;
        const float alpha = fast_exp2(st.m - ms);
        st.m = mn;
        float pr;
        (void)Mma<T>::round(fast_exp2(sc - ms), pr);
        st.lsum = st.lsum * alpha + (q == 0 ? pr : 0.f);
        // O^T fragment nn of lane (n, q): d = 16 nn + 4 q + i
#pragma unroll
        for (int nn = 0; nn < Gm::NN; ++nn) {
            const uint2 vw = *(const uint2 *)(new_v + (16 * nn + 4 * q) * 2);
            float v4[4];
            if constexpr (std::is_same<T, F16>::value) {
                v4[0] = (float)__builtin_bit_cast(_Float16, (uint16_t)(vw.x & 0xffffu));
                v4[1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(vw.x >> 16));
                v4[2] = (float)__builtin_bit_cast(_Float16, (uint16_t)(vw.y & 0xffffu));
                v4[3] = (float)__builtin_bit_cast(_Float16, (uint16_t)(vw.y >> 16));
            } else {
                v4[0] = __uint_as_float(vw.x << 16);
                v4[1] = __uint_as_float(vw.x & 0xffff0000u);
                v4[2] = __uint_as_float(vw.y << 16);
                v4[3] = __uint_as_float(vw.y & 0xffff0000u);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) st.o[nn][i] = st.o[nn][i] * alpha + pr * v4[i];
        }
    }
    // normaliser of head n over the 4 lanes of its column
    st.lsum = sum_over_column(st.lsum);
}

// Merge the waves' states through LDS (the staging area; every wave's loads of the range
// are complete) and write, per query head g of the group, either the normalised output
// row out_row0 + g (ws_max == nullptr) or the partial (max, sum, weighted value sums)
// at index idx0 + g * idx_stride of the workspace arrays; rows outside row_mask are not
// written.  Called by every thread; leaves LDS free for the next range.
template <typename T, int D, int G>
__device__ __forceinline__ void finish(const WaveState<D> &st, uint8_t *lds, int *sm_bad, int wave, int lane,
                                       void *out, int64_t out_row0, float *ws_max, float *ws_sum, float *ws_acc,
                                       int64_t idx0, int64_t idx_stride, uint32_t row_mask = 0xffffffffu) {
    constexpr int NN = Geom<D>::NN;
    const int n = lane & 15;
    const int q = lane >> 4;
    __syncthreads();
    float *sm_m = (float *)lds;     // [MW][G]
    float *sm_l = sm_m + MW * G;    // [MW][G]
    float *sm_acc = sm_l + MW * G;  // [MW][G][D]
    if (threadIdx.x == 0) *sm_bad = 0;
    __syncthreads();
    if (st.bad) *sm_bad = 1;
    if (n < G) {
        if (q == 0) {
            sm_m[wave * G + n] = st.m;
            sm_l[wave * G + n] = st.lsum;
        }
#pragma unroll
        for (int nn = 0; nn < NN; ++nn)
#pragma unroll
            for (int i = 0; i < 4; ++i) sm_acc[(wave * G + n) * D + 16 * nn + 4 * q + i] = st.o[nn][i];
    }
    __syncthreads();
    const bool any_bad = *sm_bad != 0;
    for (int t = threadIdx.x; t < G * D; t += MW * 64) {
        const int g = t / D;
        const int j = t - g * D;
        if (!((row_mask >> g) & 1u)) continue;  // a row this workgroup does not own
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
        if (ws_max) {
            const int64_t pi = idx0 + g * idx_stride;
            if (j == 0) {
                ws_max[pi] = any_bad ? NAN : M;
                ws_sum[pi] = Lsum;
            }
            ws_acc[pi * D + j] = A;
        } else {
            float ov = Lsum > 0.f ? A / Lsum : 0.f;
            if (any_bad) ov = NAN;
            store_out<T>(out, (out_row0 + g) * D + j, ov);
        }
    }
    __syncthreads();
}

template <typename T, int D, int G, bool SPLIT, bool NT>
__global__ __launch_bounds__(MW * 64) __attribute__((amdgpu_waves_per_eu(2))) void decode_mfma_kernel(
    void *__restrict__ out, const uint8_t *__restrict__ query, const uint8_t *__restrict__ key_cache,
    const uint8_t *__restrict__ value_cache, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ context_lens, float *__restrict__ ws_max, float *__restrict__ ws_sum,
    float *__restrict__ ws_acc, int max_blocks_per_seq, int num_seqs, int num_kv_heads,
    int log2_block, int num_blocks, int partition_size, int max_partitions, float scale_log2,
    const uint8_t *__restrict__ new_key, const uint8_t *__restrict__ new_value, uint8_t *key_out,
    uint8_t *value_out) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

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

    __shared__ __attribute__((aligned(16))) uint8_t lds[MW * Geom<D>::WAVE_LDS];
    static_assert((2 * MW * G + MW * G * D) * 4 <= MW * Geom<D>::WAVE_LDS, "merge area must fit the staging area");
    __shared__ int sm_bad;

    WaveState<D> st;
    st.bad = ctx < 0;
    // the newest token (given in new_key / new_value) belongs to the range holding ctx - 1
    const bool app = new_key != nullptr && ctx >= 1 && end == ctx;
    const int64_t nrow = (int64_t)(s * num_kv_heads + kvh) * Geom<D>::ROW;
    attend_range<T, D, G, NT>(st, lds + wave * Geom<D>::WAVE_LDS, query, key_cache, value_cache,
                              block_tables + (int64_t)s * max_blocks_per_seq, max_blocks_per_seq, s, kvh,
                              num_kv_heads, log2_block, num_blocks, start, end, scale_log2, wave, lane,
                              app ? new_key + nrow : nullptr, app ? new_value + nrow : nullptr, key_out,
                              value_out);
    const int64_t row0 = (int64_t)s * num_q_heads + kvh * G;
    if (SPLIT)
        finish<T, D, G>(st, lds, &sm_bad, wave, lane, nullptr, 0, ws_max, ws_sum, ws_acc,
                        row0 * max_partitions + part, max_partitions);
    else
        finish<T, D, G>(st, lds, &sm_bad, wave, lane, out, row0, nullptr, nullptr, nullptr, 0, 0);
}

// Balanced split on the matrix cores (balanced.h): CT-token chunks, one worker per
// workgroup, and PA_BAL_ITEM_UNITS units ahead of each item's chunks in the list (a
// range that holds only such units of an item skips it).  The workgroup walks its range
// item by item; within an item its waves take the range's chunks in turn, as the
// one-pass kernel does for a whole context, and at the item's end they merge and write
// the item's partial.
template <typename T, int D, int G, bool NT>
__global__ __launch_bounds__(MW * 64) __attribute__((amdgpu_waves_per_eu(2))) void decode_mfma_balanced_kernel(
    const uint8_t *__restrict__ query, const uint8_t *__restrict__ key_cache,
    const uint8_t *__restrict__ value_cache, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ context_lens, int32_t *__restrict__ ws_hdr, float *__restrict__ ws_max,
    float *__restrict__ ws_sum, float *__restrict__ ws_acc, int max_blocks_per_seq, int num_seqs,
    int num_kv_heads, int log2_block, int num_blocks, float scale_log2, const uint8_t *__restrict__ new_key,
    const uint8_t *__restrict__ new_value, uint8_t *key_out, uint8_t *value_out) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int S = num_seqs;
    constexpr int OV = PA_BAL_ITEM_UNITS;

    __shared__ __attribute__((aligned(16))) uint8_t lds[MW * Geom<D>::WAVE_LDS];
    static_assert((BAL_MAX_SEQS + 1) * 4 <= MW * Geom<D>::WAVE_LDS, "chunk prefix must fit the staging area");
    static_assert((2 * MW * G + MW * G * D) * 4 <= MW * Geom<D>::WAVE_LDS, "merge area must fit the staging area");
    __shared__ int sm_bad;

    // chunks per sequence and their prefix, in the staging area until the range is
    // located (wave 0 scans 64 sequences a step)
    int *sm_pre = (int *)lds;
    if (wave == 0) {
        int carry = 0;
        for (int base = 0; base < S; base += 64) {
            const int s = base + lane;
            const int c = s < S ? context_lens[s] : 0;
            int v = c > 0 ? (c + CT - 1) / CT + OV : 0;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int t = __shfl_up(v, o);
                if (lane >= o) v += t;
            }
            if (s < S) sm_pre[s + 1] = carry + v;
            carry += __shfl(v, 63);
        }
        if (lane == 0) sm_pre[0] = 0;
    }
    __syncthreads();
    auto pre = [&](int s) -> int { return __builtin_amdgcn_readfirstlane(sm_pre[s]); };

    const int per_head = pre(S);
    const int total = per_head * num_kv_heads;
    const int W = gridDim.x;
    const int per = (total + W - 1) / W;
    if (blockIdx.x == 0) {
        if (threadIdx.x == 0) {
            ws_hdr[0] = per_head;
            ws_hdr[1] = per;
            ws_hdr[2] = W;
            ws_hdr[3] = OV;
        }
        for (int t = threadIdx.x; t <= S; t += MW * 64) ws_hdr[BAL_HDR + t] = sm_pre[t];
    }
    const int w = xcd_remap(blockIdx.x, gridDim.x);
    const int g_begin = w * per;
    const int g_end = min(total, g_begin + per);

    // first item of the range: KV head, sequence, chunk within the sequence
    int kvh = num_kv_heads, s = 0, c = 0;
    if (per > 0 && g_begin < total) {
        kvh = g_begin / per_head;
        const int r = g_begin - kvh * per_head;
        int lo = 0, hi = S - 1;  // smallest s with pre(s + 1) > r
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (pre(mid + 1) > r)
                hi = mid;
            else
                lo = mid + 1;
        }
        s = lo;
        c = r - pre(lo);
    }
    __syncthreads();  // the prefix is dead: the staging area is the waves' from here
    if (per == 0 || g_begin >= total) return;  // the whole workgroup

    for (int g = g_begin; g < g_end;) {
        const int ctx = __builtin_amdgcn_readfirstlane(context_lens[s]);
        const int nc = (ctx + CT - 1) / CT;  // > 0: the list holds only non-empty items
        // units c .. c + take of the item: OV for its start, then its chunks
        const int take = min(nc + OV - c, g_end - g);
        const int c0 = max(c - OV, 0), c1 = c + take - OV;  // its chunks in this range
        if (c1 > c0) {
            WaveState<D> st;
            st.bad = false;
            const int seg_end = min(ctx, c1 * CT);
            // the item's last segment holds the newest token
            const bool app = new_key != nullptr && seg_end == ctx;
            const int64_t nrow = (int64_t)(s * num_kv_heads + kvh) * Geom<D>::ROW;
            attend_range<T, D, G, NT>(st, lds + wave * Geom<D>::WAVE_LDS, query, key_cache, value_cache,
                                      block_tables + (int64_t)s * max_blocks_per_seq, max_blocks_per_seq, s,
                                      kvh, num_kv_heads, log2_block, num_blocks, c0 * CT, seg_end, scale_log2,
                                      wave, lane, app ? new_key + nrow : nullptr, app ? new_value + nrow : nullptr,
                                      key_out, value_out);
            const int64_t slot = (int64_t)w + (int64_t)kvh * S + s;
            finish<T, D, G>(st, lds, &sm_bad, wave, lane, nullptr, 0, ws_max, ws_sum, ws_acc, slot * G, 1);
        }
        g += take;
        // next non-empty item
        c = 0;
        if (g < g_end) {
            do {
                if (++s == S) {
                    s = 0;
                    ++kvh;
                }
            } while (__builtin_amdgcn_readfirstlane(context_lens[s]) <= 0);
        }
    }
}

// Shared-prefix pass (pa_decode_grouped): one workgroup per (group, KV head).  A group
// is a run of consecutive sequences whose tables start with the same physical blocks
// ([cpai] §6: forked sequences share their prompt's blocks); the workgroup reads the K/V
// tiles of the group's shared partitions once for all members, whose queries (one query
// head per KV head) fill the rows of the score product, and writes each served member's
// partial (max, sum, weighted value sums) for the whole shared span at (sequence, head)
// of ws_max / ws_sum / ws_acc, which the one-pass vector kernel folds into its own state
// for the member's later tokens.  Which members are served is group_serves's decision:
// each workgroup checks its own members (one wave per member), and the same launch
// carries ceil(S / MW) more workgroups that record the decision for every sequence in
// seq_group / seq_parts (one wave per sequence) for the vector kernel that follows.
template <typename T, int D, int G, bool NT>
__global__ __launch_bounds__(MW * 64) __attribute__((amdgpu_waves_per_eu(2))) void decode_mfma_grouped_kernel(
    const uint8_t *__restrict__ query, const uint8_t *__restrict__ key_cache,
    const uint8_t *__restrict__ value_cache, GroupPlanArgs plan, int32_t *__restrict__ seq_group,
    int32_t *__restrict__ seq_parts, float *__restrict__ ws_max, float *__restrict__ ws_sum,
    float *__restrict__ ws_acc, int num_kv_heads, float scale_log2) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ngw = plan.num_groups * num_kv_heads;  // shared-span workgroups
    if ((int)blockIdx.x >= ngw) {
        // the plan: one wave per sequence
        const int s = ((int)blockIdx.x - ngw) * MW + wave;
        if (s >= plan.num_seqs) return;
        int j, parts;
        const bool ok = group_serves(plan, s, lane, j, parts);
        if (lane == 0) {
            seq_group[s] = ok ? j : -1;
            seq_parts[s] = ok ? parts : 0;
        }
        return;
    }
    const int kvh = blockIdx.x % num_kv_heads;
    const int j = blockIdx.x / num_kv_heads;
    // the group's record, read together
    const int s0 = plan.group_start[j];
    const int s1 = plan.group_start[j + 1];
    const int parts = plan.group_parts[j];
    const int members = s1 - s0;
    if ((s0 < 0) | (members < 1) | (members > G) | (s0 > plan.num_seqs - members) | (parts < 1) |
        (parts > plan.max_group_parts))
        return;

    __shared__ __attribute__((aligned(16))) uint8_t lds[MW * Geom<D>::WAVE_LDS];
    static_assert((2 * MW * G + MW * G * D) * 4 <= MW * Geom<D>::WAVE_LDS, "merge area must fit the staging area");
    __shared__ int sm_bad;
    __shared__ uint32_t sm_rows[MW];
    // the members this pass serves: member i checked by wave i mod MW
    uint32_t mine_rows = 0;
    for (int i = wave; i < members; i += MW)
        if (group_serves_in(plan, s0 + i, j, s0, s0 + members, parts, lane)) mine_rows |= 1u << i;
    if (lane == 0) sm_rows[wave] = mine_rows;
    __syncthreads();
    uint32_t rows = 0;
#pragma unroll
    for (int w = 0; w < MW; ++w) rows |= sm_rows[w];
    rows = __builtin_amdgcn_readfirstlane(rows);
    if (rows == 0) return;

    WaveState<D> st;
    st.bad = false;
    attend_range<T, D, G, NT>(st, lds + wave * Geom<D>::WAVE_LDS, query, key_cache, value_cache,
                              plan.block_tables + (int64_t)s0 * plan.max_blocks_per_seq, plan.max_blocks_per_seq,
                              s0, kvh, num_kv_heads, plan.log2_block, plan.num_blocks, 0, parts * plan.span,
                              scale_log2, wave, lane, nullptr, nullptr, nullptr, nullptr, rows);
    // member i's partial at (sequence s0 + i, head kvh)
    finish<T, D, G>(st, lds, &sm_bad, wave, lane, nullptr, 0, ws_max, ws_sum, ws_acc,
                    (int64_t)s0 * num_kv_heads + kvh, num_kv_heads, rows);
}

template <typename T, int D, int G>
int launch_grouped_t(const DecodeArgs &a) {
    GroupPlanArgs plan;
    plan.block_tables = a.block_tables;
    plan.context_lens = a.context_lens;
    plan.group_start = a.group_start;
    plan.group_parts = a.group_parts;
    plan.num_seqs = a.num_seqs;
    plan.num_groups = a.num_groups;
    plan.max_blocks_per_seq = a.max_blocks_per_seq;
    plan.log2_block = __builtin_ctz(a.block_size);
    plan.num_blocks = a.num_blocks;
    plan.span = a.group_span;
    plan.group_rows = a.group_rows;
    plan.max_group_parts = a.max_group_parts;
    const int64_t grid = (int64_t)a.num_groups * a.num_kv_heads + (a.num_seqs + MW - 1) / MW;
    if (grid > 0x7fffffff) return fail(PA_ERR_UNSUPPORTED, "grid of %lld workgroups", (long long)grid);
    auto kernel = a.cached_kv ? decode_mfma_grouped_kernel<T, D, G, false> : decode_mfma_grouped_kernel<T, D, G, true>;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(MW * 64), 0, (hipStream_t)a.stream, (const uint8_t *)a.query,
                       (const uint8_t *)a.key_cache, (const uint8_t *)a.value_cache, plan, a.seq_group, a.seq_parts,
                       a.ws_max, a.ws_sum, a.ws_acc, a.num_kv_heads, a.scale_log2);
    return check_launch("decode_mfma_grouped");
}

template <typename T, int D>
int launch_grouped_d(const DecodeArgs &a) {
    switch (a.group_rows) {
        case 2: return launch_grouped_t<T, D, 2>(a);
        case 4: return launch_grouped_t<T, D, 4>(a);
        case 8: return launch_grouped_t<T, D, 8>(a);
        case 16: return launch_grouped_t<T, D, 16>(a);
    }
    return fail(PA_ERR_UNSUPPORTED, "group rows %d", a.group_rows);
}

template <typename T>
int launch_grouped(const DecodeArgs &a) {
    if (a.head_dim == 64) return launch_grouped_d<T, 64>(a);
    if (a.head_dim == 128) return launch_grouped_d<T, 128>(a);
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d", a.head_dim);
}

template <typename T, int D, int G, bool NT>
int launch_balanced(const DecodeArgs &a) {
    auto kernel = decode_mfma_balanced_kernel<T, D, G, NT>;
    static int resident = 0;  // workgroups the device holds at once (per instantiation)
    if (resident == 0) {
        int dev = 0, cus = 0, per_cu = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void *)kernel, MW * 64, 0) == hipSuccess)
            resident = cus * (PA_MFMA_BAL_PER_CU > 0 && per_cu > PA_MFMA_BAL_PER_CU ? PA_MFMA_BAL_PER_CU
                              : per_cu > 0 ? per_cu : 1);
    }
    if (resident <= 0) return fail(PA_ERR_HIP, "occupancy query failed");
    const int workers = resident > a.max_workers ? a.max_workers : resident;  // workgroups
    const int log2b = __builtin_ctz(a.block_size);
    hipLaunchKernelGGL(kernel, dim3(workers), dim3(MW * 64), 0, (hipStream_t)a.stream,
                       (const uint8_t *)a.query, (const uint8_t *)a.key_cache, (const uint8_t *)a.value_cache,
                       a.block_tables, a.context_lens, a.ws_hdr, a.ws_max, a.ws_sum, a.ws_acc,
                       a.max_blocks_per_seq, a.num_seqs, a.num_kv_heads, log2b, a.num_blocks, a.scale_log2,
                       (const uint8_t *)a.new_key, (const uint8_t *)a.new_value, (uint8_t *)a.key_out,
                       (uint8_t *)a.value_out);
    const int rc = check_launch("decode_mfma_balanced");
    if (rc != PA_OK) return rc;
    return launch_balanced_merge<T, D, G>(a);
}

template <typename T, int D, int G, bool NT>
int launch_t(const DecodeArgs &a) {
    if (a.partition_size < 0) return launch_balanced<T, D, G, NT>(a);
    const int log2b = __builtin_ctz(a.block_size);
    const bool split = a.partition_size > 0;
    const unsigned grid = (unsigned)a.num_seqs * a.num_kv_heads * (split ? a.max_partitions : 1);
    hipStream_t st = (hipStream_t)a.stream;
    if (split) {
        hipLaunchKernelGGL((decode_mfma_kernel<T, D, G, true, NT>), dim3(grid), dim3(MW * 64), 0, st,
                           a.out, (const uint8_t *)a.query, (const uint8_t *)a.key_cache,
                           (const uint8_t *)a.value_cache, a.block_tables, a.context_lens, a.ws_max,
                           a.ws_sum, a.ws_acc, a.max_blocks_per_seq, a.num_seqs, a.num_kv_heads,
                           log2b, a.num_blocks, a.partition_size, a.max_partitions, a.scale_log2,
                           (const uint8_t *)a.new_key, (const uint8_t *)a.new_value, (uint8_t *)a.key_out,
                           (uint8_t *)a.value_out);
        const int rc = check_launch("decode_mfma (partitions)");
        if (rc != PA_OK) return rc;
        return launch_lse_merge(a);
    }
    hipLaunchKernelGGL((decode_mfma_kernel<T, D, G, false, NT>), dim3(grid), dim3(MW * 64), 0, st,
                       a.out, (const uint8_t *)a.query, (const uint8_t *)a.key_cache,
                       (const uint8_t *)a.value_cache, a.block_tables, a.context_lens, nullptr,
                       nullptr, nullptr, a.max_blocks_per_seq, a.num_seqs, a.num_kv_heads, log2b,
                       a.num_blocks, 0, 1, a.scale_log2, (const uint8_t *)a.new_key,
                       (const uint8_t *)a.new_value, (uint8_t *)a.key_out, (uint8_t *)a.value_out);
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
