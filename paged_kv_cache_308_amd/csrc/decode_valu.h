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
//  * one pass: work items run longest sequence first (every workgroup sorts the
//    batch's context lengths, a few hundred instructions), KV head fastest, so no
//    long sequence starts in the last round; partitions: workgroup ids are remapped
//    so that each XCD runs a contiguous range of work items (partition fastest, then
//    sequence, then KV head).  Either way the XCDs get equal shares, and the
//    sequences of one KV head share an XCD's L2 when their tables point at the same
//    blocks (shared prefixes).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "internal.h"
#include "balanced.h"
#include "kernel_common.h"

namespace pa {
namespace valu {

#ifndef PA_VALU_WAVES
#define PA_VALU_WAVES 8
#endif
#ifndef PA_VALU_LOADS
#define PA_VALU_LOADS 4
#endif
#ifndef PA_FP8_LOADS
#define PA_FP8_LOADS 2
#endif
constexpr int NW = PA_VALU_WAVES;  // waves per workgroup
constexpr int NL = PA_VALU_LOADS;  // wave loads (of K and of V) per chunk

// Wave loads per chunk for a storage policy and group size.  E4M3 pools: two (measured
// on llama-7B-shaped batches: 73 us against 85 us with four, whose 136 registers per
// lane leave room for one workgroup per CU instead of two), and one with 8 query heads
// per KV head, whose widened codes and state need the registers.
template <typename KV, int G>
constexpr int loads_per_chunk() {
    return KV::scaled ? (G >= 8 ? PA_FP8_LOADS / 2 : PA_FP8_LOADS) : NL;
}

// How the kernels read one lane's slice of a token row (SB bytes of K or V).
//  SameKV<T>:     pools in the query's type T; 16-byte slices of 16 / sizeof(T)
//                 elements.
//  E4M3KV<T, SB>: pools of E4M3 codes with a scale per (block, KV head); query and
//                 output in T (f16 or bf16).  Slices of SB = 16 or 8 codes: 8 halves
//                 the value sums a lane holds per query head, which keeps grouped
//                 heads (4 or 8 per KV head) in registers.  Codes are widened exactly
//                 to T pairs for the packed dot products and to fp32 for the value
//                 sums; the block scales are applied to the score (keys) and to the
//                 token's weight (values).
template <typename T>
struct SameKV {
    using Q = T;
    using Word = u32x4;
    static constexpr int slice_bytes = 16;
    static constexpr int kv_bytes = T::bytes;
    static constexpr int epl = 16 / T::bytes;
    static constexpr bool scaled = false;
    struct QSlice {
        u32x4 w;
    };
    __device__ static QSlice load_q(const uint8_t *p) { return {*(const u32x4 *)p}; }
    __device__ static float dot(const QSlice &q, const Word &k) { return dot16<T>(q.w, k); }
    __device__ static void values(const Word &v, float (&f)[epl]) { to_f32<T>(v, f); }
    // this lane's slice of a token row given in the query's type (the newest token),
    // as stored in the pool: the same bytes
    __device__ static Word from_new(const uint8_t *p, float) { return *(const Word *)p; }
    // elements 4j .. 4j+3 of the slice
    __device__ static void values4(const Word &v, int j, float (&f)[4]) {
        float all[epl];
        to_f32<T>(v, all);
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = all[4 * j + e];
    }
};

template <typename T, int SB>
struct E4M3KV {
    static_assert(T::bytes == 2, "E4M3 pools take a 16-bit query");
    static_assert(SB == 16 || SB == 8, "slice bytes");
    using Q = T;
    using Word = typename std::conditional<SB == 16, u32x4, u32x2>::type;
    static constexpr int slice_bytes = SB;
    static constexpr int kv_bytes = 1;
    static constexpr int epl = SB;
    static constexpr bool scaled = true;
    struct QSlice {
        u32x4 w[SB / 8];  // SB elements of T
    };
    __device__ static QSlice load_q(const uint8_t *p) {
        QSlice q;
#pragma unroll
        for (int i = 0; i < SB / 8; ++i) q.w[i] = *(const u32x4 *)(p + 16 * i);
        return q;
    }
    // codes 8j .. 8j+7 of the slice widened to four T pairs
    __device__ static u32x4 widen8(const Word &k, int j) {
        const uint32_t a = k[2 * j], b = k[2 * j + 1];  // scalar copies: see to_f32<F16>
        return u32x4{e4m3_pair<T>(a, false), e4m3_pair<T>(a, true), e4m3_pair<T>(b, false),
                     e4m3_pair<T>(b, true)};
    }
    __device__ static float dot(const QSlice &q, const Word &k) {
        float s = dot16<T>(q.w[0], widen8(k, 0));
        if constexpr (SB == 16) s += dot16<T>(q.w[1], widen8(k, 1));
        return s;
    }
    __device__ static void values(const Word &v, float (&f)[SB]) { e4m3_to_f32<SB / 4>(v, f); }
    // codes of P consecutive elements of a token row given in T (the newest token; their
    // bits packed from the low half in h), packed from the low byte: each element's
    // code of x / scale, the scatter's rounding bit for bit
    template <int P>
    __device__ static uint32_t encode_run(uint32_t h, float scale) {
        static_assert(P == 1 || P == 2, "elements per lane");
        uint32_t c = 0;
#pragma unroll
        for (int e = 0; e < P; ++e) {
            const uint32_t bits = (h >> (16 * e)) & 0xffffu;
            float x;
            if constexpr (std::is_same<T, F16>::value)
                x = (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
            else
                x = __uint_as_float(bits << 16);
            c |= e4m3_encode(x / scale) << (8 * e);
        }
        return c;
    }
    // codes 4j .. 4j+3 of the slice
    __device__ static void values4(const Word &v, int j, float (&f)[4]) {
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        const uint32_t x = v[j];  // scalar copy: see to_f32<F16>
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)x, false);
        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)x, true);
        f[0] = lo[0];
        f[1] = lo[1];
        f[2] = hi[0];
        f[3] = hi[1];
    }
};

// One chunk of the online softmax for this lane's token rows.  k[i], v[i] hold this
// lane's slice of token row `tok_row0 + i * TPW` (rows at or past `end` are masked
// when `tail`).  ksl[i]: factor from the dot product to the exp2-domain score of the
// rows of load i (scale * log2(e), times the block's key scale for E4M3 pools);
// vsc[i]: their value scale (E4M3 pools only).  m, l, acc: fp32 running max (exp2
// domain), sum of weights and weighted value sums of this lane's rows, for each of the
// G query heads.
template <typename KV, int G, int NL, int LPT, int TPW>
__device__ inline void chunk_update(const typename KV::QSlice (&qv)[G], const typename KV::Word (&k)[NL],
                                    const typename KV::Word (&v)[NL], const float (&ksl)[NL],
                                    const float (&vsc)[NL],
                                    int tok_row0, int end, bool tail, float (&m)[G], float (&l)[G],
                                    float (&acc)[G][KV::epl]) {
    constexpr int EPL = KV::epl;
    float sc[G][NL];
    bool valid[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        valid[i] = !tail || (tok_row0 + i * TPW < end);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float dot = row_sum<LPT>(KV::dot(qv[g], k[i]));
            sc[g][i] = valid[i] ? dot * ksl[i] : -INFINITY;
        }
    }
    // weights, then the value sums: acc = acc * alpha + sum_i p_i v_i, element by element
    // in token order; values are widened four at a time, once for all G heads
    float p[G][NL];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float cm = sc[g][0];
#pragma unroll
        for (int i = 1; i < NL; ++i) cm = fmaxf(cm, sc[g][i]);
        const float mn = fmaxf(m[g], cm);
        const float ms = mn == -INFINITY ? 0.f : mn;
        const float alpha = fast_exp2(m[g] - ms);
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            p[g][i] = fast_exp2(sc[g][i] - ms);
            psum += p[g][i];
            if constexpr (KV::scaled) p[g][i] *= vsc[i];  // weight of the dequantised value
        }
        l[g] = l[g] * alpha + psum;
        m[g] = mn;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] *= alpha;
    }
    typename KV::Word w[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        w[i] = v[i];
        if (tail && !valid[i]) w[i] = typename KV::Word{};  // never multiply a slot past ctx
    }
#pragma unroll
    for (int j = 0; j < EPL / 4; ++j) {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            float f[4];
            KV::values4(w[i], j, f);
#pragma unroll
            for (int g = 0; g < G; ++g) {
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[g][4 * j + e] = fmaf(p[g][i], f[e], acc[g][4 * j + e]);
            }
        }
    }
}

// Merge the states of a wave's token rows (lanes col, col + LPT, ... hold the same
// dims) with log-sum-exp weights; afterwards every row holds the wave's state.
template <int G, int EPL, int LPT>
__device__ inline void merge_rows(float (&m)[G], float (&l)[G], float (&acc)[G][EPL]) {
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
}

// Launch shape of the partitioned / one-pass kernel per storage policy and group size
// (the macros exist for tuning builds; the defaults are the measured best).
// E4M3 pools: 4-wave workgroups.  Their 86 registers per lane allow 5 waves per SIMD,
// which 8-wave workgroups cannot fill (2 per CU); measured on llama-7B-shaped batches:
// 76 us against 83-86 us with 8 waves, the time of a copy of the kernel with the
// arithmetic taken out.
#ifndef PA_FP8_WAVES
#define PA_FP8_WAVES 4
#endif
#ifndef PA_VALU_WAVES_PER_EU
#define PA_VALU_WAVES_PER_EU 1
#endif
#ifndef PA_FP8_WAVES_PER_EU
#define PA_FP8_WAVES_PER_EU 1
#endif
// Pools in the query's type: 4-wave workgroups for one pass (4 per CU at 115 registers),
// 8 for partitions.  Measured: llama-7B-shaped batches 122.4 against 123.0 us with 8 waves
// in one pass; the private tokens of grouped shared-prefix batches (items of ~140 tokens)
// 99 against 107 us per step; partitions of 512 tokens 306 against 309 us with 8 waves.
#ifndef PA_VALU_WAVES_ONE_PASS
#define PA_VALU_WAVES_ONE_PASS 4
#endif
// Waves (one item each) per workgroup of the one-wave-per-item form.  One: the prefix
// batch's 2,560 private items then spread over the CUs a wave at a time (about ten each)
// instead of in workgroups of four, which left some CUs with twelve and others with
// eight; measured 37.7 against 40.3 us for the pass (2 waves 39.6, 8 waves 56.0).
#ifndef PA_VALU_SOLO_WAVES
#define PA_VALU_SOLO_WAVES 1
#endif
template <typename KV, int G, bool SPLIT, bool SOLO = false>
constexpr int waves_per_group() {
    return SOLO ? PA_VALU_SOLO_WAVES : (KV::scaled ? PA_FP8_WAVES : (SPLIT ? NW : PA_VALU_WAVES_ONE_PASS));
}
// Waves per SIMD the register allocation must allow (1 = no constraint).
template <typename KV, int G>
constexpr int min_waves_per_eu() {
    return KV::scaled ? PA_FP8_WAVES_PER_EU : PA_VALU_WAVES_PER_EU;
}

// One pass with one wave per work item (SOLO): each wave streams a whole (sequence, KV
// head) item and writes its output from registers; a workgroup holds NWG consecutive
// items.  For batches of short items (the private tokens after a shared-prefix pass,
// ~140 tokens each), where splitting an item over the workgroup's waves leaves each wave
// two chunks and the cross-wave merge, the sort and the launch of many small
// workgroups dominate.
// E4M3 pools: 1 reads a block's K/V scales with vector loads issued beside its codes and
// applies them when the chunk is used; 0 reads them with scalar loads when the block is
// looked up (a wait for any scalar load waits for all of them, so each chunk then waits
// for the next block's scales before it can be used).
#ifndef PA_FP8_VSCALE
#define PA_FP8_VSCALE 1
#endif
#ifndef PA_VALU_SOLO
#define PA_VALU_SOLO 0  // 0: one wave per item after a shared-prefix pass only; 1: always; -1: never
#endif
template <typename KV, int D, int G, bool SPLIT, bool NT, bool SOLO = false>
__global__ __launch_bounds__((waves_per_group<KV, G, SPLIT, SOLO>() * 64))
__attribute__((amdgpu_waves_per_eu(min_waves_per_eu<KV, G>()))) void decode_valu_kernel(
    void *__restrict__ out, const uint8_t *__restrict__ query, const uint8_t *__restrict__ key_cache,
    const uint8_t *__restrict__ value_cache, const float *__restrict__ k_scales,
    const float *__restrict__ v_scales, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ context_lens, float *__restrict__ ws_max, float *__restrict__ ws_sum,
    float *__restrict__ ws_acc, int max_blocks_per_seq, int num_seqs, int num_kv_heads,
    int log2_block, int num_blocks, int partition_size, int max_partitions, float scale_log2,
    const uint8_t *__restrict__ new_key, const uint8_t *__restrict__ new_value, uint8_t *key_out,
    uint8_t *value_out, const int32_t *__restrict__ skip_parts) {
    using T = typename KV::Q;
    constexpr int NWG = waves_per_group<KV, G, SPLIT, SOLO>();
    constexpr int QB = T::bytes;            // query / output element bytes
    constexpr int EPL = KV::epl;            // elements per lane per row
    constexpr int SB = KV::slice_bytes;
    constexpr int ROW_BYTES = D * KV::kv_bytes;
    constexpr int LPT = ROW_BYTES / SB;     // lanes per token row
    constexpr int TPW = 64 / LPT;           // token rows per wave load
    constexpr int NLK = loads_per_chunk<KV, G>();
    constexpr int C = NLK * TPW;             // tokens per chunk

    static_assert(!(SOLO && SPLIT), "one wave per item is a one-pass form");
    const int lane = threadIdx.x & 63;
    // wave-uniform: keeps table lookups on the scalar unit and branches scalar
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row = lane / LPT;
    const int col = lane % LPT;
    // the waves that share this wave's work item, and this wave's place among them
    constexpr int NWI = SOLO ? 1 : NWG;
    const int iw = SOLO ? 0 : wave;

    int part = 0, s, kvh;
    if constexpr (SPLIT) {
        // work item order: partition fastest, then sequence, then KV head, so every
        // XCD's contiguous range holds whole sequences (balanced) and a head's sequences
        // are neighbours (shared-prefix siblings land on one XCD)
        const int L = xcd_remap(blockIdx.x, gridDim.x);
        part = L % max_partitions;
        const int rest = L / max_partitions;
        s = rest % num_seqs;
        kvh = rest / num_seqs;
    } else {
        // One pass: workgroups are dispatched in index order, KV head fastest, sequences
        // longest first, so the longest items start in the first round and the last
        // rounds hold short ones (no tail of one long sequence).  Workgroup w runs on
        // XCD w % 8: with a multiple of 8 KV heads, one head's sequences share an XCD.
        const int item = SOLO ? (int)blockIdx.x * NWG + wave : (int)blockIdx.x;
        kvh = item % num_kv_heads;
        int rank = item / num_kv_heads;
        if constexpr (KV::scaled && !SOLO) {
            // E4M3 pools read a K and a V scale per (block, KV head); a block's heads share one
            // line of each scale array.  In head-fastest order XCD x (workgroup w = 8k + x) runs
            // heads x, x + 8, ... of every sequence and fetches the whole line of every block;
            // here it runs the contiguous heads hx x .. hx x + hx - 1 (hx = H_kv / 8) and
            // fetches only their part.  Sequences still start in longest-first order.
            if (num_kv_heads % 8 == 0) {
                const int hx = num_kv_heads / 8;
                const int k = item / 8;
                rank = k / hx;
                kvh = hx * (item % 8) + k % hx;
            }
        }
        if (SOLO && rank >= num_seqs) rank = num_seqs - 1;  // past the batch: sorts with the rest, then leaves
        // (one wave per item: every item of such a batch is resident at once, so the order
        // does not matter and the sort is skipped)
        __shared__ uint32_t sm_order[NWG * 64];
        s = !SOLO && num_seqs <= NWG * 64 ? longest_first<NWG * 64>(context_lens, num_seqs, rank, sm_order) : rank;
        s = __builtin_amdgcn_readfirstlane(s);
        // no barrier follows in the one-wave-per-item form
        if (SOLO && item >= num_seqs * num_kv_heads) return;
    }
    const int num_q_heads = num_kv_heads * G;

    const int ctx = context_lens[s];
    int start = 0, end = ctx;
    if (SPLIT) {
        start = part * partition_size;
        if (ctx < 0 || start >= ctx) return;  // nothing here (the merge handles bad lengths)
        end = min(ctx, start + partition_size);
    }
    // One pass after a shared-prefix pass (pa_decode_grouped): that pass attended to the
    // first skip_parts[s] spans of partition_size tokens of this sequence and left its
    // partial in ws_max / ws_sum / ws_acc at (s, query head); this workgroup starts after
    // them and folds the partial in at the end.  The plan guarantees start <= ctx - 1.
    int prefix_spans = 0;
    if (!SPLIT && skip_parts != nullptr) {
        prefix_spans = __builtin_amdgcn_readfirstlane(skip_parts[s]);
        if (prefix_spans > 0) start = prefix_spans * partition_size;
    }
    // one wave per item: the shared-prefix partial (written by the previous launch) is
    // loaded now, its latency behind the loop, rather than after it
    float pre_m[SOLO ? G : 1], pre_l[SOLO ? G : 1], pre_a[SOLO ? G : 1][SOLO ? EPL : 1];
    if constexpr (SOLO) {
        if (skip_parts != nullptr) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int64_t pi = (int64_t)s * num_kv_heads * G + kvh * G + g;
                pre_m[g] = ws_max[pi];
                pre_l[g] = ws_sum[pi];
#pragma unroll
                for (int e = 0; e < EPL; ++e) pre_a[g][e] = ws_acc[pi * D + col * EPL + e];
            }
        }
    }

    const int block_size = 1 << log2_block;
    const int32_t *table = block_tables + (int64_t)s * max_blocks_per_seq;
    const int64_t head_off = (int64_t)kvh * block_size * ROW_BYTES;
    const int64_t block_bytes = (int64_t)num_kv_heads * block_size * ROW_BYTES;
    // This wave's first table entry, read beside the context length instead of after it
    // (the first chunk's position does not depend on the length).
    const int lb0 = (start + iw * C) >> log2_block;
    const int32_t pb0 = lb0 < max_blocks_per_seq ? table[lb0] : -1;

    // this lane's slice of every query head of the group
    typename KV::QSlice qv[G];
#pragma unroll
    for (int g = 0; g < G; ++g)
        qv[g] = KV::load_q(query + ((int64_t)(s * num_q_heads + kvh * G + g) * D + col * EPL) * QB);

    float m[G], l[G], acc[G][EPL];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
    }
    bool bad = ctx < 0;

    // Newest token given in new_key / new_value (fused scatter): this workgroup, if its
    // range holds position ctx - 1, stores it into the pool and attends to it from the
    // given values after the loop; the loop reads the pool up to ctx - 1 only (the pool
    // is never read at the slot being written).
    const bool append = new_key != nullptr && ctx >= 1 && start <= ctx - 1 && ctx - 1 < end;
    const int end_all = end;
    if (append) end = ctx - 1;

    const int ntok = ctx < 0 ? 0 : end - start;
    const int nfull = ntok / C;
    const bool has_tail = (ntok % C) != 0;

    // The wave that would take the next chunk handles the newest token.  Before the loop
    // it looks up the token's slot and loads the given values (their latency hides
    // behind the loop); after the loop it stores them into the pool (E4M3: rounded by
    // all 64 lanes, D / 64 elements each) and attends to them with row 0 of its lanes
    // (the other rows masked).  The loop never reads that slot.
    const bool app_here = append && iw == (nfull + (has_tail ? 1 : 0)) % NWI;
    constexpr int AP = D / 64;  // E4M3: elements of the newest row per lane
    static_assert(AP * 64 == D, "head_dim");
    typename KV::Word app_k[1] = {typename KV::Word{}}, app_v[1] = {typename KV::Word{}};
    uint32_t app_rk = 0, app_rv = 0;  // E4M3: this lane's AP raw elements of T
    int64_t app_base = -1;
    float app_ks = 1.f, app_vs = 1.f;
    if (app_here) {
        const int t = ctx - 1;
        const int lb = t >> log2_block;
        if (lb < max_blocks_per_seq) {
            const int32_t pb = table[lb];
            if (pb >= 0 && pb < num_blocks) {
                app_base = (int64_t)pb * block_bytes + head_off + (int64_t)(t & (block_size - 1)) * ROW_BYTES;
                if constexpr (KV::scaled) {
                    app_ks = k_scales[(int64_t)pb * num_kv_heads + kvh];
                    app_vs = v_scales[(int64_t)pb * num_kv_heads + kvh];
                }
            }
        }
        if (app_base < 0) bad = true;
        if constexpr (KV::scaled) {
            const int64_t src = ((int64_t)(s * num_kv_heads + kvh) * D + lane * AP) * QB;
            if constexpr (AP == 2) {
                app_rk = *(const uint32_t *)(new_key + src);
                app_rv = *(const uint32_t *)(new_value + src);
            } else {
                app_rk = *(const uint16_t *)(new_key + src);
                app_rv = *(const uint16_t *)(new_value + src);
            }
        } else if (row == 0) {
            const int64_t src = ((int64_t)(s * num_kv_heads + kvh) * D + col * EPL) * QB;
            app_k[0] = KV::from_new(new_key + src, app_ks);
            app_v[0] = KV::from_new(new_value + src, app_vs);
        }
    }

    // Byte offset of the first row of wave load i of chunk c (uniform), or -1 when the
    // load lies past `end` or its table entry is outside the pool.  The last block
    // looked up is remembered: the loads of a chunk usually share one block.
    // A load with no data (past `end` in the tail chunk, or through a bad entry) reads
    // block 0's first rows instead (always inside the pool; masked or discarded
    // later): no branch around a load, because one makes the compiler wait for every
    // outstanding load.
    int cached_lb = -1;
    int64_t cached_base = -1;
    float cached_ks = 0.f, cached_vs = 0.f;  // E4M3 pools: the block's scales
    int64_t cached_si = 0;                   // E4M3 pools: the block's place in the scale arrays
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
                const int32_t pb = lb == lb0 ? pb0 : table[lb];
                if (pb < 0 || pb >= num_blocks) {
                    bad = true;
                } else {
                    cached_base = (int64_t)pb * block_bytes + head_off;
                    if constexpr (KV::scaled) {
                        cached_si = (int64_t)pb * num_kv_heads + kvh;
                        if (!PA_FP8_VSCALE) {
                            cached_ks = k_scales[cached_si];
                            cached_vs = v_scales[cached_si];
                        }
                    }
                }
            }
        }
        if (cached_base < 0) return -1;
        return cached_base + (int64_t)(tok & (block_size - 1)) * ROW_BYTES;
    };

    struct Chunk {
        typename KV::Word k[NLK], v[NLK];
        float ksl[NLK], vsc[NLK];
        bool sok[NLK];
    };
    // tail: the chunk that holds `end`; there a lane whose row lies at or past `end` reads
    // block 0's first rows instead (cached after the first such read; masked like any row
    // past the end), so the rows past the context in the last block are not fetched
    auto issue = [&](Chunk &b, int c, bool tail = false) {
#pragma unroll
        for (int i = 0; i < NLK; ++i) {
            int64_t off = load_offset(c, i);
            b.ksl[i] = scale_log2;
            b.vsc[i] = 1.f;
            b.sok[i] = off >= 0;
            if constexpr (KV::scaled) {
                if (PA_FP8_VSCALE) {
                    // the block's scales by vector loads beside its codes, applied when the
                    // chunk is used: vector loads are counted in order, so using this chunk
                    // never waits for the next one's (scalar loads are waited for all at once)
                    int64_t si = off < 0 ? 0 : cached_si;
                    asm volatile("" : "+v"(si));
                    b.ksl[i] = k_scales[si];
                    b.vsc[i] = v_scales[si];
                } else {
                    b.ksl[i] = off < 0 ? 0.f : scale_log2 * cached_ks;
                    b.vsc[i] = off < 0 ? 0.f : cached_vs;
                }
            }
            off = off < 0 ? 0 : off;
            if (tail && start + c * C + i * TPW + row >= end) off = 0;
            b.k[i] = kv_load<NT>((const typename KV::Word *)(key_cache + off + lane * SB));
            b.v[i] = kv_load<NT>((const typename KV::Word *)(value_cache + off + lane * SB));
        }
    };
    auto consume = [&](const Chunk &b, int c, bool tail) {
        if constexpr (KV::scaled && PA_FP8_VSCALE) {
            float ksl[NLK], vsc[NLK];
#pragma unroll
            for (int i = 0; i < NLK; ++i) {
                ksl[i] = b.sok[i] ? scale_log2 * b.ksl[i] : 0.f;
                vsc[i] = b.sok[i] ? b.vsc[i] : 0.f;
            }
            chunk_update<KV, G, NLK, LPT, TPW>(qv, b.k, b.v, ksl, vsc, start + c * C + row, end, tail, m, l, acc);
        } else {
            chunk_update<KV, G, NLK, LPT, TPW>(qv, b.k, b.v, b.ksl, b.vsc, start + c * C + row, end, tail, m, l,
                                              acc);
        }
    };

    // This wave's full chunks are iw, iw + NWI, ...  The steady-state loop always
    // has a next chunk to prefetch, so its loads are unconditional and the compiler
    // waits only for the chunk being reduced; the last one or two run after it.
    {
        const int mine = nfull > iw ? (nfull - iw + NWI - 1) / NWI : 0;
        Chunk A, Bf;
        if (mine > 0) {
            issue(A, iw);
            int j = 0;
            for (; j + 2 < mine; j += 2) {
                issue(Bf, iw + (j + 1) * NWI);
                consume(A, iw + j * NWI, false);
                issue(A, iw + (j + 2) * NWI);
                consume(Bf, iw + (j + 1) * NWI, false);
            }
            if (j + 1 < mine) {
                issue(Bf, iw + (j + 1) * NWI);
                consume(A, iw + j * NWI, false);
                consume(Bf, iw + (j + 1) * NWI, false);
            } else {
                consume(A, iw + j * NWI, false);
            }
        }
        if (has_tail && (nfull % NWI) == iw) {
            issue(A, nfull, true);
            consume(A, nfull, true);
        }
    }

    if (app_here) {
        if constexpr (KV::scaled) {
            __shared__ __align__(16) uint8_t sm_new_all[SOLO ? NWG : 1][2][D];
            uint8_t(&sm_new)[2][D] = sm_new_all[SOLO ? wave : 0];
            const uint32_t ck = KV::template encode_run<AP>(app_rk, app_ks);
            const uint32_t cv = KV::template encode_run<AP>(app_rv, app_vs);
            if constexpr (AP == 2) {
                *(uint16_t *)(sm_new[0] + lane * 2) = (uint16_t)ck;
                *(uint16_t *)(sm_new[1] + lane * 2) = (uint16_t)cv;
                if (app_base >= 0) {
                    *(uint16_t *)(key_out + app_base + lane * 2) = (uint16_t)ck;
                    *(uint16_t *)(value_out + app_base + lane * 2) = (uint16_t)cv;
                }
            } else {
                sm_new[0][lane] = (uint8_t)ck;
                sm_new[1][lane] = (uint8_t)cv;
                if (app_base >= 0) {
                    key_out[app_base + lane] = (uint8_t)ck;
                    value_out[app_base + lane] = (uint8_t)cv;
                }
            }
            // row 0 gathers its slices (LDS operations of one wave complete in order)
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            if (row == 0) {
                app_k[0] = *(const typename KV::Word *)(sm_new[0] + col * SB);
                app_v[0] = *(const typename KV::Word *)(sm_new[1] + col * SB);
            }
        } else if (row == 0 && app_base >= 0) {
            *(typename KV::Word *)(key_out + app_base + col * SB) = app_k[0];
            *(typename KV::Word *)(value_out + app_base + col * SB) = app_v[0];
        }
        const float ksl1[1] = {KV::scaled ? scale_log2 * app_ks : scale_log2};
        const float vsc1[1] = {app_vs};
        chunk_update<KV, G, 1, LPT, TPW>(qv, app_k, app_v, ksl1, vsc1, row, 1, true, m, l, acc);
    }
    end = end_all;

    merge_rows<G, EPL, LPT>(m, l, acc);

    if constexpr (SOLO) {
        // the item's only wave: row 0 writes its slices of every head's output, after
        // folding in the shared-prefix partial if there is one
        if (row == 0) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int h = kvh * G + g;
                const int64_t pi = (int64_t)s * num_q_heads + h;
                float M = m[g], m0 = -INFINITY, l0 = 0.f;
                bool bad0 = false;
                if (prefix_spans > 0) {
                    m0 = pre_m[g];
                    l0 = pre_l[g];
                    bad0 = m0 != m0;
                    if (!bad0) M = fmaxf(M, m0);
                }
                const float Ms = M == -INFINITY ? 0.f : M;
                const float f = fast_exp2(m[g] - Ms);
                const float f0 = prefix_spans > 0 && !bad0 ? fast_exp2(m0 - Ms) : 0.f;
                const float Lsum = l[g] * f + l0 * f0;
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    const int j = col * EPL + e;
                    float A = acc[g][e] * f;
                    if (prefix_spans > 0 && !bad0) A += pre_a[g][e] * f0;
                    float o = Lsum > 0.f ? A / Lsum : 0.f;
                    if (bad || bad0) o = NAN;
                    store_out<T>(out, pi * D + j, o);
                }
            }
        }
        return;
    }

    // merge the waves through LDS
    __shared__ float sm_m[NWG][G], sm_l[NWG][G], sm_acc[NWG][G][D];
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
    for (int t = threadIdx.x; t < G * D; t += NWG * 64) {
        const int g = t / D;
        const int j = t - g * D;
        const int h = kvh * G + g;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NWG; ++w) M = fmaxf(M, sm_m[w][g]);
        float m0 = -INFINITY, l0 = 0.f, a0 = 0.f;  // the shared-prefix partial, if any
        bool bad0 = false;
        if (!SPLIT && prefix_spans > 0) {
            const int64_t pi = (int64_t)s * num_q_heads + h;
            m0 = ws_max[pi];
            l0 = ws_sum[pi];
            a0 = ws_acc[pi * D + j];
            bad0 = m0 != m0;
            M = fmaxf(M, m0);
        }
        const float Ms = M == -INFINITY ? 0.f : M;
        float Lsum = 0.f, A = 0.f;
#pragma unroll
        for (int w = 0; w < NWG; ++w) {
            const float f = fast_exp2(sm_m[w][g] - Ms);
            Lsum += sm_l[w][g] * f;
            A += sm_acc[w][g][j] * f;
        }
        if (!SPLIT && prefix_spans > 0 && !bad0) {
            const float f = fast_exp2(m0 - Ms);
            Lsum += l0 * f;
            A += a0 * f;
        }
        if (SPLIT) {
            const int64_t pi = ((int64_t)s * num_q_heads + h) * max_partitions + part;
            if (j == 0) {
                ws_max[pi] = any_bad ? NAN : M;
                ws_sum[pi] = Lsum;
            }
            ws_acc[pi * D + j] = A;
        } else {
            float o = Lsum > 0.f ? A / Lsum : 0.f;
            if (any_bad || bad0) o = NAN;
            store_out<T>(out, ((int64_t)s * num_q_heads + h) * D + j, o);
        }
    }
}

// Log-sum-exp merge of the partition partials of one (sequence, query head):
//   M = max_p m_p,  L = sum_p l_p 2^(m_p - M),  out = sum_p 2^(m_p - M) acc_p / L.
// The merge is latency-bound (a few KB per wave), so the loads are issued together:
// lane p holds partition p's max and sum (64 partitions a round), the first 8
// partitions' value sums are loaded before the context length is even known (every
// slot below max_partitions lies in the workspace; unused ones are never counted), and
// later value sums 8 partitions at a time.  Weights reach the other lanes by readlane.
template <typename T, int D>
__global__ __launch_bounds__(64) void lse_merge_kernel(
    void *__restrict__ out, const float *__restrict__ ws_max, const float *__restrict__ ws_sum,
    const float *__restrict__ ws_acc, const int32_t *__restrict__ context_lens, int num_q_heads,
    int partition_size, int max_partitions) {
    constexpr int JP = D / 64;  // output elements per lane
    constexpr int PB = 8;       // partitions whose value sums are loaded together
    const int lane = threadIdx.x;
    const int sh = blockIdx.x;  // s * H_q + h
    const int s = sh / num_q_heads;
    const int64_t obase = (int64_t)sh * D;
    const float *mp = ws_max + (int64_t)sh * max_partitions;
    const float *lp = ws_sum + (int64_t)sh * max_partitions;
    const float *ap = ws_acc + (int64_t)sh * max_partitions * D + lane;
    float a0[PB][JP];
#pragma unroll
    for (int u = 0; u < PB; ++u)
#pragma unroll
        for (int jj = 0; jj < JP; ++jj) a0[u][jj] = u < max_partitions ? ap[u * D + 64 * jj] : 0.f;
    const int ctx = context_lens[s];
    const int n = ctx <= 0 ? 0 : (ctx + partition_size - 1) / partition_size;
    if (ctx < 0 || n > max_partitions) {
        for (int j = lane; j < D; j += 64) store_out<T>(out, obase + j, NAN);
        return;
    }
    // the maximum (and any NaN partial, from a bad table entry) over every partition
    float xf = -INFINITY, lf = 0.f;  // this lane's partition of the first round
    float M = -INFINITY;
    bool bad = false;
    for (int p0 = 0; p0 < n; p0 += 64) {
        const int p = p0 + lane;
        const float x = p < n ? mp[p] : -INFINITY;
        if (p0 == 0) {
            xf = x;
            lf = p < n ? lp[p] : 0.f;
        }
        bad |= x != x;
        M = fmaxf(M, x);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    const bool any_bad = __any(bad);
    const float Ms = M == -INFINITY ? 0.f : M;
    float Lsum = 0.f, A[JP];
#pragma unroll
    for (int jj = 0; jj < JP; ++jj) A[jj] = 0.f;
    for (int p0 = 0; p0 < n; p0 += 64) {
        const int p = p0 + lane;
        const float x = p0 == 0 ? xf : (p < n ? mp[p] : -INFINITY);
        const float l = p0 == 0 ? lf : (p < n ? lp[p] : 0.f);
        const float w = p < n ? fast_exp2(x - Ms) : 0.f;
        Lsum += l * w;
        const int cnt = min(64, n - p0);
        for (int i = 0; i < cnt; i += PB) {
            float a[PB][JP];
#pragma unroll
            for (int u = 0; u < PB; ++u)
#pragma unroll
                for (int jj = 0; jj < JP; ++jj)
                    a[u][jj] = p0 + i == 0 ? a0[u][jj] : (i + u < cnt ? ap[(int64_t)(p0 + i + u) * D + 64 * jj] : 0.f);
#pragma unroll
            for (int u = 0; u < PB; ++u) {
                if (i + u >= cnt) break;
                const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), i + u));
#pragma unroll
                for (int jj = 0; jj < JP; ++jj) A[jj] += wu * a[u][jj];
            }
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) Lsum += __shfl_xor(Lsum, o);
#pragma unroll
    for (int jj = 0; jj < JP; ++jj) {
        float o = Lsum > 0.f ? A[jj] / Lsum : 0.f;
        if (any_bad) o = NAN;
        store_out<T>(out, obase + lane + 64 * jj, o);
    }
}

// ------------------------------------------------------------------ balanced split
//
// The list, ranges, partial slots and header are those of balanced.h, with C-token
// chunks and one worker per wave: each of the W resident waves streams its range with
// the same double-buffered pipeline, so no wave waits for a long sequence and no
// sequence waits for a free wave.

constexpr int NWB = 4;  // waves per workgroup of the balanced kernel

template <typename KV, int D, int G, bool NT>
__global__ __launch_bounds__(NWB * 64) void decode_balanced_kernel(
    const uint8_t *__restrict__ query, const uint8_t *__restrict__ key_cache,
    const uint8_t *__restrict__ value_cache, const float *__restrict__ k_scales,
    const float *__restrict__ v_scales, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ context_lens, int32_t *__restrict__ ws_hdr, float *__restrict__ ws_max,
    float *__restrict__ ws_sum, float *__restrict__ ws_acc, int max_blocks_per_seq, int num_seqs,
    int num_kv_heads, int log2_block, int num_blocks, float scale_log2) {
    constexpr int QB = KV::Q::bytes;
    constexpr int EPL = KV::epl;
    constexpr int SB = KV::slice_bytes;
    constexpr int ROW_BYTES = D * KV::kv_bytes;
    constexpr int LPT = ROW_BYTES / SB;
    constexpr int TPW = 64 / LPT;
    constexpr int NLK = loads_per_chunk<KV, G>();
    constexpr int C = NLK * TPW;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row = lane / LPT;
    const int col = lane % LPT;
    const int S = num_seqs;
    const int num_q_heads = num_kv_heads * G;

    // chunks per sequence and their prefix, in LDS (wave 0 scans 64 sequences a step)
    __shared__ int sm_pre[BAL_MAX_SEQS + 1];
    if (wave == 0) {
        int carry = 0;
        for (int base = 0; base < S; base += 64) {
            const int s = base + lane;
            const int c = s < S ? context_lens[s] : 0;
            int v = c > 0 ? (c + C - 1) / C : 0;
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
    const int W = gridDim.x * NWB;
    const int per = (total + W - 1) / W;
    if (blockIdx.x == 0) {
        if (threadIdx.x == 0) {
            ws_hdr[0] = per_head;
            ws_hdr[1] = per;
            ws_hdr[2] = W;
            ws_hdr[3] = 0;
        }
        for (int t = threadIdx.x; t <= S; t += NWB * 64) ws_hdr[BAL_HDR + t] = sm_pre[t];
    }
    // consecutive workers share an XCD (shared-prefix siblings are neighbours in the list)
    const int w = xcd_remap(blockIdx.x, gridDim.x) * NWB + wave;
    const int g_begin = w * per;
    const int g_end = min(total, g_begin + per);
    if (per == 0 || g_begin >= total) return;

    // position in the list: KV head, sequence, chunk of the sequence
    struct Pos {
        int kvh, s, c, n, ctx;
    };
    auto locate = [&](int g) -> Pos {
        Pos p;
        p.kvh = g / per_head;
        const int r = g - p.kvh * per_head;
        int lo = 0, hi = S - 1;  // smallest s with pre(s + 1) > r
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (pre(mid + 1) > r)
                hi = mid;
            else
                lo = mid + 1;
        }
        p.s = lo;
        p.c = r - pre(lo);
        p.n = pre(lo + 1) - pre(lo);
        p.ctx = context_lens[lo];
        return p;
    };
    auto advance = [&](Pos &p) {
        if (++p.c < p.n) return;
        p.c = 0;
        do {
            if (++p.s == S) {
                p.s = 0;
                ++p.kvh;
            }
            p.n = pre(p.s + 1) - pre(p.s);
        } while (p.n == 0 && p.kvh < num_kv_heads);
        p.ctx = context_lens[p.s];
    };

    const int block_size = 1 << log2_block;
    const int64_t block_bytes = (int64_t)num_kv_heads * block_size * ROW_BYTES;

    struct Chunk {
        typename KV::QSlice q[G];
        typename KV::Word k[NLK], v[NLK];
        float ksl[NLK], vsc[NLK];
        Pos p;
        bool bad;
    };
    // Loads of chunk p.  As in the partitioned kernel every chunk issues the same loads
    // (rows past ctx, a bad table entry or a position past the list read block 0's first
    // rows and are masked or discarded), so the compiler's waits stay exact.
    auto issue = [&](Chunk &b, const Pos &p) {
        b.p = p;
        b.bad = false;
        const bool live = p.kvh < num_kv_heads;
        const int s = live ? p.s : 0;
        const int kvh = live ? p.kvh : 0;
        const int32_t *table = block_tables + (int64_t)s * max_blocks_per_seq;
        int cached_lb = -1;
        int64_t cached_base = 0;
        float cached_ks = 0.f, cached_vs = 0.f;
#pragma unroll
        for (int i = 0; i < NLK; ++i) {
            const int tok = p.c * C + i * TPW;
            int64_t off = 0;
            b.ksl[i] = scale_log2;
            b.vsc[i] = 1.f;
            if (live && tok < p.ctx) {
                const int lb = tok >> log2_block;
                if (lb != cached_lb) {
                    cached_lb = lb;
                    cached_base = -1;
                    if (lb < max_blocks_per_seq) {
                        const int32_t pb = table[lb];
                        if (pb >= 0 && pb < num_blocks) {
                            cached_base = (int64_t)pb * block_bytes + (int64_t)kvh * block_size * ROW_BYTES;
                            if constexpr (KV::scaled) {
                                cached_ks = k_scales[(int64_t)pb * num_kv_heads + kvh];
                                cached_vs = v_scales[(int64_t)pb * num_kv_heads + kvh];
                            }
                        }
                    }
                }
                if (cached_base < 0)
                    b.bad = true;
                else
                    off = cached_base + (int64_t)(tok & (block_size - 1)) * ROW_BYTES;
                if constexpr (KV::scaled) {
                    b.ksl[i] = scale_log2 * cached_ks;
                    b.vsc[i] = cached_vs;
                }
            }
            b.k[i] = kv_load<NT>((const typename KV::Word *)(key_cache + off + lane * SB));
            b.v[i] = kv_load<NT>((const typename KV::Word *)(value_cache + off + lane * SB));
        }
#pragma unroll
        for (int g = 0; g < G; ++g)
            b.q[g] = KV::load_q(query + ((int64_t)(s * num_q_heads + kvh * G + g) * D + col * EPL) * QB);
    };

    float m[G], l[G], acc[G][EPL];
    auto reset = [&]() {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            m[g] = -INFINITY;
            l[g] = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
        }
    };
    reset();
    bool item_bad = false;

    auto consume = [&](const Chunk &b, int g) {
        const Pos &p = b.p;
        const int tok0 = p.c * C;
        chunk_update<KV, G, NLK, LPT, TPW>(b.q, b.k, b.v, b.ksl, b.vsc, tok0 + row, p.ctx, tok0 + C > p.ctx,
                                          m, l, acc);
        item_bad |= b.bad;
        if (p.c == p.n - 1 || g == g_end - 1) {
            // this wave's share of the item is complete: write its partial
            merge_rows<G, EPL, LPT>(m, l, acc);
            const int64_t slot = (int64_t)w + p.kvh * S + p.s;
            if (row == 0) {
#pragma unroll
                for (int gg = 0; gg < G; ++gg) {
#pragma unroll
                    for (int e = 0; e < EPL; ++e) ws_acc[(slot * G + gg) * D + col * EPL + e] = acc[gg][e];
                    if (col == 0) {
                        ws_max[slot * G + gg] = item_bad ? NAN : m[gg];
                        ws_sum[slot * G + gg] = l[gg];
                    }
                }
            }
            reset();
            item_bad = false;
        }
    };

    const int mine = g_end - g_begin;
    Pos ip = locate(g_begin);  // position of the next chunk to issue
    Chunk A, Bf;
    issue(A, ip);
    advance(ip);
    int j = 0;
    for (; j + 2 < mine; j += 2) {
        issue(Bf, ip);
        advance(ip);
        consume(A, g_begin + j);
        issue(A, ip);
        advance(ip);
        consume(Bf, g_begin + j + 1);
    }
    if (j + 1 < mine) {
        issue(Bf, ip);
        consume(A, g_begin + j);
        consume(Bf, g_begin + j + 1);
    } else {
        consume(A, g_begin + j);
    }
}

// Waves of one balanced launch: as many as can be resident at once on this device.
template <typename K>
int balanced_workers(K kernel) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void *)kernel, NWB * 64, 0) != hipSuccess)
        return 0;
    return cus * (per_cu > 0 ? per_cu : 1) * NWB;
}

template <typename KV, int D, int G, bool NT>
int launch_balanced(const DecodeArgs &a) {
    auto kernel = decode_balanced_kernel<KV, D, G, NT>;
    static int workers = 0;  // per instantiation; the library runs on one device type
    if (workers == 0) workers = balanced_workers(kernel);
    if (workers <= 0) return fail(PA_ERR_HIP, "occupancy query failed");
    if (workers > a.max_workers) workers = a.max_workers - a.max_workers % NWB;
    hipStream_t st = (hipStream_t)a.stream;
    hipLaunchKernelGGL(kernel, dim3(workers / NWB), dim3(NWB * 64), 0, st, (const uint8_t *)a.query,
                       (const uint8_t *)a.key_cache, (const uint8_t *)a.value_cache, a.k_scales,
                       a.v_scales, a.block_tables, a.context_lens, a.ws_hdr, a.ws_max, a.ws_sum, a.ws_acc,
                       a.max_blocks_per_seq, a.num_seqs, a.num_kv_heads, __builtin_ctz(a.block_size),
                       a.num_blocks, a.scale_log2);
    int rc = check_launch("decode_balanced");
    if (rc != PA_OK) return rc;
    return launch_balanced_merge<typename KV::Q, D, G>(a);
}

template <typename KV, int D, int G, bool NT>
int launch_t(const DecodeArgs &a) {
    if (a.partition_size < 0) return launch_balanced<KV, D, G, NT>(a);
    const int log2b = __builtin_ctz(a.block_size);
    const bool split = a.partition_size > 0;
    const unsigned grid = (unsigned)a.num_seqs * a.num_kv_heads * (split ? a.max_partitions : 1);
    hipStream_t st = (hipStream_t)a.stream;
    if (split) {
        hipLaunchKernelGGL((decode_valu_kernel<KV, D, G, true, NT>), dim3(grid),
                           dim3(waves_per_group<KV, G, true>() * 64), 0, st,
                           a.out, (const uint8_t *)a.query, (const uint8_t *)a.key_cache,
                           (const uint8_t *)a.value_cache, a.k_scales, a.v_scales, a.block_tables,
                           a.context_lens, a.ws_max, a.ws_sum, a.ws_acc, a.max_blocks_per_seq, a.num_seqs,
                           a.num_kv_heads, log2b, a.num_blocks, a.partition_size, a.max_partitions,
                           a.scale_log2, (const uint8_t *)a.new_key, (const uint8_t *)a.new_value,
                           (uint8_t *)a.key_out, (uint8_t *)a.value_out, nullptr);
        const int rc = check_launch("decode_valu (partitions)");
        if (rc != PA_OK) return rc;
        return launch_lse_merge(a);
    }
    // one wave per item for the private tokens after a shared-prefix pass (short items;
    // pa_decode_grouped takes one query head per KV head and 16-bit pools)
    constexpr bool solo_built = PA_VALU_SOLO > 0 || (PA_VALU_SOLO == 0 && G == 1 && !KV::scaled);
    const bool solo = solo_built && (PA_VALU_SOLO > 0 || a.skip_parts != nullptr);
    constexpr int NWG1 = waves_per_group<KV, G, false>();
    constexpr int NWS = waves_per_group<KV, G, false, true>();
    auto kernel = decode_valu_kernel<KV, D, G, false, NT, false>;
    if constexpr (solo_built)
        if (solo) kernel = decode_valu_kernel<KV, D, G, false, NT, true>;
    const unsigned grid1 = solo ? (unsigned)(((int64_t)a.num_seqs * a.num_kv_heads + NWS - 1) / NWS) : grid;
    hipLaunchKernelGGL(kernel, dim3(grid1), dim3((solo ? NWS : NWG1) * 64), 0, st,
                       a.out, (const uint8_t *)a.query, (const uint8_t *)a.key_cache,
                       (const uint8_t *)a.value_cache, a.k_scales, a.v_scales, a.block_tables,
                       a.context_lens, a.ws_max, a.ws_sum, a.ws_acc, a.max_blocks_per_seq, a.num_seqs,
                       a.num_kv_heads, log2b, a.num_blocks, a.group_span, 1, a.scale_log2,
                       (const uint8_t *)a.new_key, (const uint8_t *)a.new_value, (uint8_t *)a.key_out,
                       (uint8_t *)a.value_out, a.skip_parts);
    return check_launch(solo ? "decode_valu (one wave per item)" : "decode_valu");
}

template <typename KV, int D, int G>
int by_cache(const DecodeArgs &a) {
    return a.cached_kv ? launch_t<KV, D, G, false>(a) : launch_t<KV, D, G, true>(a);
}

template <typename KV, int D>
int by_group(const DecodeArgs &a) {
    switch (a.num_q_heads / a.num_kv_heads) {
        case 1: return by_cache<KV, D, 1>(a);
        case 2: return by_cache<KV, D, 2>(a);
        case 4: return by_cache<KV, D, 4>(a);
        case 8: return by_cache<KV, D, 8>(a);
        case 16: return by_cache<KV, D, 16>(a);
    }
    return fail(PA_ERR_UNSUPPORTED, "group %d", a.num_q_heads / a.num_kv_heads);
}

template <typename KV>
int by_dim(const DecodeArgs &a) {
    if (a.head_dim == 64) return by_group<KV, 64>(a);
    if (a.head_dim == 128) return by_group<KV, 128>(a);
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d", a.head_dim);
}

// E4M3 pools: 16-code slices for 1 or 2 query heads per KV head, 8-code slices for 4
// and 8 (a lane then holds 8 fp32 value sums per head, as with 16-bit pools).
template <typename T, int D>
int e4m3_by_group(const DecodeArgs &a) {
    switch (a.num_q_heads / a.num_kv_heads) {
        case 1: return by_cache<E4M3KV<T, 16>, D, 1>(a);
        case 2: return by_cache<E4M3KV<T, 16>, D, 2>(a);
        case 4: return by_cache<E4M3KV<T, 8>, D, 4>(a);
        case 8: return by_cache<E4M3KV<T, 8>, D, 8>(a);
    }
    return fail(PA_ERR_UNSUPPORTED, "group %d with E4M3 pools", a.num_q_heads / a.num_kv_heads);
}

template <typename T>
int e4m3_by_dim(const DecodeArgs &a) {
    if (a.head_dim == 64) return e4m3_by_group<T, 64>(a);
    if (a.head_dim == 128) return e4m3_by_group<T, 128>(a);
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
