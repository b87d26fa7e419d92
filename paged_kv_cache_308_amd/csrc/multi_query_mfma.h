#pragma once
// Several causal query tokens per sequence over the paged cache, on the matrix cores
// (gfx950 MFMA): the chunked-prefill / prefix-cache-hit case ("PagedAttention 深度解析"
// (5ulink.com) §六 item 5) of the same attention through the block table ("PagedAttention"
// concept report (compassingai.com) §5 and §8).  Sequence s has n_s query tokens, the
// last n_s positions of its context (their K/V already cached); the token at position
// p attends to the cached tokens t <= p.
//
// A workgroup takes one (KV head, sequence, tile of 128 query rows), a row being one
// (query token, query head of the group) pair: 128 / g tokens times the g heads that
// share the KV head.  Each of its four waves owns 32 rows (two 16-row fragments that
// share every operand read).  The workgroup walks the keys its rows can see ([0, last
// row's position]) in tiles of 32 keys (64 at d = 64, the same bytes); every tile is
// loaded from HBM once, through the block table, into double-buffered LDS (K and V rows
// on padded strides) while the previous tile is being used,
// and all four waves read it there.  Per tile and wave:
//
//   S^T[t][r]  = sum_d K[t][d] Q[r][d]          A = K rows (16 keys x 32 d), B = Q^T
//   O^T[d][r] += sum_t V[t][d] P[r][t]          A = V^T (16 d x 32 keys),   B = P^T
//
// on v_mfma_f32_16x16x32_{f16,bf16}.  Lane l supplies A[l%16][8(l/16)..+8] and
// B[8(l/16)..+8][l%16] and receives D[4(l/16)..+4][l%16], so the score fragment holds,
// per lane, one row's scores for keys 4q..4q+3 and 16+4q..16+4q+3: exactly a P^T
// operand once the V^T operand uses the same k order (two LDS transpose reads,
// ds_read_b64_tr_b16, of the V rows).  The causal mask compares each key's position with its row's; a
// wave skips tiles past its own last row.  Softmax is fp32 online in the exp2 domain;
// P enters the second product rounded to the storage type and the normaliser sums the
// rounded weights (on the matrix cores, P against a ones operand).  Rows are written by
// the wave that owns them (no merge).
//
// Row tiles are numbered fastest, then sequence, then KV head, and spread over the XCDs
// in contiguous ranges, so the row tiles that read the same sequence's blocks share an
// XCD's L2 (K and V are read with cacheable loads).
#include <hip/hip_runtime.h>

#include "decode_mfma.h"
#include "internal.h"
#include "kernel_common.h"

namespace pa {
namespace mq {

using mfma::Mma;
using mfma::f32x4;
constexpr int MW = 4;  // waves per workgroup
#ifndef PA_MQ_FRAGS
#define PA_MQ_FRAGS 2
#endif
#ifndef PA_MQ_KEYS
#define PA_MQ_KEYS 32
#endif
// The loop is latency-bound (each wave's chain of LDS reads, score products, max,
// exponentials and value products), so occupancy wins over prefetch depth: one key tile
// in flight and registers held to 168 so that 3 waves share each SIMD (388 us against
// 455 us with two tiles in flight at 2 waves; a few bytes of spill at d = 128).
#ifndef PA_MQ_DEPTH
#define PA_MQ_DEPTH 1  // key tiles in flight beyond the one in use (1 or 2)
#endif
#ifndef PA_MQ_WAVES_PER_EU
#define PA_MQ_WAVES_PER_EU 3  // waves per SIMD the register allocation must allow
#endif
// Tuning switches: PA_MQ_VPREFETCH reads a tile's V^T operands right after the score
// product, before the softmax (their LDS latency behind the exponentials); PA_MQ_PRIO
// raises the wave's issue priority around its runs of matrix-core instructions.
#ifndef PA_MQ_VPREFETCH
#define PA_MQ_VPREFETCH 0
#endif
#ifndef PA_MQ_PRIO
#define PA_MQ_PRIO 0
#endif
// 16-row query fragments per wave.  Four halve the LDS reads per product but need more
// than 256 registers (one wave per SIMD), which measured 1.4x slower than two.
constexpr int RF = PA_MQ_FRAGS;
constexpr int ROWS = 16 * RF * MW;   // query rows per workgroup
static_assert(PA_MQ_KEYS % 32 == 0 && (RF == 1 || RF == 2 || RF == 4), "tile shape");

// Two fp32 weights rounded to T (to nearest even) and packed, the first in the low half
// (one v_cvt_pk_{f16,bf16}_f32 on gfx950).
template <typename T>
__device__ inline uint32_t round2(float a, float b);
template <>
__device__ inline uint32_t round2<F16>(float a, float b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{a, b}), h2));
}
template <>
__device__ inline uint32_t round2<BF16>(float a, float b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{a, b}), b2));
}

template <typename T, int D, int G>
__global__ __launch_bounds__(MW * 64) __attribute__((amdgpu_waves_per_eu(PA_MQ_WAVES_PER_EU))) void multi_query_kernel(
    void *__restrict__ out, const uint8_t *__restrict__ query, const uint8_t *__restrict__ key_cache,
    const uint8_t *__restrict__ value_cache, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ context_lens, const int32_t *__restrict__ query_start,
    int max_blocks_per_seq, int num_seqs, int num_kv_heads, int num_query_tokens, int tiles_per_seq,
    int max_query_len, int log2_block, int num_blocks, float scale_log2) {
    constexpr int ROW = D * 2;             // bytes per token row
    constexpr int KT = PA_MQ_KEYS * (D == 64 ? 2 : 1);  // keys per tile: the same bytes at d = 64
    constexpr int NKK = D / 32;            // 32-wide d steps of the score product
    constexpr int NN = D / 16;             // 16-row d fragments of the output
    constexpr int NT = KT / 16;            // 16-key score operands per tile
    constexpr int NH = KT / 32;            // 32-key value products per tile
    constexpr int KROW = ROW + 16;         // LDS stride of a key row (16 lanes x 16 bytes: no bank conflict)
    constexpr int KBYTES = KT * KROW;
    // V rows as they are, read transposed by ds_read_b64_tr_b16; a 32-byte pad keeps the
    // 16 rows one operand read touches in different banks
    constexpr int VROW = ROW + 32;
    constexpr int BUF = KBYTES + KT * VROW;  // one tile: K rows, then V rows
    constexpr int PARTS = ROW / 16;        // 16-byte pieces of a row
    constexpr int NCH = KT * PARTS / (MW * 64);  // pieces of K (and of V) per thread per tile
    static_assert(NCH * MW * 64 == KT * PARTS && NCH % 2 == 0, "tile pieces must divide over the workgroup");

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15;  // query row of a fragment / key row within a 16-key operand
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
    if (nq <= 0 || ROWS * tile >= rows) return;
    const bool bad_len = ctx < 0 || nq > ctx || nq > max_query_len;

    // this lane's rows (one per fragment f: token ti, head g) and their positions; the
    // wave's and the workgroup's last positions bound the keys they read
    const int wrow0 = ROWS * tile + 16 * RF * wave;  // first row of the wave
    int pos[RF], gh[RF];
    int64_t orow[RF];
    bool io_ok[RF];
#pragma unroll
    for (int f = 0; f < RF; ++f) {
        const int r = wrow0 + 16 * f + n;
        const bool ok = r < rows;
        const int ti = (ok ? r : rows - 1) / G;
        gh[f] = (ok ? r : rows - 1) % G;
        pos[f] = ctx - nq + ti;
        orow[f] = (int64_t)q0 + ti;
        io_ok[f] = ok && orow[f] >= 0 && orow[f] < num_query_tokens;
    }
    const int wave_end = wrow0 < rows ? ctx - nq + (min(rows, wrow0 + 16 * RF) - 1) / G + 1 : 0;
    const int wg_last = min(rows, ROWS * tile + ROWS) - 1;
    const int end = bad_len ? 0 : ctx - nq + wg_last / G + 1;  // keys the workgroup reads

    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * BUF];

    const int block_size = 1 << log2_block;
    const int32_t *table = block_tables + (int64_t)s * max_blocks_per_seq;
    const int64_t head_off = (int64_t)kvh * block_size * ROW;
    const int64_t block_bytes = (int64_t)num_kv_heads * block_size * ROW;

    // Q^T operands: lane holds Q[row n of fragment f][32 kk + 8 q .. +8]; rows past the
    // sequence are zero
    u32x4 qb[RF][NKK];
#pragma unroll
    for (int f = 0; f < RF; ++f)
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            qb[f][kk] = u32x4{0, 0, 0, 0};
            if (io_ok[f])
                qb[f][kk] = *(const u32x4 *)(query + ((orow[f] * num_q_heads + kvh * G + gh[f]) * D + 32 * kk +
                                                      8 * q) * 2);
        }

    // Scores stay unscaled until the exponent: exp2(s * x - m) with s = |scale * log2 e| > 0,
    // so the running max can be taken on raw products (a negative scale flips the sign
    // of q instead, which is exact).
    const float sl = fabsf(scale_log2);
    if (scale_log2 < 0.f) {
#pragma unroll
        for (int f = 0; f < RF; ++f)
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) qb[f][kk] ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
    }
    // first key position any of the wave's rows cannot see: tiles below it need no mask
    const int wave_first_pos = ctx - nq + min(wrow0, rows - 1) / G;

    // Per row: m, the reference max the weights are taken against (scaled; the same in a
    // column's 4 lanes); o, the weighted value sums; osum, the sum of the rounded weights,
    // formed on the matrix cores as the product of P with a ones operand (every element
    // of a lane's fragment holds its row's sum).  The reference only moves, and o and
    // osum are only rescaled, when a row's max exceeds it by more than 2^RESCALE_LOG2,
    // so the weights stay in (0, 2^RESCALE_LOG2]: the result is the same up to rounding.
    constexpr float RESCALE_LOG2 = 8.f;
    const uint32_t one2 = std::is_same<T, F16>::value ? 0x3C003C00u : 0x3F803F80u;  // two 1.0s
    const u32x4 ones = u32x4{one2, one2, one2, one2};
    float m[RF];
    f32x4 o[RF][NN], osum[RF];
#pragma unroll
    for (int f = 0; f < RF; ++f) {
        m[f] = -INFINITY;
        osum[f] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NN; ++i) o[f][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    bool bad = bad_len;

    const int ntiles = (end + KT - 1) / KT;

    // Global loads of key tile t: this thread's NCH pieces of K and of V.  Each 16-key
    // group lies in one block (B >= 16); the NT block ids are looked up once per tile
    // (scalar loads).  Keys at or past `end`, and pieces of a bad block, load block 0's
    // first row instead (inside the pool) and are stored as zeros.
    struct Stage {
        u32x4 k[NCH], v[NCH];
        bool ok[NCH];
        bool full;  // every piece of the tile is valid (uniform): no zeroing needed
    };
    // Pieces 2i and 2i+1 of a thread are the same 16 bytes of two neighbouring keys.
    // Everything that depends only on the thread is computed once: a piece's key, its
    // byte offset inside its 16-key group of rows, and its LDS destinations.
    int pkey[NCH], prow[NCH], kst[NCH], vst[NCH / 2];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = threadIdx.x + (i / 2) * MW * 64;  // pair index over the tile
        const int part = c % PARTS;
        pkey[i] = 2 * (c / PARTS) + (i & 1);
        prow[i] = (pkey[i] & 15) * ROW + part * 16;
        kst[i] = pkey[i] * KROW + part * 16;
        if ((i & 1) == 0) vst[i / 2] = pkey[i] * VROW + part * 16;  // the pair's second key: + VROW
    }
    auto load_tile = [&](Stage &st, int t) {
        const int k0 = t * KT;
        // byte offset of each 16-key group's first row (uniform), -1 if not valid
        int64_t base[NT];
        bool full = k0 + KT <= end;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            base[j] = -1;
            const int kj = k0 + 16 * j;
            if (kj < end) {
                const int lb = kj >> log2_block;
                if (lb < max_blocks_per_seq) {
                    const int32_t pb = table[lb];
                    if (pb >= 0 && pb < num_blocks)
                        base[j] = (int64_t)pb * block_bytes + head_off + (int64_t)(kj & (block_size - 1)) * ROW;
                }
                if (base[j] < 0) bad = true;
            }
            full = full && base[j] >= 0;
        }
        st.full = full;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            int64_t b = base[0];
#pragma unroll
            for (int j = 1; j < NT; ++j)
                if ((pkey[i] >> 4) == j) b = base[j];
            st.ok[i] = k0 + pkey[i] < end && b >= 0;
            const int64_t off = st.ok[i] ? b + prow[i] : 0;
            st.k[i] = *(const u32x4 *)(key_cache + off);
            st.v[i] = *(const u32x4 *)(value_cache + off);
        }
    };
    // K and V rows as they are (padded strides)
    auto store_tile = [&](const Stage &st, uint8_t *buf) {
#pragma unroll
        for (int i = 0; i < NCH; i += 2) {
            u32x4 k0w = st.k[i], k1w = st.k[i + 1], v0w = st.v[i], v1w = st.v[i + 1];
            if (!st.full) {
                if (!st.ok[i]) k0w = v0w = u32x4{0, 0, 0, 0};
                if (!st.ok[i + 1]) k1w = v1w = u32x4{0, 0, 0, 0};
            }
            *(u32x4 *)(buf + kst[i]) = k0w;
            *(u32x4 *)(buf + kst[i + 1]) = k1w;
            uint8_t *vt = buf + KBYTES + vst[i / 2];
            *(u32x4 *)vt = v0w;
            *(u32x4 *)(vt + VROW) = v1w;
        }
    };
    // V^T operand reads: d = 16 nn + n, keys of group g = 8h + q (+4): the swizzle of
    // d depends on nn only, so a lane needs one base per swizzle value
    // ds_read_b64_tr_b16 (checked on gfx950): within each 16-lane group, lane j receives
    // element j % 4 of the 8-byte reads of lanes 4k + j / 4, k = 0..3.  Lane (n, q) reads
    // row 4q + n / 4, columns 16 nn + 4 (n % 4) .. +3, so lane (n, q) receives
    // V[keys 4q .. 4q + 3][d = 16 nn + n]: the V^T operand's k order.
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    const int vrd0 = (4 * q + (n >> 2)) * VROW + 8 * (n & 3);
    auto compute_tile = [&](const uint8_t *buf, int t) {
        const int k0 = t * KT;
        // scores S^T: lane holds keys k0 + 16 tt + 4 q + i of row n of each fragment
        float sc[RF][NT][4];
        if (PA_MQ_PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            f32x4 acc[RF];
#pragma unroll
            for (int f = 0; f < RF; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                const u32x4 ka = *(const u32x4 *)(buf + (16 * tt + n) * KROW + (32 * kk + 8 * q) * 2);
#pragma unroll
                for (int f = 0; f < RF; ++f) acc[f] = Mma<T>::run(ka, qb[f][kk], acc[f]);
            }
#pragma unroll
            for (int f = 0; f < RF; ++f)
#pragma unroll
                for (int i = 0; i < 4; ++i) sc[f][tt][i] = acc[f][i];
        }
        if (PA_MQ_PRIO) __builtin_amdgcn_s_setprio(0);
        // V^T operand reads for this tile (see below), issued before the softmax
        auto read_v = [&](int nn, int h) -> u32x4 {
            const uint8_t *r0 = buf + KBYTES + vrd0 + (32 * h) * VROW + 32 * nn;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(r0));
            const s16x4 hi =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(r0 + 16 * VROW));
            const uint2 lw = __builtin_bit_cast(uint2, lo), hw = __builtin_bit_cast(uint2, hi);
            return u32x4{lw.x, lw.y, hw.x, hw.y};
        };
        u32x4 vpre[PA_MQ_VPREFETCH ? NN : 1][NH];
        if (PA_MQ_VPREFETCH) {
#pragma unroll
            for (int nn = 0; nn < (PA_MQ_VPREFETCH ? NN : 1); ++nn)
#pragma unroll
                for (int h = 0; h < NH; ++h) vpre[nn][h] = read_v(nn, h);
        }
        if (k0 + KT - 1 > wave_first_pos) {  // a diagonal tile: mask keys past each row
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                for (int f = 0; f < RF; ++f)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (k0 + 16 * tt + 4 * q + i > pos[f]) sc[f][tt][i] = -INFINITY;
        }
        // P^T operands per 32-key half h: k slot j < 4 -> key 32h + 4q + j,
        // j >= 4 -> key 32h + 16 + 4q + j - 4
        u32x4 pb[RF][NH];
        float alpha[RF];
        bool grow = false;
#pragma unroll
        for (int f = 0; f < RF; ++f) {
            float cm = sc[f][0][0];
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) cm = fmaxf(cm, sc[f][tt][i]);
            cm = max_over_column(cm);
            const float mt = cm * sl;  // this tile's max of the row (-inf: nothing visible)
            const bool g = mt > m[f] + RESCALE_LOG2;
            alpha[f] = g ? fast_exp2(m[f] - mt) : 1.f;
            m[f] = g ? mt : m[f];
            grow |= g;
            const float ms = m[f] == -INFINITY ? 0.f : m[f];
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                uint32_t pk[4];
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int i = 0; i < 4; i += 2)
                        pk[2 * u + i / 2] = round2<T>(fast_exp2(fmaf(sc[f][2 * h + u][i], sl, -ms)),
                                                      fast_exp2(fmaf(sc[f][2 * h + u][i + 1], sl, -ms)));
                pb[f][h] = u32x4{pk[0], pk[1], pk[2], pk[3]};
            }
        }
        // V^T operand per 16-row d fragment and half: keys 32h + 4q..+3 and 32h + 16 + 4q..+3
        // of d = 16 nn + n (two transpose reads of the V rows, read_v), shared by the fragments
        // rescale only when some row's reference moved (otherwise every alpha is 1)
        if (__any(grow)) {
#pragma unroll
            for (int f = 0; f < RF; ++f) {
                osum[f] *= alpha[f];
#pragma unroll
                for (int nn = 0; nn < NN; ++nn) o[f][nn] *= alpha[f];
            }
        }
        if (PA_MQ_PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int f = 0; f < RF; ++f) osum[f] = Mma<T>::run(ones, pb[f][h], osum[f]);
#pragma unroll
        for (int nn = 0; nn < NN; ++nn) {
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                // keys 32h + 4q .. +3, then 32h + 16 + 4q .. +3, of d = 16 nn + n
                const u32x4 va = PA_MQ_VPREFETCH ? vpre[PA_MQ_VPREFETCH ? nn : 0][h] : read_v(nn, h);
#pragma unroll
                for (int f = 0; f < RF; ++f) o[f][nn] = Mma<T>::run(va, pb[f][h], o[f][nn]);
            }
        }
        if (PA_MQ_PRIO) __builtin_amdgcn_s_setprio(0);
    };

    // While tile t is used from LDS, tile t + 1 is being loaded into registers (and with
    // PA_MQ_DEPTH 2, tile t + 2 as well).  Loads past the last tile read block 0's first
    // row (all masked) instead of being skipped, so the compiler's waits stay exact.
    if (PA_MQ_DEPTH == 1 && ntiles > 0) {
        Stage st;
        load_tile(st, 0);
        store_tile(st, lds);
        __syncthreads();
        for (int t = 0; t < ntiles; ++t) {
            load_tile(st, t + 1);
            if (t * KT < wave_end) compute_tile(lds + (t & 1) * BUF, t);
            if (t + 1 < ntiles) store_tile(st, lds + ((t + 1) & 1) * BUF);
            __syncthreads();
        }
    } else if (ntiles > 0) {
        Stage sa, sb;
        load_tile(sa, 0);
        load_tile(sb, 1);
        store_tile(sa, lds);
        __syncthreads();
        // next: the stage holding tile t + 1; spare: free, receives tile t + 2
        auto step = [&](Stage &next, Stage &spare, int t) {
            load_tile(spare, t + 2);
            if (t * KT < wave_end) compute_tile(lds + (t & 1) * BUF, t);
            if (t + 1 < ntiles) store_tile(next, lds + ((t + 1) & 1) * BUF);
            __syncthreads();
        };
        for (int t = 0; t < ntiles; t += 2) {
            step(sb, sa, t);
            if (t + 1 < ntiles) step(sa, sb, t + 1);
        }
    }

    __shared__ int sm_bad;
    if (threadIdx.x == 0) sm_bad = 0;
    __syncthreads();
    if (bad) sm_bad = 1;
    __syncthreads();
    const bool any_bad = sm_bad != 0;
    // each wave writes its own rows; the normaliser of a row sums its column's 4 lanes
#pragma unroll
    for (int f = 0; f < RF; ++f) {
        const float l = osum[f][0];
        if (!io_ok[f]) continue;
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const int64_t obase = (orow[f] * num_q_heads + kvh * G + gh[f]) * D;
#pragma unroll
        for (int nn = 0; nn < NN; ++nn)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float ov = any_bad ? NAN : o[f][nn][i] * inv;
                store_out<T>(out, obase + 16 * nn + 4 * q + i, ov);
            }
    }
}

template <typename T, int D, int G>
int launch_t(const DecodeArgs &a) {
    const int tiles = (a.max_query_len * G + ROWS - 1) / ROWS;
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
